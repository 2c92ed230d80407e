"""Helpers for the GPU parity tests: moving synthetic inputs to the device and
the benchmark spec's tolerance check.  No arithmetic of the method lives here."""
from __future__ import annotations

import sys

import numpy as np
import torch

DEV = torch.device("cuda:0")


def note(msg: str) -> None:
    """Name the case before a GPU step, flushed, so a failing run says where it was."""
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def u8(arr: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(arr).view(np.uint8).reshape(-1).copy()).to(DEV)


def bf16(bits: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(bits, dtype=np.uint16)
    return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16).to(DEV)


def f32(arr: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32).copy()).to(DEV)


def bits(t: torch.Tensor) -> np.ndarray:
    """BF16 device tensor -> numpy uint16 bit patterns."""
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def values(t: torch.Tensor) -> np.ndarray:
    """Device tensor (bf16 or fp32) -> float64 numpy."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def row_errors(y: np.ndarray, y_ref: np.ndarray) -> tuple[float, np.ndarray]:
    """max over rows of max|y - y_ref| / max(1, max|y_ref| of the row); and the per-row ratios."""
    y = np.asarray(y, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    bound = np.maximum(1.0, np.abs(y_ref).max(axis=1))
    ratio = np.abs(y - y_ref).max(axis=1) / bound
    return float(ratio.max()), ratio


def assert_close_rows(y, y_ref, rel: float = 1e-2, what: str = "") -> float:
    """The bar: max|y - y_ref| <= rel * max(1, max|y_ref| of the row), every row."""
    y = np.asarray(y, np.float64)
    assert y.shape == np.shape(y_ref), (y.shape, np.shape(y_ref))
    assert np.isfinite(y).all(), f"{what}: non-finite outputs"
    worst, _ = row_errors(y, y_ref)
    assert worst <= rel, f"{what}: worst row error {worst:.3e} > {rel}"
    return worst


def weight_dev(w) -> tuple[torch.Tensor, torch.Tensor | None]:
    """synth.Weight -> (raw bytes on device, fp32 scales on device or None)."""
    return u8(w.raw()), (f32(w.scale) if w.scale is not None else None)
