"""The seeded input generator: determinism, prefix stability, encodings."""
import numpy as np
import torch

import synth


def test_deterministic_and_prefix_stable():
    a = synth.normal_f32(123, 600, 37, 0.02)
    b = synth.normal_f32(123, 600, 37, 0.02)
    assert np.array_equal(a, b)
    c = synth.normal_f32(123, 10, 37, 0.02)
    assert np.array_equal(a[:10], c)
    assert not np.array_equal(a, synth.normal_f32(124, 600, 37, 0.02))
    assert abs(a.std() - 0.02) < 0.001


def test_bf16_bits_match_torch():
    x = synth.normal_f32(5, 300, 300, 3.0)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(synth.bf16_bits(x), ref)


def test_fp8_rows_scale_and_range():
    w = synth.weight(7, 50, 200, synth.FP8)
    assert w.data.dtype == np.uint8 and w.scale.shape == (50,)
    vals = torch.from_numpy(w.data).view(torch.float8_e4m3fn).float().numpy()
    assert np.isfinite(vals).all()
    assert (np.abs(vals).max(axis=1) == 448.0).all()  # every row reaches full scale
    x = synth.normal_f32(7, 50, 200, 0.02)
    err = np.abs(vals * w.scale[:, None] - x)
    assert (err <= np.abs(x) * 2 ** -4 + w.scale[:, None] * 2 ** -9 + 1e-12).all()


def test_seed_formula():
    assert synth.seed_for(2, 3, 1) == 20301
    assert synth.seed_for(3, 15, 50) == 31550
