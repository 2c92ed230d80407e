"""CPU oracle for the flat-weight reassembly path -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct NumPy (float64) restatement of what the
path computes, written from the weight-sharding page (zdszero.github.io,
"weight_sharding"), the vLLM PR #50656 report (prhub.com.cn) and the
sharded-matrices notes (copecc.github.io, "HowToScaleYourModel / Sharded
Matrices").  It shares no code with the HIP library and imports nothing
from it.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path never calls it and
has no CPU fallback.

Modules
-------
layout      flat layout plan, pack, reassembly, zero-copy views
numerics    BF16 / FP8-E4M3FN decoding, BF16 round-to-nearest-even, SiLU
gemm        projection, gate_up -> SiLU*up -> down MLP, sharded-matmul cases
accounting  slot memory and transfer-byte closed forms
scheduler   lookahead / ping-pong launch-and-wait sequence and its checker

Every function here is pinned by a CPU test in ``tests/test_oracle_*.py``.
"""

from . import accounting, gemm, layout, numerics, scheduler  # noqa: F401
