"""fp64 CPU oracle for rotation + Lloyd-Max weight quantization and its fused linear layers.

TEST INFRASTRUCTURE ONLY. Nothing in the product path (the HIP library and its Python
binding) may import, call, link or execute this package. Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` use it.

The oracle is plain, slow and written to be checked by eye against the method's
description ("How it works" page of turboquant-mlx, sections "Quantizing a weight, with
no data", "The ternary tier (1.58 bits)" and "Running a quantized layer"). It shares no
code, table or constant generator with the HIP library.

Modules
  codebook  Lloyd iteration on the N(0,1) density -> centroids, thresholds, distortion
  hadamard  Sylvester / Paley Hadamard matrices, Kronecker H_K, SplitMix64 signs, rotation
  encode    rotate -> group RMS -> fp16 scale -> snap -> pack (bits or trits), unpack, dequant
  ops       qmv, gather_qmv, multi_gather_qmv, gather_qmm by their definitions

Parity pins live in ``tests/test_oracle_*.py``. Every function here is pinned by at least
one check that does not re-use its own formula; see the test files for which.
"""

from . import codebook, hadamard, encode, ops  # noqa: F401
