"""MI355X (gfx950) weight-only int4 GEMM: C[M,N] = A[M,K] . dequant(B).

The compute path is the HIP library ``libw4a16.so`` built from ``csrc/``;
``w4a16`` is its thin ctypes binding. The library is loaded on first use and
a missing build raises immediately: there is no fallback path.
"""
from . import synthetic  # noqa: F401  (random inputs only; no arithmetic)
from . import w4a16  # noqa: F401  (binding; loads the library on first call)
from . import op  # noqa: F401  (registers torch.ops.w4a16.gemm; calls go through the binding)
