"""MI355X (gfx950) weight-only int4 GEMM: C[M,N] = A[M,K] . dequant(B).

The compute path is the HIP library ``libw4a16.so`` built from ``csrc/``;
``w4a16`` is its thin ctypes binding. The library is loaded on first use and
a missing build raises immediately: there is no fallback path.
"""
from . import synthetic  # noqa: F401  (random inputs only; no arithmetic)


def __getattr__(name):
    # Load the binding lazily so that ``synthetic`` (and the CPU tests of the
    # oracle that use it) import without a built library.
    if name == "w4a16":
        from . import w4a16 as mod
        return mod
    raise AttributeError(name)
