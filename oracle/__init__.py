"""CPU oracle of the weight-only int4 GEMM (test infrastructure only).

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` may import this package. The HIP library never does.
"""
from .w4a16_oracle import *  # noqa: F401,F403
from .w4a16_oracle import (F16, BF16, DTYPES, SUPPORTED_GROUP_SIZES, TOLERANCE,
                           to_f32, rne_bits, unpack_int4, pack_int4, check,
                           dequant_fp32, dequant_tile, gemm_f32, gemm,
                           bruteforce_f64, within_tolerance)
