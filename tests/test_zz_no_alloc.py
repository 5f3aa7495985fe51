"""The entry point that allocates nothing (``w4a16_gemm_noalloc``) against
the allocating one (``w4a16_gemm``), through the C ABI.

Its scratch is a fixed device array shared by every call on the GPU and
keeping the last call's contents, so the test makes calls in a row with a
smaller problem second: the second must not see the first one's partials or
counters. Each output must equal ``w4a16_gemm``'s bit for bit (the same
kernels with deterministic reductions) and lie within 2e-2 of the oracle.
Shapes split K (decode hand-off, prefill partials) so the array is used.
"""
import ctypes

import numpy as np
import pytest
import torch

from weight_only_int4_unpack_amd import w4a16 as W
from helpers import TORCH_DT, assert_within_tolerance, dev_to_bits, random_problem

pytestmark = pytest.mark.gpu

# (M, K, N, G, dtype, zero points), larger first within each sequence
SEQUENCES = [
    [(5, 5120, 17408, 128, "bf16", False), (2, 2048, 1024, 64, "fp16", True)],   # decode split-K
    [(64, 4096, 4096, 32, "fp16", True), (20, 1024, 768, 128, "bf16", False)],  # prefill K splits
    [(8, 2112, 5120, 64, "fp16", True), (1, 512, 256, 32, "bf16", True)],
]


def _existing(p, out, bias=None):
    """The allocating entry point (w4a16_gemm / w4a16_gemm_bias) on the
    current stream."""
    args = W.gemm_args(p.a, p.b_q_d, p.s, p.qz_d, p.G, 8, out)
    L = W.lib()
    st = L.w4a16_gemm(*args) if bias is None else \
        L.w4a16_gemm_bias(*args[:6], ctypes.c_void_p(bias.data_ptr()), *args[6:])
    assert st == W.OK, W.last_error()
    return out


@pytest.mark.parametrize("seq", range(len(SEQUENCES)))
def test_noalloc_two_calls_match_allocating_entry(seq):
    for i, (M, K, N, G, dtype, zp) in enumerate(SEQUENCES[seq]):
        print(f"noalloc seq {seq} call {i}: M={M} K={K} N={N} G={G} {dtype} zp={zp}", flush=True)
        p = random_problem(M, K, N, G, dtype, zp, seed=700 + 10 * seq + i)
        plan = W.plan(M, K, N, G, zp, TORCH_DT[dtype])
        assert plan.splits > 1 or i == 1 and seq == 2     # the array is used
        assert plan.workspace_bytes <= W.NOALLOC_SCRATCH_BYTES
        got = torch.empty((M, N), dtype=TORCH_DT[dtype], device="cuda")
        W.gemm_noalloc(p.a, p.b_q_d, p.s, p.qz_d, G, 8, got)
        ref = _existing(p, torch.empty_like(got))
        torch.cuda.synchronize()
        g, r = dev_to_bits(got), dev_to_bits(ref)
        assert np.array_equal(g, r), f"call {i}: {int((g != r).sum())} outputs differ"
        assert_within_tolerance(g, p.oracle_gemm(), dtype, f"noalloc call {i}")


def test_noalloc_bias_and_repeat():
    p = random_problem(4, 4096, 2048, 128, "bf16", False, seed=760)
    bias = torch.randn(2048, device="cuda").to(torch.bfloat16)
    ref = _existing(p, torch.empty((4, 2048), dtype=torch.bfloat16, device="cuda"), bias)
    for _ in range(3):
        got = torch.empty_like(ref)
        W.gemm_noalloc(p.a, p.b_q_d, p.s, None, 128, 8, got, bias=bias)
        torch.cuda.synchronize()
        assert torch.equal(got, ref)


def test_noalloc_refuses_more_than_the_array():
    # a decode split-K problem whose partials exceed the fixed array: refused
    # before anything is launched
    M, K, N = 8, 16384, 131072
    need = W.workspace_bytes(M, K, N, 128, torch.bfloat16)
    assert need > W.NOALLOC_SCRATCH_BYTES
    fake = ctypes.c_void_p(0x10000)
    st = W.lib().w4a16_gemm_noalloc(fake, fake, fake, None, 128, 8, None, fake, M, K, N, W.BF16,
                                    None)
    assert st == W.ERR_WORKSPACE and "fixed array" in W.last_error()
