"""GPU parity of the bias epilogue (``w4a16_gemm_bias``) against the oracle.

The bias is ``[N]`` in the activation dtype, added in fp32 to the product
before the one cast, indexed by output column (PR #40977 "RDNA hybrid
W4A16", Code section; its Review section reports the prior kernel's bias
indexed by a row count). Every epilogue that writes the output is covered:
decode without and with a K split (last-arrival sum), prefill without a
split and the prefill split reduction. Each case first checks which launch
the selector picks, so a change of plan cannot silently skip an epilogue.
"""
import numpy as np
import pytest
import torch

import oracle as O
from weight_only_int4_unpack_amd import synthetic
from weight_only_int4_unpack_amd import w4a16 as W
from helpers import assert_within_tolerance, bits_to_dev, dev_to_bits, make_problem, random_problem, TORCH_DT

pytestmark = pytest.mark.gpu

# (M, K, N, G, dtype, zero points, expected route, expected K splits > 1)
CASES = [
    (4, 256, 512, 128, "fp16", False, W.ROUTE_DECODE, False),     # decode, one split
    (1, 4096, 4096, 32, "fp16", True, W.ROUTE_DECODE, True),      # decode, last-arrival sum
    (5, 4096, 4104, 32, "bf16", True, W.ROUTE_DECODE, True),      # N % 32 != 0: no ring
    (9, 4096, 4096, 32, "bf16", True, W.ROUTE_PREFILL, True),     # few rows: ring, K split
    (8, 2112, 520, 64, "fp16", True, W.ROUTE_DECODE, True),       # ragged N
    (2000, 256, 4104, 64, "fp16", True, W.ROUTE_PREFILL, False),  # prefill, ragged N and M
    (300, 512, 264, 32, "fp16", False, W.ROUTE_PREFILL, True),    # prefill split, ragged N
    (16, 4096, 4096, 32, "fp16", True, W.ROUTE_PREFILL, True),    # prefill split reduction
    (64, 1024, 768, 1024, "bf16", True, W.ROUTE_PREFILL, True),   # per-channel
]
IDS = [f"M{c[0]}_K{c[1]}_N{c[2]}_G{c[3]}_{c[4]}" for c in CASES]


def _check_plan(p, route, split):
    pl = W.plan(p.M, p.K, p.N, p.G, p.qz is not None, TORCH_DT[p.dtype])
    assert pl.route == route and (pl.splits > 1) == split, pl.as_dict()


def _bias(N, dtype, seed):
    return synthetic.random_bits((N,), dtype, seed, 2.0)


@pytest.mark.parametrize("M,K,N,G,dtype,zp,route,split", CASES, ids=IDS)
def test_bias_parity(M, K, N, G, dtype, zp, route, split):
    p = random_problem(M, K, N, G, dtype, zp, seed=40 + M)
    _check_plan(p, route, split)
    bias = _bias(N, dtype, 41 + M)
    got = dev_to_bits(W.gemm(p.a, p.b_q_d, p.s, p.qz_d, G, 8, bias=bits_to_dev(bias, dtype)))
    want = O.gemm(p.a_bits, p.b_q, p.s_bits, p.qz, G, 8, dtype, bias_bits=bias)
    assert_within_tolerance(got, want, dtype, "bias")
    # the bias really entered: without it the outputs move
    nob = dev_to_bits(p.gpu_gemm())
    assert not np.array_equal(got, nob)


@pytest.mark.parametrize("M,K,N,G,dtype,zp,route,split", CASES, ids=IDS)
def test_bias_alone_bitwise(M, K, N, G, dtype, zp, route, split):
    # zero activations: the product is exactly 0, the output is the bias
    p = random_problem(M, K, N, G, dtype, zp, seed=50 + M)
    _check_plan(p, route, split)
    bias = _bias(N, dtype, 51 + M)
    a0 = torch.zeros_like(p.a)
    got = dev_to_bits(W.gemm(a0, p.b_q_d, p.s, p.qz_d, G, 8, bias=bits_to_dev(bias, dtype)))
    assert np.array_equal(got, np.broadcast_to(bias, (M, N)))


@pytest.mark.parametrize("M,K,N,G,dtype,zp,route,split", CASES, ids=IDS)
def test_bias_exact_integer_bitwise(M, K, N, G, dtype, zp, route, split):
    # A in {-1, 0, 1} (16 nonzeros per row), S = 2^-4, bias in 2^-4 steps:
    # every partial sum is exact in fp32, so any summation order gives the
    # oracle's bits
    rng = np.random.default_rng(60 + M)
    a = np.zeros((M, K), np.float32)
    for m in range(M):
        idx = rng.choice(K, size=16, replace=False)
        a[m, idx] = rng.choice([-1.0, 1.0], size=16)
    d = {"a_bits": O.rne_bits(a, dtype),
         "q": rng.integers(0, 16, size=(K, N), dtype=np.uint8),
         "s_bits": O.rne_bits(np.full((K // G, N), 1.0 / 16, np.float32), dtype),
         "z": rng.integers(0, 16, size=(K // G, N), dtype=np.uint8) if zp else None}
    p = make_problem(d, M, K, N, G, dtype)
    _check_plan(p, route, split)
    bias = O.rne_bits(rng.integers(-64, 65, size=N).astype(np.float32) / 16, dtype)
    got = dev_to_bits(W.gemm(p.a, p.b_q_d, p.s, p.qz_d, G, 8, bias=bits_to_dev(bias, dtype)))
    want = O.gemm(p.a_bits, p.b_q, p.s_bits, p.qz, G, 8, dtype, bias_bits=bias)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("M,K,N,G,dtype,zp,route,split", CASES, ids=IDS)
def test_bias_read_in_bounds(M, K, N, G, dtype, zp, route, split):
    # the bias sits between NaN canaries; a read past either end of [N] would
    # turn outputs into NaN
    p = random_problem(M, K, N, G, dtype, zp, seed=70 + M)
    bias = _bias(N, dtype, 71 + M)
    guard = 64  # elements: keeps the bias 16-byte aligned
    buf = torch.full((guard + N + guard,), float("nan"), dtype=TORCH_DT[dtype], device="cuda")
    buf[guard:guard + N] = bits_to_dev(bias, dtype)
    got = dev_to_bits(W.gemm(p.a, p.b_q_d, p.s, p.qz_d, G, 8, bias=buf[guard:guard + N]))
    assert not np.isnan(O.to_f32(got, dtype)).any()
    want = O.gemm(p.a_bits, p.b_q, p.s_bits, p.qz, G, 8, dtype, bias_bits=bias)
    assert_within_tolerance(got, want, dtype, "bias between canaries")


def test_bias_one_hot_columns():
    # a one-hot bias with zero activations lights exactly its column
    M, K, N, G = 5, 4096, 4096, 32
    p = random_problem(M, K, N, G, "fp16", True, seed=80)
    a0 = torch.zeros_like(p.a)
    for n0 in (0, 255, 256, N - 1):
        b = torch.zeros(N, dtype=torch.float16, device="cuda")
        b[n0] = 1.0
        got = W.gemm(a0, p.b_q_d, p.s, p.qz_d, G, 8, bias=b).float().cpu()
        want = torch.zeros(M, N)
        want[:, n0] = 1.0
        assert torch.equal(got, want), n0


def test_bias_zero_equals_no_bias_and_inputs_untouched():
    for M in (5, 100):
        p = random_problem(M, 1024, 512, 64, "bf16", True, seed=90 + M)
        zero = torch.zeros(p.N, dtype=torch.bfloat16, device="cuda")
        snap = [t.clone() for t in (p.a, p.b_q_d, p.s, p.qz_d, zero)]
        got = dev_to_bits(W.gemm(p.a, p.b_q_d, p.s, p.qz_d, p.G, 8, bias=zero))
        assert np.array_equal(got, dev_to_bits(p.gpu_gemm()))
        torch.cuda.synchronize()
        for t, s in zip((p.a, p.b_q_d, p.s, p.qz_d, zero), snap):
            assert torch.equal(t, s)


def test_bias_argument_checks():
    p = random_problem(4, 256, 512, 128, "fp16", False, seed=95)
    with pytest.raises(ValueError):
        W.gemm(p.a, p.b_q_d, p.s, None, 128, 8, bias=torch.zeros(p.N - 8, dtype=torch.float16,
                                                                  device="cuda"))
    with pytest.raises(ValueError):
        W.gemm(p.a, p.b_q_d, p.s, None, 128, 8, bias=torch.zeros(p.N, dtype=torch.bfloat16,
                                                                  device="cuda"))
    with pytest.raises(W.W4A16Error) as e:   # misaligned: the library reports ALIGN
        buf = torch.zeros(p.N + 8, dtype=torch.float16, device="cuda")
        W.gemm(p.a, p.b_q_d, p.s, None, 128, 8, bias=buf[1:p.N + 1])
    assert e.value.status == W.ERR_ALIGN
