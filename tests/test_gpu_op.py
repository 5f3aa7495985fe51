"""GPU tests of the opaque operator ``torch.ops.w4a16.gemm``.

The operator runs the same library call as the binding (bitwise equal), stays
within tolerance of the oracle, passes torch's operator checks, and under a
graph compiler keeps choosing its launch from the runtime M: one compiled
function called with decode and prefill sizes gives what the eager calls give
(PR #51453 "Register the Triton W4A16 GEMM as a custom op", Motivation: a tile
choice frozen at trace time slowed decode).
"""
import numpy as np
import pytest
import torch

import oracle as O
from weight_only_int4_unpack_amd import op
from weight_only_int4_unpack_amd import w4a16 as W
from helpers import assert_within_tolerance, bits_to_dev, dev_to_bits, random_problem, TORCH_DT

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M,K,N,G,dtype,zp", [
    (1, 4096, 4096, 32, "fp16", True),
    (5, 5120, 2048, 128, "bf16", False),
    (300, 512, 264, 32, "fp16", False),
])
def test_op_equals_binding_and_oracle(M, K, N, G, dtype, zp):
    p = random_problem(M, K, N, G, dtype, zp, seed=110 + M)
    got = dev_to_bits(op.gemm(p.a, p.b_q_d, p.s, p.qz_d, G))
    assert np.array_equal(got, dev_to_bits(p.gpu_gemm()))
    assert_within_tolerance(got, p.oracle_gemm(), dtype, "op")
    bias = O.rne_bits(np.linspace(-1, 1, N).astype(np.float32), dtype)
    got = dev_to_bits(op.gemm(p.a, p.b_q_d, p.s, p.qz_d, G, 8, bits_to_dev(bias, dtype)))
    want = O.gemm(p.a_bits, p.b_q, p.s_bits, p.qz, G, 8, dtype, bias_bits=bias)
    assert_within_tolerance(got, want, dtype, "op with bias")


def test_opcheck():
    p = random_problem(4, 256, 512, 128, "fp16", True, seed=120)
    torch.library.opcheck(torch.ops.w4a16.gemm.default, (p.a, p.b_q_d, p.s, p.qz_d, 128, 8, None),
                          test_utils=("test_schema", "test_faketensor"))


def test_compiled_call_routes_on_runtime_m():
    K, N, G = 1024, 2048, 64
    fn = torch.compile(lambda a, b_q, s, z: op.gemm(a, b_q, s, z, G), backend="aot_eager",
                       dynamic=True, fullgraph=True)
    for M in (1, 5, 64, 700):
        p = random_problem(M, K, N, G, "bf16", True, seed=130)
        got = dev_to_bits(fn(p.a, p.b_q_d, p.s, p.qz_d))
        assert np.array_equal(got, dev_to_bits(p.gpu_gemm())), M
    routes = {W.plan(M, K, N, G, True, TORCH_DT["bf16"]).route for M in (1, 5, 64, 700)}
    assert routes == {W.ROUTE_DECODE, W.ROUTE_PREFILL}


def test_kpacked_op_equals_binding_and_oracle():
    M, K, N, G, dtype = 5, 1024, 520, 128, "bf16"
    p = random_problem(M, K, N, G, dtype, True, seed=130)
    d_q = O.unpack_int4(p.b_q).T                      # [N, K] uint4 of the same weights
    w = torch.from_numpy(O.pack_int4_kshuffle(np.ascontiguousarray(d_q))).cuda()
    s_nk = np.ascontiguousarray(p.s_bits.T)
    z_nk = np.ascontiguousarray(O.unpack_int4(p.qz).T)
    s_d = bits_to_dev(s_nk, dtype)
    z_d = torch.from_numpy(z_nk).cuda()
    got = dev_to_bits(op.gemm_kpacked(p.a, w, s_d, z_d, G))
    assert np.array_equal(got, dev_to_bits(W.gemm_kpacked(p.a, w, s_d, z_d, G)))
    want = O.gemm_kpacked(p.a_bits, O.pack_int4_kshuffle(np.ascontiguousarray(d_q)), s_nk, z_nk,
                          G, 8, dtype)
    assert_within_tolerance(got, want, dtype, "kpacked op")
    torch.library.opcheck(torch.ops.w4a16.gemm_kpacked.default, (p.a, w, s_d, z_d, G, 8, None),
                          test_utils=("test_schema", "test_faketensor"))
