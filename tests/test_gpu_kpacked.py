"""GPU parity of the K-packed GEMM (``w4a16_gemm_kpacked``) against the oracle.

Weights are int32 ``[N, K/8]`` in ExLlama nibble order, scales and zero points
``[N, K/G]`` (PR #40977 "RDNA hybrid W4A16", Impl. item 4 and Code section).
The kernel takes one of three numerics paths: G a multiple of 128 (or G == K)
folds the scale into fp32 round sums; fp16 with G = 32, 64 multiplies
rounded tiles (2^-11 relative per weight); bf16 with G = 32, 64 keeps the
exact operand and folds per 32-K chunk, since rounded bf16 tiles leave the
tolerance over a long K (pinned on the CPU in test_oracle.py).
Cases cover both paths in both dtypes, ragged K rounds (K % 128 != 0), ragged
N (N % 16 != 0), several 16-row blocks, per-channel groups and the full-size
decode shape on sampled columns. The activation rows of a 16-row block are
staged in LDS when they fit in 60 KB (M = 6 at K = 5120 does not; 16 rows at
K = 1856 do), so both operand paths are covered.
"""
import numpy as np
import pytest
import torch

import oracle as O
from weight_only_int4_unpack_amd import synthetic
from weight_only_int4_unpack_amd import w4a16 as W
from helpers import assert_within_tolerance, bits_to_dev, dev_to_bits

pytestmark = pytest.mark.gpu

# (M, K, N, G, dtype, zero points)
CASES = [
    (4, 256, 512, 128, "fp16", False),      # tiny, fold
    (3, 256, 40, 128, "bf16", True),        # fold bf16 with zero points, ragged N
    (8, 2112, 5120, 64, "fp16", True),      # tile path, K = 16.5 rounds
    (1, 4096, 4096, 32, "fp16", True),      # tile path, G = 32
    (6, 4096, 4096, 32, "bf16", True),      # bf16 tile path
    (16, 640, 48, 64, "bf16", False),       # bf16 tile, one full row block
    (17, 1024, 100, 1024, "fp16", True),    # per-channel, two row blocks, ragged N
    (33, 2112, 72, 2112, "bf16", False),    # per-channel, partial last round, three row blocks
    (2, 96, 24, 32, "fp16", True),          # one partial round (three chunks)
    (5, 512, 1000, 128, "bf16", False),     # fold, N % 16 = 8
    (6, 5120, 1040, 128, "bf16", False),    # rows just over the LDS staging limit: global loads
    (16, 1856, 48, 64, "fp16", True),       # 16 staged rows just under the limit
]
IDS = [f"M{c[0]}_K{c[1]}_N{c[2]}_G{c[3]}_{c[4]}_{'zp' if c[5] else 'sym'}" for c in CASES]


def _problem(M, K, N, G, dtype, has_zp, seed):
    d = synthetic.draw(M, K, N, G, dtype, has_zp, family=700 + seed)
    w = O.pack_int4_kshuffle(np.ascontiguousarray(d["q"].T))
    s_nk = np.ascontiguousarray(d["s_bits"].T)
    z_nk = None if d["z"] is None else np.ascontiguousarray(d["z"].T).astype(np.uint8)
    return d, w, s_nk, z_nk


def _run(d, w, s_nk, z_nk, G, dtype, bias=None, a_bits=None):
    a = bits_to_dev(d["a_bits"] if a_bits is None else a_bits, dtype)
    zd = None if z_nk is None else torch.from_numpy(z_nk).cuda()
    bd = None if bias is None else bits_to_dev(bias, dtype)
    out = W.gemm_kpacked(a, torch.from_numpy(w).cuda(), bits_to_dev(s_nk, dtype), zd, G, 8,
                         bias=bd)
    torch.cuda.synchronize()
    return dev_to_bits(out)


@pytest.mark.parametrize("M,K,N,G,dtype,zp", CASES, ids=IDS)
def test_kpacked_parity(M, K, N, G, dtype, zp):
    d, w, s_nk, z_nk = _problem(M, K, N, G, dtype, zp, M + K % 97)
    got = _run(d, w, s_nk, z_nk, G, dtype)
    want = O.gemm_kpacked(d["a_bits"], w, s_nk, z_nk, G, 8, dtype)
    assert_within_tolerance(got, want, dtype, "kpacked")


@pytest.mark.parametrize("M,K,N,G,dtype,zp", CASES[:8], ids=IDS[:8])
def test_kpacked_exact_integer_bitwise(M, K, N, G, dtype, zp):
    # A in {-1, 0, 1} (12 nonzeros per row) and S = 2^-4: every product and
    # partial sum is exact in fp32 on either numerics path, so the output
    # bits must equal the oracle's
    rng = np.random.default_rng(80 + M)
    a = np.zeros((M, K), np.float32)
    for m in range(M):
        idx = rng.choice(K, size=12, replace=False)
        a[m, idx] = rng.choice([-1.0, 1.0], size=12)
    a_bits = O.rne_bits(a, dtype)
    q = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    z_nk = rng.integers(0, 16, size=(N, K // G), dtype=np.uint8) if zp else None
    s_nk = O.rne_bits(np.full((N, K // G), 0.0625, np.float32), dtype)
    w = O.pack_int4_kshuffle(q)
    got = _run({"a_bits": a_bits}, w, s_nk, z_nk, G, dtype)
    want = O.gemm_kpacked(a_bits, w, s_nk, z_nk, G, 8, dtype)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("M,K,N,G,dtype,zp", [CASES[1], CASES[3], CASES[6]],
                         ids=[IDS[1], IDS[3], IDS[6]])
def test_kpacked_bias(M, K, N, G, dtype, zp):
    d, w, s_nk, z_nk = _problem(M, K, N, G, dtype, zp, 5 + M)
    bias = synthetic.random_bits((N,), dtype, 90 + M, 2.0)
    got = _run(d, w, s_nk, z_nk, G, dtype, bias=bias)
    want = O.gemm_kpacked(d["a_bits"], w, s_nk, z_nk, G, 8, dtype, bias_bits=bias)
    assert_within_tolerance(got, want, dtype, "kpacked bias")
    alone = _run(d, w, s_nk, z_nk, G, dtype, bias=bias, a_bits=np.zeros_like(d["a_bits"]))
    assert np.array_equal(alone, np.broadcast_to(bias, (M, N)))


# Long K with small groups and zero points: where rounded bf16 tiles fail
# (K = 5120, 8192, 16384 at G = 32 and 64), in both dtypes, on every column.
LONG_K = [(M, K, N, G, dt) for (M, K, N) in ((8, 5120, 1024), (16, 8192, 512), (16, 16384, 256))
          for G in (32, 64) for dt in ("bf16", "fp16")]


@pytest.mark.parametrize("M,K,N,G,dtype", LONG_K,
                         ids=[f"M{c[0]}_K{c[1]}_N{c[2]}_G{c[3]}_{c[4]}" for c in LONG_K])
def test_kpacked_small_groups_long_k(M, K, N, G, dtype):
    d, w, s_nk, z_nk = _problem(M, K, N, G, dtype, True, 30 + K // 1024 + G)
    got = _run(d, w, s_nk, z_nk, G, dtype)
    want = O.gemm_kpacked(d["a_bits"], w, s_nk, z_nk, G, 8, dtype)
    assert_within_tolerance(got, want, dtype, f"kpacked K={K} G={G}")


@pytest.mark.parametrize("M", [1, 5])
def test_kpacked_full_size_decode_sampled(M):
    # the decode shape at full size (K = 5120, N = 17408, bf16, G = 128):
    # every row, 512 sampled columns including both ends
    K, N, G, dtype = 5120, 17408, 128, "bf16"
    d, w, s_nk, z_nk = _problem(M, K, N, G, dtype, False, 60 + M)
    got = _run(d, w, s_nk, z_nk, G, dtype)
    cols = np.unique(np.concatenate([[0, 15, 16, N - 1], np.random.default_rng(M).choice(N, 508)]))
    want = O.gemm_kpacked(d["a_bits"], w, s_nk, z_nk, G, 8, dtype, cols=cols)
    assert_within_tolerance(got[:, cols], want, dtype, "kpacked full size")


def test_kpacked_agrees_with_n_packed_route():
    # the same weights in both layouts through both entry points
    M, K, N, G, dtype = 5, 2048, 1024, 128, "fp16"
    d, w, s_nk, z_nk = _problem(M, K, N, G, dtype, True, 3)
    got_k = _run(d, w, s_nk, z_nk, G, dtype)
    a = bits_to_dev(d["a_bits"], dtype)
    got_n = dev_to_bits(W.gemm(a, torch.from_numpy(O.pack_int4(d["q"])).cuda(),
                               bits_to_dev(d["s_bits"], dtype),
                               torch.from_numpy(O.pack_int4(d["z"])).cuda(), G, 8))
    want = O.gemm(d["a_bits"], O.pack_int4(d["q"]), d["s_bits"], O.pack_int4(d["z"]), G, 8, dtype)
    assert_within_tolerance(got_k, want, dtype, "kpacked")
    assert_within_tolerance(got_n, want, dtype, "n-packed")


def test_kpacked_m_zero_and_errors():
    a = torch.zeros((0, 256), dtype=torch.float16, device="cuda")
    w = torch.zeros((64, 32), dtype=torch.int32, device="cuda")
    s = torch.ones((64, 2), dtype=torch.float16, device="cuda")
    assert W.gemm_kpacked(a, w, s, None, 128).shape == (0, 64)
    with pytest.raises(ValueError):
        W.gemm_kpacked(torch.zeros((1, 256), dtype=torch.float16, device="cuda"), w,
                       s.t().contiguous(), None, 128)
