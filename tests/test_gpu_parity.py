"""GPU parity: the HIP library against the CPU oracle, through the C ABI.

* dequantised tiles: bit-exact (``w4a16_dequant`` vs ``oracle.dequant_tile``);
* GEMM outputs: ``|gpu - oracle| <= 2e-2 * max(1, |oracle|)`` after the cast
  to the output dtype, element by element (full arrays at small sizes,
  sampled rows/columns at the full workload sizes);
* exact-arithmetic inputs (small integers times powers of two), one-hot
  activations and q == z: bit-exact, on both routes;
* determinism, output canaries, input immutability and edge shapes.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle as O
from weight_only_int4_unpack_amd import w4a16 as W
from helpers import (assert_within_tolerance, bits_to_dev, dev_to_bits, make_problem,
                     random_problem, workload_problem, TORCH_DT)

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _plan(p, route, L=0, mode=-1):
    return W.plan(p.M, p.K, p.N, p.G, p.qz is not None, TORCH_DT[p.dtype], route=route,
                  steps_per_wave=L, decode_mode=mode)


def _routes(M):
    """(label, plan factory) pairs that apply to a problem with M rows: the
    selector's choice, the prefill kernel, and every decode mode."""
    out = [("auto", lambda p: None), ("prefill", lambda p: _plan(p, W.ROUTE_PREFILL))]
    if 1 <= M <= 16:
        def big(p):   # the fast layout takes 1, 2, 4 or 8 steps per wavefront
            return 4 if (p.N % 16 == 0 and p.K % 8 == 0) else 1

        def sit(p):   # the rounded-weight operand (mode 0) is fp16 only
            return _plan(p, W.ROUTE_DECODE, L=big(p), mode=0 if p.dtype == "fp16" else 2)
        out += [("decode_sit", sit),
                ("decode_multi", lambda p: _plan(p, W.ROUTE_DECODE, L=big(p), mode=2)),
                ("decode_onegroup", lambda p: _plan(p, W.ROUTE_DECODE, L=1, mode=1)),
                ("decode_L2", lambda p: _plan(p, W.ROUTE_DECODE, L=min(2, big(p))))]
    return out


# ---------------------------------------------------------------- dequant probe
@pytest.mark.parametrize("K,N,G,dtype,zp", [
    (256, 512, 128, "fp16", False),
    (2112, 5120, 64, "fp16", True),
    (4096, 4096, 32, "fp16", True),
    (4096, 4096, 4096, "fp16", True),
    (5120, 2048, 128, "bf16", False),
    (1024, 1024, 64, "bf16", True),
    (129, 520, 129, "bf16", True),
    (64, 520, 32, "fp16", False),
])
def test_dequant_probe_bit_exact(K, N, G, dtype, zp):
    p = random_problem(1, K, N, G, dtype, zp, seed=K + N + G)
    got = dev_to_bits(W.dequant(p.b_q_d, p.s, p.qz_d, G, 8))
    want = O.dequant_tile(p.b_q, p.s_bits, p.qz, G, 8, dtype)
    assert np.array_equal(got, want), f"{int((got != want).sum())} mismatching weights"


def test_dequant_probe_zp_bias_values():
    for zp in (0, 7, 15):
        p = random_problem(1, 128, 256, 64, "fp16", False, seed=40 + zp, zp_bias=zp)
        got = dev_to_bits(W.dequant(p.b_q_d, p.s, None, 64, zp))
        assert np.array_equal(got, O.dequant_tile(p.b_q, p.s_bits, None, 64, zp, "fp16"))


# ---------------------------------------------------------------- parity grid
# The M grid is the page's reference test grid (PR #40977, Code section:
# 1, the skinny-batch limit 5, one past it, and 64), from the golden file.
_PAGE_GRID = json.load(open(os.path.join(GOLDEN, "pages_parity_grid.json")))
GRID = [(M, dtype, G, zp) for M in _PAGE_GRID["m_grid"] for dtype in ("fp16", "bf16")
        for G in (32, 64, 128, 512) for zp in (False, True)]
assert _PAGE_GRID["group_size_reported_broken"] in (32, 64, 128, 512)


@pytest.mark.parametrize("M,dtype,G,zp", GRID)
def test_gemm_parity_grid(M, dtype, G, zp):
    K, N = 512, 768
    p = random_problem(M, K, N, G, dtype, zp, seed=M * 7 + G)
    want = p.oracle_gemm()
    for label, mk in _routes(M):
        got = dev_to_bits(p.gpu_gemm(plan=mk(p)))
        assert_within_tolerance(got, want, dtype, f"M={M} {dtype} G={G} zp={zp} {label}")


# ---------------------------------------------------------------- prefill tiles
# Several 64 x 256 prefill tiles in both directions with ragged tails (M = 200
# = 3 x 64 + 8, N = 520 = 2 x 256 + 8), every group span (G = 32, 64, 128 and
# per-channel: 20, 10, 5 and 1 groups), both dtypes, with and without zero
# points; K = 608 (K % 64 == 32) takes the variant that clamps the last stage.
PREFILL_GRID = [(640, G, dtype, zp) for G in (32, 64, 128, 640) for dtype in ("fp16", "bf16")
                for zp in (False, True)] + [(608, 32, "fp16", True), (608, 32, "bf16", False),
                                            (608, 608, "bf16", True)]


@pytest.mark.parametrize("K,G,dtype,zp", PREFILL_GRID)
def test_prefill_tiles_parity(K, G, dtype, zp):
    M, N = 200, 520
    p = random_problem(M, K, N, G, dtype, zp, seed=K + G + (7 if zp else 0))
    plan = _plan(p, W.ROUTE_PREFILL)
    assert plan.block_m == 64 and plan.grid >= 4 * 3
    got = dev_to_bits(p.gpu_gemm(plan=plan))
    assert_within_tolerance(got, p.oracle_gemm(), dtype, f"K={K} G={G} {dtype} zp={zp}")


# Tiles of 32 rows (few rows, K splits): several tiles with a ragged last one
# (M = 40 and 64 over 32-row tiles, M = 12 and 16 in one), every group span,
# both dtypes, zero points, ragged N; and bit for bit on exact inputs,
# through the selector's own plan.
SMALL_TILES = [(M, G, dtype, zp) for M in (12, 16, 40, 64) for G in (32, 64, 128, 1024)
               for dtype in ("fp16", "bf16") for zp in (False, True) if (G + M) % 3 != 1]


@pytest.mark.parametrize("M,G,dtype,zp", SMALL_TILES)
def test_small_prefill_tiles_parity(M, G, dtype, zp):
    K, N = 1024, 776
    p = random_problem(M, K, N, G, dtype, zp, seed=M * 3 + G)
    plan = _plan(p, W.ROUTE_PREFILL)
    assert plan.block_m == 32 and plan.splits > 1
    assert_within_tolerance(dev_to_bits(p.gpu_gemm(plan=plan)), p.oracle_gemm(), dtype,
                            f"M={M} G={G} {dtype} zp={zp} bm={plan.block_m}")


@pytest.mark.parametrize("M,dtype", [(16, "bf16"), (40, "fp16"), (9, "fp16"), (64, "bf16")])
def test_small_prefill_tiles_exact_bitwise(M, dtype):
    q = _exact_problem(M, 2048, 520, 128, dtype, True, seed=90 + M)
    plan = _plan(q, W.ROUTE_PREFILL)
    assert plan.block_m == 32
    got = dev_to_bits(q.gpu_gemm(plan=plan))
    want = q.oracle_gemm()
    assert np.array_equal(got, want), f"M={M}: {int((got != want).sum())} differ"


# The LDS-ring prefill (64-row tiles, K % 64 == 0, N % 32 == 0):
# ragged M (200 = 3 x 64 + 8) and N (544 = 2 x 256 + 32: the last tile's
# weight pieces past N are clamped), both dtypes, with and without zero
# points (without them bf16 takes seeded partials). Unsplit, the stage counts
# KT walk every tail of the loop (it runs four stages per trip while seven
# remain, then 1..6); split, every split has one to three stages.
RING_K = [(64 * kt, 64) for kt in (1, 2, 3, 4, 5, 6, 9, 10, 11)] + \
         [(64 * kt, 128) for kt in (2, 4, 6, 10)] + [(192, 192), (448, 448)] + \
         [(64 * kt, 32) for kt in (1, 2, 5, 7)]


@pytest.mark.parametrize("K,G", RING_K)
@pytest.mark.parametrize("dtype,zp", [("bf16", False), ("bf16", True), ("fp16", False), ("fp16", True)])
def test_prefill_ring_parity(K, G, dtype, zp):
    M, N = 200, 544
    p = random_problem(M, K, N, G, dtype, zp, seed=K + 3 * G + (5 if zp else 0))
    KT = K // 64
    unit = 2 if G == 128 else 1
    for stages in sorted({KT, unit, 3 * unit}):
        plan = W.plan(M, K, N, G, zp, TORCH_DT[dtype], route=W.ROUTE_PREFILL, steps_per_wave=stages)
        blk = 512 if G == 32 else 256
        assert plan.block_m == 64 and plan.lds_bytes == 4 * (2 * 64 * 64 * 2 + 4 * blk)
        got = dev_to_bits(p.gpu_gemm(plan=plan))
        assert_within_tolerance(got, p.oracle_gemm(), dtype,
                                f"K={K} G={G} {dtype} zp={zp} stages={stages} splits={plan.splits}")


# The ring's 32-row tiles (few rows, K splits): M within one tile (12, 16) or
# over two with a ragged second (40, 64), every group span, both dtypes,
# zero points, N % 256 = 32; the selector's split and a forced one.
RING_SMALL = [(M, G, dtype, zp) for M in (12, 16, 40, 64) for G in (32, 64, 128, 1024)
              for dtype in ("fp16", "bf16") for zp in (False, True) if (G + M + zp) % 3 != 1]


@pytest.mark.parametrize("M,G,dtype,zp", RING_SMALL)
def test_prefill_ring_small_tiles_parity(M, G, dtype, zp):
    K, N = 1024, 800
    p = random_problem(M, K, N, G, dtype, zp, seed=M * 5 + G + 1)
    for stages in (0, 6 if G == 128 else 3):
        plan = W.plan(M, K, N, G, zp, TORCH_DT[dtype], route=W.ROUTE_PREFILL, steps_per_wave=stages)
        blk = 512 if G == 32 else 256
        assert plan.block_m == 32 and plan.splits > 1
        assert plan.lds_bytes == 4 * (32 * 64 * 2 + 64 * 128 + 4 * blk)
        assert_within_tolerance(dev_to_bits(p.gpu_gemm(plan=plan)), p.oracle_gemm(), dtype,
                                f"M={M} G={G} {dtype} zp={zp} splits={plan.splits}")


# bit for bit on exact inputs through the ring, unsplit and split
@pytest.mark.parametrize("dtype,zp,G", [("bf16", False, 128), ("bf16", True, 64), ("fp16", True, 128),
                                         ("bf16", False, 640), ("bf16", True, 32), ("fp16", False, 32)])
def test_prefill_ring_exact_bitwise(dtype, zp, G):
    M, K, N = 136, 640, 800
    q = _exact_problem(M, K, N, G, dtype, zp, seed=700 + G)
    for stages in (K // 64, 2):
        plan = W.plan(M, K, N, G, zp, TORCH_DT[dtype], route=W.ROUTE_PREFILL, steps_per_wave=stages)
        got = dev_to_bits(q.gpu_gemm(plan=plan))
        want = q.oracle_gemm()
        assert np.array_equal(got, want), f"stages={stages}: {int((got != want).sum())} differ"


# bf16 prefill with groups of 128 over a long K (8576 = 67 groups), unsplit
# and with forced K splits of 35 and 3 groups, so that splits start at group
# offsets other than 0; tolerance against the oracle and the exact-arithmetic
# case bit for bit.
@pytest.mark.parametrize("stages", [0, 70, 6])
def test_prefill_bf16_long_k_splits(stages):
    M, K, N, G = 100, 8576, 520, 128
    p = random_problem(M, K, N, G, "bf16", False, seed=300 + stages)
    plan = W.plan(M, K, N, G, False, torch.bfloat16, route=W.ROUTE_PREFILL,
                  steps_per_wave=stages if stages else K // 64)
    assert plan.splits == (1 if stages == 0 else -(-(K // 64) // stages))
    got = dev_to_bits(p.gpu_gemm(plan=plan))
    assert_within_tolerance(got, p.oracle_gemm(), "bf16", f"stages={stages}")
    q = _exact_problem(M, K, N, G, "bf16", False, seed=310 + stages)
    got = dev_to_bits(q.gpu_gemm(plan=plan))
    want = q.oracle_gemm()
    assert np.array_equal(got, want), f"stages={stages}: {int((got != want).sum())} differ"


# per-channel scales take the decode route up to 16 rows where the ring
# prefill does not apply or win (fewer splits above 8 rows); aligned K with
# N % 32 != 0, and ragged K, through the selector's own plan
@pytest.mark.parametrize("M", [9, 12, 16])
@pytest.mark.parametrize("K,N,dtype", [(4096, 4104, "fp16"), (2120, 520, "bf16")])
def test_per_channel_decode_route_mid_m(M, K, N, dtype):
    p = random_problem(M, K, N, K, dtype, True, seed=400 + M + K)
    plan = W.plan(M, K, N, K, True, TORCH_DT[dtype])
    assert plan.route == W.ROUTE_DECODE and plan.decode_mode == 1
    assert_within_tolerance(dev_to_bits(p.gpu_gemm()), p.oracle_gemm(), dtype, f"M={M} K={K}")


# ---------------------------------------------------------------- workloads
def _check_workload(name, rows=None, cols=None, routes=True):
    p = workload_problem(name)
    labels = _routes(p.M) if routes else [("auto", lambda q: None)]
    want = p.oracle_gemm(rows=rows, cols=cols)
    for label, mk in labels:
        out = dev_to_bits(p.gpu_gemm(plan=mk(p)))
        if rows is not None:
            out = out[np.asarray(rows)]
        if cols is not None:
            out = out[:, np.asarray(cols)]
        assert_within_tolerance(out, want, p.dtype, f"{name} {label}")


def test_workload_tiny():
    _check_workload("tiny")


def test_workload_k2112():
    _check_workload("k2112")


@pytest.mark.parametrize("name", ["decode_m1", "decode_m5"])
def test_workload_decode_sampled(name):
    rng = np.random.default_rng(3)
    cols = np.unique(np.concatenate([np.arange(0, 64), np.arange(17408 - 64, 17408),
                                     rng.choice(17408, 512, replace=False)]))
    _check_workload(name, cols=cols)


def test_workload_prefill_sampled():
    rng = np.random.default_rng(4)
    rows = np.unique(np.concatenate([[0, 1, 255, 256, 2047], rng.choice(2048, 59, replace=False)]))
    cols = np.unique(np.concatenate([np.arange(0, 32), np.arange(17408 - 32, 17408),
                                     rng.choice(17408, 448, replace=False)]))
    _check_workload("prefill", rows=rows, cols=cols, routes=False)


@pytest.mark.parametrize("m", [1, 2, 4, 5, 6, 16, 64, 256])
def test_workload_sweep(m):
    _check_workload(f"sweep_m{m}", routes=m <= 16)


def test_workload_sweep_m4096_sampled():
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, 4095], rng.choice(4096, 126, replace=False)]))
    _check_workload("sweep_m4096", rows=rows, routes=False)


def test_workload_sweep_per_channel():
    _check_workload("sweep_pc16")


# ---------------------------------------------------------------- exact pins
def _exact_problem(M, K, N, G, dtype, zp, seed):
    rng = np.random.default_rng(seed)
    a = np.zeros((M, K), np.float32)
    for m in range(M):
        idx = rng.choice(K, size=16, replace=False)
        a[m, idx] = rng.choice([-1.0, 1.0], size=16)
    d = {"a_bits": O.rne_bits(a, dtype),
         "q": rng.integers(0, 16, size=(K, N), dtype=np.uint8),
         "s_bits": O.rne_bits(np.full((K // G, N), 1.0 / 16, np.float32), dtype),
         "z": rng.integers(0, 16, size=(K // G, N), dtype=np.uint8) if zp else None}
    return make_problem(d, M, K, N, G, dtype)


@pytest.mark.parametrize("M,K,N,G,dtype,zp", [
    (4, 4096, 512, 128, "bf16", False),
    (8, 2112, 640, 64, "fp16", True),
    (16, 4096, 512, 32, "fp16", True),
    (64, 1024, 768, 1024, "bf16", True),
    (300, 512, 256, 32, "fp16", False),
])
def test_exact_arithmetic_bitwise(M, K, N, G, dtype, zp):
    p = _exact_problem(M, K, N, G, dtype, zp, seed=M + K)
    want = p.oracle_gemm()
    for label, mk in _routes(M):
        got = dev_to_bits(p.gpu_gemm(plan=mk(p)))
        assert np.array_equal(got, want), f"{label}: {int((got != want).sum())} differ"


@pytest.mark.parametrize("dtype,G,zp", [("fp16", 32, True), ("bf16", 128, False),
                                        ("fp16", 64, False), ("bf16", 256, True)])
def test_one_hot_rows_bitwise(dtype, G, zp):
    K, N = 256, 512
    p = random_problem(1, K, N, G, dtype, zp, seed=G)
    ks = [0, 1, 31, 32, 100, 127, 128, 255, 7, 200, 64, 65, 96, 33]
    a = np.zeros((len(ks), K), np.float32)
    for i, k in enumerate(ks):
        a[i, k] = 1.0
    p.a_bits = O.rne_bits(a, dtype)
    p.a = bits_to_dev(p.a_bits, dtype)
    p.M = len(ks)
    tile = O.dequant_tile(p.b_q, p.s_bits, p.qz, G, 8, dtype)[ks]
    for label, mk in _routes(p.M):
        got = dev_to_bits(p.gpu_gemm(plan=mk(p)))
        assert np.array_equal(got, tile), f"{label}: {int((got != tile).sum())} differ"


@pytest.mark.parametrize("dtype,zp", [("fp16", True), ("bf16", False)])
def test_q_equals_z_gives_zero(dtype, zp):
    M, K, N, G = 8, 512, 512, 64
    rng = np.random.default_rng(9)
    z = rng.integers(0, 16, size=(K // G, N), dtype=np.uint8) if zp else None
    q = np.repeat(z, G, axis=0) if zp else np.full((K, N), 8, np.uint8)
    d = {"a_bits": O.rne_bits(rng.standard_normal((M, K)).astype(np.float32), dtype), "q": q,
         "s_bits": O.rne_bits(rng.uniform(1e-3, 1e-2, (K // G, N)).astype(np.float32), dtype),
         "z": z}
    p = make_problem(d, M, K, N, G, dtype)
    bound = _factored_zero_bound(p, zp)
    for label, mk in _routes(M):
        pl = mk(p)
        got = O.to_f32(dev_to_bits(p.gpu_gemm(plan=pl)), dtype)
        eff = pl if pl is not None else W.plan(M, K, N, G, zp, TORCH_DT[dtype])
        if eff.route == W.ROUTE_DECODE and eff.decode_mode != 0 or \
                eff.route == W.ROUTE_PREFILL and dtype == "bf16":
            # factored form s (sum a (base + q) - (base + z) sum a): the two
            # fp32 sums cancel up to their rounding, within the bound below
            assert np.all(np.abs(got) <= bound), (label, float(np.abs(got).max()))
        else:
            # exact operand q - z = 0 (fp16 prefill) or the exact tile (mode 0)
            assert np.all(got == 0.0), label


def _factored_zero_bound(p, zp):
    """Bound on |out| when q == z in the factored forms (exact result 0). For
    output (m, n) and one group: S^ = fl(sum a) over at most G terms errs by at
    most g_G A (A = sum |a|, g_n = n u / (1 - n u), u = 2^-24); the operand is
    b + q = b (b = base + z <= B: bf16 128 + 15, fp16 1024 + 15).
    Fold form: P^ = fl(sum a b) errs by at most g_G B A, and fl(P^ - b S^)
    by at most 2 g_G B A (1 + u).
    Seeded form (bf16 prefill without zero points): the partial starts from
    C0 = fl(-b S^) (|C0 + b S^| <= u B A (1 + g_G)) and accumulates the G
    products onto it, G + 1 terms each at most B A (1 + g_G): the result errs
    by at most 2 g_{G+1} B A (1 + g_G) from C0 + b S = -b (S^ - S) + (C0 + b S^),
    so |partial| <= (g_G + u + 2 g_{G+1}) B A (1 + g_G).
    Both are below (3 g_{G+1} + u) B A (1 + g_G); times s, summed over groups,
    wavefronts and splits (roundings relative to these tiny terms: factor
    1.01), and one ulp of the output type (at least its smallest subnormal)."""
    a = np.abs(O.to_f32(p.a_bits, p.dtype).astype(np.float64))             # [M, K]
    s = np.abs(O.to_f32(p.s_bits, p.dtype).astype(np.float64))             # [K/G, N]
    s_k = np.repeat(s, p.G, axis=0)                                        # [K, N]
    u = 2.0 ** -24
    g = p.G * u / (1 - p.G * u)
    g1 = (p.G + 1) * u / (1 - (p.G + 1) * u)
    B = 143.0 if p.dtype == "bf16" else 1039.0
    bound = (3 * g1 + u) * (1 + g) * B * (a @ s_k) * 1.01                  # [M, N]
    tiny = 2.0 ** -24 if p.dtype == "fp16" else 2.0 ** -133
    return bound * (1 + 2.0 ** -7) + tiny


# Linearity. Scaling S or a by 2 scales every product and every partial sum
# by 2 with no change in rounding (no overflow or underflow in the fp32
# sums), on any hardware summation that aligns in binary; the reductions are
# deterministic, so the outputs must be exactly 2C, bit for bit, on every
# route, except fp16 outputs in the subnormal range (see below). Negating a negates every product; with IEEE rounding
# to nearest every sum would negate exactly too, and on the bf16 routes and
# the fp16 prefill (integer operand) the output is exactly -C. The fp16
# matrix-core dot product is not sign-symmetric in its internal rounding
# (measured on MI355X: a few outputs in a thousand off by 1-2 ulp on the fp16
# decode routes, including the one fed plain rounded weights), so there the
# pin is -C within 2 ulp of the output on every element, and at most 1 % of
# the outputs differing at all.
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("M", [5, 100])
def test_linearity_bitwise(M, dtype):
    p = random_problem(M, 1024, 512, 64, dtype, True, seed=77)
    routes = _routes(M)
    base = {label: dev_to_bits(p.gpu_gemm(plan=mk(p))) for label, mk in routes}
    a0, s0 = p.a, p.s
    for what, factor in (("s*2", 2.0), ("a*2", 2.0), ("-a", -1.0)):
        p.a, p.s = a0, s0
        if what == "s*2":
            p.s = s0 * 2
        else:
            p.a = a0 * factor
        for label, mk in routes:
            pl = mk(p)
            bits = dev_to_bits(p.gpu_gemm(plan=pl))
            got, want = O.to_f32(bits, dtype), factor * O.to_f32(base[label], dtype)
            eff = pl if pl is not None else W.plan(M, p.K, p.N, p.G, True, TORCH_DT[dtype])
            if what == "-a" and dtype == "fp16" and eff.route == W.ROUTE_DECODE:
                # magnitudes within 2 ulp, signs opposite to the base result
                ulps = np.abs((bits & 0x7FFF).astype(np.int32) -
                              (base[label] & 0x7FFF).astype(np.int32))
                flipped = (bits >> 15) != (base[label] >> 15)
                assert np.all(flipped | (got == want)), (what, label)
                assert int(ulps.max()) <= 2 and np.mean(got != want) <= 0.01, (what, label)
            elif factor == 2.0 and dtype == "fp16":
                # outputs below the smallest normal fp16 (2^-14) round on the
                # fixed subnormal grid, where RNE(2x) and 2 RNE(x) may differ
                # by one subnormal step: bit for bit above, within 2^-23 below
                tiny = np.abs(O.to_f32(base[label], dtype)) < 2.0 ** -14
                assert np.array_equal(got[~tiny], want[~tiny]), (what, label)
                assert np.all(np.abs(got[tiny] - want[tiny]) <= 2.0 ** -23), (what, label)
            else:
                assert np.array_equal(got, want), (what, label)
    p.a, p.s = a0, s0


# ---------------------------------------------------------------- robustness
@pytest.mark.parametrize("M", [5, 8, 300])
def test_deterministic_repeat(M):
    p = random_problem(M, 4096, 4096, 32, "fp16", True, seed=5)
    for label, mk in _routes(M):
        r1 = dev_to_bits(p.gpu_gemm(plan=mk(p)))
        r2 = dev_to_bits(p.gpu_gemm(plan=mk(p)))
        assert np.array_equal(r1, r2), label


@pytest.mark.parametrize("M", [3, 70])
def test_canaries_and_inputs_untouched(M):
    p = random_problem(M, 512, 520, 128, "fp16", True, seed=11)
    snap = [t.clone() for t in (p.a, p.b_q_d, p.s, p.qz_d)]
    guard = 4096
    for label, mk in _routes(M):
        buf = torch.full((guard * 2 + M * p.N,), 12345, dtype=torch.int16, device="cuda")
        out = buf[guard:guard + M * p.N].view(torch.float16).view(M, p.N)
        p.gpu_gemm(plan=mk(p), out=out)
        torch.cuda.synchronize()
        assert torch.all(buf[:guard] == 12345) and torch.all(buf[guard + M * p.N:] == 12345), label
        assert_within_tolerance(dev_to_bits(out), p.oracle_gemm(), "fp16", label)
    for t, s in zip((p.a, p.b_q_d, p.s, p.qz_d), snap):
        assert torch.equal(t, s)


@pytest.mark.parametrize("M,K,N,G,dtype,zp", [
    (1, 2120, 520, 2120, "fp16", True),     # K % 32 != 0, N % 256 != 0
    (3, 2120, 512, 2120, "bf16", True),     # K % 32 != 0 on the fast layout: the last
    (6, 1064, 1024, 1064, "fp16", False),   # step's weight rows past K read as zeros
    (7, 129, 264, 129, "bf16", False),      # K % 8 != 0 (per-channel)
    (16, 96, 24, 32, "fp16", True),         # fewer columns than one block
    (2, 4096, 8, 128, "bf16", True),        # N = 8
    (17, 640, 1032, 64, "fp16", False),     # first prefill M, ragged N
    (129, 2120, 520, 2120, "bf16", True),   # ragged M, K and N on prefill
    (255, 64, 256, 32, "fp16", True),       # a single K tile
    (1, 256, 66048, 128, "bf16", False),    # 258 column blocks: the counter split-K hand-off
    (3, 512, 66048, 64, "fp16", True),      # same, fp16 with zero points
])
def test_edge_shapes(M, K, N, G, dtype, zp):
    p = random_problem(M, K, N, G, dtype, zp, seed=M + K + N)
    want = p.oracle_gemm()
    for label, mk in _routes(M):
        got = dev_to_bits(p.gpu_gemm(plan=mk(p)))
        assert_within_tolerance(got, want, dtype, f"{label}")


# eight 32-row steps per wavefront: the two register slots of the decode's
# ring are refilled six times; every operand mode that takes it, a K split of
# two, N = 4 x 256 + 32 (a ragged last column block)
@pytest.mark.parametrize("M,dtype,G,zp,mode", [(5, "bf16", 128, True, 2), (1, "fp16", 64, True, 2),
                                               (16, "fp16", 32, True, 0), (8, "bf16", 2048, False, 1),
                                               (3, "fp16", 2048, True, 1)])
def test_decode_eight_steps(M, dtype, G, zp, mode):
    K, N = 2048, 1056
    p = random_problem(M, K, N, G, dtype, zp, seed=880 + G + mode + M)
    plan = _plan(p, W.ROUTE_DECODE, L=8, mode=mode)
    assert (plan.steps_per_wave, plan.splits, plan.decode_mode) == (8, 2, mode)
    got = dev_to_bits(p.gpu_gemm(plan=plan))
    assert_within_tolerance(got, p.oracle_gemm(), dtype, f"L=8 mode={mode} G={G}")


# The arrival counters of the split decode sit as far apart as the counter
# region allows (one per 128-byte line for up to 64 column blocks, closer
# for more), and each launch leaves its counters zero for the next. Split
# launches with 8, 1024 and 68 column blocks (slots 32, 4 and 32 apart) on
# one stream share the library's workspace; the first shape runs again at
# the end, so a counter left nonzero anywhere would cut a hand-off short.
def test_decode_counter_slots_reused_across_strides():
    cases = [(3, 1024, 2048, 128, "fp16", True, 1, 1),     # 8 column blocks
             (1, 256, 262144, 128, "bf16", False, 1, 1),   # 1024 column blocks
             (5, 1024, 17408, 128, "bf16", False, 2, 1)]   # 68 column blocks
    probs = []
    for i, (M, K, N, G, dtype, zp, L, mode) in enumerate(cases):
        p = random_problem(M, K, N, G, dtype, zp, seed=890 + i)
        plan = _plan(p, W.ROUTE_DECODE, L=L, mode=mode)
        assert plan.splits > 1, plan.as_dict()
        cols = np.unique(np.r_[0:64, N - 64:N, np.random.default_rng(i).integers(0, N, 256)])
        probs.append((p, plan, cols, p.oracle_gemm(cols=cols)))
    for p, plan, cols, want in probs + probs[:1]:
        got = dev_to_bits(p.gpu_gemm(plan=plan))[:, cols]
        assert_within_tolerance(got, want, p.dtype, f"N={p.N} splits={plan.splits}")


# Eight wavefronts per workgroup (half the K splits at the same wavefront
# count; the planner's choice for small shapes at one or two steps per
# wavefront): every operand mode, M = 1..8 (row blocks of 4 and 8, one row per
# wavefront in the hand-off), with the staged-scale modes 0 and 2 reading
# their 256 columns' scales through the first 256 threads.
@pytest.mark.parametrize("M,K,N,G,dtype,zp,L,mode", [
    (1, 4096, 4096, 32, "fp16", True, 0, -1), (2, 4096, 4096, 32, "bf16", True, 0, -1),
    (4, 4096, 4096, 32, "fp16", False, 0, -1), (5, 4096, 4096, 32, "fp16", True, 0, -1),
    (8, 4096, 4096, 32, "bf16", False, 0, -1), (3, 8192, 4096, 32, "fp16", True, 2, 0),
    (5, 8192, 4096, 32, "bf16", True, 2, 2), (8, 8192, 4096, 64, "fp16", True, 2, 1),
    (7, 8192, 4096, 32, "fp16", True, 1, 1),
    # the selector's own plan at 32 splits of 8 wavefronts (64 with 4)
    (3, 8192, 8192, 32, "fp16", True, 0, -1), (4, 8192, 8192, 32, "bf16", False, 0, -1)])
def test_decode_eight_wavefronts(M, K, N, G, dtype, zp, L, mode):
    p = random_problem(M, K, N, G, dtype, zp, seed=970 + M + K // 1024 + L)
    plan = W.plan(M, K, N, G, zp, TORCH_DT[dtype]) if L == 0 else _plan(p, W.ROUTE_DECODE, L=L, mode=mode)
    assert plan.route == W.ROUTE_DECODE and plan.threads == 512, plan.as_dict()
    cols = np.unique(np.r_[0:64, N - 64:N, np.random.default_rng(M).integers(0, N, 256)])
    got = dev_to_bits(p.gpu_gemm(plan=None if L == 0 else plan))[:, cols]
    assert_within_tolerance(got, p.oracle_gemm(cols=cols), dtype, f"M={M} L={L} mode={plan.decode_mode}")


# From 9 to 16 rows the selector keeps the decode where each wavefront's 2 or
# more steps lie inside one group with at most 16 splits: groups of 128 and
# 64, through the selector's own plan (16-row MFMA blocks, 4 rows per
# wavefront in the hand-off)
@pytest.mark.parametrize("M", [9, 12, 16])
@pytest.mark.parametrize("K,N,G,dtype,zp", [(4096, 4096, 128, "bf16", False),
                                            (2112, 5120, 64, "fp16", True)])
def test_decode_route_mid_m_one_group(M, K, N, G, dtype, zp):
    p = random_problem(M, K, N, G, dtype, zp, seed=950 + M + G)
    plan = W.plan(M, K, N, G, zp, TORCH_DT[dtype])
    assert plan.route == W.ROUTE_DECODE and plan.decode_mode == 1 and plan.steps_per_wave >= 2
    assert plan.splits <= 16, plan.as_dict()
    assert_within_tolerance(dev_to_bits(p.gpu_gemm()), p.oracle_gemm(), dtype, f"M={M}")


# The last arrival of a split decode with several rows per wavefront (M >= 5)
# and at least two windows of splits keeps a sliding window of partial
# loads in flight, wrapping the surplus split indices of its last window and
# reading zeros for rows past M. K = 4128 is 129 steps: 33 splits at one
# step per wavefront, so the last window holds one real split. Every M from
# 5 to 16 (row blocks of 8 and 16, wavefronts with one and two rows), and
# exact-integer data for a bitwise check of M = 5, 8, 13; N = 520 (off the
# fast layout: 16-row blocks at every M) for M = 6.
@pytest.mark.parametrize("N,Ms", [(512, range(5, 17)), (520, (6,))])
def test_decode_sliding_partial_window_every_m(N, Ms):
    K, G = 4128, 32
    p16 = random_problem(16, K, N, G, "fp16", True, seed=900 + N)
    for M in Ms:
        p = make_problem({"a_bits": p16.a_bits[:M], "q": W.unpack_int4(p16.b_q),
                          "s_bits": p16.s_bits, "z": W.unpack_int4(p16.qz)}, M, K, N, G, "fp16")
        plan = _plan(p, W.ROUTE_DECODE, L=1)
        assert plan.splits == 33, plan.as_dict()
        got = dev_to_bits(p.gpu_gemm(plan=plan))
        assert_within_tolerance(got, p.oracle_gemm(), "fp16", f"M={M}")
    for M in ((5, 8, 13) if N == 512 else Ms):
        q = _exact_problem(M, K, N, G, "fp16", True, seed=910 + M)
        got = dev_to_bits(q.gpu_gemm(plan=_plan(q, W.ROUTE_DECODE, L=1)))
        assert np.array_equal(got, q.oracle_gemm()), f"M={M}"


def test_decode_every_m_up_to_16():
    p16 = random_problem(16, 1024, 1024, 128, "bf16", False, seed=21)
    for M in range(1, 17):
        p = make_problem({"a_bits": p16.a_bits[:M], "q": W.unpack_int4(p16.b_q),
                          "s_bits": p16.s_bits, "z": None}, M, 1024, 1024, 128, "bf16")
        got = dev_to_bits(p.gpu_gemm(plan=_plan(p, W.ROUTE_DECODE)))
        assert_within_tolerance(got, p.oracle_gemm(), "bf16", f"M={M}")


def test_m_zero_is_noop():
    p = random_problem(1, 256, 512, 128, "fp16", False, seed=1)
    a0 = torch.empty((0, 256), dtype=torch.float16, device="cuda")
    out = W.gemm(a0, p.b_q_d, p.s, None, 128)
    assert tuple(out.shape) == (0, 512)


def test_pages_shape_contract_gpu():
    g = json.load(open(os.path.join(GOLDEN, "pages_shape_contract.json")))
    M, K = g["a_shape"]
    N = g["b_q_shape"][1] * 8
    p = random_problem(M, K, N, g["group_size"], g["a_dtype"], False, seed=2)
    out = W.gemm(p.a, p.b_q_d, p.s, None, g["group_size"])
    assert list(out.shape) == g["out_shape"] and out.dtype == torch.float16
    assert out.device == p.a.device


def test_streams_are_respected():
    p = random_problem(5, 2048, 2048, 128, "bf16", False, seed=31)
    want = p.oracle_gemm()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        out = p.gpu_gemm()
    s.synchronize()
    assert_within_tolerance(dev_to_bits(out), want, "bf16", "side stream")


# Seeded random shapes through the selector's own plan (whatever route, split
# and mode it takes), every row and 96 sampled columns (both edges included)
# against the oracle.
def test_random_shapes_selector_plan():
    rng = np.random.default_rng(77)
    for t in range(40):
        M = int(np.exp(rng.uniform(0, np.log(300))))
        G = int(rng.choice([32, 64, 128, 0]))
        if G:
            K = G * int(rng.integers(1, 4096 // G + 1))
        else:
            K = 8 * int(rng.integers(1, 513)) + int(rng.choice([0, 0, 1]))
            G = K
        N = 8 * int(rng.integers(1, 1025))
        dtype = "fp16" if rng.integers(2) else "bf16"
        zp = bool(rng.integers(2))
        p = random_problem(M, K, N, G, dtype, zp, seed=1000 + t)
        cols = np.unique(np.r_[0:min(N, 16), max(0, N - 16):N, rng.integers(0, N, 64)])
        got = dev_to_bits(p.gpu_gemm())[:, cols]
        plan = W.plan(M, K, N, G, zp, TORCH_DT[dtype]).as_dict()
        assert_within_tolerance(got, p.oracle_gemm(cols=cols), dtype, f"{(M, K, N, G, dtype, zp)} {plan}")
