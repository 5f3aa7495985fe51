"""CPU tests of the C ABI: symbols, host pack utility, argument checks, selector.

Nothing here launches a kernel; every call either is host-only or fails its
argument checks before the library touches a device.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle as O
from weight_only_int4_unpack_amd import w4a16 as W

HAS_GPU = torch.cuda.is_available()


def test_library_exports_every_header_symbol():
    L = W.lib()
    names = W.header_functions()
    assert {"w4a16_gemm", "w4a16_gemm_bias", "w4a16_gemm_planned", "w4a16_gemm_ws",
            "w4a16_workspace_bytes", "w4a16_plan", "w4a16_plan_route",
            "w4a16_dequant", "w4a16_pack_int4", "w4a16_unpack_int4", "w4a16_last_error",
            "w4a16_version", "w4a16_gemm_kpacked", "w4a16_pack_int4_kshuffle",
            "w4a16_unpack_int4_kshuffle"} <= set(names)
    for n in names:
        assert hasattr(L, n), n
    assert W.version().startswith("w4a16-gfx950")


def test_pack_matches_oracle_bitwise():
    rng = np.random.default_rng(5)
    q = rng.integers(0, 16, size=(333, 1024), dtype=np.uint8)
    assert np.array_equal(W.pack_int4(q), O.pack_int4(q))
    assert np.array_equal(W.unpack_int4(W.pack_int4(q)), q)
    x = rng.integers(-2**31, 2**31, size=(17, 40), dtype=np.int64).astype(np.int32)
    assert np.array_equal(W.unpack_int4(x), O.unpack_int4(x))


def test_pack_printed_vectors():
    w = W.pack_int4(np.array([[0, 1, 2, 3, 4, 5, 6, 7, 15, 14, 13, 12, 11, 10, 9, 8]], np.uint8))
    assert w.tolist() == [[0x76543210, -1985229329]]


def test_pack_errors():
    with pytest.raises(W.W4A16Error) as e:
        W.pack_int4(np.full((2, 8), 16, np.uint8))
    assert e.value.status == W.ERR_VALUE and "outside 0..15" in W.last_error()
    with pytest.raises(W.W4A16Error) as e:
        W.pack_int4(np.zeros((2, 12), np.uint8))
    assert e.value.status == W.ERR_SHAPE
    with pytest.raises(W.W4A16Error):
        W.pack_int4(np.array([[300] * 8]))
    L = W.lib()
    assert L.w4a16_pack_int4(None, 2, 8, None) == W.ERR_NULL
    assert L.w4a16_pack_int4(None, 0, 8, None) == W.OK       # empty is fine


def test_kshuffle_pack_matches_oracle_bitwise():
    rng = np.random.default_rng(6)
    q = rng.integers(0, 16, size=(129, 512), dtype=np.uint8)
    assert np.array_equal(W.pack_int4_kshuffle(q), O.pack_int4_kshuffle(q))
    assert np.array_equal(W.unpack_int4_kshuffle(W.pack_int4_kshuffle(q)), q)
    x = rng.integers(-2**31, 2**31, size=(9, 24), dtype=np.int64).astype(np.int32)
    assert np.array_equal(W.unpack_int4_kshuffle(x), O.unpack_int4_kshuffle(x))
    assert W.pack_int4_kshuffle(np.arange(8, dtype=np.uint8)[None, :]).tolist() == [[0x75316420]]
    with pytest.raises(W.W4A16Error) as e:
        W.pack_int4_kshuffle(np.full((2, 8), 16, np.uint8))
    assert e.value.status == W.ERR_VALUE
    with pytest.raises(W.W4A16Error) as e:
        W.pack_int4_kshuffle(np.zeros((2, 12), np.uint8))
    assert e.value.status == W.ERR_SHAPE
    assert W.lib().w4a16_pack_int4_kshuffle(None, 2, 8, None) == W.ERR_NULL


# ------------------------------------------------------------ argument checks
FAKE = ctypes.c_void_p(0x10000)    # aligned, never dereferenced on the host


def _kp(M=1, K=5120, N=17408, G=128, dt=1, a=FAKE, w=FAKE, s=FAKE, z=None, zp=8, bias=None,
        out=FAKE):
    return W.lib().w4a16_gemm_kpacked(a, w, s, z, G, zp, bias, out, M, K, N, dt, None)


@pytest.mark.parametrize("kw,status", [
    (dict(dt=2), W.ERR_DTYPE),
    (dict(K=0), W.ERR_SHAPE),
    (dict(M=-1), W.ERR_SHAPE),
    (dict(N=0), W.ERR_SHAPE),
    (dict(K=2120, G=2120), W.ERR_SHAPE),        # K % 32
    (dict(G=16), W.ERR_GROUP),
    (dict(G=96), W.ERR_GROUP),
    (dict(K=2112, G=128), W.ERR_SHAPE),         # K % G
    (dict(a=None), W.ERR_NULL),
    (dict(w=None), W.ERR_NULL),
    (dict(s=None), W.ERR_NULL),
    (dict(out=None), W.ERR_NULL),
    (dict(zp=16), W.ERR_ZP),
    (dict(a=ctypes.c_void_p(0x10008)), W.ERR_ALIGN),
    (dict(w=ctypes.c_void_p(0x10004)), W.ERR_ALIGN),
    (dict(bias=ctypes.c_void_p(0x10002)), W.ERR_ALIGN),
])
def test_gemm_kpacked_rejections(kw, status):
    assert _kp(**kw) == status
    assert W.last_error() != ""


def test_gemm_kpacked_accepts_odd_n_and_any_zero_alignment():
    assert _kp(M=0, a=None, w=None, s=None, out=None) == W.OK
    for kw in (dict(N=17), dict(z=ctypes.c_void_p(0x10003), zp=99), dict(K=2112, G=2112)):
        st = _kp(**kw)
        assert st == (W.ERR_DEVICE if not HAS_GPU else st), kw


def _gemm(a=FAKE, b=FAKE, s=FAKE, z=None, G=128, zp=8, out=FAKE, M=4, K=256, N=512, dt=W.F16):
    return W.lib().w4a16_gemm(a, b, s, z, G, zp, out, M, K, N, dt, None)


@pytest.mark.parametrize("kw,status", [
    (dict(dt=2), W.ERR_DTYPE),
    (dict(N=516), W.ERR_SHAPE),
    (dict(K=0), W.ERR_SHAPE),
    (dict(M=-1), W.ERR_SHAPE),
    (dict(G=16), W.ERR_GROUP),
    (dict(G=96), W.ERR_GROUP),
    (dict(G=100, K=200), W.ERR_GROUP),
    (dict(K=2112, G=128), W.ERR_SHAPE),
    (dict(a=None), W.ERR_NULL),
    (dict(out=None), W.ERR_NULL),
    (dict(s=None), W.ERR_NULL),
    (dict(zp=16), W.ERR_ZP),
    (dict(zp=-1), W.ERR_ZP),
    (dict(a=ctypes.c_void_p(0x10008)), W.ERR_ALIGN),
    (dict(z=ctypes.c_void_p(0x10004)), W.ERR_ALIGN),
])
def test_gemm_rejections(kw, status):
    assert _gemm(**kw) == status
    assert W.last_error() != ""


def _gemm_bias(bias, a=FAKE, out=FAKE, M=4, K=256, N=512, dt=W.F16):
    return W.lib().w4a16_gemm_bias(a, FAKE, FAKE, None, 128, 8, bias, out, M, K, N, dt, None)


def test_gemm_bias_checks():
    # a misaligned bias is rejected before any device work; shape, NULL and
    # M = 0 rules are those of w4a16_gemm
    assert _gemm_bias(ctypes.c_void_p(0x10002)) == W.ERR_ALIGN
    assert "bias" in W.last_error()
    assert _gemm_bias(FAKE, N=516) == W.ERR_SHAPE
    assert _gemm_bias(FAKE, a=None) == W.ERR_NULL
    assert _gemm_bias(FAKE, M=0, a=None, out=None) == W.OK
    if not HAS_GPU:   # a valid call (with or without bias) reaches the device check
        assert _gemm_bias(FAKE) == W.ERR_DEVICE
        assert _gemm_bias(None) == W.ERR_DEVICE


def test_group_64_is_kept_not_substituted():
    # both routes plan groups of 64 as given (the decode route with its exact
    # one-fold operand, as the group holds a wavefront's two steps)
    p = W.plan(8, 2112, 5120, 64, True, torch.float16)
    assert p.route == W.ROUTE_DECODE and p.decode_mode == 1 and p.steps_per_wave == 2
    assert W.plan(8, 2112, 5120, 64, True, torch.float16, route=W.ROUTE_PREFILL).route == W.ROUTE_PREFILL
    # a non-multiple K for G=64 is an error, never a fallback to another G
    assert _gemm(M=8, K=2100, N=5120, G=64) == W.ERR_SHAPE


def test_m_zero_is_noop_even_with_null_pointers():
    assert _gemm(M=0, a=None, out=None) == W.OK


def test_zero_point_bias_ignored_when_qzeros_given():
    # zp_bias is only checked for symmetric calls; with qzeros it is unused
    st = _gemm(z=FAKE, zp=99)
    assert st == (W.ERR_DEVICE if not HAS_GPU else st)


@pytest.mark.skipif(HAS_GPU, reason="checks the no-device error path")
def test_valid_call_without_device_reports_device_error():
    assert _gemm() == W.ERR_DEVICE
    assert "device" in W.last_error()


def test_python_wrapper_validates_shapes():
    a = torch.zeros((4, 256), dtype=torch.float16)
    b = torch.zeros((256, 64), dtype=torch.int32)
    s = torch.zeros((2, 512), dtype=torch.float16)
    with pytest.raises(ValueError):
        W.gemm(a, b, torch.zeros((2, 256), dtype=torch.float16))    # scales shape
    with pytest.raises(ValueError):
        W.gemm(a, b, s.to(torch.bfloat16))                           # scales dtype
    with pytest.raises(ValueError):
        W.gemm(a, b, s, qzeros=torch.zeros((2, 32), dtype=torch.int32))
    with pytest.raises(ValueError):
        W.gemm(a, b[:128], s)                                         # K mismatch
    with pytest.raises(ValueError):
        W.gemm(a, b, s)                                               # CPU tensors


# ------------------------------------------------------------ selector
def test_selector_routes_on_runtime_m():
    D, P = W.ROUTE_DECODE, W.ROUTE_PREFILL
    # K = N = 4096, fp16 groups of 32: decode up to 8 rows, one step per
    # wavefront inside its group (mode 1), 8 wavefronts per workgroup: 16
    # splits over 256 workgroups (32 over 512 with 4); the prefill above
    for M in (1, 2, 4, 5, 6, 8):
        p = W.plan(M, 4096, 4096, 32, True, torch.float16)
        assert (p.route, p.steps_per_wave, p.decode_mode, p.splits, p.threads) == (D, 1, 1, 16, 512), M
    for M in (9, 16, 17, 64, 256, 2048, 4096):
        assert W.plan(M, 4096, 4096, 32, True, torch.float16).route == P
    assert W.plan(0, 4096, 4096, 32, True, torch.float16).route == W.ROUTE_NONE
    # K = N = 8192, fp16 groups of 32: mode 1 takes 64 splits of 4 wavefronts
    # or 32 of 8; up to 4 rows (M * S <= 128) the decode with 8, from 5 rows
    # the ring prefill's K split (N <= 8192)
    p = W.plan(1, 8192, 8192, 32, True, torch.float16)
    assert (p.route, p.decode_mode, p.splits * p.threads // 64) == (D, 1, 256)
    for M in (2, 3, 4):
        p = W.plan(M, 8192, 8192, 32, True, torch.float16)
        assert (p.route, p.decode_mode, p.steps_per_wave, p.splits, p.threads) == (D, 1, 1, 32, 512), M
    for M in (5, 8):
        assert W.plan(M, 8192, 8192, 32, True, torch.float16).route == P
    # ... but wide N keeps the decode, with the rounded weights (mode 0)
    p = W.plan(5, 5120, 17408, 32, True, torch.float16)
    assert (p.route, p.decode_mode, p.steps_per_wave) == (D, 0, 4)
    # groups of 128: 4 steps of a wavefront inside one group, so the decode
    # up to 16 rows (few splits), the prefill above
    for M, route in ((1, D), (2, D), (4, D), (8, D), (9, D), (16, D), (17, P)):
        assert W.plan(M, 4096, 4096, 128, False, torch.bfloat16).route == route, M
    p = W.plan(16, 4096, 4096, 128, False, torch.bfloat16)
    assert (p.steps_per_wave, p.splits, p.decode_mode) == (4, 8, 1)
    # ... unless above 8 rows the splits would exceed 16 (K = 14336: 28)
    assert W.plan(8, 14336, 4096, 128, True, torch.float16).route == D
    assert W.plan(16, 14336, 4096, 128, True, torch.float16).route == P
    # above 8 rows the workgroup target halves, but not below 64
    p = W.plan(16, 2048, 2048, 128, False, torch.bfloat16)
    assert (p.route, p.steps_per_wave, p.grid) == (D, 2, 64)
    assert W.plan(4, 8192, 4096, 128, False, torch.bfloat16).route == D
    assert W.plan(4, 2048, 2048, 128, False, torch.bfloat16).route == D
    assert W.plan(4, 4096, 14336, 128, False, torch.bfloat16).route == D
    assert W.plan(8, 5120, 17408, 128, False, torch.bfloat16).route == D
    # K % 64 != 0 or N % 32 != 0 (no ring): decode up to 8 rows
    assert W.plan(8, 4160 - 32, 4096, 4128, True, torch.float16).route == D
    assert W.plan(8, 4096, 4104, 128, True, torch.float16).route == D
    # per-channel scales: the decode route up to 16 rows, with fewer splits
    # above 8 rows
    for M in (9, 12, 16):
        for N in (14336, 4096):
            p = W.plan(M, 4096, N, 4096, True, torch.float16)
            assert p.route == D and p.decode_mode == 1
    assert W.plan(8, 4096, 4096, 4096, True, torch.float16).steps_per_wave == 2
    assert W.plan(16, 4096, 4096, 4096, True, torch.float16).steps_per_wave == 4
    assert W.plan(17, 4096, 14336, 4096, True, torch.float16).route == P


def test_selector_decode_shapes():
    p = W.plan(1, 5120, 17408, 128, False, torch.bfloat16)
    nb = 17408 // 256
    assert p.block_n == 256 and p.grid == nb * p.splits
    assert p.steps_per_wave in (1, 2, 4, 8)
    assert p.splits * 4 * p.steps_per_wave >= 5120 // 32
    assert (p.splits - 1) * 4 * p.steps_per_wave < 5120 // 32        # no empty split
    # 4 steps per wavefront (one group of 128 rows) at 3 wavefronts per SIMD:
    # 680 workgroups resident at once; 8 steps would span two groups
    assert p.steps_per_wave == 4 and p.decode_mode == 1 and p.grid == 680
    assert W.plan(1, 5120, 17408, 128, False, torch.bfloat16, route=W.ROUTE_DECODE,
                  steps_per_wave=8).decode_mode == 2
    # K = 2112 is 66 steps of 32 rows; groups of 64 hold a wavefront's 2 steps,
    # so the exact operand with one in-place fold (mode 1) applies
    p = W.plan(8, 2112, 5120, 64, True, torch.float16, route=W.ROUTE_DECODE)
    assert p.splits * 4 * p.steps_per_wave >= 66
    assert p.steps_per_wave == 2 and p.decode_mode == 1
    # fp16 groups of 32 with 2 steps per wavefront: the rounded weight (mode 0)
    q = W.plan(1, 4096, 4096, 32, True, torch.float16, route=W.ROUTE_DECODE, steps_per_wave=2)
    assert q.decode_mode == 0
    assert p.workspace_bytes >= p.splits * 8 * 5120 * 4 or p.splits == 1
    # partials of 4 wavefronts, then scales and packed zeros of the staged groups
    ng = 4 * p.steps_per_wave // 2 + 1
    assert p.lds_bytes == 4 * 8 * 256 * 4 + ng * 256 * 2 + ng * 32 * 4
    # bf16 with groups of 32 cannot keep 2 or 4 steps in one group
    p = W.plan(4, 4096, 4096, 32, True, torch.bfloat16, route=W.ROUTE_DECODE, steps_per_wave=4)
    assert p.decode_mode == 2
    # per-channel: one group spans every step
    assert W.plan(8, 4096, 4096, 4096, True, torch.float16, route=W.ROUTE_DECODE).decode_mode == 1


def test_selector_prefill_tiles():
    p = W.plan(2048, 5120, 17408, 128, False, torch.bfloat16)
    assert (p.block_m, p.block_n, p.block_k) == (64, 256, 64)
    assert p.grid % 8 == 0 and p.grid >= 32 * 68
    # K % 64 == 0, N % 32 == 0: the operands go through the LDS ring, 4 slots of
    # two 8 KB tiles and four per-wavefront blocks of scales, zero points and
    # activation sums (256 bytes; 512 for groups of 32, two per stage)
    assert p.lds_bytes == 4 * (2 * 64 * 64 * 2 + 4 * 256)
    assert p.splits == 1                       # 2176 tiles: no K split
    assert W.plan(2048, 5120, 17408, 32, False, torch.bfloat16).lds_bytes == \
        4 * (2 * 64 * 64 * 2 + 4 * 512)
    # K % 64 != 0 (or N % 32 != 0): the double-buffered activation tile
    assert W.plan(2048, 5000, 17408, 5000, False, torch.bfloat16).lds_bytes == 2 * 64 * 80 * 2
    assert W.plan(2048, 5120, 17400, 128, False, torch.bfloat16).lds_bytes == 2 * 64 * 80 * 2
    q = W.plan(100, 4096, 4096, 32, True, torch.float16)
    assert q.grid == 2 * 16 * q.splits and q.splits > 1     # 32 tiles, K split


@pytest.mark.parametrize("M,K,N,G", [(64, 4096, 4096, 32), (256, 4096, 4096, 32),
                                     (17, 640, 1032, 64), (200, 640, 520, 128),
                                     (64, 608, 520, 32), (32, 5120, 17408, 128),
                                     (16, 4096, 4096, 4096), (300, 2112, 5120, 64)])
def test_selector_prefill_splits(M, K, N, G):
    p = W.plan(M, K, N, G, True, torch.bfloat16, route=W.ROUTE_PREFILL)
    # tile rows: 64, or 32 for M <= 64 when K % 64 == 0 and K splits
    assert p.block_m == (64 if K % 64 or M > 64 or p.splits == 1 else 32)
    ring = K % 64 == 0 and N % 32 == 0
    blk = 512 if G == 32 and K != 32 else 256
    assert p.lds_bytes == (4 * (p.block_m * 64 * 2 + 64 * 128 + 4 * blk) if ring
                           else 2 * p.block_m * 80 * 2)
    tiles = -(-M // p.block_m) * -(-N // 256)
    KT = -(-K // 64)
    S, ks = p.splits, p.steps_per_wave
    assert 1 <= S <= 32
    assert S * ks >= KT and (S - 1) * ks < KT             # every split has stages
    if G == 128 and G != K:
        assert ks % 2 == 0                               # whole groups of 128 rows
    if S > 1:
        assert tiles < 256 and ks >= 2
        # counter region, then the partials of the real rows only
        assert p.workspace_bytes == W.WORKSPACE_COUNTER_BYTES + S * M * N * 4
    # a forced split reproduces exactly; invalid ones are rejected
    f = W.plan(M, K, N, G, True, torch.bfloat16, route=W.ROUTE_PREFILL, steps_per_wave=ks)
    assert (f.splits, f.steps_per_wave, f.grid) == (S, ks, p.grid)
    assert p.grid % 8 == 0 and p.grid >= tiles * S


def test_forced_routes_and_errors():
    p = W.plan(5, 4096, 4096, 32, True, torch.float16, route=W.ROUTE_PREFILL)
    assert p.route == W.ROUTE_PREFILL
    with pytest.raises(W.W4A16Error) as e:
        W.plan(17, 4096, 4096, 32, True, torch.float16, route=W.ROUTE_DECODE)
    assert e.value.status == W.ERR_PLAN
    p = W.plan(4, 4096, 4096, 32, True, torch.float16, route=W.ROUTE_DECODE, steps_per_wave=1)
    assert p.steps_per_wave == 1 and p.splits == 4096 // 32 // (p.threads // 64)
    p = W.plan(4, 4096, 4096, 32, True, torch.float16, route=W.ROUTE_DECODE, decode_mode=2)
    assert p.decode_mode == 2
    for bad in (dict(steps_per_wave=3), dict(decode_mode=3),
                dict(steps_per_wave=4, decode_mode=1)):       # 4 steps straddle groups of 1
        with pytest.raises(W.W4A16Error) as e:
            W.plan(4, 4096, 4096, 32, True, torch.float16, route=W.ROUTE_DECODE, **bad)
        assert e.value.status == W.ERR_PLAN
    # shapes off the fast layout run one step per wavefront
    assert W.plan(4, 2120, 520, 2120, True, torch.float16).steps_per_wave == 1
    with pytest.raises(W.W4A16Error):
        W.plan(4, 2120, 520, 2120, True, torch.float16, route=W.ROUTE_DECODE, steps_per_wave=2)


def test_prefill_forced_split_errors():
    with pytest.raises(W.W4A16Error):     # 3 stages would cut a 128-row group
        W.plan(64, 4096, 4096, 128, False, torch.bfloat16, route=W.ROUTE_PREFILL, steps_per_wave=3)
    with pytest.raises(W.W4A16Error):     # 64 stages, 1 per split: 64 > 32 splits
        W.plan(64, 4096, 4096, 32, False, torch.bfloat16, route=W.ROUTE_PREFILL, steps_per_wave=1)
    p = W.plan(64, 4096, 4096, 32, False, torch.bfloat16, route=W.ROUTE_PREFILL, steps_per_wave=16)
    assert p.splits == 4 and p.block_m == 32 and p.grid == (64 // 32) * 16 * 4


def test_planned_call_rejects_mismatched_plan():
    p = W.plan(4, 4096, 4096, 32, True, torch.float16)
    p.grid += 1
    st = W.lib().w4a16_gemm_planned(FAKE, FAKE, FAKE, FAKE, 32, 8, FAKE, 4, 4096, 4096, W.F16,
                                    ctypes.byref(p), None)
    assert st == W.ERR_PLAN


# ------------------------------------------------------------ workspace
def test_workspace_bytes_follow_the_plan():
    # decode at the 5120 x 17408 shape: 10 splits of fp32 partials after the
    # counter region; M = 5 has five rows of them
    for M in (1, 5):
        p = W.plan(M, 5120, 17408, 128, False, torch.bfloat16)
        assert p.splits == 10
        n = W.workspace_bytes(M, 5120, 17408, 128, torch.bfloat16)
        assert n == p.workspace_bytes == W.WORKSPACE_COUNTER_BYTES + 10 * M * 17408 * 4
    # unsplit launches need none: the 256 x 512 tiny problem, the fp16 prefill
    assert W.workspace_bytes(4, 256, 512, 128, torch.float16) == 0
    assert W.workspace_bytes(2048, 5120, 17408, 128, torch.float16) == 0
    assert W.workspace_bytes(0, 5120, 17408, 128, torch.bfloat16) == 0
    # the bf16 prefill through the ring: the activation sums of its 40 groups
    # for the rows padded to 64, after the counter region
    assert W.workspace_bytes(2048, 5120, 17408, 128, torch.bfloat16) == \
        W.WORKSPACE_COUNTER_BYTES + 40 * 2048 * 4
    assert W.workspace_bytes(300, 5120, 17408, 5120, torch.bfloat16) == \
        W.WORKSPACE_COUNTER_BYTES + 1 * 320 * 4
    assert W.workspace_bytes(2048, 5120, 17408, 32, torch.bfloat16) == \
        W.WORKSPACE_COUNTER_BYTES + 160 * 2048 * 4
    # K % 64 != 0: no ring, the sums stay in the GEMM
    assert W.workspace_bytes(2048, 5024, 17408, 32, torch.bfloat16) == 0
    # fewer CUs, fewer splits wanted: never more scratch than for 256
    assert W.workspace_bytes(64, 4096, 4096, 32, torch.float16, num_cus=32) <= \
        W.workspace_bytes(64, 4096, 4096, 32, torch.float16)


def test_workspace_bytes_errors():
    L = W.lib()
    n = ctypes.c_int64(-1)
    assert L.w4a16_workspace_bytes(1, 256, 512, 128, W.F16, 256, None) == W.ERR_NULL
    assert L.w4a16_workspace_bytes(1, 256, 512, 128, 7, 256, ctypes.byref(n)) == W.ERR_DTYPE
    assert L.w4a16_workspace_bytes(1, 256, 516, 128, W.F16, 256, ctypes.byref(n)) == W.ERR_SHAPE
    assert L.w4a16_workspace_bytes(1, 256, 512, 96, W.F16, 256, ctypes.byref(n)) == W.ERR_GROUP
    assert L.w4a16_workspace_bytes(1, 2112, 512, 128, W.F16, 256, ctypes.byref(n)) == W.ERR_SHAPE
    assert n.value == -1     # untouched on error


def _gemm_ws(ws=FAKE, nbytes=1 << 30, M=5, K=4096, N=4096, G=128, dt=W.F16, bias=None, a=FAKE):
    return W.lib().w4a16_gemm_ws(a, FAKE, FAKE, None, G, 8, bias, FAKE, M, K, N, dt, ws, nbytes,
                                 None)


def test_gemm_ws_rejections():
    need = W.workspace_bytes(5, 4096, 4096, 128, torch.float16)
    assert need > 0
    assert _gemm_ws(nbytes=need - 1) == W.ERR_WORKSPACE
    assert "workspace" in W.last_error()
    assert _gemm_ws(ws=None, nbytes=0) == W.ERR_NULL
    assert _gemm_ws(nbytes=-1) == W.ERR_WORKSPACE
    assert _gemm_ws(ws=ctypes.c_void_p(0x10008)) == W.ERR_ALIGN
    assert _gemm_ws(bias=ctypes.c_void_p(0x10002)) == W.ERR_ALIGN
    assert _gemm_ws(a=None) == W.ERR_NULL
    assert _gemm_ws(G=96) == W.ERR_GROUP
    assert _gemm_ws(M=0, ws=None, nbytes=0, a=None) == W.OK
    if not HAS_GPU:   # valid arguments reach the device check
        assert _gemm_ws(nbytes=need) == W.ERR_DEVICE
        # a problem without split needs no workspace at all
        assert _gemm_ws(ws=None, nbytes=0, M=4, K=256, N=512) == W.ERR_DEVICE


def test_bf16_decode_mode_0_rejected():
    # the rounded-weight operand of decode mode 0 is fp16 only: bf16 rounding
    # (2^-8 per weight) over a long K leaves the tolerance
    with pytest.raises(W.W4A16Error) as e:
        W.plan(4, 4096, 4096, 32, True, torch.bfloat16, route=W.ROUTE_DECODE, decode_mode=0)
    assert e.value.status == W.ERR_PLAN and "fp16" in W.last_error()
    assert W.plan(4, 4096, 4096, 32, True, torch.float16, route=W.ROUTE_DECODE,
                  decode_mode=0).decode_mode == 0
    # the selector never picks it for bf16
    for G in (32, 64, 128, 4096):
        for M in range(1, 9):
            for N in (4096, 14336):
                p = W.plan(M, 4096, N, G, True, torch.bfloat16)
                assert p.route != W.ROUTE_DECODE or p.decode_mode != 0


def test_k_limit_and_counter_limit():
    # K above 2^24 would overflow the 32-bit byte offsets of a row block
    assert _gemm(M=1, K=1 << 25, N=8, G=1 << 25) == W.ERR_SHAPE
    assert "2^24" in W.last_error()
    assert _kp(M=1, K=1 << 25, N=8, G=1 << 25) == W.ERR_SHAPE
    # more column blocks than the counter region serves: the selector takes
    # the prefill route, and a forced split decode is refused
    N = 4097 * 256
    assert W.plan(1, 4096, N, 128, False, torch.bfloat16).route == W.ROUTE_PREFILL
    with pytest.raises(W.W4A16Error) as e:
        W.plan(1, 4096, N, 128, False, torch.bfloat16, route=W.ROUTE_DECODE)
    assert e.value.status == W.ERR_PLAN
    assert W.plan(1, 4096, 4096 * 256, 128, False, torch.bfloat16).route == W.ROUTE_DECODE


def test_plan_invariants_over_random_shapes():
    # the selector's plans on 4000 seeded random shapes: every plan is one the
    # kernels can run, covers K exactly once and asks for enough scratch
    rng = np.random.default_rng(2024)
    D, P = W.ROUTE_DECODE, W.ROUTE_PREFILL
    for _ in range(4000):
        M = int(np.exp(rng.uniform(0, np.log(4096))))
        G = int(rng.choice([32, 64, 128, 0]))
        if G:
            K = G * int(rng.integers(1, 16384 // G + 1))
        else:
            K = 8 * int(rng.integers(1, 2049)) + int(rng.choice([0, 0, 0, 1]))   # K % 8 != 0 now and then
            G = K
        N = 8 * int(np.exp(rng.uniform(0, np.log(8192))))
        dt = torch.float16 if rng.integers(2) else torch.bfloat16
        zp = bool(rng.integers(2))
        p = W.plan(M, K, N, G, zp, dt)
        d = p.as_dict()
        what = (M, K, N, G, dt, zp, d)
        assert d["lds_bytes"] <= 160 * 1024, what
        assert W.workspace_bytes(M, K, N, G, dt) >= d["workspace_bytes"], what
        if d["route"] == D:
            KS, L, S, Wv = -(-K // 32), d["steps_per_wave"], d["splits"], d["threads"] // 64
            assert M <= 16 and L in (1, 2, 4, 8), what
            assert Wv == 4 or (Wv == 8 and L <= 2 and M <= 8 and N % 16 == 0 and K % 8 == 0), what
            assert S == -(-KS // (Wv * L)) and (S - 1) * Wv * L < KS, what     # K once, no empty split
            assert d["grid"] == -(-N // 256) * S, what
            assert d["decode_mode"] in (0, 1, 2), what
            if d["decode_mode"] == 0:
                assert dt == torch.float16, what
            if d["decode_mode"] == 1:
                assert G == K or (G // 32) % L == 0, what                      # steps inside one group
            if N % 16 or K % 8:
                assert L == 1, what
            if S > 1:
                assert d["workspace_bytes"] >= W.WORKSPACE_COUNTER_BYTES + S * M * N * 4, what
        else:
            assert d["route"] == P, what
            KT, bm, S = -(-K // 64), d["block_m"], d["splits"]
            assert bm in (32, 64) and S == -(-KT // d["steps_per_wave"]), what
            units = -(-M // bm) * -(-N // 256) * S                              # tiles x splits,
            assert d["grid"] == -(-units // 8) * 8, what                         # padded to the 8 XCDs
            if S > 1:
                assert d["workspace_bytes"] >= W.WORKSPACE_COUNTER_BYTES + S * M * N * 4, what
            assert M > 1 or N <= 8192 or K % 8, what   # one row takes the decode on wide N
