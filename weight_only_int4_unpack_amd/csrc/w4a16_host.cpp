// Host side of the C ABI in include/w4a16.h: argument checks, the runtime
// route/tile selector, launches and the host pack utility.
//
// Checks follow the kernel-selection rules of PR #43731
// "TritonW4A16LinearKernel as CUDA fallback" (Code section, can_implement):
// fp16/bf16 activations only, N % 8 == 0, and a group size from the
// supported set or equal to the full K; no input is a silent substitute
// (PR #40977 "RDNA hybrid W4A16", Review section: group size 64 was run with
// the parameters of 128). The route and tiles are picked from the runtime
// shape on every call (PR #51453 "Register the Triton W4A16 GEMM as a custom
// op", Motivation and implementation item 1).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/w4a16.h"
#include "w4a16_internal.h"

namespace {

thread_local std::string g_last_error;

w4a16_status fail(w4a16_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

w4a16_status check_shape(int64_t M, int64_t K, int64_t N, int32_t G, int32_t dtype) {
  if (dtype != W4A16_F16 && dtype != W4A16_BF16)
    return fail(W4A16_ERR_DTYPE, "dtype %d: only fp16 (0) and bf16 (1) activations are supported",
                (int)dtype);
  if (M < 0 || K <= 0 || N <= 0)
    return fail(W4A16_ERR_SHAPE, "need M >= 0, K > 0, N > 0 (got M=%lld K=%lld N=%lld)",
                (long long)M, (long long)K, (long long)N);
  if (N % 8 != 0)
    return fail(W4A16_ERR_SHAPE, "N=%lld must be divisible by 8 (8 int4 values per int32)",
                (long long)N);
  if (!(G == 32 || G == 64 || G == 128 || (int64_t)G == K))
    return fail(W4A16_ERR_GROUP, "group size %d not supported (32, 64, 128 or K=%lld)", (int)G,
                (long long)K);
  if (K % G != 0)
    return fail(W4A16_ERR_SHAPE, "K=%lld is not a multiple of group size %d", (long long)K,
                (int)G);
  // 32-bit index limits of the kernels: rows, columns, per-row offsets, and
  // the byte offsets of one prefill row block ((64 - 1) * K * 2 < 2^32 needs
  // K < 2^25; K <= 2^24 leaves a margin)
  const int64_t lim = (int64_t)1 << 31;
  if (K > ((int64_t)1 << 24))
    return fail(W4A16_ERR_SHAPE, "K=%lld exceeds 2^24 (32-bit byte offsets of a row block)",
                (long long)K);
  if (N >= lim || M >= lim || (K / G) * N >= lim || M * K >= lim * 64 || K * (N / 8) >= lim * 64)
    return fail(W4A16_ERR_SHAPE, "problem too large for 32-bit row/column indexing");
  return W4A16_OK;
}

w4a16_status check_ptrs(const void* a, const void* b_q, const void* scales, const void* qzeros,
                        const void* out, int32_t zp_bias) {
  if (!a || !b_q || !scales || !out)
    return fail(W4A16_ERR_NULL, "a, b_q, scales and out must be non-NULL");
  if (!qzeros && (zp_bias < 0 || zp_bias > 15))
    return fail(W4A16_ERR_ZP, "zp_bias=%d must lie in 0..15", (int)zp_bias);
  if (!aligned16(a) || !aligned16(b_q) || !aligned16(scales) || !aligned16(out) ||
      (qzeros && !aligned16(qzeros)))
    return fail(W4A16_ERR_ALIGN, "device pointers must be 16-byte aligned");
  return W4A16_OK;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ---------------------------------------------------------------------------
// selector
// ---------------------------------------------------------------------------
// Decode launch: 256 columns per workgroup, 4 wavefronts of L steps each.
// L (1, 2, 4 or 8) is the smallest that keeps the wavefront count within two
// resident wavefronts per SIMD, so every wavefront streams from the start and
// none waits for a second round. Mode: fp16 with groups of 32 or 64 folds
// the scale into each weight (cheap packed fp16 ops); otherwise the scale is
// applied per group to the fp32 partial, with one group per wavefront when
// the wavefront's steps cannot straddle a group boundary.
int decode_ng_max(int64_t K, int32_t G, int64_t L, int W = w4a16::kDecodeWaves) {
  using namespace w4a16;
  if ((int64_t)G == K) return 1;
  const int64_t SG = G / kStepRows;
  return (int)std::max<int64_t>(1, (W * L) / SG + 1);
}

// Arrival counters of a split decode: one per (column block, wavefront),
// spread over the counter region as far apart as it allows, up to one per
// 128-byte line, so that the atomics on different counters do not queue on
// one line. Packed four to a line, the counter atomics of K = N = 4096 fp16
// G = 32 at M = 5 (2048 arrivals on 64 counters) took 3-4 us to return and
// the launch 14.0 us; spread, 9.6 us (M = 1, one step per wavefront: 8.7 ->
// 7.4 us).
int32_t decode_counter_stride(int64_t NB, int W) {
  using namespace w4a16;
  const int64_t slots = kCounterBytes / (int64_t)sizeof(int32_t);
  int32_t cs = 1;
  while (2 * cs <= kCounterStrideMax && 2 * cs * NB * W <= slots) cs *= 2;
  return cs;
}

// Wavefronts per workgroup of a decode launch: 8 instead of 4 halves the K
// splits (and the partials the last arrival loads) at the same wavefront
// count, where that helps: up to 8 rows, one or two steps per wavefront, at
// least 16 splits with 4 (32 at one row), and a grid that still covers every
// CU at least as evenly (whole workgroups per CU) as the 4-wavefront one.
// Measured on MI355X, 4 -> 8 wavefronts: K = N = 4096 fp16 G = 32, one step
// per wavefront, M = 1 7.3 -> 6.8 us, M = 5 8.6 -> 7.7 us; K = 5120,
// N = 17408 bf16 G = 64, two steps, M = 5 17.6 -> 15.3 us; K = N = 8192
// G = 32 M = 1 15.3 -> 14.9 us; at one row with 16-20 splits 8 lost (K =
// 2048, N = 8192: 6.6 -> 6.9 us); at the 5120 x 17408 shape with four steps
// 340 workgroups of 8 (two on some CUs, one on others) took 16.6 us against
// 12.9 us, which the evenness test keeps out.
int decode_waves(int64_t M, int64_t K, int64_t N, int64_t L, int num_cus) {
  using namespace w4a16;
  const int64_t KS = ceil_div(K, kStepRows), NB = ceil_div(N, kDecodeCols);
  const bool aligned = (N % 16 == 0) && (K % 8 == 0);
  if (!aligned || M > kAutoDecodeMaxM || L > 2) return kDecodeWaves;
  const int64_t S4 = ceil_div(KS, kDecodeWaves * L), S8 = ceil_div(KS, kDecodeWavesWide * L);
  const int64_t g4 = S4 * NB, g8 = S8 * NB;
  if (S4 < (M == 1 ? 32 : 16) || g8 < num_cus ||
      NB * kDecodeWavesWide > kCounterBytes / (int64_t)sizeof(int32_t))
    return kDecodeWaves;
  // workgroups per CU, rounded up, against the even share: 1 is perfectly even
  auto unevenness = [&](int64_t g) { return (double)ceil_div(g, num_cus) * num_cus / (double)g; };
  return unevenness(g8) <= unevenness(g4) + 1e-9 ? kDecodeWavesWide : kDecodeWaves;
}

// Steps per wavefront (L) of a decode launch when the caller leaves them
// open; *one_group tells whether the choice came from the mode 1 candidates
// below (each wavefront's steps inside one group, few splits). mode_forced
// < 0: any mode.
//
// Mode 1 comes first: it loads its scales straight into registers and folds
// once, where modes 0 and 2 stage the workgroup's scales in LDS behind a
// barrier that waits for the stream's first loads. Its candidates are the L
// whose steps fit in one group and whose K split count S stays at most 64
// at one row, 32 up to 8 rows, 16 above (each split adds partials that the
// last arrival loads), counted at the plan's wavefronts per workgroup (where
// only 8 bring S under that cap, also M * S <= 128: K = N = 8192 fp16 G = 32,
// 32 splits of 8 wavefronts against the prefill route, M = 2 14.8 vs 16.2,
// M = 4 15.8 vs 16.5 us, but M = 8 17.2 vs 16.6). Among them: the L whose grid is resident at once (3
// wavefronts per SIMD, fewer if LDS says so) and whose workgroup count is
// closest, by ratio, to max(column blocks, min(CUs, weight bytes / 32 KiB)),
// halved above 8 rows but not below 64; with none
// resident, the longest. Without a mode 1 candidate: the resident L closest
// to max(column blocks, weight bytes / 32 KiB) (halved likewise), else 8. Ties go to the
// smaller L. Measured on MI355X (graph-replayed, weights rotated), chosen
// plan against the next best: K=N=4096 fp16 G=32 M=1 L=1 7.4 us (L=2, mode
// 0: 8.3), M=5 9.3 (9.6); K=8192, N=4096 bf16 G=128 M=4 L=4 8.8 (L=2: 9.7);
// K=N=16384 fp16 G=128 M=1 L=4 31.1 (L=8, mode 2: 34.3); K=5120, N=17408
// bf16 G=64 M=5 L=2 17.2 (L=4, mode 2: 20.7); K=5120, N=17408 fp16 G=32
// M=5 L=4, mode 0, 21.1 (L=1, 40 splits: 24.9).
int64_t decode_auto_steps(int64_t M, int64_t K, int64_t N, int32_t G, int32_t dtype, int num_cus,
                          int32_t mode_forced, bool* one_group_out) {
  using namespace w4a16;
  const int64_t KS = ceil_div(K, kStepRows);
  const int64_t NB = ceil_div(N, kDecodeCols);
  const int64_t SG = ((int64_t)G == K) ? KS : G / kStepRows;
  const bool one_group = ((int64_t)G == K);
  const bool aligned = (N % 16 == 0) && (K % 8 == 0);
  auto fits_one_of = [&](int64_t l) { return one_group || (SG >= l && SG % l == 0); };
  // off the fast layout: one step per wavefront, always inside one group
  *one_group_out = true;
  if (!aligned) return 1;
  const double bytes = (double)K * (double)N / 2.0;
  // above 8 rows each split's hand-off carries twice the partials: aim at
  // half the workgroups, but not below 64 (K = N = 4096, per-channel,
  // M = 16: 4 steps per wavefront, 10.2 us, against 11.3 us with 2; K = N =
  // 2048 bf16 G = 128 M = 16: 2 steps, 7.5 us, against 8.1 with 4)
  auto aim = [&](double t) { return M > w4a16::kAutoDecodeMaxM ? std::max(t / 2.0, 64.0) : t; };
  auto resident = [&](int64_t l, int m) {
    const int64_t lds = decode_lds_bytes((int)M, decode_ng_max(K, G, (int)l));
    const int64_t by_lds = std::max<int64_t>(1, kLdsPerCu / std::max<int64_t>(1, lds));
    const int64_t per_simd = std::min<int64_t>(m == 2 ? 2 : 3, by_lds);
    return ceil_div(KS, l) * NB <= per_simd * 4 * (int64_t)num_cus;
  };
  auto closest = [&](auto&& take, double target, int64_t& L) {
    double best = 1e300;
    bool any = false;
    for (int64_t l = 1; l <= kDecodeMaxSteps; l *= 2) {
      if (!take(l)) continue;
      const double grid = (double)(ceil_div(KS, kDecodeWaves * l) * NB);
      const double d = std::fabs(std::log(grid / target));
      if (d < best - 1e-9) {
        best = d;
        L = l;
        any = true;
      }
    }
    return any;
  };
  if (mode_forced < 0 || mode_forced == 1) {
    const int64_t smax = M == 1 ? 64 : M <= w4a16::kAutoDecodeMaxM ? 32 : 16;
    // splits at the plan's own wavefront count; a candidate that only 8
    // wavefronts per workgroup bring under the cap also keeps M * S <= 128
    auto cand = [&](int64_t l) {
      if (!fits_one_of(l)) return false;
      if (mode_forced == 1 || ceil_div(KS, kDecodeWaves * l) <= smax) return true;
      const int64_t w = decode_waves(M, K, N, l, num_cus);
      const int64_t s = ceil_div(KS, w * l);
      return w == kDecodeWavesWide && s <= smax && M * s <= 128;
    };
    int64_t L = 0;
    for (int64_t l = 1; l <= kDecodeMaxSteps; l *= 2)
      if (cand(l)) L = l;  // the longest candidate
    if (L > 0) {
      *one_group_out = true;
      const double target = aim(std::max<double>((double)NB, std::min<double>((double)num_cus,
                                                                             bytes / 32768.0)));
      closest([&](int64_t l) { return cand(l) && resident(l, 1); }, target, L);
      return L;
    }
  }
  *one_group_out = false;
  auto mode_of = [&](int64_t l) {
    if (mode_forced >= 0) return (int)mode_forced;
    if (fits_one_of(l)) return 1;
    return (dtype == W4A16_F16 && G <= 64) ? 0 : 2;
  };
  int64_t L = kDecodeMaxSteps;  // nothing resident: longest streams
  const double target = aim(std::max<double>((double)NB, bytes / 32768.0));
  closest([&](int64_t l) { return (mode_of(l) != 1 || fits_one_of(l)) && resident(l, mode_of(l)); },
          target, L);
  return L;
}

w4a16_status plan_decode(int64_t M, int64_t K, int64_t N, int32_t G, int32_t dtype, int num_cus,
                         int32_t L_forced, int32_t mode_forced, w4a16_plan_t* pl) {
  using namespace w4a16;
  const int64_t KS = ceil_div(K, kStepRows);
  const int64_t NB = ceil_div(N, kDecodeCols);
  const int64_t SG = ((int64_t)G == K) ? KS : G / kStepRows;
  const bool one_group = ((int64_t)G == K);
  // shapes off the fast layout (N % 16 or K % 8 nonzero) use one step per
  // wavefront
  const bool aligned = (N % 16 == 0) && (K % 8 == 0);
  int64_t L = L_forced;
  if (L != 0 && L != 1 && L != 2 && L != 4 && L != 8)
    return fail(W4A16_ERR_PLAN, "steps per wavefront must be 1, 2, 4 or 8 (got %lld)", (long long)L);
  if (!aligned && L > 1)
    return fail(W4A16_ERR_PLAN, "N %% 16 or K %% 8 nonzero: decode runs one step per wavefront");
  auto fits_one_of = [&](int64_t l) { return one_group || (SG >= l && SG % l == 0); };
  // One group per wavefront: mode 1 (exact operand, one in-place fold after
  // the stream). Otherwise fp16 with groups of up to 64 rows feeds the rounded
  // weight (mode 0), and the rest fold per group (mode 2). (Measured on
  // MI355X: K=2112, N=5120, fp16, G=64, M=8: mode 1 9.45 us, mode 0 10.7 us;
  // K=N=4096, fp16, G=32, 2 steps per wavefront: mode 0 8.9 us, mode 2 9.6 us.)
  auto auto_mode = [&](int64_t l) {
    if (fits_one_of(l)) return 1;
    return (dtype == W4A16_F16 && G <= 64) ? 0 : 2;
  };
  if (L == 0) {
    bool in_one = false;
    L = decode_auto_steps(M, K, N, G, dtype, num_cus, mode_forced, &in_one);
  }
  int32_t mode = mode_forced;
  const bool fits_one = fits_one_of(L);
  if (mode < 0) mode = auto_mode(L);
  if (mode < 0 || mode > 2) return fail(W4A16_ERR_PLAN, "decode mode must be 0, 1 or 2");
  if (mode == 1 && !fits_one)
    return fail(W4A16_ERR_PLAN, "decode mode 1 needs the %lld steps of a wavefront inside one group",
                (long long)L);
  // Mode 0 feeds RNE_dtype((q - z) s) to the MFMA. In fp16 that is 2^-11
  // relative per weight; in bf16 (2^-8) the sum over a long K leaves the
  // 2e-2 tolerance (K = 5120, G = 32 with zero points already does), so
  // bf16 always takes the exact operand of modes 1 and 2.
  if (mode == 0 && dtype != W4A16_F16)
    return fail(W4A16_ERR_PLAN, "decode mode 0 (rounded weights) is fp16 only");
  const int W = decode_waves(M, K, N, L, num_cus);
  const int64_t S = ceil_div(KS, (int64_t)W * L);
  // the kernel addresses the split-K partials with 32-bit byte offsets
  if (S > 1 && S * M * N * 4 >= (int64_t(1) << 32))
    return fail(W4A16_ERR_PLAN, "decode split-K partials (%lld splits x %lld x %lld fp32) exceed 4 GiB",
                (long long)S, (long long)M, (long long)N);
  if (S > 1 && NB > kMaxCounterBlocks)
    return fail(W4A16_ERR_PLAN, "decode split-K needs %lld column blocks of counters (at most %lld)",
                (long long)NB, (long long)kMaxCounterBlocks);
  pl->route = W4A16_ROUTE_DECODE;
  pl->block_m = kDecodeMaxM;
  pl->block_n = kDecodeCols;
  pl->block_k = kStepRows;
  pl->decode_mode = mode;
  pl->splits = (int32_t)S;
  pl->steps_per_wave = (int32_t)L;
  pl->grid = (int32_t)(NB * S);
  pl->threads = 64 * W;
  pl->lds_bytes = decode_lds_bytes((int)M, decode_ng_max(K, G, L, W), W);
  pl->workspace_bytes = S > 1 ? (int64_t)(kCounterBytes + S * M * N * 4) : 0;
  return W4A16_OK;
}

// Prefill: 64 x 256 tiles. When there are fewer tiles than CUs, K is split
// across workgroups (whole groups per split, at least two 64-row stages
// each); each split writes an fp32 partial of the M real rows and a second,
// fully parallel kernel adds them in split order. Every split adds M x N x 8
// bytes of partial traffic, so the register-staged kernel ran best at one
// workgroup per CU (13.4 vs 14.8 us at M = 16, 32.7 vs 34.0 us at M = 256,
// K = N = 4096); the ring's 64-row tiles at two (below).
//
// Tile rows: 64, or 32 for M <= 64 when K % 64 == 0 and the launch splits
// K, so that fewer MFMA rows are padding and more workgroups fit a CU
// (K = N = 4096: M = 16 12.2 vs 13.1 us, M = 64 17.7 vs 20.0 us with 32-row
// tiles; a 2048-row prefill is faster with 64).
w4a16_status plan_prefill_bm(int64_t M, int64_t K, int64_t N, int32_t G, int32_t dtype, int num_cus,
                             int32_t ks_forced, int64_t BM, w4a16_plan_t* pl);

w4a16_status plan_prefill(int64_t M, int64_t K, int64_t N, int32_t G, int32_t dtype, int num_cus,
                          int32_t ks_forced, w4a16_plan_t* pl) {
  using namespace w4a16;
  const int64_t small = M <= 64 ? 32 : kPrefillBM;
  if (small < kPrefillBM && K % kPrefillBK == 0) {
    w4a16_plan_t q{};
    w4a16_status st = plan_prefill_bm(M, K, N, G, dtype, num_cus, ks_forced, small, &q);
    if (st != W4A16_OK) return st;
    if (q.splits > 1) {
      *pl = q;
      return W4A16_OK;
    }
  }
  return plan_prefill_bm(M, K, N, G, dtype, num_cus, ks_forced, kPrefillBM, pl);
}

w4a16_status plan_prefill_bm(int64_t M, int64_t K, int64_t N, int32_t G, int32_t dtype, int num_cus,
                             int32_t ks_forced, int64_t BM, w4a16_plan_t* pl) {
  using namespace w4a16;
  const int64_t tm = ceil_div(M, BM), tn = ceil_div(N, kPrefillBN);
  const int64_t tiles = tm * tn;
  const int64_t KT = ceil_div(K, kPrefillBK);
  const int64_t unit = ((int64_t)G != K && G == 128) ? 2 : 1;  // stages per group
  int64_t S = 1, ks = KT;
  // fewer tiles than CUs: split to about one workgroup per CU for 32-row
  // tiles, two for 64-row ring tiles (K = N = 4096, M = 256, 64 tiles: 8
  // splits 34.0 us, 4 splits 35.9 us; M = 16 and 64 on 32-row tiles are
  // fastest at 16 and 8 splits)
  const int64_t want = (int64_t)num_cus * ((BM == kPrefillBM && prefill_ring_ok(K, N, BM)) ? 2 : 1);
  if (ks_forced != 0) {
    if (ks_forced < 0 || ks_forced % unit != 0)
      return fail(W4A16_ERR_PLAN, "prefill stages per workgroup must be a positive multiple of %lld",
                  (long long)unit);
    ks = std::min<int64_t>(ks_forced, KT);
    S = ceil_div(KT, ks);
    if (S > kPrefillMaxSplits)
      return fail(W4A16_ERR_PLAN, "%lld stages per workgroup give %lld K splits (at most %d)",
                  (long long)ks_forced, (long long)S, kPrefillMaxSplits);
    if (S == 1) ks = KT;
  } else if (tiles < (int64_t)num_cus) {
    const int64_t s_max = std::max<int64_t>(1, std::min<int64_t>(kPrefillMaxSplits, KT / (2 * unit)));
    const int64_t s0 = std::min<int64_t>(s_max, ceil_div(want, tiles));
    if (s0 > 1) {
      ks = ceil_div(ceil_div(KT, s0), unit) * unit;
      S = ceil_div(KT, ks);
    }
  }
  const int64_t units = tiles * S;
  const int64_t per_xcd = ceil_div(units, kXcds);
  pl->route = W4A16_ROUTE_PREFILL;
  pl->block_m = (int32_t)BM;
  pl->block_n = kPrefillBN;
  pl->block_k = kPrefillBK;
  pl->decode_mode = 0;
  pl->splits = (int32_t)S;
  pl->steps_per_wave = (int32_t)ks;
  pl->grid = (int32_t)(per_xcd * kXcds);
  pl->threads = kPrefillThreads;
  pl->lds_bytes = prefill_ring_ok(K, N, BM) ? prefill_ring_lds_bytes(K, G, BM) : prefill_lds_bytes((int)BM);
  // K splits: counter region, then the fp32 partials; bf16 through the ring
  // without splits: counter region, then the precomputed activation sums
  pl->workspace_bytes = S > 1 ? (int64_t)(kCounterBytes + S * M * N * 4)
                        : prefill_asum_pre(K, N, G, dtype, BM, S)
                            ? (int64_t)(kCounterBytes + prefill_asum_bytes(M, K, G))
                            : 0;
  return W4A16_OK;
}

w4a16_status make_plan(int64_t M, int64_t K, int64_t N, int32_t G, int32_t dtype, int32_t num_cus,
                       int32_t route, int32_t L, int32_t mode, w4a16_plan_t* pl) {
  if (!pl) return fail(W4A16_ERR_NULL, "plan must be non-NULL");
  w4a16_status st = check_shape(M, K, N, G, dtype);
  if (st != W4A16_OK) return st;
  std::memset(pl, 0, sizeof(*pl));
  if (num_cus <= 0) num_cus = 256;
  if (M == 0) {
    pl->route = W4A16_ROUTE_NONE;
    return W4A16_OK;
  }
  // Decode for M <= 8, and up to 16 rows for per-channel scales (one group)
  // or where the decode keeps each wavefront's 2 or more steps inside one
  // group (mode 1, above; M = 16: K = 5120, N = 17408 bf16 G = 128 18.7 vs
  // 21.3 us, K = 8192, N = 4096 11.2 vs 12.7 us; M = 12, K = 4096, N = 14336
  // 13.1 vs 17.7 us; groups of 32 stay on the prefill: K = N = 4096 fp16
  // M = 16 11.3 vs 11.5 us), except where from 2 rows on, with few column tiles (N <= 8192), the
  // decode cannot keep each wavefront's steps inside one group at few enough
  // K splits (mode 1, above): there the prefill route's K split through the
  // LDS ring (32-row tiles) is faster. Measured graph-replayed on MI355X,
  // decode against prefill: K = N = 4096 fp16 G = 32 M = 2 7.6 vs 9.5, M = 5
  // 9.3 vs 9.6 us; K = 2112, N = 5120 fp16 G = 64 M = 8 7.6 vs 8.5; K = 8192,
  // N = 4096 bf16 G = 128 M = 4 8.8 vs 11.2; per-channel K = N = 4096 M = 16
  // 10.2 vs 10.7; K = N = 8192 bf16 G = 128 M = 8 14.6 vs 15.0; sent to the
  // prefill: K = N = 8192 fp16 G = 32 M = 8 (mode 1 would take 32 splits of
  // 8 wavefronts, over the M * S cap above) 17.0 against 17.2 (mode 1) and
  // 17.6 (mode 0, 2 steps). (N beyond what the
  // counter region serves, 2^20 columns, has column blocks enough to fill
  // the GPU on the prefill route's tiles.)
  if (route == 0) {
    const bool counters_ok = ceil_div(N, w4a16::kDecodeCols) <= w4a16::kMaxCounterBlocks;
    bool in_one = false;
    const int64_t L_auto = M <= w4a16::kDecodeMaxM
                               ? decode_auto_steps(M, K, N, G, dtype, num_cus, -1, &in_one)
                               : 0;
    bool decode = counters_ok && (M <= w4a16::kAutoDecodeMaxM ||
                                  (M <= w4a16::kDecodeMaxM && ((int64_t)G == K || (in_one && L_auto >= 2))));
    if (decode && M >= 2 && N <= 8192 && w4a16::prefill_ring_ok(K, N, 32) && !in_one) decode = false;
    route = decode ? W4A16_ROUTE_DECODE : W4A16_ROUTE_PREFILL;
  }
  if (route == W4A16_ROUTE_DECODE) {
    if (M > w4a16::kDecodeMaxM)
      return fail(W4A16_ERR_PLAN, "decode route needs M <= %d (got %lld)", w4a16::kDecodeMaxM,
                  (long long)M);
    st = plan_decode(M, K, N, G, dtype, num_cus, L, mode, pl);
    if (st != W4A16_OK) return st;
  } else if (route == W4A16_ROUTE_PREFILL) {
    st = plan_prefill(M, K, N, G, dtype, num_cus, L, pl);
    if (st != W4A16_OK) return st;
  } else {
    return fail(W4A16_ERR_PLAN, "unknown route %d", (int)route);
  }
  return W4A16_OK;
}

// A caller-supplied plan must be one the selector could have produced.
w4a16_status check_plan(const w4a16_plan_t* pl, int64_t M, int64_t K, int64_t N, int32_t G,
                        int32_t dtype) {
  w4a16_plan_t ref;
  w4a16_status st = make_plan(M, K, N, G, dtype, 256, pl->route, pl->steps_per_wave,
                              pl->route == W4A16_ROUTE_DECODE ? pl->decode_mode : -1, &ref);
  if (st != W4A16_OK) return st;
  if (std::memcmp(&ref, pl, sizeof(ref)) != 0)
    return fail(W4A16_ERR_PLAN, "plan does not match the problem (route %d)", (int)pl->route);
  return W4A16_OK;
}

// ---------------------------------------------------------------------------
// per-device state: architecture check, CU count, LDS limit, and the
// library's own per-stream workspaces (for the calls without one)
// ---------------------------------------------------------------------------
struct StreamWs {
  void* ptr = nullptr;
  size_t bytes = 0;
};
struct DeviceState {
  bool probed = false;
  bool ok = false;
  int num_cus = 0;
  size_t lds_per_block = 0;
  std::map<hipStream_t, StreamWs> ws;  // one workspace per stream
  std::vector<void*> retired;          // outgrown workspaces, kept until exit
};
std::mutex g_mu;
std::vector<DeviceState> g_dev;

w4a16_status device_state(DeviceState** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return fail(W4A16_ERR_DEVICE, "no HIP device available");
  }
  std::lock_guard<std::mutex> lk(g_mu);
  if ((int)g_dev.size() <= dev) g_dev.resize(dev + 1);
  DeviceState& ds = g_dev[dev];
  if (!ds.probed) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      (void)hipGetLastError();
      return fail(W4A16_ERR_DEVICE, "hipGetDeviceProperties failed for device %d", dev);
    }
    ds.probed = true;
    ds.ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    ds.num_cus = prop.multiProcessorCount;
    ds.lds_per_block = prop.sharedMemPerBlock;
  }
  if (!ds.ok) return fail(W4A16_ERR_DEVICE, "device %d is not a gfx950 (MI355X) GPU", dev);
  *out = &ds;
  return W4A16_OK;
}

// The library's workspace of `stream`, grown to at least `bytes`. Growing
// allocates a new buffer and clears its counter region on `stream` (ordered
// before the launch that needs it); the old buffer stays allocated, because
// a graph captured earlier or a launch still queued may use it. Nothing
// here synchronises. While the stream is being captured, growing would put
// an allocation and a memset node into the graph: refused instead.
w4a16_status stream_workspace(DeviceState* ds, hipStream_t stream, size_t bytes, void** ptr) {
  std::lock_guard<std::mutex> lk(g_mu);
  StreamWs& w = ds->ws[stream];
  if (w.bytes >= bytes) {
    *ptr = w.ptr;
    return W4A16_OK;
  }
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cs) != hipSuccess) {
    (void)hipGetLastError();
    cs = hipStreamCaptureStatusActive;  // e.g. the null stream while another captures
  }
  if (cs != hipStreamCaptureStatusNone)
    return fail(W4A16_ERR_WORKSPACE,
                "the launch needs %zu bytes of scratch and the stream's workspace holds %zu; it "
                "cannot grow while the stream is captured (run the problem once uncaptured, or "
                "pass a workspace to w4a16_gemm_ws)",
                bytes, w.bytes);
  const size_t sz = std::max<size_t>({bytes, 2 * w.bytes, (size_t)8 << 20});
  void* p = nullptr;
  if (hipMalloc(&p, sz) != hipSuccess) {
    (void)hipGetLastError();
    return fail(W4A16_ERR_HIP, "hipMalloc of %zu bytes of split-K scratch failed", sz);
  }
  if (hipMemsetAsync(p, 0, (size_t)w4a16::kCounterBytes, stream) != hipSuccess) {
    (void)hipGetLastError();
    (void)hipFree(p);
    return fail(W4A16_ERR_HIP, "clearing the arrival counters failed");
  }
  if (w.ptr) ds->retired.push_back(w.ptr);
  w.ptr = p;
  w.bytes = sz;
  *ptr = p;
  return W4A16_OK;
}

// One launch of `pl` with its scratch at `ws` (at least pl.workspace_bytes,
// counter region zero; unused when the plan needs none).
w4a16_status run(const w4a16::GemmArgs& g, const w4a16_plan_t& pl, void* ws, hipStream_t stream) {
  using namespace w4a16;
  hipError_t e = hipSuccess;
  if (pl.route == W4A16_ROUTE_NONE) return W4A16_OK;
  int32_t* counters = (int32_t*)ws;
  float* partials = ws ? (float*)((char*)ws + kCounterBytes) : nullptr;
  if (pl.route == W4A16_ROUTE_DECODE) {
    DecodeParams p{};
    p.dq = dq_consts(g.dtype);
    p.a = (const uint16_t*)g.a;
    p.bq = (const uint32_t*)g.b_q;
    p.sc = (const uint16_t*)g.scales;
    p.qz = (const uint32_t*)g.qzeros;
    p.bias = (const uint16_t*)g.bias;
    p.out = (uint16_t*)g.out;
    p.M = (int32_t)g.M;
    p.K = (int32_t)g.K;
    p.N = (int32_t)g.N;
    p.G = g.G;
    p.zp_bias = g.zp_bias;
    p.KS = (int32_t)ceil_div(g.K, kStepRows);
    p.SG = ((int64_t)g.G == g.K) ? p.KS : g.G / kStepRows;
    p.sg_shift = ((int64_t)g.G == g.K) ? -1 : (g.G == 32 ? 0 : g.G == 64 ? 1 : 2);
    p.W = pl.threads / 64;
    p.ng_max = decode_ng_max(g.K, g.G, pl.steps_per_wave, p.W);
    p.L = pl.steps_per_wave;
    p.S = pl.splits;
    p.NB = (int32_t)ceil_div(g.N, kDecodeCols);
    if (pl.splits > 1) {
      p.ws = partials;
      p.counters = counters;
      p.cstride = decode_counter_stride(p.NB, p.W);
    }
    e = launch_decode(p, g.dtype, g.qzeros != nullptr, pl.decode_mode, pl.grid, pl.lds_bytes,
                      stream);
  } else {
    PrefillParams p{};
    p.dq = dq_consts(g.dtype);
    p.a = (const uint16_t*)g.a;
    p.bq = (const uint32_t*)g.b_q;
    p.sc = (const uint16_t*)g.scales;
    p.qz = (const uint32_t*)g.qzeros;
    p.bias = pl.splits > 1 ? nullptr : (const uint16_t*)g.bias;  // split: the reduction adds it
    p.out = (uint16_t*)g.out;
    p.M = (int32_t)g.M;
    p.K = (int32_t)g.K;
    p.N = (int32_t)g.N;
    p.G = g.G;
    p.zp_bias = g.zp_bias;
    p.g_shift = g.G == 32 ? 5 : g.G == 64 ? 6 : g.G == 128 ? 7 : 0;
    p.bm = pl.block_m;
    p.ring = prefill_ring_ok(g.K, g.N, pl.block_m) ? 1 : 0;
    if (prefill_asum_pre(g.K, g.N, g.G, g.dtype, pl.block_m, pl.splits)) {
      AsumParams ap{};
      ap.a = (const uint16_t*)g.a;
      ap.out = (float*)((char*)ws + kCounterBytes);
      ap.M = (int32_t)g.M;
      ap.K = (int32_t)g.K;
      ap.G = g.G;
      ap.rows = (int32_t)prefill_asum_rows(g.M);
      ap.scale = (g.qzeros == nullptr && g.G != g.K) ? -(128.0f + (float)g.zp_bias) : 1.0f;
      e = launch_asum(ap, stream);
      if (e != hipSuccess)
        return fail(W4A16_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
      p.asum = ap.out;
      p.asum_rows = ap.rows;
    }
    p.tiles_m = (int32_t)ceil_div(g.M, pl.block_m);
    p.tiles_n = (int32_t)ceil_div(g.N, kPrefillBN);
    p.tiles = p.tiles_m * p.tiles_n;
    p.per_xcd = pl.grid / kXcds;
    p.band = (int32_t)std::min<int64_t>(kPrefillBand, p.tiles_m);
    p.S = pl.splits;
    p.kt_split = pl.steps_per_wave;
    if (pl.splits > 1) p.ws = partials;
    e = launch_prefill(p, g.dtype, g.qzeros != nullptr, pl.grid, stream);
    if (e == hipSuccess && pl.splits > 1) {
      PrefillReduceParams r{};
      r.ws = partials;
      r.bias = (const uint16_t*)g.bias;
      r.out = (uint16_t*)g.out;
      r.M = (int32_t)g.M;
      r.N = (int32_t)g.N;
      r.S = pl.splits;
      e = launch_prefill_reduce(r, g.dtype, stream);
    }
  }
  if (e != hipSuccess) return fail(W4A16_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return W4A16_OK;
}

// Where a call's scratch comes from.
enum class WsMode { Library, Caller, Static };

w4a16_status gemm_common(const void* a, const int32_t* b_q, const void* scales,
                         const int32_t* qzeros, int32_t G, int32_t zp_bias, const void* bias,
                         void* out, int64_t M, int64_t K, int64_t N, int32_t dtype,
                         const w4a16_plan_t* forced, void* stream, WsMode wsm = WsMode::Library,
                         void* ws = nullptr, int64_t ws_bytes = 0) {
  w4a16_status st = check_shape(M, K, N, G, dtype);
  if (st != W4A16_OK) return st;
  if (M == 0) return W4A16_OK;
  st = check_ptrs(a, b_q, scales, qzeros, out, zp_bias);
  if (st != W4A16_OK) return st;
  if (bias && !aligned16(bias)) return fail(W4A16_ERR_ALIGN, "bias must be 16-byte aligned");
  if (wsm == WsMode::Caller) {
    if (ws_bytes < 0) return fail(W4A16_ERR_WORKSPACE, "ws_bytes must be >= 0");
    if (ws && !aligned16(ws)) return fail(W4A16_ERR_ALIGN, "workspace must be 16-byte aligned");
  }
  if (forced) {
    st = check_plan(forced, M, K, N, G, dtype);
    if (st != W4A16_OK) return st;
  }
  // a caller's workspace is checked against the plan for 256 CUs before
  // any device call (so the check runs without a GPU), and again below
  // against the plan for the current device's CU count
  auto check_ws = [&](const w4a16_plan_t& q) -> w4a16_status {
    if (wsm != WsMode::Caller || q.workspace_bytes == 0) return W4A16_OK;
    if (!ws)
      return fail(W4A16_ERR_NULL, "the launch needs %lld bytes of workspace and none was given",
                  (long long)q.workspace_bytes);
    if (ws_bytes < q.workspace_bytes)
      return fail(W4A16_ERR_WORKSPACE, "the launch needs %lld bytes of workspace, %lld given",
                  (long long)q.workspace_bytes, (long long)ws_bytes);
    return W4A16_OK;
  };
  if (wsm == WsMode::Static) {  // the fixed array's size, checked without a device
    w4a16_plan_t pre;
    st = make_plan(M, K, N, G, dtype, 256, 0, 0, -1, &pre);
    if (st != W4A16_OK) return st;
    if (pre.workspace_bytes > w4a16::kStaticScratchBytes)
      return fail(W4A16_ERR_WORKSPACE,
                  "the launch needs %lld bytes of scratch; the fixed array holds %lld",
                  (long long)pre.workspace_bytes, (long long)w4a16::kStaticScratchBytes);
  }
  if (wsm == WsMode::Caller) {
    w4a16_plan_t pre;
    if (forced) {
      pre = *forced;
    } else {
      st = make_plan(M, K, N, G, dtype, 256, 0, 0, -1, &pre);
      if (st != W4A16_OK) return st;
    }
    st = check_ws(pre);
    if (st != W4A16_OK) return st;
  }
  DeviceState* ds = nullptr;
  st = device_state(&ds);
  if (st != W4A16_OK) return st;
  w4a16_plan_t pl;
  if (forced) {
    pl = *forced;
  } else {
    st = make_plan(M, K, N, G, dtype, ds->num_cus, 0, 0, -1, &pl);
    if (st != W4A16_OK) return st;
  }
  if (const char* lg = std::getenv("W4A16_LOG")) {
    if (lg[0] == '1')
      std::fprintf(stderr,
                   "[w4a16] M=%lld K=%lld N=%lld G=%d route=%d bm=%d splits=%d L=%d mode=%d grid=%d\n",
                   (long long)M, (long long)K, (long long)N, (int)G, pl.route, pl.block_m, pl.splits,
                   pl.steps_per_wave, pl.decode_mode, pl.grid);
  }
  void* scratch = nullptr;
  if (pl.workspace_bytes > 0) {
    if (wsm == WsMode::Caller) {
      st = check_ws(pl);
      if (st != W4A16_OK) return st;
      scratch = ws;
    } else if (wsm == WsMode::Static) {
      if (pl.workspace_bytes > w4a16::kStaticScratchBytes)
        return fail(W4A16_ERR_WORKSPACE,
                    "the launch needs %lld bytes of scratch; the fixed array holds %lld",
                    (long long)pl.workspace_bytes, (long long)w4a16::kStaticScratchBytes);
      const hipError_t e = w4a16::static_scratch((hipStream_t)stream, &scratch);
      if (e != hipSuccess)
        return fail(W4A16_ERR_HIP, "fixed scratch array: %s", hipGetErrorString(e));
    } else {
      st = stream_workspace(ds, (hipStream_t)stream, (size_t)pl.workspace_bytes, &scratch);
      if (st != W4A16_OK) return st;
    }
  }
  w4a16::GemmArgs g{a, b_q, scales, qzeros, bias, out, M, K, N, G, zp_bias, dtype};
  return run(g, pl, scratch, (hipStream_t)stream);
}

}  // namespace

extern "C" {

w4a16_status w4a16_gemm(const void* a, const int32_t* b_q, const void* scales,
                        const int32_t* qzeros, int32_t group_size, int32_t zp_bias, void* out,
                        int64_t M, int64_t K, int64_t N, int32_t dtype, void* stream) {
  return gemm_common(a, b_q, scales, qzeros, group_size, zp_bias, nullptr, out, M, K, N, dtype,
                     nullptr, stream);
}

w4a16_status w4a16_gemm_bias(const void* a, const int32_t* b_q, const void* scales,
                             const int32_t* qzeros, int32_t group_size, int32_t zp_bias,
                             const void* bias, void* out, int64_t M, int64_t K, int64_t N,
                             int32_t dtype, void* stream) {
  return gemm_common(a, b_q, scales, qzeros, group_size, zp_bias, bias, out, M, K, N, dtype,
                     nullptr, stream);
}

w4a16_status w4a16_gemm_planned(const void* a, const int32_t* b_q, const void* scales,
                                const int32_t* qzeros, int32_t group_size, int32_t zp_bias,
                                void* out, int64_t M, int64_t K, int64_t N, int32_t dtype,
                                const w4a16_plan_t* plan, void* stream) {
  if (!plan) return fail(W4A16_ERR_NULL, "plan must be non-NULL");
  return gemm_common(a, b_q, scales, qzeros, group_size, zp_bias, nullptr, out, M, K, N, dtype,
                     plan, stream);
}

w4a16_status w4a16_workspace_bytes(int64_t M, int64_t K, int64_t N, int32_t group_size,
                                   int32_t dtype, int32_t num_cus, int64_t* bytes) {
  if (!bytes) return fail(W4A16_ERR_NULL, "bytes must be non-NULL");
  w4a16_plan_t pl;
  w4a16_status st = make_plan(M, K, N, group_size, dtype, num_cus, 0, 0, -1, &pl);
  if (st != W4A16_OK) return st;
  *bytes = pl.workspace_bytes;
  return W4A16_OK;
}

w4a16_status w4a16_gemm_ws(const void* a, const int32_t* b_q, const void* scales,
                           const int32_t* qzeros, int32_t group_size, int32_t zp_bias,
                           const void* bias, void* out, int64_t M, int64_t K, int64_t N,
                           int32_t dtype, void* workspace, int64_t ws_bytes, void* stream) {
  return gemm_common(a, b_q, scales, qzeros, group_size, zp_bias, bias, out, M, K, N, dtype,
                     nullptr, stream, WsMode::Caller, workspace, ws_bytes);
}

w4a16_status w4a16_gemm_noalloc(const void* a, const int32_t* b_q, const void* scales,
                                const int32_t* qzeros, int32_t group_size, int32_t zp_bias,
                                const void* bias, void* out, int64_t M, int64_t K, int64_t N,
                                int32_t dtype, void* stream) {
  return gemm_common(a, b_q, scales, qzeros, group_size, zp_bias, bias, out, M, K, N, dtype,
                     nullptr, stream, WsMode::Static);
}

w4a16_status w4a16_plan(int64_t M, int64_t K, int64_t N, int32_t group_size, int32_t has_zp,
                        int32_t dtype, int32_t num_cus, w4a16_plan_t* plan) {
  (void)has_zp;
  return make_plan(M, K, N, group_size, dtype, num_cus, 0, 0, -1, plan);
}

w4a16_status w4a16_plan_route(int64_t M, int64_t K, int64_t N, int32_t group_size, int32_t has_zp,
                              int32_t dtype, int32_t num_cus, int32_t route, int32_t steps_per_wave,
                              int32_t decode_mode, w4a16_plan_t* plan) {
  (void)has_zp;
  if (route != W4A16_ROUTE_DECODE && route != W4A16_ROUTE_PREFILL)
    return fail(W4A16_ERR_PLAN, "route must be decode (1) or prefill (2), got %d", (int)route);
  return make_plan(M, K, N, group_size, dtype, num_cus, route, steps_per_wave, decode_mode, plan);
}

w4a16_status w4a16_dequant(const int32_t* b_q, const void* scales, const int32_t* qzeros,
                           int32_t group_size, int32_t zp_bias, void* w_out, int64_t K, int64_t N,
                           int32_t dtype, void* stream) {
  w4a16_status st = check_shape(1, K, N, group_size, dtype);
  if (st != W4A16_OK) return st;
  if (!b_q || !scales || !w_out) return fail(W4A16_ERR_NULL, "b_q, scales and w_out must be non-NULL");
  if (!qzeros && (zp_bias < 0 || zp_bias > 15))
    return fail(W4A16_ERR_ZP, "zp_bias=%d must lie in 0..15", (int)zp_bias);
  if (!aligned16(b_q) || !aligned16(scales) || !aligned16(w_out) || (qzeros && !aligned16(qzeros)))
    return fail(W4A16_ERR_ALIGN, "device pointers must be 16-byte aligned");
  DeviceState* ds = nullptr;
  st = device_state(&ds);
  if (st != W4A16_OK) return st;
  w4a16::DequantParams p{w4a16::dq_consts(dtype), (const uint32_t*)b_q,  (const uint16_t*)scales,
                         (const uint32_t*)qzeros,   (uint16_t*)w_out,       (int32_t)K,
                         (int32_t)N,                group_size,             zp_bias};
  hipError_t e = w4a16::launch_dequant(p, dtype, qzeros != nullptr, (hipStream_t)stream);
  if (e != hipSuccess) return fail(W4A16_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return W4A16_OK;
}

w4a16_status w4a16_pack_int4(const uint8_t* q, int64_t rows, int64_t cols, int32_t* packed) {
  if (rows < 0 || cols < 0 || cols % 8 != 0)
    return fail(W4A16_ERR_SHAPE, "need rows >= 0 and cols a non-negative multiple of 8");
  if (rows * cols == 0) return W4A16_OK;
  if (!q || !packed) return fail(W4A16_ERR_NULL, "q and packed must be non-NULL");
  const int64_t words = cols / 8;
  for (int64_t r = 0; r < rows; ++r) {
    const uint8_t* src = q + r * cols;
    int32_t* dst = packed + r * words;
    for (int64_t w = 0; w < words; ++w) {
      uint32_t v = 0;
      for (int j = 0; j < 8; ++j) {
        const uint8_t x = src[8 * w + j];
        if (x > 15)
          return fail(W4A16_ERR_VALUE, "value %u at (%lld, %lld) is outside 0..15", (unsigned)x,
                      (long long)r, (long long)(8 * w + j));
        v |= (uint32_t)x << (4 * j);
      }
      dst[w] = (int32_t)v;
    }
  }
  return W4A16_OK;
}

w4a16_status w4a16_unpack_int4(const int32_t* packed, int64_t rows, int64_t cols, uint8_t* q) {
  if (rows < 0 || cols < 0 || cols % 8 != 0)
    return fail(W4A16_ERR_SHAPE, "need rows >= 0 and cols a non-negative multiple of 8");
  if (rows * cols == 0) return W4A16_OK;
  if (!q || !packed) return fail(W4A16_ERR_NULL, "q and packed must be non-NULL");
  const int64_t words = cols / 8;
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t w = 0; w < words; ++w) {
      const uint32_t v = (uint32_t)packed[r * words + w];
      for (int j = 0; j < 8; ++j) q[r * cols + 8 * w + j] = (uint8_t)((v >> (4 * j)) & 0xFu);
    }
  return W4A16_OK;
}

w4a16_status w4a16_gemm_kpacked(const void* a, const int32_t* w, const void* scales,
                                const uint8_t* zeros, int32_t group_size, int32_t zp_bias,
                                const void* bias, void* out, int64_t M, int64_t K, int64_t N,
                                int32_t dtype, void* stream) {
  if (dtype != W4A16_F16 && dtype != W4A16_BF16)
    return fail(W4A16_ERR_DTYPE, "dtype %d: only fp16 (0) and bf16 (1) activations are supported",
                (int)dtype);
  if (M < 0 || K <= 0 || N <= 0)
    return fail(W4A16_ERR_SHAPE, "need M >= 0, K > 0, N > 0 (got M=%lld K=%lld N=%lld)",
                (long long)M, (long long)K, (long long)N);
  if (K % 32 != 0)
    return fail(W4A16_ERR_SHAPE, "K=%lld must be a multiple of 32 for the K-packed layout",
                (long long)K);
  if (!(group_size == 32 || group_size == 64 || group_size == 128 || group_size == K))
    return fail(W4A16_ERR_GROUP, "group size %d not supported (32, 64, 128 or K=%lld)",
                (int)group_size, (long long)K);
  if (K % group_size != 0)
    return fail(W4A16_ERR_SHAPE, "K=%lld is not a multiple of group size %d", (long long)K,
                (int)group_size);
  if (K > (1ll << 24) || M * K >= (1ll << 31) || M * N >= (1ll << 31) ||
      N * (K / 8) >= (1ll << 31) || M > 65535ll * w4a16::kKpRows)
    return fail(W4A16_ERR_SHAPE, "problem too large for 32-bit row/column indexing");
  if (M == 0) return W4A16_OK;
  if (!a || !w || !scales || !out)
    return fail(W4A16_ERR_NULL, "a, w, scales and out must be non-NULL");
  if (!zeros && (zp_bias < 0 || zp_bias > 15))
    return fail(W4A16_ERR_ZP, "zp_bias=%d must lie in 0..15", (int)zp_bias);
  if (!aligned16(a) || !aligned16(w) || !aligned16(scales) || !aligned16(out) ||
      (bias && !aligned16(bias)))
    return fail(W4A16_ERR_ALIGN, "device pointers (zeros excepted) must be 16-byte aligned");
  DeviceState* ds = nullptr;
  w4a16_status st = device_state(&ds);
  if (st != W4A16_OK) return st;
  // activation rows go to LDS when they fit the staging limit and, with the
  // kernel's static reduction array, the device's LDS per workgroup
  const size_t stage_lds = w4a16::kpacked_lds_bytes(M, K);
  const bool stage = stage_lds <= (size_t)w4a16::kKpLdsStageMax &&
                     stage_lds + w4a16::kKpRedBytes <= ds->lds_per_block;
  w4a16::KPackedParams p{};
  p.dq = w4a16::dq_consts(dtype);
  p.a = (const uint16_t*)a;
  p.w = (const uint32_t*)w;
  p.sc = (const uint16_t*)scales;
  p.zp = zeros;
  p.bias = (const uint16_t*)bias;
  p.out = (uint16_t*)out;
  p.M = (int32_t)M;
  p.K = (int32_t)K;
  p.N = (int32_t)N;
  p.G = group_size;
  p.zp_bias = zp_bias;
  p.g_shift = group_size == K ? -1 : (group_size == 32 ? 0 : group_size == 64 ? 1 : 2);
  const int64_t rounds = (K / 32 + 3) / 4;
  p.rpw = (int32_t)ceil_div(rounds, w4a16::kKpThreads / 64);
  // a 128-K round stays inside one group when G is a multiple of 128 or the
  // whole of K: the scale can then multiply fp32 round sums
  const bool fold = group_size % 128 == 0 || group_size == K;
  hipError_t e =
      w4a16::launch_kpacked(p, dtype, zeros != nullptr, fold, stage, (hipStream_t)stream);
  if (e != hipSuccess) return fail(W4A16_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return W4A16_OK;
}

w4a16_status w4a16_pack_int4_kshuffle(const uint8_t* q, int64_t N, int64_t K, int32_t* packed) {
  if (N < 0 || K < 0 || K % 8 != 0)
    return fail(W4A16_ERR_SHAPE, "need N >= 0 and K a non-negative multiple of 8");
  if (N * K == 0) return W4A16_OK;
  if (!q || !packed) return fail(W4A16_ERR_NULL, "q and packed must be non-NULL");
  // nibble p of a word holds K offset 2p (p < 4) or 2(p - 4) + 1 (p >= 4)
  for (int64_t n = 0; n < N; ++n)
    for (int64_t c = 0; c < K / 8; ++c) {
      const uint8_t* src = q + n * K + 8 * c;
      uint32_t v = 0;
      for (int p = 0; p < 8; ++p) {
        const int off = p < 4 ? 2 * p : 2 * (p - 4) + 1;
        if (src[off] > 15)
          return fail(W4A16_ERR_VALUE, "value %u at (%lld, %lld) is outside 0..15",
                      (unsigned)src[off], (long long)n, (long long)(8 * c + off));
        v |= (uint32_t)src[off] << (4 * p);
      }
      packed[n * (K / 8) + c] = (int32_t)v;
    }
  return W4A16_OK;
}

w4a16_status w4a16_unpack_int4_kshuffle(const int32_t* packed, int64_t N, int64_t K, uint8_t* q) {
  if (N < 0 || K < 0 || K % 8 != 0)
    return fail(W4A16_ERR_SHAPE, "need N >= 0 and K a non-negative multiple of 8");
  if (N * K == 0) return W4A16_OK;
  if (!q || !packed) return fail(W4A16_ERR_NULL, "q and packed must be non-NULL");
  for (int64_t n = 0; n < N; ++n)
    for (int64_t c = 0; c < K / 8; ++c) {
      const uint32_t v = (uint32_t)packed[n * (K / 8) + c];
      for (int p = 0; p < 8; ++p)
        q[n * K + 8 * c + (p < 4 ? 2 * p : 2 * (p - 4) + 1)] = (uint8_t)((v >> (4 * p)) & 0xFu);
    }
  return W4A16_OK;
}

const char* w4a16_last_error(void) { return g_last_error.c_str(); }

const char* w4a16_version(void) { return "w4a16-gfx950 0.1.0"; }

}  // extern "C"
