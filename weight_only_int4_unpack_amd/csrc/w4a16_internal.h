// Internal interface between the host side (validation, selector, launches)
// and the gfx950 kernels. Every tile constant lives here once, so the host's
// LDS accounting and the kernels' arrays cannot drift apart (PR #40977,
// Review section: a hard-coded LDS size disagreed with the host-side check).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/w4a16.h"

namespace w4a16 {

// ---- decode route (skinny split-K, MFMA 16x16x32 with M padded to 16)
constexpr int kDecodeMaxM = 16;        // rows of one MFMA tile
constexpr int kDecodeCols = 256;       // output columns per workgroup
constexpr int kDecodeWaves = 4;        // wavefronts per workgroup
constexpr int kDecodeWavesWide = 8;    // ... on small shapes at one or two steps per wavefront
constexpr int kDecodeThreads = 64 * kDecodeWaves;
constexpr int kStepRows = 32;          // K rows per MFMA step
constexpr int kDecodeMaxSteps = 8;     // most 32-row steps one wavefront streams
constexpr int kAutoDecodeMaxM = 8;     // selector: decode for 1 <= M <= this (prefill with K splits wins above)

// ---- prefill route (tiled MFMA)
constexpr int kPrefillBM = 64;         // rows per workgroup tile (32 for few rows, with K splits)
constexpr int kPrefillBN = 256;        // output columns per workgroup (4 waves x 64)
constexpr int kPrefillBK = 64;         // K rows per pipeline stage
constexpr int kPrefillThreads = 256;
constexpr int kPrefillLdsRowHalves = kPrefillBK + 16;  // A-tile row: 160 B, no bank conflicts for the b128 operand reads

constexpr int kPrefillBand = 8;         // tile rows per band of the tile order
constexpr int kPrefillMaxSplits = 32;   // most K splits of one prefill tile
constexpr int kXcds = 8;                // MI355X: workgroups round-robin over 8 XCDs
constexpr int64_t kLdsPerCu = 160 * 1024;  // gfx950 LDS per CU

// ---- scratch memory of the split-K routes. Every workspace (the caller's,
// the library's per-stream one, the fixed device array) starts with a region
// of arrival counters that must be zero before first use and that every
// completed launch leaves zero; the fp32 partials follow it, so that no
// launch ever writes partials where another expects zeroed counters.
constexpr int64_t kCounterBytes = W4A16_WORKSPACE_COUNTER_BYTES;
// decode column blocks the region serves: one int32 counter per wavefront each
constexpr int64_t kMaxCounterBlocks = kCounterBytes / (kDecodeWaves * (int64_t)sizeof(int32_t));
// most int32 slots between consecutive counters (one counter per 128 B line)
constexpr int32_t kCounterStrideMax = 32;
// the fixed device array of the entry point that allocates nothing
constexpr int64_t kStaticPartialBytes = 32ll << 20;
constexpr int64_t kStaticScratchBytes = kCounterBytes + kStaticPartialBytes;
static_assert(kStaticScratchBytes == W4A16_NOALLOC_SCRATCH_BYTES, "header and library agree");

// partial sums of the W wavefronts, then the staged scales (halves) and
// packed zero points (words) of at most ng_max groups
inline int decode_lds_bytes(int M, int ng_max, int W = kDecodeWaves) {
  return W * M * kDecodeCols * (int)sizeof(float) + ng_max * kDecodeCols * 2 +
         ng_max * (kDecodeCols / 8) * 4;
}
inline int prefill_lds_bytes(int bm) {
  return 2 * bm * kPrefillLdsRowHalves * 2;
}
// Prefill through an LDS ring: every operand of a 64-row K stage (activation
// tile, packed weight tile, the group's scales, zero points and precomputed
// activation sums) is copied by the load units straight into one of
// kRingSlots LDS slots, kRingSlots - 1 stages ahead of the stage being
// multiplied, without passing through registers. Taken when K % 64 == 0 and
// N % 32 == 0 (every 16-byte weight piece of a tile row then lies inside the
// row), for 64-row tiles and for the 32-row tiles of K-split launches.
constexpr int kRingSlots = 4;
constexpr int kRingWeightBytes = kPrefillBK * kPrefillBN / 2;  // 64 K rows x 256 nibbles
// Slot layout: the activation tile (bm rows x 128 B), the weight tile, then
// per wavefront a block with its 64 columns' scales (128 B per group),
// zero-point words (32 B per group) and 16 rows' activation sums (64 B per
// group) of the stage's groups: one group per stage in 256 bytes (scales at
// 0, zero points at 128, sums at 160), or, for groups of 32, two groups in
// 512 bytes (scales at 0 and 128, zero points at 256 and 288, sums at 320
// and 384).
constexpr int ring_a_bytes(int bm) { return bm * kPrefillBK * 2; }
constexpr int ring_aux_off(int bm) { return ring_a_bytes(bm) + kRingWeightBytes; }
constexpr int ring_aux_bytes(bool two_groups) { return two_groups ? 512 : 256; }
constexpr int ring_slot_bytes(int bm, bool two_groups) {
  return ring_aux_off(bm) + 4 * ring_aux_bytes(two_groups);
}
constexpr int ring_bytes(int bm, bool two_groups) { return kRingSlots * ring_slot_bytes(bm, two_groups); }
static_assert(ring_slot_bytes(32, false) % 16 == 0 && ring_slot_bytes(64, true) % 16 == 0,
              "16-byte aligned slots");
static_assert(2 * ring_bytes(64, true) <= kLdsPerCu, "two ring workgroups per CU");
inline bool prefill_ring_ok(int64_t K, int64_t N, int64_t bm) {
  return (bm == kPrefillBM || bm == 32) && K % kPrefillBK == 0 && N % 32 == 0 && N <= (1 << 26);
}
inline int prefill_ring_lds_bytes(int64_t K, int32_t G, int64_t bm) {
  return ring_bytes((int)bm, G == 32 && K != 32);
}
// bf16 through the ring without K splits: the activation sums of every
// (group, row), which the factored numerics need at each group's fold, come
// from a pass over A before the GEMM (asum_kernel: the same MFMA chain
// against a ones operand that the GEMM would run per wavefront, so the
// values are bit-identical) instead of four times per tile inside the GEMM.
// They sit in the workspace after the counter region, [K/G][rows padded to
// 64] fp32, and reach the GEMM through the ring's per-wavefront blocks.
// Without zero points (and G < K) they are stored times -(128 + zp_bias)
// and start each group's partial sums.
inline int64_t prefill_asum_rows(int64_t M) { return (M + kPrefillBM - 1) / kPrefillBM * kPrefillBM; }
inline bool prefill_asum_pre(int64_t K, int64_t N, int32_t G, int32_t dtype, int64_t bm, int64_t S) {
  (void)G;
  return dtype == W4A16_BF16 && S == 1 && bm == kPrefillBM && prefill_ring_ok(K, N, bm);
}
inline int64_t prefill_asum_bytes(int64_t M, int64_t K, int32_t G) {
  return (K / G) * prefill_asum_rows(M) * (int64_t)sizeof(float);
}

// Constants of the nibble-to-float step, passed as kernel arguments so that
// the compiler keeps them in registers (see the kernels' dequantisation).
struct DqConsts {
  uint32_t magic;  // 0x64006400 (fp16) or 0x43004300 (bf16)
  uint32_t m_lo;   // 0x000F000F
  uint32_t m_hi;   // 0x00F000F0
  uint32_t zero;   // 0: mixed into the magic so that it lives in a vector register
};
inline DqConsts dq_consts(int dtype) {
  return DqConsts{dtype == W4A16_F16 ? 0x64006400u : 0x43004300u, 0x000F000Fu, 0x00F000F0u, 0u};
}

struct GemmArgs {
  const void* a;
  const int32_t* b_q;
  const void* scales;
  const int32_t* qzeros;  // nullable
  const void* bias;       // nullable: [N] in the activation dtype, added in fp32
  void* out;
  int64_t M, K, N;
  int32_t G, zp_bias, dtype;
};

struct DecodeParams {
  DqConsts dq;
  const uint16_t* a;
  const uint32_t* bq;
  const uint16_t* sc;
  const uint32_t* qz;
  const uint16_t* bias;  // nullable [N]
  uint16_t* out;
  float* ws;          // [S, M, N] fp32 partials (S > 1)
  int32_t* counters;  // [NB][W] arrival counters per wavefront, zero between launches,
                      // cstride int32 apart
  int32_t M, K, N, G, zp_bias;
  int32_t KS;         // K steps of 32 rows
  int32_t SG;         // steps per group
  int32_t sg_shift;   // log2(SG); -1 when one group spans every step
  int32_t ng_max;     // most groups one workgroup's steps touch
  int32_t L;          // steps per wavefront
  int32_t S;          // splits across workgroups
  int32_t NB;         // column blocks
  int32_t cstride;    // int32 slots from one arrival counter to the next
  int32_t W;          // wavefronts per workgroup (kDecodeWaves or kDecodeWavesWide)
};

struct PrefillParams {
  DqConsts dq;
  const uint16_t* a;
  const uint32_t* bq;
  const uint16_t* sc;
  const uint32_t* qz;
  const uint16_t* bias;  // nullable [N] (unused when S > 1: the reduction adds it)
  uint16_t* out;
  int32_t M, K, N, G, zp_bias;
  int32_t bm;         // rows per workgroup tile: 64, or 32 (K splits only)
  int32_t ring;       // 1: operands staged through the LDS ring (prefill_ring_ok holds)
  const float* asum;  // precomputed activation sums [K/G][asum_rows] (prefill_asum_pre), else null
  int32_t asum_rows;
  int32_t g_shift;    // log2(G) when G is 32, 64 or 128 (unused when G == K)
  int32_t tiles_m, tiles_n, tiles, per_xcd;
  int32_t band;       // tile rows per band of the workgroup -> tile order
  int32_t S;          // K splits (1: no cross-workgroup hand-off)
  int32_t kt_split;   // 64-row K stages per split
  float* ws;          // fp32 partials [S][M][N] (S > 1)
};
struct PrefillReduceParams {
  const float* ws;    // [S][M][N] fp32 partials
  const uint16_t* bias;  // nullable [N]
  uint16_t* out;      // [M][N]
  int32_t M, N, S;
};

struct AsumParams {
  const uint16_t* a;  // [M, K] bf16
  float* out;         // [K/G][rows] fp32, rows = prefill_asum_rows(M)
  int32_t M, K, G, rows;
  float scale;        // 1, or -(128 + zp_bias) without zero points and G < K
};

struct DequantParams {
  DqConsts dq;
  const uint32_t* bq;
  const uint16_t* sc;
  const uint32_t* qz;
  uint16_t* w;
  int32_t K, N, G, zp_bias;
};

// K-packed layout: weights [N, K/8] int32 in ExLlama nibble order, scales
// and zero points [N, K/G]. One workgroup per 16 columns x 16 rows.
struct KPackedParams {
  DqConsts dq;
  const uint16_t* a;
  const uint32_t* w;
  const uint16_t* sc;
  const uint8_t* zp;     // nullable: zp_bias for every group
  const uint16_t* bias;  // nullable [N]
  uint16_t* out;
  int32_t M, K, N, G, zp_bias;
  int32_t g_shift;       // log2(G / 32) for G = 32, 64, 128; -1 when G == K
  int32_t rpw;           // 128-K rounds per wavefront
};
constexpr int kKpThreads = 512;  // 8 wavefronts
constexpr int kKpCols = 16;
constexpr int kKpRows = 16;
// LDS of the K-packed kernel: a static array through which wavefronts 1..7
// hand their 16x16 sums to wavefront 0, plus (when it fits) the block's
// activation rows, each padded by 16 bytes, as dynamic LDS. The rows are
// staged only up to kKpLdsStageMax bytes (more costs occupancy and measured
// no faster) and never beyond what the device gives one workgroup.
constexpr int kKpRedBytes = (kKpThreads / 64 - 1) * 64 * 16;
constexpr int kKpLdsStageMax = 60 * 1024;
inline size_t kpacked_lds_bytes(int64_t M, int64_t K) {
  const int64_t mb = M < kKpRows ? M : kKpRows;
  return (size_t)(mb * (K + 8) * 2);
}

hipError_t launch_decode(const DecodeParams& p, int dtype, bool has_zp, int mode,
                         int grid, int lds_bytes, hipStream_t stream);
hipError_t launch_prefill(const PrefillParams& p, int dtype, bool has_zp, int grid, hipStream_t stream);
hipError_t launch_prefill_reduce(const PrefillReduceParams& p, int dtype, hipStream_t stream);
hipError_t launch_asum(const AsumParams& p, hipStream_t stream);
// stage: the activation rows go to LDS (the host checked that
// kpacked_lds_bytes + kKpRedBytes fits the device's per-workgroup LDS)
hipError_t launch_kpacked(const KPackedParams& p, int dtype, bool has_zp, bool fold, bool stage,
                          hipStream_t stream);
// Entry point without allocation: the device address of this device's copy
// of the fixed scratch array (kStaticScratchBytes, counter region zeroed on
// first use on the device, on `stream`).
hipError_t static_scratch(hipStream_t stream, void** ptr);
hipError_t launch_dequant(const DequantParams& p, int dtype, bool has_zp,
                          hipStream_t stream);

}  // namespace w4a16
