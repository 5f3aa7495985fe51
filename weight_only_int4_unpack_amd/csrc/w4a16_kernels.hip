// gfx950 kernels of the weight-only int4 GEMM  C[M,N] = A[M,K] . dequant(B).
//
// Arithmetic follows PR #40977 "RDNA hybrid W4A16", Code section (the test's
// reference: w = (q - z) * s with fp32 accumulation and one final cast); the
// packed operand layout follows PR #51453 "Register the Triton W4A16 GEMM as
// a custom op", implementation item 1 (b_q is [K, N/8], N = 8 * columns).
//
// Layout facts used everywhere below:
//   * b_q word (k, c) holds columns 8c..8c+7 of row k, value j in bits
//     [4j, 4j+4).
//   * The MFMA v_mfma_f32_16x16x32_{f16,bf16} contracts 32 k per
//     instruction; lane l supplies row/column (l & 15) of its operand and 8
//     k-values chosen by lane group (l >> 4). The k-to-slot mapping is the
//     same function for both operands, so any consistent assignment of
//     logical k to (lane group, slot) is valid; here slot s of lane group g
//     is logical row 8g + s of the 32-row step.
//   * The accumulator of lane l holds rows 4(l >> 4) + v (v = 0..3) of
//     column (l & 15).
//
// Dequantisation ("magic number"): OR-ing a uint4 into the low mantissa bits
// of a float with unit ulp gives base + q exactly: fp16 0x6400 is 1024
// (ulp 1), bf16 0x4300 is 128 (ulp 1). With two rows of four values in one
// 32-bit word (row r in bits 0..15, row r+1 in bits 16..31) one AND-OR makes
// a packed pair {base + q[r], base + q[r+1]} of one column. For fp16 the
// value in bits 4..7 can be taken in place as 1024 + 16 q.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "w4a16_internal.h"

namespace w4a16 {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

struct F16 {
  static constexpr bool kIsF16 = true;
  static constexpr float kBase = 1024.0f;
  static constexpr uint32_t kOnePair = 0x3C003C00u;
};
struct BF16 {
  static constexpr bool kIsF16 = false;
  static constexpr float kBase = 128.0f;
  static constexpr uint32_t kOnePair = 0x3F803F80u;
};

template <typename T>
__device__ __forceinline__ f32x4 mfma(u32x4 a, u32x4 b, f32x4 c);
template <>
__device__ __forceinline__ f32x4 mfma<F16>(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}
template <>
__device__ __forceinline__ f32x4 mfma<BF16>(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ float widen(F16, uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}
__device__ __forceinline__ float widen(BF16, uint32_t h) {
  return __builtin_bit_cast(float, h << 16);
}
__device__ __forceinline__ uint16_t narrow(F16, float x) {
  return __builtin_bit_cast(uint16_t, (_Float16)x);
}
__device__ __forceinline__ uint16_t narrow(BF16, float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

// The dequantisation masks and the dtype's magic pattern arrive as kernel
// arguments (DqConsts, filled by the host), so the compiler cannot fold them:
// with literal operands it would emit an AND and an OR (a gfx9 VOP3 takes no
// two literals); with register operands it selects one v_and_or_b32.
struct DqRegs {
  uint32_t mag;    // T::kMagic
  uint32_t m_lo;   // 0x000F000F
  uint32_t m_hi;   // 0x00F000F0
};
// The magic is made per-lane (xor with threadIdx & 0) so that it is held in
// a vector register: v_and_or_b32 reads at most one scalar operand here.
__device__ __forceinline__ DqRegs dq_regs(const DqConsts& d) {
  return DqRegs{d.magic ^ (threadIdx.x & d.zero), d.m_lo, d.m_hi};
}

// Pair {row r, row r+1} of column e (0..3) of Y as base + q (fp16, e odd:
// base + 16 q).
template <typename T, int E>
__device__ __forceinline__ uint32_t magic_pair(uint32_t y, const DqRegs& k) {
  if constexpr (T::kIsF16) {
    const uint32_t src = (E >= 2) ? (y >> 8) : y;
    return (src & ((E & 1) ? k.m_hi : k.m_lo)) | k.mag;
  } else {
    return ((y >> (4 * E)) & k.m_lo) | k.mag;
  }
}

// A 64-bit right shift of the word pair {y1, y0}: y1 >> s in the high word,
// y0 >> s in the low word save for y1's low bits, which enter from bit 32 - s
// up (s <= 12: bit 20 and above).
template <int S>
__device__ __forceinline__ uint64_t shr64(uint64_t y) {
  static_assert(S > 0 && S <= 12, "shift");
  uint64_t r;
  asm("v_lshrrev_b64 %0, %1, %2" : "=v"(r) : "n"(S), "v"(y));
  return r;
}
// magic_pair of four words (two row pairs each). Where a pair needs a shift
// (bf16 e > 0: 4e; fp16 e >= 2: 8), one 64-bit shift serves two words: the
// masks keep bits 0..7 and 16..23 only, below the bits the other word
// shifts in (bf16 2048 x 5120 x 17408 prefill 348.6 -> 338.4 us, decode
// M = 1 13.97 -> 13.47 us). PAIRED = false keeps one 32-bit shift per word:
// on the few-row fp16 routes that feed the integer operand (K-split
// prefill) or the rounded one (decode mode 0) it measured as fast or faster
// (K = N = 4096, M = 5: 9.47 against 9.68 us).
template <typename T, int E, bool PAIRED = true>
__device__ __forceinline__ u32x4 magic_op(const uint32_t* y, const DqRegs& mag) {
  constexpr int S = T::kIsF16 ? (E >= 2 ? 8 : 0) : 4 * E;
  if constexpr (S == 0 || !PAIRED) {
    return u32x4{magic_pair<T, E>(y[0], mag), magic_pair<T, E>(y[1], mag),
                 magic_pair<T, E>(y[2], mag), magic_pair<T, E>(y[3], mag)};
  } else {
    const uint32_t m = (T::kIsF16 && (E & 1)) ? mag.m_hi : mag.m_lo;
    const uint64_t s01 = shr64<S>(((uint64_t)y[1] << 32) | y[0]);
    const uint64_t s23 = shr64<S>(((uint64_t)y[3] << 32) | y[2]);
    return u32x4{((uint32_t)s01 & m) | mag.mag, ((uint32_t)(s01 >> 32) & m) | mag.mag,
                 ((uint32_t)s23 & m) | mag.mag, ((uint32_t)(s23 >> 32) & m) | mag.mag};
  }
}
// ---------------------------------------------------------------------------
// Exact dequantisation of one pair to RNE_dtype((q - z) * s).
//   fp16: (base + q) - (base + z) is the exact integer q - z (for e odd,
//         (1024 + 16q)/16 - (64 + z)); one packed multiply rounds it once.
//   bf16: (128 + q) * s and (128 + z) * s are exact in fp32, so one fp32 FMA
//         gives (q - z) * s exactly; the bf16 conversion rounds once.
// ---------------------------------------------------------------------------
struct ColF16 {
  f16x2 bias;   // {b, b}, b = 1024 + z (e even) or 64 + z (e odd)
  f16x2 scale;  // {s, s}
};
struct ColBF16 {
  float scale;  // s
  float c;      // -(128 + z) * s, exact
};
template <typename T>
struct Col;
template <>
struct Col<F16> { using type = ColF16; };
template <>
struct Col<BF16> { using type = ColBF16; };

template <int E>
__device__ __forceinline__ ColF16 make_col(F16, uint32_t s_bits, uint32_t z) {
  ColF16 c;
  const _Float16 b = (_Float16)(float)((E & 1) ? 64u + z : 1024u + z);
  const _Float16 s = __builtin_bit_cast(_Float16, (uint16_t)s_bits);
  c.bias = f16x2{b, b};
  c.scale = f16x2{s, s};
  return c;
}
template <int E>
__device__ __forceinline__ ColBF16 make_col(BF16, uint32_t s_bits, uint32_t z) {
  ColBF16 c;
  c.scale = __builtin_bit_cast(float, s_bits << 16);
  c.c = -(128.0f + (float)z) * c.scale;
  return c;
}

template <int E>
__device__ __forceinline__ uint32_t exact_from_magic(F16, uint32_t mg, const ColF16& c) {
  f16x2 h = __builtin_bit_cast(f16x2, mg);
  if constexpr (E & 1) {
    const f16x2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
    h = __builtin_elementwise_fma(h, sixteenth, -c.bias);
  } else {
    h = h - c.bias;
  }
  h = h * c.scale;
  return __builtin_bit_cast(uint32_t, h);
}
// fp16 pair of column e as the exact integer q - z (no scale): the prefill
// operand when the scale is applied to fp32 sums instead.
template <int E>
__device__ __forceinline__ uint32_t int_from_magic(uint32_t mg, f16x2 bias) {
  f16x2 h = __builtin_bit_cast(f16x2, mg);
  if constexpr (E & 1) {
    const f16x2 sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
    h = __builtin_elementwise_fma(h, sixteenth, -bias);
  } else {
    h = h - bias;
  }
  return __builtin_bit_cast(uint32_t, h);
}
// The bias {b, b} is built from z's bits: fp16 1024 + z is 0x6400 | z, and
// 64 + z (e odd: (1024 + 16q) / 16 - (64 + z)) is 0x5400 | 16z.
template <int E>
__device__ __forceinline__ u32x4 int_op(const uint32_t* y, const DqRegs& mag, uint32_t z) {
  const uint32_t b = (E & 1) ? (0x5400u | (z << 4)) : (0x6400u | z);
  const f16x2 bias = __builtin_bit_cast(f16x2, b * 0x10001u);
  const u32x4 m = magic_op<F16, E, false>(y, mag);
  return u32x4{int_from_magic<E>(m[0], bias), int_from_magic<E>(m[1], bias),
               int_from_magic<E>(m[2], bias), int_from_magic<E>(m[3], bias)};
}
// fp16 operand RNE((q - z) * s) of column e: the exact integer q - z (as in
// int_op) times the scale in one packed multiply, which rounds once. Same
// value as exact_pair (and the oracle's rounded tile), with the bias and the
// scale pair built from bits.
template <int E>
__device__ __forceinline__ u32x4 tile_op(const uint32_t* y, const DqRegs& mag, uint32_t z,
                                         uint32_t s_bits) {
  const uint32_t b = (E & 1) ? (0x5400u | (z << 4)) : (0x6400u | z);
  const f16x2 bias = __builtin_bit_cast(f16x2, b * 0x10001u);
  const f16x2 sc = __builtin_bit_cast(f16x2, (s_bits & 0xFFFFu) * 0x10001u);
  const u32x4 m = magic_op<F16, E>(y, mag);
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    r[i] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, int_from_magic<E>(m[i], bias)) * sc);
  return r;
}
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
template <int E>
__device__ __forceinline__ uint32_t exact_from_magic(BF16, uint32_t p, const ColBF16& c) {
  const f32x2 v = {__builtin_fmaf(__builtin_bit_cast(float, p << 16), c.scale, c.c),
                   __builtin_fmaf(__builtin_bit_cast(float, p & 0xFFFF0000u), c.scale, c.c)};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));  // one RNE each
}
template <int E, typename T>
__device__ __forceinline__ uint32_t exact_pair(T, uint32_t y, const DqRegs& mag,
                                               const typename Col<T>::type& c) {
  return exact_from_magic<E>(T{}, magic_pair<T, E>(y, mag), c);
}

__device__ __forceinline__ uint32_t nib(uint32_t w, int j) { return (w >> (4 * j)) & 0xFu; }

// A scale as a plain fp32 register (xor with threadIdx & 0): keeps the
// compiler from folding its fp16 -> fp32 conversion into every FMA that uses
// it as a mixed-precision v_fma_mix_f32, which measured at a fraction of the
// rate of v_fma_f32 in the folds (fp16 prefill at 4096^3: 387 -> 217 us).
__device__ __forceinline__ float plain_f32(float x, uint32_t zero) {
  return __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, x) ^ (threadIdx.x & zero));
}

// Activation loads read an in-bounds (clamped) address and clear the value
// afterwards where it lies past K. Selecting between the activation pointer
// and a zero block instead would make the load a flat one, and a pending flat
// load makes the compiler wait for every outstanding load (vmcnt(0)) before
// the first use of any of them, so nothing would overlap the stream.
// Two rows' half-words h (0: columns 0..3, 1: columns 4..7) of words w0, w1
// joined into one Y word (row of w0 in the low half).
__device__ __forceinline__ uint32_t join_rows(uint32_t w0, uint32_t w1, int h) {
  return __builtin_amdgcn_perm(w1, w0, h ? 0x07060302u : 0x05040100u);
}

// ---------------------------------------------------------------------------
// Decode: M <= 16. A workgroup owns 256 output columns and a contiguous range
// of W L steps of 32 K-rows; each of its W wavefronts (4, or 8 where the
// planner halves the K splits) streams L of them
// through a ring of D = min(L, 2) register slots: the loads of D steps are in
// flight from the start, and each slot is refilled with step j + D as soon as
// step j has been consumed. Lane (g, c) loads, per step, rows 8g..8g+7 of
// words 2c, 2c+1 of the block (16 columns) and feeds 16 MFMAs (column offset
// t = 0..15: column 16c + t). Loads never branch: row and column indices are
// clamped into the arrays; rows past K meet a zero activation and columns
// past N are never stored. The scales and zero points of the groups the
// workgroup touches are staged in LDS once.
//
// MODE selects where scale and zero point enter:
//   kSit:    the MFMA operand is the exact dequantised weight RNE((q-z)s).
//   kOneGrp: the operand is base + q (exact); the wavefront's steps lie in
//            one group, whose scale and zero point are applied once:
//              sum_k a (q - z) s = s (sum_k a (base + q) - (base + z) sum_k a),
//            with sum_k a from one extra MFMA against a ones operand.
//   kMulti:  as kOneGrp, but a wavefront may span groups: each group's
//            partial is folded into a second accumulator at its last step.
// Partials of the W wavefronts meet in LDS; partials of the S workgroups of
// one column block meet in an fp32 scratch buffer through write-through
// (agent-scope) stores, and the last workgroup to arrive (arrival counter)
// adds them in split order and writes the output, so the result does not
// depend on arrival order. No cache-wide flush is needed: the partials never
// sit dirty in a per-XCD L2, and they are read back with agent-scope loads.
// ---------------------------------------------------------------------------
enum { kSit = 0, kOneGrp = 1, kMulti = 2 };
// Two slots: with four, a CU's oldest wavefronts (served first) drew all
// their data before the next ones got any, so the last workgroup's steps all
// arrived at the end and were computed one after another; with two, each
// wavefront's later steps are requested as its earlier ones are consumed
// (decode 5120 x 17408 bf16: M = 1 13.02 -> 12.78 us, M = 5 14.38 -> 14.18 us).
constexpr int kRing = 2;

template <typename T, int E>
__device__ __forceinline__ u32x4 exact_op(const uint32_t* y, const DqRegs& mag, uint32_t s_bits,
                                          uint32_t z) {
  const auto cc = make_col<E>(T{}, s_bits, z);
  const u32x4 m = magic_op<T, E, false>(y, mag);
  return u32x4{exact_from_magic<E>(T{}, m[0], cc), exact_from_magic<E>(T{}, m[1], cc),
               exact_from_magic<E>(T{}, m[2], cc), exact_from_magic<E>(T{}, m[3], cc)};
}

__device__ __forceinline__ uint32_t half_of(const u32x4 (&sv)[2], int t) {
  const uint32_t w = sv[t >> 3][(t >> 1) & 3];
  return (t & 1) ? (w >> 16) : (w & 0xFFFFu);
}

// Four adjacent fp32 partials at byte offset `off` of the split-K scratch,
// stored and loaded as one 16-byte buffer access with the sc1 cache policy
// (write-through on stores, a fresh read past the per-XCD L2 on loads): a
// workgroup on any XCD reads what another wrote once the arrival counter
// says it is there. The buffer's record count bounds every access.
constexpr int kSc1 = 16;  // cache-policy operand: sc1
__device__ __forceinline__ __amdgpu_buffer_rsrc_t scratch_rsrc(float* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(base, 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ void store_wt4(__amdgpu_buffer_rsrc_t r, uint32_t off, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, (int)off, 0, kSc1);
}
__device__ __forceinline__ f32x4 load_wt4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kSc1));
}
// the same with a wave-uniform part of the offset in the scalar operand
__device__ __forceinline__ f32x4 load_wt4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(f32x4,
                            __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, kSc1));
}
// Four adjacent outputs, rounded to the activation type, in one 8-byte store.
template <typename T>
__device__ __forceinline__ void store_out4(T, uint16_t* dst, f32x4 v) {
  *(u32x2*)dst = u32x2{(uint32_t)narrow(T{}, v[0]) | ((uint32_t)narrow(T{}, v[1]) << 16),
                       (uint32_t)narrow(T{}, v[2]) | ((uint32_t)narrow(T{}, v[3]) << 16)};
}

// Bias of four adjacent output columns widened to fp32 (zeros without bias).
// It is added to the fp32 result before the one rounding to the output type,
// indexed by output column only (never by row).
template <typename T>
__device__ __forceinline__ f32x4 bias4(T, const uint16_t* bias, int col) {
  if (bias == nullptr) return f32x4{0.f, 0.f, 0.f, 0.f};
  const u32x2 b = *(const u32x2*)(bias + col);
  return f32x4{widen(T{}, b.x & 0xFFFFu), widen(T{}, b.x >> 16), widen(T{}, b.y & 0xFFFFu),
               widen(T{}, b.y >> 16)};
}

// One ring slot: the packed weights (8 rows x 2 words) and the activation
// operand of one 32-row step.
struct DecodeSlot {
  u32x2 w[8];
  u32x4 a;
};

// MT: M rounded up to 4, 8 or 16 (compile-time row count of the reductions).
// SLIDE: the last arrival keeps a sliding window of partial loads in flight
// (several rows, more splits than one window). W: wavefronts per workgroup
// (4, or 8 for half the K splits on small shapes).
template <typename T, bool HAS_ZP, int MODE, bool ALIGNED, int L, int MT, bool SLIDE, int W>
__global__ __launch_bounds__(64 * W, 2) void decode_kernel(DecodeParams p) {
  constexpr int D = L < kRing ? L : kRing;
  extern __shared__ __attribute__((aligned(16))) float red[];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int g = lane >> 4;
  const int c = lane & 15;
  const int b = blockIdx.x % p.NB;
  const int s = blockIdx.x / p.NB;
  const int N8 = p.N >> 3;
  const int M = p.M;
  const int word0 = b * (kDecodeCols / 8) + 2 * c;
  // clamped indices: every load below is in bounds without a branch
  const int wc0 = min(word0, N8 - 1);
  const int wc1 = min(word0 + 1, N8 - 1);
  const int wcv = ALIGNED ? min(word0, N8 - 2) : 0;  // 8-byte aligned pair
  // rows c >= M load row M - 1: their MFMA rows are computed and never stored
  const int mrow = min(c, M - 1);
  const uint16_t* arow = p.a + (int64_t)mrow * p.K;
  const DqRegs mag = dq_regs(p.dq);

  const int wg_beg = s * W * L;
  const int wg_last = min(wg_beg + W * L, p.KS) - 1;
  const int step_beg = wg_beg + wave * L;
  const int nsteps = max(0, min(L, p.KS - step_beg));
  auto group_of = [&](int st) { return p.sg_shift < 0 ? 0 : (st >> p.sg_shift); };
  const int g_lo = group_of(wg_beg);
  const int ngroups = group_of(wg_last) - g_lo + 1;

  // LDS: red[W][M][256] floats | scales[ng_max][256] halves | zeros[ng_max][32] words
  uint16_t* lds_sc = (uint16_t*)(red + W * M * kDecodeCols);
  uint32_t* lds_z = (uint32_t*)(lds_sc + p.ng_max * kDecodeCols);

  // ---- ring prologue: the first D steps' loads
  auto issue = [&](int j, DecodeSlot& sl) {
    const int st = min(step_beg + j, p.KS - 1);
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int row = min(st * kStepRows + 8 * g + r, p.K - 1);
      const uint32_t* src = p.bq + (int64_t)row * N8;
      if constexpr (ALIGNED) {
        sl.w[r] = *(const u32x2*)(src + wcv);
      } else {
        sl.w[r] = u32x2{src[wc0], src[wc1]};
      }
    }
    const int k = st * kStepRows + 8 * g;
    if constexpr (ALIGNED) {  // K % 8 == 0: a whole 8-element piece or none
      const u32x4 v = *(const u32x4*)(arow + min(k, p.K - 8));
      sl.a = k < p.K ? v : u32x4{0u, 0u, 0u, 0u};
    } else {
      uint32_t h[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t v = arow[min(k + e, p.K - 1)];
        h[e] = k + e < p.K ? v : 0u;
      }
      sl.a = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                   h[6] | (h[7] << 16)};
    }
  };
  DecodeSlot ring[D];
#pragma unroll
  for (int j = 0; j < D; ++j) issue(j, ring[j]);
  __builtin_amdgcn_sched_barrier(0);

  // ---- kOneGrp: the lane's 16 scales and zero points of its wavefront's one
  // group go straight to registers (used once, after the stream)
  u32x4 sv1[2];
  u32x2 zv1;
  if constexpr (MODE == kOneGrp) {
    const int grp = group_of(min(step_beg, p.KS - 1));
    const int col_lane = b * kDecodeCols + 16 * c;
    const uint16_t* srow = p.sc + (int64_t)grp * p.N;
    if constexpr (ALIGNED) {  // N % 16 == 0: 16 scales in two aligned pieces
      const uint16_t* sp = srow + min(col_lane, p.N - 16);
      sv1[0] = *(const u32x4*)sp;
      sv1[1] = *(const u32x4*)(sp + 8);
    } else {
      uint32_t h[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) h[e] = srow[min(col_lane + e, p.N - 1)];
#pragma unroll
      for (int q = 0; q < 2; ++q)
        sv1[q] = u32x4{h[8 * q] | (h[8 * q + 1] << 16), h[8 * q + 2] | (h[8 * q + 3] << 16),
                       h[8 * q + 4] | (h[8 * q + 5] << 16), h[8 * q + 6] | (h[8 * q + 7] << 16)};
    }
    if constexpr (HAS_ZP) {
      const uint32_t* zp = p.qz + (int64_t)grp * N8;
      zv1 = u32x2{zp[wc0], zp[wc1]};
    } else {
      const uint32_t zb = (uint32_t)p.zp_bias * 0x11111111u;
      zv1 = u32x2{zb, zb};
    }
  }
  // ---- the other modes stage this workgroup's scales and zero points in LDS
  if constexpr (MODE != kOneGrp) {
    const int colc = min(b * kDecodeCols + tid, p.N - 1);
    if (tid < kDecodeCols)
      for (int gi = 0; gi < ngroups; ++gi)
        lds_sc[gi * kDecodeCols + tid] = p.sc[(int64_t)(g_lo + gi) * p.N + colc];
    if constexpr (HAS_ZP) {
      for (int i = tid; i < ngroups * 32; i += 64 * W) {
        const int gi = i >> 5, wi = min(b * 32 + (i & 31), N8 - 1);
        lds_z[i] = p.qz[(int64_t)(g_lo + gi) * N8 + wi];
      }
    }
  }
  if constexpr (MODE != kOneGrp) __syncthreads();
  auto lds_scales = [&](int st, u32x4 (&sv)[2], u32x2& zv) {
    const int gi = group_of(st) - g_lo;
    const uint16_t* sp = lds_sc + gi * kDecodeCols + 16 * c;
    sv[0] = *(const u32x4*)sp;
    sv[1] = *(const u32x4*)(sp + 8);
    if constexpr (HAS_ZP) {
      zv = *(const u32x2*)(lds_z + gi * 32 + 2 * c);
    } else {
      const uint32_t zb = (uint32_t)p.zp_bias * 0x11111111u;
      zv = u32x2{zb, zb};
    }
  };

  f32x4 acc[16];
  f32x4 R[16];
  f32x4 Rs = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int t = 0; t < 16; ++t) {
    acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    R[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const u32x4 ones = u32x4{T::kOnePair, T::kOnePair, T::kOnePair, T::kOnePair};

  // ---- stream the steps
#pragma unroll
  for (int j = 0; j < L; ++j) {
    DecodeSlot& sl = ring[j % D];
    const int st = step_beg + j;
    if (j < nsteps) {
      uint32_t Y[2][2][4];  // [word][half][row pair]
#pragma unroll
      for (int w = 0; w < 2; ++w)
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int i = 0; i < 4; ++i) Y[w][h][i] = join_rows(sl.w[2 * i][w], sl.w[2 * i + 1][w], h);
      if constexpr (MODE == kSit) {
        u32x4 sv[2];
        u32x2 zv;
        lds_scales(st, sv, zv);
#pragma unroll
        for (int t = 0; t < 16; ++t) {
          const uint32_t* y = Y[t >> 3][(t >> 2) & 1];
          const uint32_t sb = half_of(sv, t);
          const uint32_t z = nib(zv[t >> 3], t & 7);
          u32x4 bop;
          switch (t & 3) {
            case 0: bop = exact_op<T, 0>(y, mag, sb, z); break;
            case 1: bop = exact_op<T, 1>(y, mag, sb, z); break;
            case 2: bop = exact_op<T, 2>(y, mag, sb, z); break;
            default: bop = exact_op<T, 3>(y, mag, sb, z); break;
          }
          acc[t] = mfma<T>(sl.a, bop, acc[t]);
        }
      } else {
#pragma unroll
        for (int t = 0; t < 16; ++t) {
          const uint32_t* y = Y[t >> 3][(t >> 2) & 1];
          u32x4 bop;
          switch (t & 3) {
            case 0: bop = magic_op<T, 0>(y, mag); break;
            case 1: bop = magic_op<T, 1>(y, mag); break;
            case 2: bop = magic_op<T, 2>(y, mag); break;
            default: bop = magic_op<T, 3>(y, mag); break;
          }
          R[t] = mfma<T>(sl.a, bop, R[t]);
        }
        Rs = mfma<T>(sl.a, ones, Rs);
        const bool group_last =
            p.sg_shift >= 0 && (((st + 1) & ((1 << p.sg_shift) - 1)) == 0);
        // kOneGrp folds once, in place, after the loop
        const bool fold = (MODE == kMulti) && (group_last || (j + 1 == nsteps));
        if (fold) {
          u32x4 sv[2];
          u32x2 zv;
          lds_scales(st, sv, zv);
#pragma unroll
          for (int t = 0; t < 16; ++t) {
            const bool odd16 = T::kIsF16 && (t & 1);
            const float sc =
                plain_f32(widen(T{}, half_of(sv, t)) * (odd16 ? 0.0625f : 1.0f), p.dq.zero);
            const float bias = T::kBase + (float)nib(zv[t >> 3], t & 7) * (odd16 ? 16.0f : 1.0f);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const float part = __builtin_fmaf(-bias, Rs[v], R[t][v]);
              acc[t][v] = __builtin_fmaf(sc, part, acc[t][v]);
            }
            R[t] = f32x4{0.f, 0.f, 0.f, 0.f};
          }
          Rs = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
    }
    if (j + D < L) issue(j + D, sl);
    __builtin_amdgcn_sched_barrier(0);
  }
  // kOneGrp: the wavefront's steps lie in one group; fold R in place (a
  // wavefront without steps keeps its zero partial)
  if constexpr (MODE == kOneGrp) {
    if (nsteps > 0) {
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const bool odd16 = T::kIsF16 && (t & 1);
        const float sc =
            plain_f32(widen(T{}, half_of(sv1, t)) * (odd16 ? 0.0625f : 1.0f), p.dq.zero);
        const float bias = T::kBase + (float)nib(zv1[t >> 3], t & 7) * (odd16 ? 16.0f : 1.0f);
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (v < M) R[t][v] = sc * __builtin_fmaf(-bias, Rs[v], R[t][v]);
      }
    }
  }
  f32x4 (&res)[16] = *[&]() -> f32x4 (*)[16] {
    if constexpr (MODE == kOneGrp) return &R; else return &acc;
  }();

  // ---- the W wavefronts' partials meet in LDS: red[wave][m][256]
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int m = 4 * g + v;
    if (m < M) {
      float* dst = red + (wave * M + m) * kDecodeCols + 16 * c;
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4)
        *(f32x4*)(dst + 4 * t4) = f32x4{res[4 * t4][v], res[4 * t4 + 1][v], res[4 * t4 + 2][v],
                                        res[4 * t4 + 3][v]};
    }
  }
  __syncthreads();

  // Wavefront w owns rows w, w + W, ... (< M) and lane l columns b*256 + 4l
  // .. 4l + 3 of them: 16-byte LDS reads and 8-byte global accesses keep this
  // epilogue short, which matters because the last arrival of a column block
  // runs it once, from a cold instruction cache, on the kernel's critical path.
  constexpr int RPT = (MT + W - 1) / W;  // rows per wavefront
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int col4 = b * kDecodeCols + 4 * lane;
  const bool col_ok = col4 < p.N;  // N % 8 == 0: all four columns or none
  const uint32_t lane_off = (uint32_t)min(col4, p.N - 4) * 4u;  // bytes
  const uint32_t row_bytes = (uint32_t)p.N * 4u;
  // the planner keeps the S x M x N fp32 partials below 4 GiB
  const __amdgpu_buffer_rsrc_t wsr = scratch_rsrc(p.ws, (uint32_t)(p.S * M) * row_bytes);
  f32x4 part[RPT];
#pragma unroll
  for (int r = 0; r < RPT; ++r) {
    const int m = wv + W * r;
    if (m < M) {
      f32x4 v = *(const f32x4*)(red + m * kDecodeCols + 4 * lane);
#pragma unroll
      for (int w = 1; w < W; ++w)
        v += *(const f32x4*)(red + (w * M + m) * kDecodeCols + 4 * lane);
      part[r] = v;
    }
  }
  if (p.S == 1) {
    if (col_ok) {
      const f32x4 bv = bias4(T{}, p.bias, col4);
#pragma unroll
      for (int r = 0; r < RPT; ++r)
        if (wv + W * r < M)
          store_out4(T{}, p.out + (int64_t)(wv + W * r) * p.N + col4, part[r] + bv);
    }
    return;
  }
  // Wavefront wv hands its rows over on its own: it publishes them, waits
  // until its stores are complete, and counts itself in on the counter of
  // (column block, wavefront); the last of the S arrivals adds them up.
  if (wv >= M) return;  // no rows
  if (col_ok) {
#pragma unroll
    for (int r = 0; r < RPT; ++r)
      if (wv + W * r < M)
        store_wt4(wsr, (uint32_t)(s * M + wv + W * r) * row_bytes + lane_off, part[r]);
  }
  // Ordering of the hand-off. The partials are stored, and later loaded,
  // with the device-scope cache policy (sc1): on gfx950 a store with that
  // scope is written through to the device's point of coherence and a load
  // with it is served from there, never from a possibly stale per-XCD L2.
  // vmcnt counts the whole wavefront's stores: once it reads zero every
  // lane's partials are complete at device scope, so the counter (a device-
  // scope atomic) cannot move before them. The last arrival issues its loads
  // only after the atomic's value has come back (it branches on it), and
  // they read at device scope. Compiler barriers keep the compiler from
  // moving memory operations across these points. A language-level agent
  // fence would do the same with a write-back and an invalidation of the
  // whole L2 (buffer_wbl2 / buffer_inv sc1): measured on MI355X at the
  // 5120 x 17408 decode shape, 13.5 -> 38 us per launch at M = 1 and
  // 15 -> 84 us at M = 5, for no change in what this code relies on.
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  int32_t* counter = p.counters + (b * W + wv) * p.cstride;
  int prev = 0;
  if (lane == 0)
    prev = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (__builtin_amdgcn_readfirstlane(prev) != p.S - 1) return;
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  // last arrival: add the S partials of each row in split order, QB splits'
  // loads of the wavefront's rows in flight (the partial buffer holds S x M
  // rows of row_bytes; every real load below lies inside it)
  if (lane == 0) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  constexpr int QB = RPT <= 2 ? 16 : 4;
  const int S = p.S;
  const uint32_t split_bytes = (uint32_t)M * row_bytes;
  f32x4 sum[RPT];
#pragma unroll
  for (int r = 0; r < RPT; ++r) sum[r] = f32x4{0.f, 0.f, 0.f, 0.f};
  if constexpr (!SLIDE) {
    // windows of QB splits: their loads, then their adds (one round trip
    // per window)
    for (int q0 = 0; q0 < S; q0 += QB) {
      f32x4 tq[QB][RPT];
#pragma unroll
      for (int u = 0; u < QB; ++u)
        if (q0 + u < S) {
#pragma unroll
          for (int r = 0; r < RPT; ++r)
            if (wv + W * r < M)
              tq[u][r] = load_wt4(wsr, (uint32_t)(wv + W * r) * row_bytes + lane_off,
                                  (uint32_t)(q0 + u) * split_bytes);
        }
#pragma unroll
      for (int u = 0; u < QB; ++u)
        if (q0 + u < S) {
#pragma unroll
          for (int r = 0; r < RPT; ++r)
            if (wv + W * r < M) sum[r] += tq[u][r];
        }
    }
  } else {
    // S >= 2 QB, several rows: a window in flight throughout, a partial's
    // register slot refilled with the load QB splits ahead as soon as it is
    // added. Every load is issued without a branch and every loaded value is
    // consumed, so that the waits count loads in order instead of draining
    // them; the scheduling barriers keep each add next to its refill. Split
    // indices past S wrap to q - S (distinct splits already added, in the
    // scalar offset); a row past M gets a vector offset past the buffer's
    // end, where the bounds check of buffer loads returns zeros without a
    // memory access, and its sum is never stored. (With one row the
    // compiler copies the loaded slots and drains the loads at every window,
    // so one row keeps the windows above.)
    static_assert(RPT >= 2, "sliding window: several rows");
    uint32_t row_off[RPT];
#pragma unroll
    for (int r = 0; r < RPT; ++r)
      row_off[r] = wv + W * r < M ? (uint32_t)(wv + W * r) * row_bytes + lane_off
                                  : (uint32_t)S * split_bytes;
    auto split_off = [&](int q) { return (uint32_t)(q < S ? q : q - S) * split_bytes; };
    f32x4 tq[QB][RPT];
#pragma unroll
    for (int u = 0; u < QB; ++u)
#pragma unroll
      for (int r = 0; r < RPT; ++r) tq[u][r] = load_wt4(wsr, row_off[r], split_off(u));
    int q0 = 0;
    for (; q0 + QB < S; q0 += QB) {  // windows with another after them: all QB splits real
#pragma unroll
      for (int u = 0; u < QB; ++u) {
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
          sum[r] += tq[u][r];
          tq[u][r] = load_wt4(wsr, row_off[r], split_off(q0 + QB + u));
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int u = 0; u < QB; ++u) {  // the last window: splits q0 + u < S
      const bool real = q0 + u < S;
#pragma unroll
      for (int r = 0; r < RPT; ++r) {
        const f32x4 t = sum[r] + tq[u][r];
#pragma unroll
        for (int v = 0; v < 4; ++v) sum[r][v] = real ? t[v] : sum[r][v];
      }
    }
  }
  if (col_ok) {
    const f32x4 bv = bias4(T{}, p.bias, col4);
#pragma unroll
    for (int r = 0; r < RPT; ++r)
      if (wv + W * r < M)
        store_out4(T{}, p.out + (int64_t)(wv + W * r) * p.N + col4, sum[r] + bv);
  }
}

// Workgroup -> (output tile, K split). Workgroups go round-robin over the 8
// XCDs, so XCD x runs blockIdx x, x+8, ...; it is given the contiguous range
// [x * per_xcd, (x + 1) * per_xcd) of the units, which are ordered split by
// split and, within a split, in a banded tile order: bands of `band` tile
// rows, walked column by column, rows fastest. The ~64 tiles an XCD runs at
// once then form a compact block (e.g. 8 rows x 8 columns), so the
// activation rows and weight columns they read are shared in that XCD's L2.
__device__ __forceinline__ bool prefill_tile(const PrefillParams& p, int& tm, int& tn, int& split) {
  const int xcd = blockIdx.x % kXcds;
  int L = xcd * p.per_xcd + blockIdx.x / kXcds;
  if (L >= p.tiles * p.S) return false;
  split = L / p.tiles;  // units with one split index are consecutive
  L -= split * p.tiles;
  const int full = p.tiles_m / p.band;          // bands of `band` rows
  const int in_full = full * p.band * p.tiles_n;
  if (L < in_full) {
    const int b = L / (p.band * p.tiles_n);
    const int r = L - b * p.band * p.tiles_n;
    tn = r / p.band;
    tm = b * p.band + (r - tn * p.band);
  } else {
    const int rows = p.tiles_m - full * p.band;  // last, shorter band
    const int r = L - in_full;
    tn = r / rows;
    tm = full * p.band + (r - tn * rows);
  }
  return true;
}

// A load from a wave-uniform base plus a per-lane 32-bit byte offset (lets
// the compiler use the scalar-base form of the global load).
template <typename V>
__device__ __forceinline__ V ldg(const char* base, uint32_t off) {
  return *(const V*)(base + off);
}

// Global -> LDS copies of the prefill ring (gfx950 global_load_lds): lane i
// reads `size` bytes at sbase + voff and the load unit writes them to LDS
// byte address lds + i * size; no register receives data. They are issued
// here rather than through the compiler's builtin because the compiler,
// seeing the ring's slots as one array, would wait for every copy in flight
// (vmcnt(0)) before each read of any slot, and the ring exists to keep the
// copies of later stages in flight meanwhile. The kernel therefore waits for
// them itself (ring_wait) and contains no other vector-memory loads while a
// copy can be in flight. m0 is set inside the statement (the one nop covers
// the m0 write -> LDS-copy hazard).
typedef __attribute__((address_space(3))) unsigned char lds_byte;
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const lds_byte*)p;
}
// The base address in scalar registers (its value is wave-uniform).
__device__ __forceinline__ const void* scalar_ptr(const void* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}
// LDS destination = lds (wave-uniform) + OFF (a compile-time byte offset).
// The scalar add that forms m0 also writes SCC, which the compiler may be
// carrying between the two halves of a 64-bit address add around this
// statement: SCC is declared clobbered (without it, a carry lost here put a
// pointer 4 GiB low whenever its low half wrapped, and the load faulted).
template <int OFF>
__device__ __forceinline__ void copy16_to_lds(const void* sbase, uint32_t voff, uint32_t lds) {
  static_assert(OFF >= 0 && OFF < (1 << 20), "LDS offset");
  asm volatile("s_add_u32 m0, %2, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(scalar_ptr(sbase)), "s"(__builtin_amdgcn_readfirstlane(lds)), "n"(OFF)
               : "memory", "scc");
}
// Two 1 KB blocks with one m0: the instruction offset moves the global and
// the LDS address alike, so the first block goes at m0 - 1024 (its lane
// offset passed plus 1024, never below zero) and the second at m0.
template <int OFF>
__device__ __forceinline__ void copy16x2_to_lds(const void* sbase, uint32_t voff0p, uint32_t voff1,
                                                uint32_t lds) {
  static_assert(OFF >= 0 && OFF + 1024 < (1 << 20), "LDS offset");
  asm volatile(
      "s_add_u32 m0, %3, %4\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %2 offset:-1024\n\t"
      "global_load_lds_dwordx4 %1, %2"
      :
      : "v"(voff0p), "v"(voff1), "s"(scalar_ptr(sbase)), "s"(__builtin_amdgcn_readfirstlane(lds)),
        "n"(OFF + 1024)
      : "memory", "scc");
}
// 4 bytes per lane from the lane's own address
template <int OFF>
__device__ __forceinline__ void copy4_to_lds_lane(const void* src, uint32_t lds) {
  static_assert(OFF >= 0 && OFF < (1 << 20), "LDS offset");
  asm volatile("s_add_u32 m0, %1, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :
               : "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds)), "n"(OFF)
               : "memory", "scc");
}
// Wait until at most N of this wavefront's vector-memory operations are in
// flight (they complete in issue order); also a compiler barrier for memory.
template <int N>
__device__ __forceinline__ void ring_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// ---------------------------------------------------------------------------
// Prefill: workgroup tile 64 x 256, K staged 64 rows (two 32-row slabs) at a
// time. The A tile goes through LDS (double-buffered) and is read by all 4
// wavefronts; each wavefront owns 64 output columns and turns exactly the
// weights it multiplies into MFMA operands: lane (g, c) reads, per slab,
// rows 8g..8g+7 of columns 4c..4c+3 of its 64 (one 16-bit piece of a packed
// word per row, two rows per register) and forms four operands (column
// 4c + e, e = 0..3).
//
// Numerics (factored, as in the decode kernel's grouped modes): the operand
// is the exact integer base + q (fp16, e odd: 1024 + 16q); one more MFMA
// against a ones operand gives each row's activation sum over the slab. For
// each group, in fp32,
//     sum_k a (q - z) s = s' (part - (base + z') sum_k a),
// with part = sum_k a (base + q) and s' = s, z' = z (fp16 e odd: s/16, 16z),
// folded into the output accumulator at the group's last slab. No weight is
// rounded to fp16/bf16: the products are exact and only fp32 sums round.
// GS = G / 32 slabs per group (1, 2 or 4); GS = 0: one group spans all of K
// and the fold is done once, on the output accumulator, at the end.
//
// Loads never branch: rows and columns are clamped into the arrays, rows past
// M are computed and not stored, activation columns past K are cleared.
// The K loop is unrolled twice so the two weight buffers swap roles without
// copies (a group of 4 slabs is exactly one unrolled body). Workgroup ids are
// spread so that the tiles of one XCD share A rows. Two workgroups fit a CU.
// KM = 0: K % 64 == 0 and no load is checked against K. KM = 1, 2: the
// stage that holds row K - 1 clamps weight rows and clears activations past
// K; activations load in 16-byte pieces (KM = 1, K % 8 == 0) or one at a time.
// ---------------------------------------------------------------------------
// BM: rows per workgroup tile, 64 (two workgroups per CU, 252 VGPRs) or, for
// few rows, 32 (fewer padding rows in the MFMAs, fewer registers, three
// workgroups per CU; measured at K = N = 4096: M = 64 in 17.7 us with 32-row
// tiles against 20.0 us with 64-row tiles, M = 16 12.2 against 13.1 us, while
// the 2048-row prefill takes 506 us with 32-row tiles against 426 us, each
// weight being dequantised twice as often). 16-row tiles were slower than 32
// at M = 16 (14.3 us; with four workgroups per CU they spilled to scratch).
template <typename T, bool HAS_ZP, int GS, int KM, bool SPLIT, int BM, bool RING>
__global__ __launch_bounds__(kPrefillThreads, (BM == 64 || RING) ? 2 : 3) void prefill_kernel(
    PrefillParams p) {
  static_assert(BM == 32 || BM == 64, "tile rows");
  static_assert(!RING || (KM == 0 && (BM == 64 || SPLIT)), "ring: full stages; 32-row tiles split K");
  constexpr int RH = kPrefillLdsRowHalves;
  constexpr int MB = BM / 16;
  constexpr int AP = BM / 32;  // 16-byte A pieces per thread per stage
  constexpr int kLds = RING ? ring_bytes(BM, GS == 1) : 2 * BM * RH * 2;
  __shared__ __attribute__((aligned(16))) unsigned char smem[kLds];
  auto As = reinterpret_cast<uint16_t(*)[BM * RH]>(smem);

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int g = lane >> 4;
  const int c = lane & 15;

  int tm, tn, split;
  if (!prefill_tile(p, tm, tn, split)) return;
  const int m0 = tm * BM;
  const int ncol = tn * kPrefillBN + wave * 64 + 4 * c;  // this lane's 4 columns
  const int ncolc = min(ncol, p.N - 4);
  const int N4 = p.N >> 2;  // 16-bit pieces per weight row
  const uint16_t* bq16 = (const uint16_t*)p.bq + (ncolc >> 2);
  const int KT = (p.K + kPrefillBK - 1) / kPrefillBK;
  // this workgroup's K stages [kt_beg, kt_end): whole groups per split
  const int kt_beg = SPLIT ? split * p.kt_split : 0;
  const int kt_end = SPLIT ? min(KT, kt_beg + p.kt_split) : KT;
  const DqRegs mag = dq_regs(p.dq);
  const u32x4 ones = u32x4{T::kOnePair, T::kOnePair, T::kOnePair, T::kOnePair};
  const f32x4 zero4 = f32x4{0.f, 0.f, 0.f, 0.f};
  // Unsplit fp16 with groups of 32 or 64 rows (GS = 1, 2): the operand is
  // the weight itself, RNE_fp16((q - z) * s) (relative error 2^-11 per
  // weight), so no per-group fold is needed; folding every 32 or 64 rows made
  // these shapes bound by the fold's fp32 FMAs (4096^3, G = 32: 207 -> 187
  // us). The K-split kernel serves small, latency-bound tile counts, where
  // the scale multiply in front of the MFMAs measured slower than the fold
  // behind them (M = 256: 33.5 -> 38.9 us), so it keeps the integer operand.
  // Other fp16 groups: the operand is the exact integer q - z (one packed
  // subtract or FMA per pair), so no activation sums are needed; bf16 keeps
  // base + q.
  constexpr bool kTile = T::kIsF16 && (GS == 1 || GS == 2) && !SPLIT;
  constexpr bool kIntOp = T::kIsF16 && !kTile;
  // bf16 ring without K splits: activation sums precomputed (p.asum). With
  // one zero point for every column (b = base + zp_bias) and groups below K,
  // the pass stores -b * sum a instead, and each group's partials start from
  // it rather than from zero, so the fold is acc += s * part (one FMA per
  // output instead of two).
  constexpr bool kPreSum = RING && !SPLIT && !T::kIsF16;
  constexpr bool kInitSum = kPreSum && !HAS_ZP && GS > 0;

  f32x4 acc[MB][4];   // output accumulator
  f32x4 part[MB][4];  // current group's sum of a (base + q)   (GS > 0)
  f32x4 asum[MB];     // current group's (GS = 0: all of K's) sum of a
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    asum[i] = zero4;
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[i][t] = zero4;
  }

  // ---- loaders. Full stages (all 64 rows inside K) address every load as a
  // wave-uniform base plus one per-lane 32-bit byte offset; the last stage,
  // when K % 64 != 0, clamps weight rows and clears activations past K.
  // Rows past M are clamped to M - 1 once, in the per-lane offsets.
  uint32_t a_off[AP];
#pragma unroll
  for (int j = 0; j < AP; ++j)
    a_off[j] = (uint32_t)(((min(m0 + j * 32 + (tid >> 3), p.M - 1) - m0) * p.K + (tid & 7) * 8) * 2);
  const char* a_base = (const char*)(p.a + (int64_t)m0 * p.K);
  const uint32_t b_off = (uint32_t)((8 * g * N4 + (ncolc >> 2)) * 2);
  const uint32_t s_off = (uint32_t)(ncolc * 2);
  const uint32_t z_off = (uint32_t)((ncolc >> 2) * 2);
  const int KF = p.K / kPrefillBK;  // full stages

  // ---- LDS ring (RING). A slot holds one stage: the activation tile (64
  // rows x 128 B), the weight tile (64 K rows x 128 B: 256 columns of
  // nibbles), and per wavefront a block with its 64 columns' scales and
  // packed zero-point words and its 16 rows' precomputed activation sums for
  // the stage's group, or two groups when G = 32 (layout beside
  // ring_aux_bytes). Tiles are stored in 1 KB blocks of 8 rows; within a row
  // the 16-byte pieces are permuted (XOR) so that the operand reads meet
  // distinct LDS banks: activation row r keeps piece j at j ^ (r & 7) (the
  // 16 rows one MFMA operand read spans hit 8 distinct pieces per 8 lanes);
  // weight row k keeps piece j at j ^ 2((k >> 3) & 3) (the 4 rows one
  // 16-bit read spans, 8 apart, hit 4 distinct piece pairs). Each wavefront
  // copies blocks 2w and 2w + 1 of both tiles and fills its own block: one
  // copy of 4 bytes per lane, two for two groups with zero points or sums.
  constexpr bool kTwo = GS == 1;                 // two groups per stage
  constexpr int kAuxB = ring_aux_bytes(kTwo);
  constexpr int kSlotB = ring_slot_bytes(BM, kTwo);
  constexpr int kBOff = ring_a_bytes(BM);        // weight tile
  constexpr int kAuxOff = ring_aux_off(BM);      // per-wavefront blocks
  constexpr int kABlk = BM / 32;                 // activation blocks each wavefront copies
  constexpr int kSumOff = kTwo ? 320 : 160;      // sums of the stage's (first) group in a block
  constexpr bool kAux2 = kTwo && (HAS_ZP || kPreSum);
  constexpr int kCopies = kABlk + 3 + (kAux2 ? 1 : 0);  // copies per wavefront per stage
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  uint32_t a_dma[2] = {0u, 0u}, b_dma[2] = {0u, 0u};
  uint32_t a_rd[2] = {0u, 0u}, b_rd = 0u, b_sel = 0u, s_rd = 0u, z_rd = 0u, ring_lds = 0u;
  // per lane: source of its 4 bytes of the block for the stage's first
  // group, and the bytes between groups (second copy: aux2_*)
  const char* aux_src = nullptr;
  const char* aux2_src = nullptr;
  uint32_t aux_step = 0u, aux2_step = 0u;
  if constexpr (RING) {
    ring_lds = lds_addr(smem);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int blk = 2 * wv + j;
      const int row = 8 * blk + (lane >> 3);
      const int bp = (lane & 7) ^ (2 * (blk & 3));
      const int cc = min(tn * 8 + bp, p.N / 32 - 1) - tn * 8;  // pieces past N: clamped, never stored
      b_dma[j] = (uint32_t)(row * (p.N / 2) + cc * 16);
      // activation blocks: kABlk per wavefront (rows 8 kABlk w + 8j + lane / 8)
      const int arow = 8 * (kABlk * wv + j) + (lane >> 3);
      const int ap = (lane & 7) ^ (arow & 7);
      a_dma[j] = (uint32_t)((min(m0 + arow, p.M - 1) - m0) * p.K * 2 + ap * 16);
    }
    const int col0 = tn * kPrefillBN + wv * 64;
    auto scale_src = [&](int l) {  // scale pair of columns col0 + 2l, 2l + 1
      return (const char*)p.sc + (int64_t)min(col0 + 2 * l, p.N - 2) * 2;
    };
    auto zero_src = [&](int l) {   // zero-point word of columns col0 + 8l .. 8l + 7
      return (const char*)p.qz + (int64_t)min(col0 / 8 + l, p.N / 8 - 1) * 4;
    };
    auto sum_src = [&](int l) {    // activation sum of tile row 16w + l
      return (const char*)(p.asum + m0 + 16 * wv + l);
    };
    const uint32_t s_step = (uint32_t)(p.N * 2), z_step = (uint32_t)(p.N / 2);
    const uint32_t a_step = (uint32_t)(p.asum_rows * 4);
    if constexpr (!kTwo) {
      // lanes 0..31: scale pairs; 32..39: zero-point words; 40..55 (kPreSum):
      // activation sums; the rest repeat lane 0's pair into the block's pad
      if (HAS_ZP && lane >= 32 && lane < 40) {
        aux_src = zero_src(lane - 32);
        aux_step = z_step;
      } else if (kPreSum && lane >= 40 && lane < 56) {
        aux_src = sum_src(lane - 40);
        aux_step = a_step;
      } else {
        aux_src = scale_src(lane < 32 ? lane : 0);
        aux_step = s_step;
      }
    } else {
      // first copy: lanes 0..31 the first group's scale pairs, 32..63 the
      // second's; second copy: lanes 0..15 zero-point words (8 per group),
      // 16..47 activation sums (16 per group), the rest repeat lane 0's pair
      aux_src = scale_src(lane & 31) + (lane >> 5) * s_step;
      aux_step = s_step;
      if (HAS_ZP && lane < 16) {
        aux2_src = zero_src(lane & 7) + (lane >> 3) * z_step;
        aux2_step = z_step;
      } else if (kPreSum && lane >= 16 && lane < 48) {
        aux2_src = sum_src((lane - 16) & 15) + ((lane - 16) >> 4) * a_step;
        aux2_step = a_step;
      } else {
        aux2_src = scale_src(0);
        aux2_step = s_step;
      }
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) a_rd[ks] = (uint32_t)(c * 128 + (((ks * 4 + g) ^ (c & 7)) * 16));
    // the dword holding the lane's 16 bits of a weight row (its half: c & 1)
    b_rd = (uint32_t)(kBOff + 8 * g * 128 + (((2 * wave + (c >> 3)) ^ (2 * g)) * 16) + (c & 6) * 2);
    b_sel = (c & 1) ? 0x07060302u : 0x05040100u;
    s_rd = (uint32_t)(kAuxOff + wave * kAuxB + 8 * c);
    z_rd = (uint32_t)(kAuxOff + wave * kAuxB + (kTwo ? 256 : 128) + 2 * c);
  }
  // the copies of stage kt into slot SL = (kt - kt_beg) % kRingSlots (a
  // compile-time constant)
  auto ring_issue = [&](int kt, auto slc) {
    constexpr int SO = decltype(slc)::value * kSlotB;
    const uint32_t wa = ring_lds + kABlk * wv * 1024;              // this wavefront's activation blocks,
    const uint32_t wb = ring_lds + 2 * wv * 1024;                  // weight blocks
    const uint32_t waux = ring_lds + wv * kAuxB;                   // and scale/zero/sum block
    const char* ab = (const char*)p.a + ((int64_t)m0 * p.K + (int64_t)kt * kPrefillBK) * 2;
    if constexpr (kABlk == 2)
      copy16x2_to_lds<SO>(ab, a_dma[0] + 1024u, a_dma[1], wa);
    else
      copy16_to_lds<SO>(ab, a_dma[0], wa);
    const char* bb = (const char*)p.bq + (int64_t)kt * kPrefillBK * (p.N / 2) + tn * (kPrefillBN / 2);
    copy16x2_to_lds<SO + kBOff>(bb, b_dma[0] + 1024u, b_dma[1], wb);
    const int grp = GS == 0 ? 0 : ((kt * kPrefillBK) >> p.g_shift);  // the stage's first group
    copy4_to_lds_lane<SO + kAuxOff>(aux_src + (uint64_t)grp * aux_step, waux);
    if constexpr (kAux2)
      copy4_to_lds_lane<SO + kAuxOff + 256>(aux2_src + (uint64_t)grp * aux2_step, waux);
  };

  auto load_a = [&](int kt, u32x4 (&ar)[AP]) {
    if (KM == 0 || kt < KF) {
#pragma unroll
      for (int j = 0; j < AP; ++j) ar[j] = ldg<u32x4>(a_base + kt * (kPrefillBK * 2), a_off[j]);
    } else {
#pragma unroll
      for (int j = 0; j < AP; ++j) {
        const int row = min(m0 + j * 32 + (tid >> 3), p.M - 1);
        const int k = kt * kPrefillBK + (tid & 7) * 8;
        const uint16_t* arow = p.a + (int64_t)row * p.K;
        if constexpr (KM == 1) {
          const u32x4 v = *(const u32x4*)(arow + min(k, p.K - 8));
          ar[j] = k < p.K ? v : u32x4{0u, 0u, 0u, 0u};
        } else {
          uint32_t h[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint32_t v = arow[min(k + e, p.K - 1)];
            h[e] = k + e < p.K ? v : 0u;
          }
          ar[j] = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                        h[6] | (h[7] << 16)};
        }
      }
    }
  };
  auto store_a = [&](int buf, const u32x4 (&ar)[AP]) {
#pragma unroll
    for (int j = 0; j < AP; ++j) {
      const int row = j * 32 + (tid >> 3);
      *(u32x4*)&As[buf][row * RH + (tid & 7) * 8] = ar[j];
    }
  };
  // One slab's weights (rows 8g..8g+7, two rows per register) and, for a
  // slab that closes a group, that group's 4 scales and packed zero points.
  struct Slab {
    u16x2 q[4];
    u32x2 s;
    uint32_t z;
    bool valid;
  };
  // POS: slab position within the unrolled body (0..3)
  auto load_slab = [&](int kt, int half, Slab& sl, auto posc) {
    constexpr int POS = decltype(posc)::value;
    constexpr bool closes = GS > 0 && (POS + 1) % (GS > 0 ? GS : 1) == 0;
    const int k0 = kt * kPrefillBK + 32 * half;
    if ((KM == 0 || kt < KF) && GS >= 2) {
      // buffer loads: a resource based at row k0 (scalar), the lane's fixed
      // byte offset, and a scalar row offset per load, so that no load needs
      // vector address arithmetic (global loads here cost one 64-bit add
      // each; bf16 G = 128 at the 2048 x 5120 x 17408 shape: 439 -> 425 us).
      // With one slab per group (GS = 1) the kernel sits at the register
      // limit and the compiler then issues these loads one pair at a time,
      // so that case, and the per-channel one (GS = 0, not measured faster),
      // keep the global loads below.
      const __amdgpu_buffer_rsrc_t br = __builtin_amdgcn_make_buffer_rsrc(
          (void*)((const char*)p.bq + (int64_t)k0 * (N4 * 2)), 0, -1, 0x00020000);
#pragma unroll
      for (int r = 0; r < 4; ++r)
        sl.q[r] = u16x2{__builtin_amdgcn_raw_buffer_load_b16(br, (int)b_off, (2 * r) * (N4 * 2), 0),
                        __builtin_amdgcn_raw_buffer_load_b16(br, (int)b_off, (2 * r + 1) * (N4 * 2), 0)};
    } else if (KM == 0 || kt < KF) {
      const char* rb = (const char*)p.bq + (int64_t)k0 * (N4 * 2);
#pragma unroll
      for (int r = 0; r < 4; ++r)
        sl.q[r] = u16x2{ldg<uint16_t>(rb + (int64_t)(2 * r) * (N4 * 2), b_off),
                        ldg<uint16_t>(rb + (int64_t)(2 * r + 1) * (N4 * 2), b_off)};
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int r0 = min(k0 + 8 * g + 2 * r, p.K - 1);
        const int r1 = min(k0 + 8 * g + 2 * r + 1, p.K - 1);
        sl.q[r] = u16x2{bq16[(int64_t)r0 * N4], bq16[(int64_t)r1 * N4]};
      }
    }
    const int grp = GS == 0 ? 0 : (min(k0, p.K - 1) >> p.g_shift);
    if constexpr (closes || kTile) {
      sl.s = ldg<u32x2>((const char*)p.sc + (int64_t)grp * p.N * 2, s_off);
      sl.valid = KM == 0 || k0 < p.K;
    }
    // zero points: where the scale is applied (factored form), or with every
    // slab's weights (fp16 integer or weight operand)
    if constexpr (HAS_ZP && (closes || kIntOp || kTile))
      sl.z = ldg<uint16_t>((const char*)p.qz + (int64_t)grp * N4 * 2, z_off);
  };
  // Fold a group's partial into the output accumulator (scales s_bits of the
  // lane's 4 columns, their packed zero points z4). GS = 0: acc holds the
  // partial itself. fp16 (integer operand q - z): acc += s * part; bf16
  // (operand base + q): acc += s' * (part - (base + z') * sum a).
  auto col_consts = [&](u32x2 s_bits, uint32_t z4, bool valid, float (&sc)[4], float (&bias)[4]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t sb = (e < 2 ? s_bits.x : s_bits.y) >> (16 * (e & 1));
      const float z = (float)(HAS_ZP ? nib(z4, e) : (uint32_t)p.zp_bias);
      const bool odd16 = !kIntOp && T::kIsF16 && (e & 1);
      sc[e] = plain_f32(valid ? widen(T{}, sb & 0xFFFFu) * (odd16 ? 0.0625f : 1.0f) : 0.f,
                        p.dq.zero);
      bias[e] = T::kBase + z * (odd16 ? 16.0f : 1.0f);
    }
  };
  auto fold_block = [&](const float (&sc)[4], const float (&bias)[4], const f32x4& as,
                        const f32x4 (&src)[4], f32x4 (&dst)[4]) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float d = (kIntOp || kInitSum) ? src[e][v] : __builtin_fmaf(-bias[e], as[v], src[e][v]);
        dst[e][v] = GS > 0 ? __builtin_fmaf(sc[e], d, dst[e][v]) : sc[e] * d;
      }
  };
  // Activation operand of row block i, 32-row half ks: from LDS buffer `buf`,
  // or (RING) from the slot at byte offset `buf`.
  auto aop_at = [&](uint32_t buf, int ks, int i) -> u32x4 {
    if constexpr (RING)
      return *(const u32x4*)(smem + buf + a_rd[ks] + i * 16 * kPrefillBK * 2);
    else
      return *(const u32x4*)&As[buf][(i * 16 + c) * RH + ks * 32 + 8 * g];
  };
  // A slab's weights, scales and zero points from the ring slot at byte
  // offset `so` (RING): rows 2r and 2r + 1 of the lane's 8 in one register,
  // from one two-dword LDS read (the dwords of both rows that hold the
  // lane's 16 bits, 128 bytes apart) and one byte permute.
  auto ring_slab = [&](uint32_t so, int ks, Slab& sl, auto posc) {
    constexpr int POS = decltype(posc)::value;
    constexpr bool closes = GS > 0 && (POS + 1) % (GS > 0 ? GS : 1) == 0;
    const uint32_t* bp = (const uint32_t*)(smem + so + b_rd + ks * 32 * 128);
#pragma unroll
    for (int r = 0; r < 4; ++r)
      sl.q[r] = __builtin_bit_cast(u16x2, __builtin_amdgcn_perm(bp[(2 * r + 1) * 32], bp[(2 * r) * 32], b_sel));
    const uint32_t gk = kTwo ? ks : 0;  // the slab's group within the stage
    if constexpr (closes || kTile) {
      sl.s = *(const u32x2*)(smem + so + s_rd + gk * 128);
      sl.valid = true;
    }
    if constexpr (HAS_ZP && (closes || kIntOp || kTile))
      sl.z = *(const uint16_t*)(smem + so + z_rd + gk * 32);
    constexpr bool opens = GS > 0 && POS % (GS > 0 ? GS : 1) == 0;
    if constexpr (kPreSum && (kInitSum ? opens : closes)) {
#pragma unroll
      for (int i = 0; i < MB; ++i)
        asum[i] = *(const f32x4*)(smem + so + kAuxOff + i * kAuxB + kSumOff + gk * 64 + 16 * g);
    }
  };
  // The MFMAs of one slab (LDS buffer `buf`, 32-row half `ks`). With one
  // slab per group (GS = 1) each row block is folded right after its MFMAs,
  // so only one row block's partials are live.
  auto slab = [&](int buf, int ks, const Slab& sl, auto posc) {
    constexpr int POS = decltype(posc)::value;
    constexpr bool opens = GS > 0 && POS % (GS > 0 ? GS : 1) == 0;
    constexpr bool closes = GS > 0 && (POS + 1) % (GS > 0 ? GS : 1) == 0;
    uint32_t Y[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) Y[r] = __builtin_bit_cast(uint32_t, sl.q[r]);
    u32x4 bop[4];
    if constexpr (kTile) {
      // rows past K (K tail) meet zero activations; their clamped weights and
      // scales are finite, so they add exact zeros
      const uint32_t z4 = HAS_ZP ? sl.z : (uint32_t)p.zp_bias * 0x1111u;
      bop[0] = tile_op<0>(Y, mag, nib(z4, 0), sl.s.x);
      bop[1] = tile_op<1>(Y, mag, nib(z4, 1), sl.s.x >> 16);
      bop[2] = tile_op<2>(Y, mag, nib(z4, 2), sl.s.y);
      bop[3] = tile_op<3>(Y, mag, nib(z4, 3), sl.s.y >> 16);
#pragma unroll
      for (int i = 0; i < MB; ++i) {
        const u32x4 aop = aop_at(buf, ks, i);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[i][e] = mfma<T>(aop, bop[e], acc[i][e]);
      }
      return;
    } else if constexpr (kIntOp) {
      const uint32_t z4 = HAS_ZP ? sl.z : (uint32_t)p.zp_bias * 0x1111u;
      bop[0] = int_op<0>(Y, mag, nib(z4, 0));
      bop[1] = int_op<1>(Y, mag, nib(z4, 1));
      bop[2] = int_op<2>(Y, mag, nib(z4, 2));
      bop[3] = int_op<3>(Y, mag, nib(z4, 3));
    } else {
      bop[0] = magic_op<T, 0>(Y, mag);
      bop[1] = magic_op<T, 1>(Y, mag);
      bop[2] = magic_op<T, 2>(Y, mag);
      bop[3] = magic_op<T, 3>(Y, mag);
    }
    float sc[4], bias[4];
    if constexpr (closes) col_consts(sl.s, HAS_ZP ? sl.z : 0u, sl.valid, sc, bias);
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      const u32x4 aop = aop_at(buf, ks, i);
      if constexpr (GS == 1) {
        const f32x4 as = (kIntOp || kInitSum) ? zero4 : kPreSum ? asum[i] : mfma<T>(aop, ones, zero4);
        f32x4 pt[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) pt[e] = mfma<T>(aop, bop[e], kInitSum ? asum[i] : zero4);
        fold_block(sc, bias, as, pt, acc[i]);
      } else {
        if constexpr (!kIntOp && !kPreSum) asum[i] = mfma<T>(aop, ones, opens ? zero4 : asum[i]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if constexpr (GS > 0)
            part[i][e] = mfma<T>(aop, bop[e], opens ? (kInitSum ? asum[i] : zero4) : part[i][e]);
          else
            acc[i][e] = mfma<T>(aop, bop[e], acc[i][e]);
        }
      }
    }
    if constexpr (closes && GS > 1) {
#pragma unroll
      for (int i = 0; i < MB; ++i) fold_block(sc, bias, asum[i], part[i], acc[i]);
    }
  };
  // The magic-operand path of slab() in two parts, so that a stage can form
  // its second slab's operands between the first slab's MFMAs: the
  // operands of a slab, and its MFMAs (then its fold), with hook(i) called
  // after row block i's MFMAs (i < MB).
  auto slab_ops = [&](const Slab& sl, u32x4 (&bop)[4]) {
    uint32_t Y[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) Y[r] = __builtin_bit_cast(uint32_t, sl.q[r]);
    bop[0] = magic_op<T, 0>(Y, mag);
    bop[1] = magic_op<T, 1>(Y, mag);
    bop[2] = magic_op<T, 2>(Y, mag);
    bop[3] = magic_op<T, 3>(Y, mag);
  };
  auto slab_mma = [&](uint32_t buf, int ks, const Slab& sl, const u32x4 (&bop)[4], auto posc,
                      auto&& hook) {
    constexpr int POS = decltype(posc)::value;
    constexpr bool opens = GS > 0 && POS % (GS > 0 ? GS : 1) == 0;
    constexpr bool closes = GS > 0 && (POS + 1) % (GS > 0 ? GS : 1) == 0;
    float sc[4], bias[4];
    if constexpr (closes) col_consts(sl.s, HAS_ZP ? sl.z : 0u, sl.valid, sc, bias);
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      const u32x4 aop = aop_at(buf, ks, i);
      if constexpr (!kPreSum) asum[i] = mfma<T>(aop, ones, opens ? zero4 : asum[i]);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        part[i][e] = mfma<T>(aop, bop[e], opens ? (kInitSum ? asum[i] : zero4) : part[i][e]);
      hook(i);
    }
    if constexpr (closes) {
#pragma unroll
      for (int i = 0; i < MB; ++i) fold_block(sc, bias, asum[i], part[i], acc[i]);
    }
  };
  // One stage (P: 0 or 1 within the unrolled body; LD: stage kt+1 exists):
  // prefetch stage kt+1 (A to registers, weights to `nxt`), compute stage
  // kt, publish the A tile.
  u32x4 a_next[AP];
  auto stage = [&](int kt, const Slab (&cur)[2], Slab (&nxt)[2], auto pc, auto ldc) {
    constexpr int P = decltype(pc)::value;
    constexpr bool LD = decltype(ldc)::value;
    const int buf = kt & 1;
    if constexpr (LD) {
      load_a(kt + 1, a_next);
      load_slab(kt + 1, 0, nxt[0], std::integral_constant<int, 2 * (1 - P)>{});
      load_slab(kt + 1, 1, nxt[1], std::integral_constant<int, 2 * (1 - P) + 1>{});
    }
    slab(buf, 0, cur[0], std::integral_constant<int, 2 * P>{});
    slab(buf, 1, cur[1], std::integral_constant<int, 2 * P + 1>{});
    if constexpr (LD) store_a(buf ^ 1, a_next);
    __syncthreads();
  };
  using C0 = std::integral_constant<int, 0>;
  using C1 = std::integral_constant<int, 1>;
  using Yes = std::true_type;
  using No = std::false_type;

  if constexpr (RING) {
    // Stage kt (LATER: stages already issued after kt, 0..2; ISSUE: stage
    // kt + 3 exists): wait for this wavefront's copies of stage kt, then the
    // barrier (every wavefront's copies of kt have landed, and every
    // wavefront is done with stage kt - 1, whose slot the copies of stage
    // kt + 3 then reuse), then multiply stage kt out of its slot.
    // stage kt in slot SL = (kt - kt_beg) % kRingSlots
    auto rstage = [&](int kt, auto slc, auto laterc, auto issuec) {
      constexpr int SL = decltype(slc)::value;
      constexpr int P = SL & 1;  // kt - kt_beg even: P = 0 (opens a two-stage group)
      constexpr int LATER = decltype(laterc)::value;
      static_assert(kRingSlots == 4, "three stages in flight, slots alternate parity");
      if constexpr (LATER >= 0) {
        ring_wait<kCopies * LATER>();
      } else {  // the last stages: LATER = kt_end - 1 - kt
        const int later = kt_end - 1 - kt;
        if (later >= 2) ring_wait<2 * kCopies>(); else if (later == 1) ring_wait<kCopies>(); else ring_wait<0>();
      }
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (decltype(issuec)::value)
        ring_issue(kt + kRingSlots - 1, std::integral_constant<int, (SL + kRingSlots - 1) % kRingSlots>{});
      constexpr uint32_t so = SL * kSlotB;
      if constexpr (!kTile && !kIntOp && GS > 1) {
        // the second slab's operands formed between the first slab's MFMAs
        // (one nibble position per row block), so that a wavefront's own
        // VALU work runs while its matrix-core work does
        using Q0 = std::integral_constant<int, 2 * P>;
        using Q1 = std::integral_constant<int, 2 * P + 1>;
        Slab s0, s1;
        ring_slab(so, 0, s0, Q0{});
        ring_slab(so, 1, s1, Q1{});
        u32x4 b0[4], b1[4];
        slab_ops(s0, b0);
        uint32_t Y1[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) Y1[r] = __builtin_bit_cast(uint32_t, s1.q[r]);
        // nibble positions 4i / MB .. 4(i + 1) / MB - 1 behind row block i
        auto form = [&](int e) {
          switch (e) {
            case 0: b1[0] = magic_op<T, 0>(Y1, mag); break;
            case 1: b1[1] = magic_op<T, 1>(Y1, mag); break;
            case 2: b1[2] = magic_op<T, 2>(Y1, mag); break;
            default: b1[3] = magic_op<T, 3>(Y1, mag); break;
          }
        };
        slab_mma(so, 0, s0, b0, Q0{}, [&](int i) {
#pragma unroll
          for (int e = i * 4 / MB; e < (i + 1) * 4 / MB; ++e) form(e);
        });
        slab_mma(so, 1, s1, b1, Q1{}, [](int) {});
      } else {
        Slab sl;
        ring_slab(so, 0, sl, std::integral_constant<int, 2 * P>{});
        slab(so, 0, sl, std::integral_constant<int, 2 * P>{});
        ring_slab(so, 1, sl, std::integral_constant<int, 2 * P + 1>{});
        slab(so, 1, sl, std::integral_constant<int, 2 * P + 1>{});
      }
    };
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using S2 = std::integral_constant<int, 2>;
    using S3 = std::integral_constant<int, 3>;
    using L2 = std::integral_constant<int, 2>;
    using Lr = std::integral_constant<int, -1>;
    if (kt_beg < kt_end) ring_issue(kt_beg, S0{});
    if (kt_beg + 1 < kt_end) ring_issue(kt_beg + 1, S1{});
    if (kt_beg + 2 < kt_end) ring_issue(kt_beg + 2, S2{});
    // kt_beg is even whenever a group spans two stages, so even slots open groups.
    // Four stages per trip while every one of them still issues a later stage.
    int kt = kt_beg;
    for (; kt + 6 < kt_end; kt += 4) {
      rstage(kt, S0{}, L2{}, Yes{});
      rstage(kt + 1, S1{}, L2{}, Yes{});
      rstage(kt + 2, S2{}, L2{}, Yes{});
      rstage(kt + 3, S3{}, L2{}, Yes{});
    }
    // the last 1..6 stages (kt - kt_beg is a multiple of 4: slots start at 0)
    if (kt < kt_end) rstage(kt, S0{}, Lr{}, std::false_type{});
    if (kt + 3 < kt_end) ring_issue(kt + 3, S3{});
    if (kt + 1 < kt_end) rstage(kt + 1, S1{}, Lr{}, std::false_type{});
    if (kt + 4 < kt_end) ring_issue(kt + 4, S0{});
    if (kt + 2 < kt_end) rstage(kt + 2, S2{}, Lr{}, std::false_type{});
    if (kt + 5 < kt_end) ring_issue(kt + 5, S1{});
    if (kt + 3 < kt_end) rstage(kt + 3, S3{}, Lr{}, std::false_type{});
    if (kt + 4 < kt_end) rstage(kt + 4, S0{}, Lr{}, std::false_type{});
    if (kt + 5 < kt_end) rstage(kt + 5, S1{}, Lr{}, std::false_type{});
  } else {
    Slab B0[2], B1[2];
    load_a(kt_beg, a_next);
    load_slab(kt_beg, 0, B0[0], C0{});
    load_slab(kt_beg, 1, B0[1], C1{});
    store_a(kt_beg & 1, a_next);
    __syncthreads();
    // kt_beg is even whenever a group spans two stages, so P = 0 opens groups
    int kt = kt_beg;
    for (; kt + 2 < kt_end; kt += 2) {
      stage(kt, B0, B1, C0{}, Yes{});
      stage(kt + 1, B1, B0, C1{}, Yes{});
    }
    if (kt + 2 == kt_end) {
      stage(kt, B0, B1, C0{}, Yes{});
      stage(kt + 1, B1, B0, C1{}, No{});
    } else {
      stage(kt, B0, B1, C0{}, No{});
    }
  }

  // ---- epilogue: lane holds rows i*16 + 4g + v, columns ncol + e
  const bool col_ok = ncol < p.N;
  if constexpr (GS == 0) {  // one group: fold this split's sums (the fold is linear)
    if constexpr (kPreSum) {
#pragma unroll
      for (int i = 0; i < MB; ++i) asum[i] = *(const f32x4*)(p.asum + m0 + 16 * i + 4 * g);
    }
    const u32x2 sv = *(const u32x2*)(p.sc + ncolc);
    const uint32_t z4 = HAS_ZP ? ((const uint16_t*)p.qz)[ncolc >> 2] : 0u;
    float sc[4], bias[4];
    col_consts(sv, z4, true, sc, bias);
#pragma unroll
    for (int i = 0; i < MB; ++i) fold_block(sc, bias, asum[i], acc[i], acc[i]);
  }
  auto store_out = [&](int row, float x0, float x1, float x2, float x3) {
    const uint32_t lo = (uint32_t)narrow(T{}, x0) | ((uint32_t)narrow(T{}, x1) << 16);
    const uint32_t hi = (uint32_t)narrow(T{}, x2) | ((uint32_t)narrow(T{}, x3) << 16);
    *(u32x2*)(p.out + (int64_t)row * p.N + ncol) = u32x2{lo, hi};
  };
  if constexpr (!SPLIT) {
    if (!col_ok) return;
    const f32x4 bv = bias4(T{}, p.bias, ncol);
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = m0 + i * 16 + 4 * g + v;
        if (row < p.M)
          store_out(row, acc[i][0][v] + bv[0], acc[i][1][v] + bv[1], acc[i][2][v] + bv[2],
                    acc[i][3][v] + bv[3]);
      }
    return;
  }
  // ---- K split: this split's fp32 partial goes to ws[split][row][col] for
  // the M real rows only (rows of the tile past M are never written);
  // prefill_reduce_kernel, launched next on the same stream, adds the splits
  // in order.
  if constexpr (SPLIT) {
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int row = m0 + i * 16 + 4 * g + v;
      float* d = p.ws + ((int64_t)split * p.M + row) * p.N + ncolc;
      if (col_ok && row < p.M)
        *(f32x4*)d = f32x4{acc[i][0][v], acc[i][1][v], acc[i][2][v], acc[i][3][v]};
    }
  }
}

// ---------------------------------------------------------------------------
// Activation sums for the bf16 ring prefill: out[g][r] = scale * (sum over
// group g's rows k of a[r][k]), the sum computed exactly as the prefill's
// wavefronts would (the MFMA against a ones operand, one 32-row slab after
// another, from zero). scale is 1, or -(base + zp_bias) when every column
// shares that zero point (one rounding). Workgroup = 64 rows x one group;
// wavefront w takes rows 16w .. 16w + 15. Rows past M repeat row M - 1.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void asum_kernel(AsumParams p) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4, c = lane & 15;
  const int r0 = blockIdx.x * kPrefillBM + 16 * wave;
  const int grp = blockIdx.y;
  const uint16_t* arow = p.a + (int64_t)min(r0 + c, p.M - 1) * p.K + (int64_t)grp * p.G + 8 * g;
  const u32x4 ones = u32x4{BF16::kOnePair, BF16::kOnePair, BF16::kOnePair, BF16::kOnePair};
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < p.G / 32; ++s) acc = mfma<BF16>(*(const u32x4*)(arow + 32 * s), ones, acc);
  if (c == 0) *(f32x4*)(p.out + (int64_t)grp * p.rows + r0 + 4 * g) = acc * p.scale;
}

// ---------------------------------------------------------------------------
// Prefill K-split reduction: out[m][n] = cast(sum over splits in order of
// ws[s][m][n] + bias[n]); one thread per 4 adjacent outputs, all splits'
// loads in flight at once.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void prefill_reduce_kernel(PrefillReduceParams p) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;  // 4-column piece
  const int N4 = p.N >> 2;
  if (q >= (int64_t)p.M * N4) return;
  const int m = (int)(q / N4);
  const int n = (int)(q - (int64_t)m * N4) * 4;
  const int64_t split_stride = (int64_t)p.M * p.N;
  const float* src = p.ws + (int64_t)m * p.N + n;
  f32x4 v[kPrefillMaxSplits];
#pragma unroll
  for (int s = 0; s < kPrefillMaxSplits; ++s)
    if (s < p.S) v[s] = *(const f32x4*)(src + s * split_stride);
  f32x4 sum = v[0];
#pragma unroll
  for (int s = 1; s < kPrefillMaxSplits; ++s)
    if (s < p.S) sum += v[s];
  sum += bias4(T{}, p.bias, n);
  const uint32_t lo = (uint32_t)narrow(T{}, sum[0]) | ((uint32_t)narrow(T{}, sum[1]) << 16);
  const uint32_t hi = (uint32_t)narrow(T{}, sum[2]) | ((uint32_t)narrow(T{}, sum[3]) << 16);
  *(u32x2*)(p.out + (int64_t)m * p.N + n) = u32x2{lo, hi};
}

// ---------------------------------------------------------------------------
// Dequant probe: w[k, n] = RNE((q - z) * s), written densely. Thread owns
// rows 2i, 2i+1 of one packed word (8 columns) and uses the same pair
// routine as the prefill operands.
// ---------------------------------------------------------------------------
template <typename T, bool HAS_ZP>
__global__ __launch_bounds__(256) void dequant_kernel(DequantParams p) {
  const int N8 = p.N >> 3;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t pairs = ((int64_t)p.K + 1) / 2;
  if (idx >= pairs * N8) return;
  const int wc = (int)(idx % N8);
  const int r0 = (int)(idx / N8) * 2;
  const bool has1 = r0 + 1 < p.K;
  const uint32_t w0 = p.bq[(int64_t)r0 * N8 + wc];
  const uint32_t w1 = has1 ? p.bq[(int64_t)(r0 + 1) * N8 + wc] : 0u;
  const int grp = r0 / p.G;  // rows r0, r0 + 1 share a group: G is even or G == K
  const uint32_t zw = HAS_ZP ? p.qz[(int64_t)grp * N8 + wc] : (uint32_t)p.zp_bias * 0x11111111u;
  const uint16_t* sp = p.sc + (int64_t)grp * p.N + wc * 8;
  uint16_t* o0 = p.w + (int64_t)r0 * p.N + wc * 8;
  uint16_t* o1 = o0 + p.N;
  const DqRegs mag = dq_regs(p.dq);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t y = join_rows(w0, w1, h);
    uint32_t pr[4];
    pr[0] = exact_pair<0>(T{}, y, mag, make_col<0>(T{}, sp[4 * h + 0], nib(zw, 4 * h + 0)));
    pr[1] = exact_pair<1>(T{}, y, mag, make_col<1>(T{}, sp[4 * h + 1], nib(zw, 4 * h + 1)));
    pr[2] = exact_pair<2>(T{}, y, mag, make_col<2>(T{}, sp[4 * h + 2], nib(zw, 4 * h + 2)));
    pr[3] = exact_pair<3>(T{}, y, mag, make_col<3>(T{}, sp[4 * h + 3], nib(zw, 4 * h + 3)));
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      o0[4 * h + e] = (uint16_t)(pr[e] & 0xFFFFu);
      if (has1) o1[4 * h + e] = (uint16_t)(pr[e] >> 16);
    }
  }
}

// ---------------------------------------------------------------------------
// K-packed decode (weights [N, K/8] int32, ExLlama nibble order: nibbles i and
// i + 4 of a word hold K values 2i and 2i + 1, so (w >> 4i) & 0x000F000F is a
// packed pair of consecutive K; scales and zero points [N, K/G]).
//
// A workgroup owns 16 columns x 16 activation rows and all of K, so partial
// sums never leave it. A round is 128 K. Lane l = 16j + c loads 16 bytes of
// column c: chunk 4r + j (32 K values) of round r. Its four words are the B
// operands of the round's four MFMA 16x16x32 steps; step i takes word i of
// every lane group j, and the A operand of lane l is activation row c at the
// same 8 K values. The eight wavefronts take contiguous runs of rounds and
// add up in LDS.
//   LDSA: when the block's activation rows fit (kKpLdsStageMax, rows padded by
//     16 bytes so that the 16 rows of one read fall in different banks), they
//     are copied to LDS once per workgroup and the A operands are read there;
//     otherwise each lane loads them from global memory per round.
//   FOLD (G a multiple of 128, or G == K): a round lies inside one group, so
//     the MFMAs run on unscaled operands and the scale multiplies the round's
//     fp32 sum: fp16 operand q - z (exact); bf16 operand 128 + q, with the
//     round's activation sums from MFMAs against ones, folded as
//     s * (part - (128 + z) * sum).
//   TILE (fp16, G = 32, 64): a round spans groups; the operand is the
//     rounded tile RNE_fp16((q - z) * s) of the lane's own chunk (relative
//     error 2^-11 per weight).
//   CHUNK (bf16, G = 32, 64): rounding a weight to bf16 costs 2^-8 relative,
//     which over a long K leaves the 2e-2 tolerance, so the operand stays
//     exact (128 + q) and the scale folds per group as in FOLD. For that an
//     MFMA step must lie in one group: lane l = 16j + c loads word j of each
//     of the round's four chunks (four 4-byte loads instead of one 16-byte
//     load), so step i covers chunk 4r + i alone, whose group's scale folds
//     into the step's sum (G = 64: every two steps).
// ---------------------------------------------------------------------------
constexpr int kKpU = 2;  // rounds in flight per wavefront

// pair i of a K-packed word as base + q: (nibble i, nibble i + 4)
__device__ __forceinline__ u32x4 kp_magic_op(uint32_t w, const DqRegs& k) {
  return u32x4{(w & k.m_lo) | k.mag, ((w >> 4) & k.m_lo) | k.mag, ((w >> 8) & k.m_lo) | k.mag,
               ((w >> 12) & k.m_lo) | k.mag};
}
// fp16 pairs as the exact integers q - z: (1024 + q) - (1024 + z)
__device__ __forceinline__ u32x4 kp_int_op(uint32_t w, const DqRegs& k, uint32_t z) {
  const f16x2 bias = __builtin_bit_cast(f16x2, (0x6400u | z) * 0x10001u);
  const u32x4 m = kp_magic_op(w, k);
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // through a scalar: hipcc folds a bit_cast of a vector element m[i] to
    // element 0 for every i
    const uint32_t mi = m[i];
    r[i] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, mi) - bias);
  }
  return r;
}
// fp16 rounded tile RNE((q - z) * s): the exact integer times s in one
// packed multiply, which rounds once (fp16 only: a bf16 tile rounds too
// coarsely for long K, see CHUNK below)
template <typename T>
__device__ __forceinline__ u32x4 kp_tile_op(uint32_t w, const DqRegs& k, uint32_t s_bits,
                                            uint32_t z) {
  static_assert(T::kIsF16, "rounded K-packed tiles are fp16 only");
  const u32x4 q = kp_int_op(w, k, z);
  const f16x2 sc = __builtin_bit_cast(f16x2, (s_bits & 0xFFFFu) * 0x10001u);
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t qi = q[i];  // through a scalar, as in kp_int_op
    r[i] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, qi) * sc);
  }
  return r;
}

enum { kKpFold = 0, kKpTile = 1, kKpChunk32 = 2, kKpChunk64 = 3 };

template <typename T, bool HAS_ZP, int NUM, bool LDSA>
__global__ __launch_bounds__(kKpThreads) void kpacked_kernel(KPackedParams p) {
  constexpr bool FOLD = NUM == kKpFold;
  __shared__ f32x4 red[kKpThreads / 64 - 1][64];
  static_assert(sizeof(red) == kKpRedBytes, "host LDS accounting");
  extern __shared__ __attribute__((aligned(16))) uint16_t a_lds[];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int j = lane >> 4;
  const int c = lane & 15;
  const int col = blockIdx.x * kKpCols + c;
  const int m0 = blockIdx.y * kKpRows;
  const bool row_ok = m0 + c < p.M;
  const int KC = p.K >> 5;        // 32-K chunks per column
  const int R = (KC + 3) >> 2;    // 128-K rounds
  const int r_beg = min(R, wave * p.rpw);
  const int r_end = min(R, r_beg + p.rpw);
  // clamped column and row: every load below is in bounds without a branch
  const uint32_t* wrow = p.w + (int64_t)min(col, p.N - 1) * (p.K >> 3);
  const uint16_t* arow = p.a + (int64_t)min(m0 + c, p.M - 1) * p.K;
  const int NG = p.K / p.G;
  const uint16_t* srow = p.sc + (int64_t)min(col, p.N - 1) * NG;
  const uint8_t* zrow = HAS_ZP ? p.zp + (int64_t)min(col, p.N - 1) * NG : nullptr;
  const DqRegs mag = dq_regs(p.dq);
  const u32x4 ones = {T::kOnePair, T::kOnePair, T::kOnePair, T::kOnePair};
  const u32x4 zero4 = {0u, 0u, 0u, 0u};
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const int mb = min(kKpRows, p.M - m0);
  const int astride = p.K + 8;  // elements: 16 bytes of padding per row
  if constexpr (LDSA) {
    // the block's activation rows, once per workgroup
    const int per_row = p.K >> 3;  // 16-byte pieces
    for (int idx = threadIdx.x; idx < mb * per_row; idx += kKpThreads) {
      const int rr = idx / per_row, q = idx - rr * per_row;
      *(u32x4*)(a_lds + rr * astride + 8 * q) = *(const u32x4*)(p.a + (int64_t)(m0 + rr) * p.K + 8 * q);
    }
    __syncthreads();
  }
  const uint16_t* alds = a_lds + min(c, mb - 1) * astride;

  if constexpr (NUM == kKpChunk32 || NUM == kKpChunk64) {
    constexpr int SPG = NUM == kKpChunk32 ? 1 : 2;  // MFMA steps per group
    for (int r0 = r_beg; r0 < r_end; r0 += kKpU) {
      uint32_t wv[kKpU][4], sb[kKpU][4], zb[kKpU][4];
      u32x4 av[kKpU][4];
#pragma unroll
      for (int u = 0; u < kKpU; ++u) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int ch = (r0 + u) * 4 + i;  // step i covers chunk ch alone
          const bool live = row_ok && r0 + u < r_end && ch < KC;
          const int cl = min(ch, KC - 1);
          wv[u][i] = wrow[cl * 4 + j];
          const int g = cl >> p.g_shift;
          sb[u][i] = srow[g];
          zb[u][i] = HAS_ZP ? (uint32_t)zrow[g] : (uint32_t)p.zp_bias;
          const u32x4 v = LDSA ? *(const u32x4*)(alds + cl * 32 + 8 * j)
                               : *(const u32x4*)(arow + cl * 32 + 8 * j);
          av[u][i] = live ? v : zero4;  // dead K and padding rows add zero
        }
      }
#pragma unroll
      for (int u = 0; u < kKpU; ++u) {
        if (r0 + u >= r_end) break;  // uniform over the wavefront
#pragma unroll
        for (int i0 = 0; i0 < 4; i0 += SPG) {
          f32x4 part = {0.f, 0.f, 0.f, 0.f};
          f32x4 sa = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int i = i0; i < i0 + SPG; ++i) {
            part = mfma<T>(av[u][i], kp_magic_op(wv[u][i], mag), part);
            sa = mfma<T>(av[u][i], ones, sa);
          }
          // column c's scale and zero point of this group, loaded by the lane
          const float s = widen(T{}, sb[u][i0]);
          const float base = T::kBase + (float)zb[u][i0];
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[v] = __builtin_fmaf(s, __builtin_fmaf(-base, sa[v], part[v]), acc[v]);
        }
      }
    }
  } else
  for (int r0 = r_beg; r0 < r_end; r0 += kKpU) {
    u32x4 wv[kKpU], av[kKpU][4];
    uint32_t sb[kKpU], zb[kKpU];
#pragma unroll
    for (int u = 0; u < kKpU; ++u) {
      const int ch = (r0 + u) * 4 + j;
      const bool live = row_ok && r0 + u < r_end && ch < KC;
      const int cl = min(ch, KC - 1);
      wv[u] = *(const u32x4*)(wrow + cl * 4);
      const int g = p.g_shift < 0 ? 0 : (cl >> p.g_shift);
      sb[u] = srow[g];
      zb[u] = HAS_ZP ? (uint32_t)zrow[g] : (uint32_t)p.zp_bias;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const u32x4 v = LDSA ? *(const u32x4*)(alds + cl * 32 + 8 * i)
                             : *(const u32x4*)(arow + cl * 32 + 8 * i);
        av[u][i] = live ? v : zero4;  // dead K and padding rows add zero
      }
    }
#pragma unroll
    for (int u = 0; u < kKpU; ++u) {
      if (r0 + u >= r_end) break;  // uniform over the wavefront
      if constexpr (FOLD) {
        f32x4 part = {0.f, 0.f, 0.f, 0.f};
        f32x4 sa = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if constexpr (T::kIsF16) {
            part = mfma<T>(av[u][i], kp_int_op(wv[u][i], mag, zb[u]), part);
          } else {
            part = mfma<T>(av[u][i], kp_magic_op(wv[u][i], mag), part);
            sa = mfma<T>(av[u][i], ones, sa);
          }
        }
        // lane l's outputs are column c, whose scale (and zero point) for
        // this round's group the lane loaded itself
        const float s = widen(T{}, sb[u]);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          float d = part[v];
          if constexpr (!T::kIsF16) d = __builtin_fmaf(-(T::kBase + (float)zb[u]), sa[v], d);
          acc[v] = __builtin_fmaf(s, d, acc[v]);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          acc = mfma<T>(av[u][i], kp_tile_op<T>(wv[u][i], mag, sb[u], zb[u]), acc);
      }
    }
  }

  // wavefronts 1..7 hand their sums to wavefront 0 through LDS
  if (wave > 0) red[wave - 1][lane] = acc;
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 0; w < kKpThreads / 64 - 1; ++w) acc += red[w][lane];
  if (col < p.N) {
    const float bv = p.bias ? widen(T{}, p.bias[col]) : 0.f;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int row = m0 + 4 * j + v;  // MFMA result row 4j + v, column c
      if (row < p.M) p.out[(int64_t)row * p.N + col] = narrow(T{}, acc[v] + bv);
    }
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <typename T, bool Z, int MODE, bool AL, int L, int MT, bool SLIDE, int W = kDecodeWaves>
static hipError_t decode_go(const DecodeParams& p, int grid, int lds, hipStream_t st) {
  if (lds > 65536) {  // above the default dynamic LDS limit: raise it once
    static const hipError_t once = hipFuncSetAttribute(
        (const void*)decode_kernel<T, Z, MODE, AL, L, MT, SLIDE, W>,
        hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024 - 64);
    if (once != hipSuccess) return once;
  }
  hipLaunchKernelGGL((decode_kernel<T, Z, MODE, AL, L, MT, SLIDE, W>), dim3(grid), dim3(64 * W),
                     lds, st, p);
  return hipGetLastError();
}
// rows rounded up to MT, and the last arrival's partial loads: windows one
// after another for one row per wavefront or fewer than two windows of
// splits (a window: 16 splits up to 8 rows, 4 above), else a sliding window
// (K = N = 4096 fp16 G = 32, 32 splits: M = 5 9.4 -> 8.9 us, M = 8 10.3 ->
// 9.1 us; at 20 splits, M = 5, it was 1 us slower)
template <typename T, bool Z, int MODE, bool AL, int L, int MT>
static hipError_t decode_slide(const DecodeParams& p, int grid, int lds, hipStream_t st) {
  if (p.S >= 2 * (MT <= 8 ? 16 : 4)) return decode_go<T, Z, MODE, AL, L, MT, true>(p, grid, lds, st);
  return decode_go<T, Z, MODE, AL, L, MT, false>(p, grid, lds, st);
}
template <typename T, bool Z, int MODE, bool AL, int L>
static hipError_t decode_mt(const DecodeParams& p, int grid, int lds, hipStream_t st) {
  if constexpr (AL && L <= 2) {
    // eight wavefronts per workgroup (the planner's choice for up to 8 rows
    // at one or two steps per wavefront): one row per wavefront
    if (p.W == kDecodeWavesWide) {
      if (p.M <= 4) return decode_go<T, Z, MODE, AL, L, 4, false, kDecodeWavesWide>(p, grid, lds, st);
      if (p.M <= 8) return decode_go<T, Z, MODE, AL, L, 8, false, kDecodeWavesWide>(p, grid, lds, st);
      return hipErrorInvalidValue;
    }
  }
  if (p.W != kDecodeWaves) return hipErrorInvalidValue;
  if (p.M <= 4) return decode_go<T, Z, MODE, AL, L, 4, false>(p, grid, lds, st);
  if (p.M <= 8) return decode_slide<T, Z, MODE, AL, L, 8>(p, grid, lds, st);
  return decode_slide<T, Z, MODE, AL, L, 16>(p, grid, lds, st);
}
template <typename T, bool Z, int MODE, bool AL>
static hipError_t decode_l(const DecodeParams& p, int grid, int lds, hipStream_t st) {
  if constexpr (!AL) {
    // shapes off the fast layout run one step per wavefront, 16-row reductions
    if (p.L != 1 || p.W != kDecodeWaves) return hipErrorInvalidValue;
    return decode_slide<T, Z, MODE, AL, 1, 16>(p, grid, lds, st);
  } else {
    switch (p.L) {
      case 1: return decode_mt<T, Z, MODE, AL, 1>(p, grid, lds, st);
      case 2: return decode_mt<T, Z, MODE, AL, 2>(p, grid, lds, st);
      case 4: return decode_mt<T, Z, MODE, AL, 4>(p, grid, lds, st);
      case 8: return decode_mt<T, Z, MODE, AL, 8>(p, grid, lds, st);
      default: return hipErrorInvalidValue;
    }
  }
}
template <typename T, bool Z, int MODE>
static hipError_t decode_al(const DecodeParams& p, int grid, int lds, hipStream_t st) {
  if ((p.N & 15) == 0 && (p.K & 7) == 0) return decode_l<T, Z, MODE, true>(p, grid, lds, st);
  return decode_l<T, Z, MODE, false>(p, grid, lds, st);
}
template <typename T, bool Z>
static hipError_t decode_mode(const DecodeParams& p, int mode, int grid, int lds, hipStream_t st) {
  switch (mode) {
    case kSit: return decode_al<T, Z, kSit>(p, grid, lds, st);
    case kOneGrp: return decode_al<T, Z, kOneGrp>(p, grid, lds, st);
    case kMulti: return decode_al<T, Z, kMulti>(p, grid, lds, st);
    default: return hipErrorInvalidValue;
  }
}
hipError_t launch_decode(const DecodeParams& p, int dtype, bool has_zp, int mode, int grid,
                         int lds, hipStream_t st) {
  if (dtype == W4A16_F16)
    return has_zp ? decode_mode<F16, true>(p, mode, grid, lds, st)
                  : decode_mode<F16, false>(p, mode, grid, lds, st);
  return has_zp ? decode_mode<BF16, true>(p, mode, grid, lds, st)
                : decode_mode<BF16, false>(p, mode, grid, lds, st);
}

// 64-row tiles in every variant; 32-row tiles only with K splits and
// K % 64 == 0 (the host's planner never asks for others)
template <typename T, bool Z, int GS, int KM>
static hipError_t prefill_go(const PrefillParams& p, int grid, hipStream_t st) {
  const dim3 g(grid), b(kPrefillThreads);
  if constexpr (KM == 0) {
    if (p.ring) {
      if (p.bm == 32 && p.S > 1)
        hipLaunchKernelGGL((prefill_kernel<T, Z, GS, KM, true, 32, true>), g, b, 0, st, p);
      else if (p.bm != 64)
        return hipErrorInvalidValue;
      else if (p.S > 1)
        hipLaunchKernelGGL((prefill_kernel<T, Z, GS, KM, true, 64, true>), g, b, 0, st, p);
      else
        hipLaunchKernelGGL((prefill_kernel<T, Z, GS, KM, false, 64, true>), g, b, 0, st, p);
      return hipGetLastError();
    }
  }
  if (p.ring) return hipErrorInvalidValue;
  if (p.S > 1) {
    if constexpr (KM == 0) {
      if (p.bm == 32) {
        hipLaunchKernelGGL((prefill_kernel<T, Z, GS, KM, true, 32, false>), g, b, 0, st, p);
        return hipGetLastError();
      }
    }
    if (p.bm != 64) return hipErrorInvalidValue;
    hipLaunchKernelGGL((prefill_kernel<T, Z, GS, KM, true, 64, false>), g, b, 0, st, p);
  } else {
    if (p.bm != 64) return hipErrorInvalidValue;
    hipLaunchKernelGGL((prefill_kernel<T, Z, GS, KM, false, 64, false>), g, b, 0, st, p);
  }
  return hipGetLastError();
}
template <typename T, bool Z, int GS>
static hipError_t prefill_km(const PrefillParams& p, int grid, hipStream_t st) {
  if (p.K % kPrefillBK == 0) return prefill_go<T, Z, GS, 0>(p, grid, st);
  if constexpr (GS == 0) {
    if (p.K % 8 != 0) return prefill_go<T, Z, GS, 2>(p, grid, st);
  }
  return prefill_go<T, Z, GS, 1>(p, grid, st);
}
template <typename T, bool Z>
static hipError_t prefill_gs(const PrefillParams& p, int grid, hipStream_t st) {
  if (p.G == p.K) return prefill_km<T, Z, 0>(p, grid, st);
  switch (p.G) {
    case 32: return prefill_km<T, Z, 1>(p, grid, st);
    case 64: return prefill_km<T, Z, 2>(p, grid, st);
    case 128: return prefill_km<T, Z, 4>(p, grid, st);
    default: return hipErrorInvalidValue;
  }
}
hipError_t launch_prefill_reduce(const PrefillReduceParams& p, int dtype, hipStream_t st) {
  const int64_t pieces = (int64_t)p.M * (p.N / 4);
  const int grid = (int)((pieces + 255) / 256);
  if (dtype == W4A16_F16)
    hipLaunchKernelGGL((prefill_reduce_kernel<F16>), dim3(grid), dim3(256), 0, st, p);
  else
    hipLaunchKernelGGL((prefill_reduce_kernel<BF16>), dim3(grid), dim3(256), 0, st, p);
  return hipGetLastError();
}
hipError_t launch_asum(const AsumParams& p, hipStream_t st) {
  hipLaunchKernelGGL(asum_kernel, dim3(p.rows / kPrefillBM, p.K / p.G), dim3(256), 0, st, p);
  return hipGetLastError();
}
hipError_t launch_prefill(const PrefillParams& p, int dtype, bool has_zp, int grid,
                          hipStream_t st) {
  if (dtype == W4A16_F16)
    return has_zp ? prefill_gs<F16, true>(p, grid, st) : prefill_gs<F16, false>(p, grid, st);
  return has_zp ? prefill_gs<BF16, true>(p, grid, st) : prefill_gs<BF16, false>(p, grid, st);
}

template <typename T, bool Z, int NUM>
static hipError_t kpacked_num(const KPackedParams& p, bool stage, hipStream_t st) {
  const dim3 grid((unsigned)((p.N + kKpCols - 1) / kKpCols), (unsigned)((p.M + kKpRows - 1) / kKpRows));
  if (stage) {
    hipLaunchKernelGGL((kpacked_kernel<T, Z, NUM, true>), grid, dim3(kKpThreads),
                       kpacked_lds_bytes(p.M, p.K), st, p);
  } else {
    hipLaunchKernelGGL((kpacked_kernel<T, Z, NUM, false>), grid, dim3(kKpThreads), 0, st, p);
  }
  return hipGetLastError();
}
// numerics: FOLD when a 128-K round lies in one group (G a multiple of 128,
// or G == K); otherwise TILE for fp16 and CHUNK for bf16
template <typename T, bool Z>
static hipError_t kpacked_go(const KPackedParams& p, bool fold, bool stage, hipStream_t st) {
  if (fold) return kpacked_num<T, Z, kKpFold>(p, stage, st);
  if constexpr (T::kIsF16) {
    return kpacked_num<T, Z, kKpTile>(p, stage, st);
  } else {
    if (p.g_shift == 0) return kpacked_num<T, Z, kKpChunk32>(p, stage, st);
    if (p.g_shift == 1) return kpacked_num<T, Z, kKpChunk64>(p, stage, st);
    return hipErrorInvalidValue;
  }
}
hipError_t launch_kpacked(const KPackedParams& p, int dtype, bool has_zp, bool fold, bool stage,
                          hipStream_t st) {
  if (dtype == W4A16_F16)
    return has_zp ? kpacked_go<F16, true>(p, fold, stage, st)
                  : kpacked_go<F16, false>(p, fold, stage, st);
  return has_zp ? kpacked_go<BF16, true>(p, fold, stage, st)
                : kpacked_go<BF16, false>(p, fold, stage, st);
}

template <typename T, bool Z>
static hipError_t dequant_go(const DequantParams& p, hipStream_t st) {
  const int64_t work = (((int64_t)p.K + 1) / 2) * (p.N >> 3);
  const int64_t grid = (work + 255) / 256;
  hipLaunchKernelGGL((dequant_kernel<T, Z>), dim3((unsigned)grid), dim3(256), 0, st, p);
  return hipGetLastError();
}
hipError_t launch_dequant(const DequantParams& p, int dtype, bool has_zp, hipStream_t st) {
  if (dtype == W4A16_F16) return has_zp ? dequant_go<F16, true>(p, st) : dequant_go<F16, false>(p, st);
  return has_zp ? dequant_go<BF16, true>(p, st) : dequant_go<BF16, false>(p, st);
}

}  // namespace w4a16
