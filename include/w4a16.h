/*
 * w4a16.h - C ABI of the MI355X (gfx950) weight-only int4 GEMM.
 *
 *   C[M,N] = A[M,K] . dequant(B),   dequant(B)[k,n] = (q[k,n] - z[k/G,n]) * s[k/G,n]
 *
 * Where the operation is defined (pages cited by title and section):
 *   - Operands and shapes: PR #51453 "Register the Triton W4A16 GEMM as a
 *     custom op", implementation item 1 (contiguous inputs, M,K from the
 *     activation, N = 8 * packed columns) and its Code section (the facade
 *     signature a, b_q, scales, qzeros|None, group_size, zp_bias=8; the
 *     output [M, 8*b_q.cols] in the activation's dtype; no input mutated).
 *   - Arithmetic: PR #40977 "RDNA hybrid W4A16", Code section (reference:
 *     zero points and scales repeated along K per group, (raw - zero)*scale
 *     in fp32, fp32 product, one cast to the activation dtype; symmetric
 *     weights use the constant 8).
 *   - Rejections: PR #43731 "TritonW4A16LinearKernel as CUDA fallback",
 *     Code section (can_implement: activation dtype, N % 8, g_idx, group
 *     size unless equal to the full K) and its Motivation (no kernel is an
 *     error, never a silent substitute).
 *
 * Layout (all row-major, contiguous, no padding):
 *   a       [M, K]    fp16 or bf16
 *   b_q     [K, N/8]  int32; uint4 value j of word c is column 8c+j, in
 *                     bits [4j, 4j+4) (LSB first)
 *   scales  [K/G, N]  same dtype as a
 *   qzeros  [K/G, N/8] int32 packed like b_q, or NULL (symmetric: z = zp_bias)
 *   bias    [N]       same dtype as a, or NULL (w4a16_gemm_bias only)
 *   out     [M, N]    same dtype as a
 *
 * Conventions:
 *   - Every call returns a w4a16_status; nothing is thrown or aborted. The
 *     calling thread's last message is returned by w4a16_last_error().
 *   - All argument checks run before anything is launched.
 *   - Device pointers must be 16-byte aligned; the caller owns every buffer.
 *   - GPU calls are enqueued on `stream` (a hipStream_t; NULL = the null
 *     stream) and never synchronise the device or the stream.
 *   - G (group_size) is 32, 64, 128 or K (one group per column), and K is a
 *     multiple of G. N is a multiple of 8. M = 0 is a no-op that succeeds.
 *     K is at most 2^24 (the kernels address a row block with 32-bit byte
 *     offsets).
 *
 * Scratch ("workspace"). Some launches split K across workgroups and meet in
 * fp32 partial sums in device memory (the page of PR #51453, Review section,
 * asks for split-K because small problems leave most of the GPU idle). A
 * workspace starts with W4A16_WORKSPACE_COUNTER_BYTES of arrival counters,
 * followed by the partials. The counter region must hold zeros before the
 * workspace is first used; every launch that completes leaves it zero, and
 * nothing else is ever written there, so one zeroed workspace serves any
 * sequence of calls on one stream. Two launches that run at the same time
 * (different streams) must not share a workspace.
 */
#ifndef W4A16_H
#define W4A16_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  W4A16_OK = 0,
  W4A16_ERR_NULL = 1,       /* a required pointer is NULL */
  W4A16_ERR_SHAPE = 2,      /* M < 0, K <= 0, N <= 0, N % 8, K % G, size overflow */
  W4A16_ERR_GROUP = 3,      /* G not in {32, 64, 128, K} */
  W4A16_ERR_DTYPE = 4,      /* dtype not W4A16_F16 / W4A16_BF16 */
  W4A16_ERR_ZP = 5,         /* zp_bias outside 0..15 (symmetric calls only) */
  W4A16_ERR_ALIGN = 6,      /* a device pointer is not 16-byte aligned */
  W4A16_ERR_DEVICE = 7,     /* no device, or the current device is not gfx950 */
  W4A16_ERR_HIP = 8,        /* a HIP runtime call or launch failed */
  W4A16_ERR_VALUE = 9,      /* pack: a value outside 0..15 */
  W4A16_ERR_PLAN = 10,      /* a caller-supplied plan does not fit the problem */
  W4A16_ERR_WORKSPACE = 11  /* workspace too small, or scratch that would have to be
                               allocated while the stream is being captured */
} w4a16_status;

/* Bytes of arrival counters at the start of every workspace (see above). */
#define W4A16_WORKSPACE_COUNTER_BYTES 65536

typedef enum { W4A16_F16 = 0, W4A16_BF16 = 1 } w4a16_dtype;

typedef enum {
  W4A16_ROUTE_NONE = 0,     /* M == 0: nothing to launch */
  W4A16_ROUTE_DECODE = 1,   /* skinny split-K kernel, M <= 16 */
  W4A16_ROUTE_PREFILL = 2   /* tiled MFMA kernel, any M */
} w4a16_route;

/* The launch the selector picked for one problem (all fields plain ints). */
typedef struct {
  int32_t route;            /* w4a16_route */
  int32_t block_m;          /* rows of A per workgroup tile (decode: 16) */
  int32_t block_n;          /* output columns per workgroup */
  int32_t block_k;          /* K rows per pipeline step */
  int32_t decode_mode;      /* decode: 0 = scale folded into each weight;
                               1 = scale applied once per group, one group per
                               wavefront; 2 = as 1, several groups per
                               wavefront */
  int32_t splits;           /* K splits across workgroups (1 = none) */
  int32_t steps_per_wave;   /* decode: 32-row K steps per wavefront (1, 2, 4, 8);
                               prefill: 64-row K stages per workgroup */
  int32_t grid;             /* workgroups launched */
  int32_t threads;          /* threads per workgroup */
  int32_t lds_bytes;        /* LDS per workgroup */
  int64_t workspace_bytes;  /* device scratch the launch needs: 0, or the
                               counter region plus the fp32 partials */
} w4a16_plan_t;

/*
 * w4a16_gemm - out = a . dequant(b_q, scales, qzeros) on the GPU.
 * Route and tiles are chosen from the runtime M, K, N, G on every call
 * (PR #51453 Motivation: a tile choice frozen at trace time slowed decode).
 * Scratch: the library keeps one workspace per (device, stream). When a
 * launch needs more than that stream's workspace holds, it allocates a
 * larger one (hipMalloc), zeroes its counter region on `stream`, and keeps
 * the old one allocated until the process ends (a captured graph or a
 * queued launch may still use it); it never synchronises. While `stream`
 * is being captured into a graph no allocation is made: a launch that would
 * need one fails with WORKSPACE (make one uncaptured call of the largest
 * problem first, or use w4a16_gemm_ws). Calls on different streams never
 * share scratch.
 * Errors: NULL, SHAPE, GROUP, DTYPE, ZP, ALIGN, DEVICE, HIP, WORKSPACE.
 */
w4a16_status w4a16_gemm(const void* a, const int32_t* b_q, const void* scales,
                        const int32_t* qzeros, int32_t group_size,
                        int32_t zp_bias, void* out, int64_t M, int64_t K,
                        int64_t N, int32_t dtype, void* stream);

/*
 * w4a16_gemm_bias - as w4a16_gemm, plus a bias row: out[m,n] =
 * RNE(fp32(sum_k a[m,k] w[k,n]) + fp32(bias[n])), the bias added to the
 * fp32 result before the one rounding to the output type and indexed by
 * the output column only (PR #40977 "RDNA hybrid W4A16", Code section: the
 * test's reference adds bias.float() to the fp32 product before the cast;
 * its Review section reports the prior kernel indexing the bias by a row
 * count, out of bounds). bias: device pointer to N values of `dtype`,
 * 16-byte aligned, owned by the caller, never written; NULL gives exactly
 * w4a16_gemm. Errors: those of w4a16_gemm (ALIGN for a misaligned bias).
 */
w4a16_status w4a16_gemm_bias(const void* a, const int32_t* b_q,
                             const void* scales, const int32_t* qzeros,
                             int32_t group_size, int32_t zp_bias,
                             const void* bias, void* out, int64_t M,
                             int64_t K, int64_t N, int32_t dtype,
                             void* stream);

/*
 * w4a16_gemm_planned - as w4a16_gemm, but runs the launch in `plan`
 * (obtained from w4a16_plan or w4a16_plan_route, possibly with another
 * route or split forced). The plan is checked against the problem first.
 * Errors: those of w4a16_gemm, and PLAN.
 */
w4a16_status w4a16_gemm_planned(const void* a, const int32_t* b_q,
                                const void* scales, const int32_t* qzeros,
                                int32_t group_size, int32_t zp_bias, void* out,
                                int64_t M, int64_t K, int64_t N, int32_t dtype,
                                const w4a16_plan_t* plan, void* stream);

/*
 * w4a16_workspace_bytes - the workspace w4a16_gemm_ws needs for one problem
 * (host only, no GPU call): 0 when the launch splits no K across
 * workgroups, else W4A16_WORKSPACE_COUNTER_BYTES plus the fp32 partials.
 * num_cus: compute units of the device the call will run on (256 on
 * MI355X; <= 0 means 256); w4a16_gemm_ws plans with the current device's
 * count. Written to *bytes. The split-K request this serves is PR #51453's
 * Review section; keeping scratch in caller memory keeps the call free of
 * allocation, as its Code section's non-mutating, graph-capture-friendly
 * operator needs.
 * Errors: SHAPE, GROUP, DTYPE, NULL (bytes).
 */
w4a16_status w4a16_workspace_bytes(int64_t M, int64_t K, int64_t N, int32_t group_size,
                                   int32_t dtype, int32_t num_cus, int64_t* bytes);

/*
 * w4a16_gemm_ws - as w4a16_gemm_bias (bias may be NULL), with the scratch
 * in caller memory: `workspace` (device, 16-byte aligned, owned by the
 * caller) of `ws_bytes` bytes, laid out and kept as described at the top.
 * NULL with ws_bytes 0 is accepted when the problem needs no scratch. No
 * allocation, no synchronisation: the call can be captured into a HIP graph
 * on its first use (PR #51453 Code section: mutates_args=[], so that the
 * operator is safe under CUDA-graph capture; Risks section: compile mode 3
 * with FULL_AND_PIECEWISE graphs).
 * Errors: those of w4a16_gemm_bias, and WORKSPACE (ws_bytes below
 * w4a16_workspace_bytes for the current device), NULL (workspace needed).
 */
w4a16_status w4a16_gemm_ws(const void* a, const int32_t* b_q, const void* scales,
                           const int32_t* qzeros, int32_t group_size, int32_t zp_bias,
                           const void* bias, void* out, int64_t M, int64_t K, int64_t N,
                           int32_t dtype, void* workspace, int64_t ws_bytes, void* stream);

/*
 * w4a16_gemm_noalloc - as w4a16_gemm_bias (bias may be NULL), for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc). Its scratch is a fixed
 * device array inside the library, one copy per GPU, held until the process
 * ends: W4A16_NOALLOC_SCRATCH_BYTES, i.e. the counter region plus 32 MiB of
 * fp32 partials; a problem whose split-K partials need more is refused with
 * WORKSPACE before anything runs (w4a16_workspace_bytes gives the need). The
 * call allocates nothing; its first call on a device looks up the array's
 * address and clears its counter region with a kernel on `stream`. Every
 * call on one GPU shares that GPU's array: calls that may overlap in time
 * (different streams, or several threads) race on it and must be ordered by
 * the caller, e.g. issued to one stream.
 * Errors: those of w4a16_gemm_bias, and WORKSPACE.
 */
#define W4A16_NOALLOC_SCRATCH_BYTES (W4A16_WORKSPACE_COUNTER_BYTES + (32ll << 20))
w4a16_status w4a16_gemm_noalloc(const void* a, const int32_t* b_q, const void* scales,
                                const int32_t* qzeros, int32_t group_size, int32_t zp_bias,
                                const void* bias, void* out, int64_t M, int64_t K, int64_t N,
                                int32_t dtype, void* stream);

/*
 * w4a16_plan - the launch w4a16_gemm would make (host only, no GPU call):
 * route by the real M (PR #40977 "RDNA hybrid W4A16", Impl. item 5: the
 * skinny kernel for small batches, the tiled kernel above) and tiles from
 * the runtime shape (PR #51453 Motivation and Impl. item 1: BLOCK_M/N/K
 * picked per call, never frozen at trace time).
 * num_cus: compute units of the target (256 on MI355X); <= 0 means 256.
 * Errors: SHAPE, GROUP, DTYPE, NULL (plan).
 */
w4a16_status w4a16_plan(int64_t M, int64_t K, int64_t N, int32_t group_size,
                        int32_t has_zp, int32_t dtype, int32_t num_cus,
                        w4a16_plan_t* plan);

/*
 * w4a16_plan_route - as w4a16_plan with the route forced
 * (W4A16_ROUTE_DECODE needs 1 <= M <= 16) and, for decode, the steps per
 * wavefront (1, 2, 4 or 8; 0 = selector's choice) and the decode mode
 * (0, 1, 2; -1 = selector's choice; mode 1 needs every wavefront's steps
 * inside one group; mode 0, the rounded-weight operand, is fp16 only)
 * forced; for prefill, steps_per_wave forces the 64-row K stages per
 * workgroup (0 = selector's choice; a multiple of 2 when G = 128 < K; at
 * most 32 K splits result) and decode_mode is ignored. Same passages as
 * w4a16_plan; forcing a route exists to test every kernel against the
 * reference on the same shapes (PR #40977 Code section: the reference test
 * is run across the skinny-batch boundary).
 * Errors: those of w4a16_plan, and PLAN.
 */
w4a16_status w4a16_plan_route(int64_t M, int64_t K, int64_t N,
                              int32_t group_size, int32_t has_zp,
                              int32_t dtype, int32_t num_cus, int32_t route,
                              int32_t steps_per_wave, int32_t decode_mode,
                              w4a16_plan_t* plan);

/*
 * w4a16_dequant - w_out[k,n] = RNE_dtype((q - z) * s), the dequantised
 * weight in the activation dtype, written as a dense [K, N] array (test
 * probe of the magic-number unpack of PR #40977 "RDNA hybrid W4A16",
 * Impl. item 3, with the reference's (raw - zero) * scale of its Code
 * section; the fp16 kernels that feed rounded weights to the MFMA use the
 * same device routine).
 * Errors: NULL, SHAPE, GROUP, DTYPE, ZP, ALIGN, DEVICE, HIP.
 */
w4a16_status w4a16_dequant(const int32_t* b_q, const void* scales,
                           const int32_t* qzeros, int32_t group_size,
                           int32_t zp_bias, void* w_out, int64_t K, int64_t N,
                           int32_t dtype, void* stream);

/*
 * w4a16_pack_int4 - host utility: q [rows, cols] uint8 values 0..15 ->
 * packed [rows, cols/8] int32 in the layout above (used for b_q and
 * qzeros; PR #51453 Impl. item 1: eight uint4 per int32 along N, so
 * N = 8 * packed columns). Host pointers.
 * Errors: NULL, SHAPE (cols % 8), VALUE.
 */
w4a16_status w4a16_pack_int4(const uint8_t* q, int64_t rows, int64_t cols,
                             int32_t* packed);

/*
 * w4a16_unpack_int4 - host inverse of w4a16_pack_int4 (diagnostics; the
 * nibbles come out by logical shifts, as PR #40977's Impl. item 4 extracts
 * them). Host pointers; `cols` counts unpacked columns.
 * Errors: NULL, SHAPE.
 */
w4a16_status w4a16_unpack_int4(const int32_t* packed, int64_t rows,
                               int64_t cols, uint8_t* q);

/*
 * w4a16_gemm_kpacked - the same product for weights stored K-packed, the
 * hybrid path's single buffer (PR #40977 "RDNA hybrid W4A16", Impl. item 4
 * and the Code section's module docstring):
 *   w       [N, K/8] int32: word c of row n holds K values 8c..8c+7 of
 *           column n in ExLlama order, nibble p (bits [4p, 4p+4)) holding
 *           K offset 0, 2, 4, 6, 1, 3, 5, 7 for p = 0..7, so that nibbles
 *           i and i+4 are K values 2i and 2i+1
 *           (w4a16_pack_int4_kshuffle writes it)
 *   scales  [N, K/G] in `dtype`
 *   zeros   [N, K/G] uint8 (values 0..15), or NULL (z = zp_bias)
 *   bias    [N] in `dtype`, or NULL; added to the fp32 result
 *   a [M, K] and out [M, N] as for w4a16_gemm.
 * out[m,n] = RNE(fp32(sum_k a[m,k] (q[n,k] - z[n,k/G]) s[n,k/G]) + bias[n]).
 * K must be a multiple of 32 (G in {32, 64, 128, K}); N is any positive
 * size. a, w, scales, out and bias must be 16-byte aligned; zeros need no
 * alignment. Device pointers, owned by the caller; only out is written.
 * One launch, no scratch memory, no allocation; any M (16-row blocks).
 * Errors: NULL, SHAPE, GROUP, DTYPE, ZP, ALIGN, DEVICE, HIP.
 */
w4a16_status w4a16_gemm_kpacked(const void* a, const int32_t* w,
                                const void* scales, const uint8_t* zeros,
                                int32_t group_size, int32_t zp_bias,
                                const void* bias, void* out, int64_t M,
                                int64_t K, int64_t N, int32_t dtype,
                                void* stream);

/*
 * w4a16_pack_int4_kshuffle - host utility: q [N, K] uint8 values 0..15 ->
 * packed [N, K/8] int32 in the K-packed ExLlama order of
 * w4a16_gemm_kpacked (PR #40977 "RDNA hybrid W4A16", key files and symbols:
 * the packing helper and its layout test). Host pointers.
 * Errors: NULL, SHAPE (K % 8), VALUE.
 */
w4a16_status w4a16_pack_int4_kshuffle(const uint8_t* q, int64_t N, int64_t K,
                                      int32_t* packed);

/*
 * w4a16_unpack_int4_kshuffle - host inverse of w4a16_pack_int4_kshuffle
 * (PR #40977 "RDNA hybrid W4A16", Impl. item 4: the shuffle is undone when
 * the nibbles are unpacked). Host pointers. Errors: NULL, SHAPE.
 */
w4a16_status w4a16_unpack_int4_kshuffle(const int32_t* packed, int64_t N,
                                        int64_t K, uint8_t* q);

/*
 * Message of the calling thread's last failed call ("" if none): why the
 * problem was refused, as PR #43731's can_implement (Code section) returns
 * a reason with every refusal and its Motivation treats "no kernel" as an
 * error, never a silent substitute. Owned by the library, valid until the
 * thread's next failing call.
 */
const char* w4a16_last_error(void);

/*
 * Library version string (static storage), so a caller can record which
 * build of the kernels ran (PR #40977 Impl. item 6: benchmark runs name the
 * kernel they time).
 */
const char* w4a16_version(void);

#ifdef __cplusplus
}
#endif

#endif /* W4A16_H */
