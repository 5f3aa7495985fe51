"""CPU oracle for the weight-only int4 GEMM  C[M,N] = A[M,K] . dequant(B).

TEST INFRASTRUCTURE ONLY. This module is the slow, plain reference that the
HIP library is checked against. Only the test suite, the smoke check of
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import
or run it. The library (``weight_only_int4_unpack_amd``) never imports it,
and it imports nothing from the library: the two share no code.

What it computes, and where each step comes from (pages are cited by title
and section; "Code" is the page's key-source-snippet section):

* Packed layout, [K, N] orientation. ``b_q`` is int32 ``[K, N/8]``, eight
  uint4 values per word along N, so ``N = 8 * b_q.shape[1]``; ``scales`` is
  ``[K/G, N]`` in the activation dtype (PR #51453 "Register Triton W4A16 GEMM
  as a custom op", Impl. item 1 and the Code section's fake-impl test
  shapes). ``qzeros``, when given, is ``[K/G, N/8]`` packed the same way.
* Nibble order inside a word: the pages leave it open. The reading taken
  here is sequential and LSB-first: column ``8c + j`` sits in bits
  ``[4j, 4j+4)`` of word ``c``, extracted with logical shifts (PR #40977
  "RDNA hybrid W4A16", Code section: nibbles are pulled out with shifts).
* Dequantisation ``w = (q - z) * s`` computed in fp32, where row k uses scale
  and zero-point row ``k // G`` (the reference in PR #40977's test file,
  Code section: ``repeat_interleave`` of the group rows along K, then
  ``(raw - zero) * scale`` in float). Symmetric weights have no zero-point
  tensor and use the constant ``zp_bias`` (8 for uint4b8; PR #51453 Code
  section, ``zp_bias=8`` default and the ``qzeros=None`` call).
* GEMM in fp32: ``A.float() @ W`` then one round-to-nearest-even cast to the
  activation dtype (PR #40977 Code section, reference function's last two
  lines).
* Optional bias ``[N]`` in the activation dtype: widened to fp32 and added
  to the fp32 product, by output column, before that one cast (PR #40977
  Code section: the reference adds ``bias.float()`` to the fp32 result;
  its Review section reports the prior kernel's bias indexed out of bounds
  by a row count, so the index here is the column alone).
* Rejections (PR #43731 "TritonW4A16LinearKernel as CUDA fallback", Code
  section ``can_implement``): activations not fp16/bf16, N not a multiple
  of 8, unsupported group size unless it equals the full K. The supported
  set {32, 64, 128} is not printed on the pages; it is the reading taken for
  the group sizes this build serves.

* K-packed layout (the hybrid path's single weight buffer; PR #40977 "RDNA
  hybrid W4A16", Impl. item 4 and the Code section's module docstring):
  int32 ``[N, K/8]``, eight K values of one column per word, in ExLlama's
  shuffled nibble order. The pages name the order but do not print it. The
  reading taken here is the one the shuffle exists for: nibble p holds K
  offset ``(0, 2, 4, 6, 1, 3, 5, 7)[p]``, so that masking the word shifted
  right by 4i with 0x000F000F leaves K values 2i and 2i+1 in the two 16-bit
  halves, a packed pair of consecutive K. Scales are ``[N, K/G]`` and zero
  points, when given, ``[N, K/G]`` uint8 (values 0..15), column-major like
  the weights (the test's reference takes ``[N, K//G]`` scales and zero
  points, Code section); the zero points' storage type is not given and
  one byte each is the reading taken.
* Pins: every function here is checked by ``tests/test_oracle.py`` against
facts other than itself (printed pack vectors of the stated convention,
closed forms, invariants, torch's own bf16/fp16 casts, exact integer
arithmetic and an fp64 brute force). No function is "parity unpinned".

Arrays of fp16/bf16 values are carried as ``uint16`` bit patterns plus a
dtype tag (``"fp16"`` or ``"bf16"``), because NumPy has no bfloat16.
"""
from __future__ import annotations

import numpy as np

F16 = "fp16"
BF16 = "bf16"
DTYPES = (F16, BF16)
SUPPORTED_GROUP_SIZES = (32, 64, 128)
TOLERANCE = 2e-2


# --------------------------------------------------------------------------
# bit patterns <-> fp32
# --------------------------------------------------------------------------
def to_f32(bits, dtype: str) -> np.ndarray:
    """Exact widening of fp16/bf16 bit patterns to fp32."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    if dtype == F16:
        return bits.view(np.float16).astype(np.float32)
    if dtype == BF16:
        # bf16 is the upper half of an fp32 word.
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    raise ValueError(f"unsupported dtype {dtype!r}")


def rne_bits(x, dtype: str) -> np.ndarray:
    """Round fp32 values to fp16/bf16 (round to nearest, ties to even).

    fp16 uses NumPy's cast, which rounds to nearest even. bf16 is done here
    on the bits: add 0x7FFF plus the lowest kept bit, then drop the low 16
    bits; a carry into the exponent is the correct round-up (it also turns
    the largest finite values into infinity exactly when RNE would). NaNs
    stay NaN (quiet bit forced).
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == F16:
        with np.errstate(over="ignore"):     # overflow to inf is the RNE result
            return x.astype(np.float16).view(np.uint16)
    if dtype == BF16:
        u = x.view(np.uint32).astype(np.uint64)
        r = ((u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1)))
             >> np.uint64(16)).astype(np.uint16)
        nan = np.isnan(x)
        if nan.any():
            r[nan] = ((u[nan] >> np.uint64(16)) | np.uint64(0x40)).astype(np.uint16)
        return r
    raise ValueError(f"unsupported dtype {dtype!r}")


# --------------------------------------------------------------------------
# packing
# --------------------------------------------------------------------------
def unpack_int4(packed) -> np.ndarray:
    """int32 ``[R, C]`` -> uint8 ``[R, 8C]``; value j of word c is column 8c+j.

    The word is reinterpreted as unsigned so the shifts are logical and a
    word with its sign bit set unpacks the same as any other.
    """
    p = np.ascontiguousarray(packed, dtype=np.int32).view(np.uint32)
    if p.ndim != 2:
        raise ValueError("packed array must be 2-D")
    out = np.empty((p.shape[0], p.shape[1], 8), dtype=np.uint8)
    for j in range(8):
        out[:, :, j] = (p >> np.uint32(4 * j)) & np.uint32(0xF)
    return out.reshape(p.shape[0], p.shape[1] * 8)


def pack_int4(q) -> np.ndarray:
    """uint4 values ``[R, 8C]`` (0..15) -> int32 ``[R, C]``, inverse of unpack."""
    q = np.asarray(q)
    if q.ndim != 2 or q.shape[1] % 8 != 0:
        raise ValueError("values must be 2-D with a column count divisible by 8")
    if q.size and (q.min() < 0 or q.max() > 15):
        raise ValueError("uint4 values must lie in 0..15")
    q = q.astype(np.uint32).reshape(q.shape[0], q.shape[1] // 8, 8)
    word = np.zeros(q.shape[:2], dtype=np.uint32)
    for j in range(8):
        word |= q[:, :, j] << np.uint32(4 * j)
    return word.view(np.int32)


# --------------------------------------------------------------------------
# validation (the rejections of the kernel-selection check)
# --------------------------------------------------------------------------
def check(M: int, K: int, N: int, group_size: int, dtype: str,
          has_zp: bool, zp_bias: int = 8) -> None:
    """Raise ValueError for every argument combination the method rejects."""
    if dtype not in DTYPES:
        raise ValueError("only float16/bfloat16 activations are supported")
    if M < 0 or K <= 0 or N <= 0:
        raise ValueError("need M >= 0, K > 0, N > 0")
    if N % 8 != 0:
        raise ValueError(f"N={N} must be divisible by 8 (8 int4 per int32)")
    if group_size not in SUPPORTED_GROUP_SIZES and group_size != K:
        raise ValueError(f"group size {group_size} not supported")
    if K % group_size != 0:
        raise ValueError(f"K={K} is not a multiple of group size {group_size}")
    if not has_zp and not (0 <= zp_bias <= 15):
        raise ValueError("zp_bias must lie in 0..15")


# --------------------------------------------------------------------------
# dequantisation
# --------------------------------------------------------------------------
def dequant_fp32(b_q, scales_bits, qzeros, group_size: int, zp_bias: int,
                 dtype: str, cols=None) -> np.ndarray:
    """W32[k, n] = (q[k, n] - z[k // G, n]) * s[k // G, n] in fp32.

    ``cols`` optionally restricts the result to a list of output columns
    (for sampled checks at full size); the arithmetic is the same.
    """
    b_q = np.asarray(b_q, dtype=np.int32)
    K = b_q.shape[0]
    N = b_q.shape[1] * 8
    if cols is None:
        cols = np.arange(N)
    cols = np.asarray(cols, dtype=np.int64)
    words = cols // 8
    lane = cols % 8
    # unpack only the words that hold the requested columns
    uw, inv = np.unique(words, return_inverse=True)
    Q = unpack_int4(b_q[:, uw]).reshape(K, len(uw), 8)[:, inv, lane]
    S = to_f32(scales_bits, dtype)[:, cols]
    if qzeros is None:
        Z = np.full(S.shape, float(zp_bias), dtype=np.float32)
    else:
        qz = np.asarray(qzeros, dtype=np.int32)
        Zall = unpack_int4(qz[:, uw]).reshape(qz.shape[0], len(uw), 8)
        Z = Zall[:, inv, lane].astype(np.float32)
    g = np.arange(K) // group_size
    return (Q.astype(np.float32) - Z[g, :]) * S[g, :]


def dequant_tile(b_q, scales_bits, qzeros, group_size: int, zp_bias: int,
                 dtype: str) -> np.ndarray:
    """The dequantised weight rounded once to the activation dtype (bits).

    ``(q - z) * s`` is exact in fp32 (a 5-bit integer times an 11- or 8-bit
    significand), so this is the correctly rounded dequantised weight.
    """
    return rne_bits(dequant_fp32(b_q, scales_bits, qzeros, group_size,
                                 zp_bias, dtype), dtype)


# --------------------------------------------------------------------------
# GEMM
# --------------------------------------------------------------------------
def gemm_f32(a_bits, b_q, scales_bits, qzeros, group_size: int,
             zp_bias: int, dtype: str, rows=None, cols=None,
             bias_bits=None) -> np.ndarray:
    """fp32 product ``float(A) @ W32`` (optionally only some rows/columns),
    plus ``float(bias)`` per output column when a bias is given."""
    A = to_f32(a_bits, dtype)
    if rows is not None:
        A = A[np.asarray(rows, dtype=np.int64)]
    W = dequant_fp32(b_q, scales_bits, qzeros, group_size, zp_bias, dtype,
                     cols=cols)
    C = A @ W
    if bias_bits is not None:
        b = to_f32(bias_bits, dtype)
        if cols is not None:
            b = b[np.asarray(cols, dtype=np.int64)]
        C = C + b[None, :]
    return C


def gemm(a_bits, b_q, scales_bits, qzeros, group_size: int, zp_bias: int,
         dtype: str, rows=None, cols=None, bias_bits=None) -> np.ndarray:
    """Output bits in the activation dtype: RNE of the fp32 product (plus
    bias)."""
    return rne_bits(gemm_f32(a_bits, b_q, scales_bits, qzeros, group_size,
                             zp_bias, dtype, rows=rows, cols=cols,
                             bias_bits=bias_bits), dtype)


def bruteforce_f64(a_bits, b_q, scales_bits, qzeros, group_size: int,
                   zp_bias: int, dtype: str, bias_bits=None) -> np.ndarray:
    """fp64 triple loop over plain Python numbers; tiny shapes only.

    Every weight is taken straight from its word with integer shifts, so
    this shares no vectorised indexing with ``dequant_fp32``. A bias is
    added to each output's fp64 sum.
    """
    A = to_f32(a_bits, dtype).astype(np.float64)
    B = None if bias_bits is None else to_f32(bias_bits, dtype).astype(np.float64)
    S = to_f32(scales_bits, dtype).astype(np.float64)
    bq = np.asarray(b_q, dtype=np.int64) & 0xFFFFFFFF
    qz = None if qzeros is None else np.asarray(qzeros, dtype=np.int64) & 0xFFFFFFFF
    M, K = A.shape
    N = bq.shape[1] * 8
    out = np.zeros((M, N), dtype=np.float64)
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                q = (int(bq[k, n // 8]) >> (4 * (n % 8))) & 15
                g = k // group_size
                z = zp_bias if qz is None else (int(qz[g, n // 8]) >> (4 * (n % 8))) & 15
                acc += float(A[m, k]) * float(q - z) * float(S[g, n])
            out[m, n] = acc if B is None else acc + float(B[n])
    return out


# --------------------------------------------------------------------------
# K-packed layout [N, K/8] with the ExLlama nibble order
# --------------------------------------------------------------------------
EXLLAMA_ORDER = (0, 2, 4, 6, 1, 3, 5, 7)  # K offset held by nibble p of a word


def pack_int4_kshuffle(q_nk) -> np.ndarray:
    """uint4 ``[N, K]`` (0..15, K % 8 == 0) -> int32 ``[N, K/8]``: word c of
    row n holds K values 8c..8c+7, nibble p holding offset EXLLAMA_ORDER[p]."""
    q = np.asarray(q_nk)
    if q.ndim != 2 or q.shape[1] % 8 != 0:
        raise ValueError("q must be [N, K] with K a multiple of 8")
    if q.size and (q.min() < 0 or q.max() > 15):
        raise ValueError("values must lie in 0..15")
    g = q.astype(np.uint32).reshape(q.shape[0], q.shape[1] // 8, 8)
    w = np.zeros(g.shape[:2], dtype=np.uint32)
    for p, off in enumerate(EXLLAMA_ORDER):
        w |= g[:, :, off] << np.uint32(4 * p)
    return w.view(np.int32)


def unpack_int4_kshuffle(w_nk8) -> np.ndarray:
    """int32 ``[N, K/8]`` -> uint8 ``[N, K]``, inverse of pack_int4_kshuffle."""
    w = np.asarray(w_nk8, dtype=np.int32).view(np.uint32)
    out = np.zeros((w.shape[0], w.shape[1], 8), dtype=np.uint8)
    for p, off in enumerate(EXLLAMA_ORDER):
        out[:, :, off] = (w >> np.uint32(4 * p)) & np.uint32(15)
    return out.reshape(w.shape[0], w.shape[1] * 8)


def dequant_kpacked_fp32(w_nk8, scales_nkg_bits, zeros_nkg, group_size: int,
                         zp_bias: int, dtype: str, cols=None) -> np.ndarray:
    """W32[k, n] = (q[n, k] - z[n, k // G]) * s[n, k // G] in fp32, returned
    as ``[K, N]`` (the orientation of the product); ``cols`` optionally
    selects output columns."""
    w = np.asarray(w_nk8, dtype=np.int32)
    if cols is not None:
        cols = np.asarray(cols, dtype=np.int64)
        w = w[cols]
    Q = unpack_int4_kshuffle(w).astype(np.float32)          # [n, K]
    S = to_f32(scales_nkg_bits, dtype)
    if cols is not None:
        S = S[cols]
    if zeros_nkg is None:
        Z = np.full(S.shape, float(zp_bias), dtype=np.float32)
    else:
        Z = np.asarray(zeros_nkg, dtype=np.uint8)
        Z = (Z[cols] if cols is not None else Z).astype(np.float32)
    g = np.arange(Q.shape[1]) // group_size
    return ((Q - Z[:, g]) * S[:, g]).T


def gemm_kpacked(a_bits, w_nk8, scales_nkg_bits, zeros_nkg, group_size: int,
                 zp_bias: int, dtype: str, rows=None, cols=None,
                 bias_bits=None) -> np.ndarray:
    """Output bits of ``A @ W (+ bias)`` for K-packed weights: fp32 product,
    bias added in fp32 by column, one RNE cast (as ``gemm``)."""
    A = to_f32(a_bits, dtype)
    if rows is not None:
        A = A[np.asarray(rows, dtype=np.int64)]
    C = A @ dequant_kpacked_fp32(w_nk8, scales_nkg_bits, zeros_nkg, group_size,
                                 zp_bias, dtype, cols=cols)
    if bias_bits is not None:
        b = to_f32(bias_bits, dtype)
        if cols is not None:
            b = b[np.asarray(cols, dtype=np.int64)]
        C = C + b[None, :]
    return rne_bits(C, dtype)


def within_tolerance(got_bits, want_bits, dtype: str,
                     tol: float = TOLERANCE) -> np.ndarray:
    """Elementwise ``|got - want| <= tol * max(1, |want|)`` on dtype values."""
    g = to_f32(got_bits, dtype).astype(np.float64)
    w = to_f32(want_bits, dtype).astype(np.float64)
    return np.abs(g - w) <= tol * np.maximum(1.0, np.abs(w))
