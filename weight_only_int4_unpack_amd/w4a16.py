"""ctypes binding of ``libw4a16.so`` (include/w4a16.h).

Argument marshalling only: shapes are read off the tensors, checked against
each other, and passed with raw pointers and the current HIP stream. Every
step of the computation runs in the library's kernels. There is no fallback:
if the library is missing or the device is not gfx950, calls raise.

The Python signature mirrors the facade of PR #51453 "Register the Triton
W4A16 GEMM as a custom op" (Code section): ``gemm(a, b_q, scales, qzeros,
group_size, zp_bias=8)`` returning ``[M, 8 * b_q.shape[1]]`` in ``a``'s dtype.
"""
from __future__ import annotations

import ctypes
import os
import re

import numpy as np
import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# W4A16_LIB names another build of the same ABI (the host-side sanitizer
# build used by ``sanitize.py``); by default the in-tree gfx950 library
LIB_PATH = os.environ.get("W4A16_LIB") or os.path.join(_PKG, "libw4a16.so")
HEADER = os.path.join(os.path.dirname(_PKG), "include", "w4a16.h")

OK, ERR_NULL, ERR_SHAPE, ERR_GROUP, ERR_DTYPE, ERR_ZP, ERR_ALIGN, ERR_DEVICE, \
    ERR_HIP, ERR_VALUE, ERR_PLAN, ERR_WORKSPACE = range(12)
STATUS_NAMES = ["OK", "NULL", "SHAPE", "GROUP", "DTYPE", "ZP", "ALIGN", "DEVICE",
                "HIP", "VALUE", "PLAN", "WORKSPACE"]
WORKSPACE_COUNTER_BYTES = 65536   # W4A16_WORKSPACE_COUNTER_BYTES
F16, BF16 = 0, 1
ROUTE_NONE, ROUTE_DECODE, ROUTE_PREFILL = 0, 1, 2

_DTYPE_CODE = {torch.float16: F16, torch.bfloat16: BF16}


class Plan(ctypes.Structure):
    _fields_ = [("route", ctypes.c_int32), ("block_m", ctypes.c_int32),
                ("block_n", ctypes.c_int32), ("block_k", ctypes.c_int32),
                ("decode_mode", ctypes.c_int32), ("splits", ctypes.c_int32),
                ("steps_per_wave", ctypes.c_int32), ("grid", ctypes.c_int32),
                ("threads", ctypes.c_int32), ("lds_bytes", ctypes.c_int32),
                ("workspace_bytes", ctypes.c_int64)]

    def as_dict(self):
        return {k: getattr(self, k) for k, _ in self._fields_}


class W4A16Error(RuntimeError):
    def __init__(self, status: int, message: str):
        name = STATUS_NAMES[status] if 0 <= status < len(STATUS_NAMES) else str(status)
        super().__init__(f"w4a16 error {name}: {message}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load the library once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with "
            "`python -m weight_only_int4_unpack_amd.build` (there is no fallback)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    L.w4a16_gemm.argtypes = [vp, vp, vp, vp, i32, i32, vp, i64, i64, i64, i32, vp]
    L.w4a16_gemm_bias.argtypes = [vp, vp, vp, vp, i32, i32, vp, vp, i64, i64, i64, i32, vp]
    L.w4a16_gemm_planned.argtypes = [vp, vp, vp, vp, i32, i32, vp, i64, i64, i64, i32,
                                     ctypes.POINTER(Plan), vp]
    L.w4a16_gemm_ws.argtypes = [vp, vp, vp, vp, i32, i32, vp, vp, i64, i64, i64, i32, vp, i64, vp]
    L.w4a16_workspace_bytes.argtypes = [i64, i64, i64, i32, i32, i32, ctypes.POINTER(i64)]
    L.w4a16_gemm_noalloc.argtypes = [vp, vp, vp, vp, i32, i32, vp, vp, i64, i64, i64, i32, vp]
    L.w4a16_plan.argtypes = [i64, i64, i64, i32, i32, i32, i32, ctypes.POINTER(Plan)]
    L.w4a16_plan_route.argtypes = [i64, i64, i64, i32, i32, i32, i32, i32, i32, i32,
                                   ctypes.POINTER(Plan)]
    L.w4a16_dequant.argtypes = [vp, vp, vp, i32, i32, vp, i64, i64, i32, vp]
    L.w4a16_pack_int4.argtypes = [vp, i64, i64, vp]
    L.w4a16_unpack_int4.argtypes = [vp, i64, i64, vp]
    L.w4a16_gemm_kpacked.argtypes = [vp, vp, vp, vp, i32, i32, vp, vp, i64, i64, i64, i32, vp]
    L.w4a16_pack_int4_kshuffle.argtypes = [vp, i64, i64, vp]
    L.w4a16_unpack_int4_kshuffle.argtypes = [vp, i64, i64, vp]
    for f in ("w4a16_gemm", "w4a16_gemm_bias", "w4a16_gemm_planned", "w4a16_gemm_ws",
              "w4a16_workspace_bytes", "w4a16_gemm_noalloc", "w4a16_plan", "w4a16_plan_route",
              "w4a16_dequant", "w4a16_pack_int4", "w4a16_unpack_int4", "w4a16_gemm_kpacked",
              "w4a16_pack_int4_kshuffle", "w4a16_unpack_int4_kshuffle"):
        getattr(L, f).restype = ctypes.c_int
    L.w4a16_last_error.restype = ctypes.c_char_p
    L.w4a16_last_error.argtypes = []
    L.w4a16_version.restype = ctypes.c_char_p
    L.w4a16_version.argtypes = []
    _lib = L
    return L


def header_functions() -> list[str]:
    """Names of the functions include/w4a16.h declares."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:w4a16_status|const char\*)\s+(w4a16_\w+)\s*\(",
                                 text, flags=re.M)))


def last_error() -> str:
    return lib().w4a16_last_error().decode()


def _check(status: int):
    if status != OK:
        raise W4A16Error(status, last_error())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _shapes(a, b_q, scales, qzeros, group_size):
    if a.dim() != 2 or b_q.dim() != 2 or scales.dim() != 2:
        raise ValueError("a, b_q and scales must be 2-D")
    if a.dtype not in _DTYPE_CODE:
        raise ValueError("only float16/bfloat16 activations are supported")
    if scales.dtype != a.dtype:
        raise ValueError("scales must have the activations' dtype")
    if b_q.dtype != torch.int32 or (qzeros is not None and qzeros.dtype != torch.int32):
        raise ValueError("b_q and qzeros must be int32")
    M, K = a.shape
    N = b_q.shape[1] * 8
    if b_q.shape[0] != K:
        raise ValueError(f"b_q has {b_q.shape[0]} rows, a has K={K} columns")
    if group_size <= 0 or K % group_size != 0:
        raise ValueError(f"K={K} is not a multiple of group size {group_size}")
    if tuple(scales.shape) != (K // group_size, N):
        raise ValueError(f"scales must be [{K // group_size}, {N}], got {list(scales.shape)}")
    if qzeros is not None and tuple(qzeros.shape) != (K // group_size, N // 8):
        raise ValueError(f"qzeros must be [{K // group_size}, {N // 8}], got {list(qzeros.shape)}")
    for t in (a, b_q, scales, qzeros):
        if t is not None:
            if not t.is_cuda or t.device != a.device:
                raise ValueError("all tensors must be on the same GPU")
            if not t.is_contiguous():
                raise ValueError("all tensors must be contiguous")
    return M, K, N


_NUM_CUS: dict[int, int] = {}
_WS: dict[tuple[int, int], torch.Tensor] = {}


def workspace_bytes(M: int, K: int, N: int, group_size: int, dtype, num_cus: int = 256) -> int:
    """Scratch bytes ``gemm_ws`` needs for one problem (0 if none; host only)."""
    n = ctypes.c_int64(0)
    _check(lib().w4a16_workspace_bytes(M, K, N, group_size, _DTYPE_CODE.get(dtype, dtype),
                                       num_cus, ctypes.byref(n)))
    return n.value


def _num_cus(dev: torch.device) -> int:
    i = dev.index if dev.index is not None else torch.cuda.current_device()
    if i not in _NUM_CUS:
        _NUM_CUS[i] = torch.cuda.get_device_properties(i).multi_processor_count
    return _NUM_CUS[i]


def stream_workspace(dev: torch.device, nbytes: int) -> torch.Tensor | None:
    """A workspace of at least ``nbytes`` from torch's allocator for the
    current stream of ``dev``, its counter region zero (``torch.zeros``, a
    fill kernel on that stream). Outside graph capture one workspace per
    (device, stream) is kept and reused: every completed launch leaves its
    counters zero. During capture each call gets a fresh one from the
    graph's pool (its fill is recorded in the graph), so no memory of the
    graph is ever handed to eager work."""
    if nbytes <= 0:
        return None
    stream = torch.cuda.current_stream(dev)
    key = (dev.index, stream.cuda_stream)
    if torch.cuda.is_current_stream_capturing():
        return torch.zeros(nbytes, dtype=torch.uint8, device=dev)
    ws = _WS.get(key)
    if ws is None or ws.numel() < nbytes:
        size = max(nbytes, 2 * (0 if ws is None else ws.numel()))
        ws = torch.zeros(size, dtype=torch.uint8, device=dev)
        _WS[key] = ws
    return ws


def gemm(a: torch.Tensor, b_q: torch.Tensor, scales: torch.Tensor,
         qzeros: torch.Tensor | None = None, group_size: int = 128, zp_bias: int = 8,
         out: torch.Tensor | None = None, plan: Plan | None = None,
         bias: torch.Tensor | None = None) -> torch.Tensor:
    """``a @ dequant(b_q, scales, qzeros) (+ bias)`` on the GPU, in ``a``'s dtype.

    ``bias`` (optional, ``[N]`` in ``a``'s dtype) is added to the fp32 result
    before the cast (PR #40977 "RDNA hybrid W4A16", Code section). Without a
    forced ``plan`` the call goes through ``w4a16_gemm_ws`` with a workspace
    from torch's allocator (``stream_workspace``), so it can be captured into
    a graph on first use; with one, through ``w4a16_gemm_planned`` and the
    library's per-stream workspace."""
    M, K, N = _shapes(a, b_q, scales, qzeros, group_size)
    if bias is not None:
        if plan is not None:
            raise ValueError("a forced plan runs without bias")
        if (bias.dim() != 1 or bias.shape[0] != N or bias.dtype != a.dtype
                or bias.device != a.device or not bias.is_contiguous()):
            raise ValueError(f"bias must be a contiguous [{N}] tensor of a's dtype and device")
    if out is None:
        out = torch.empty((M, N), dtype=a.dtype, device=a.device)
    elif (tuple(out.shape) != (M, N) or out.dtype != a.dtype or out.device != a.device
          or not out.is_contiguous()):
        raise ValueError("out must be a contiguous [M, N] tensor like a")
    if a.device.index == torch.cuda.current_device():
        _gemm_on_device(a, b_q, scales, qzeros, group_size, zp_bias, out, plan, bias)
    else:
        with torch.cuda.device(a.device):
            _gemm_on_device(a, b_q, scales, qzeros, group_size, zp_bias, out, plan, bias)
    return out


def _gemm_on_device(a, b_q, scales, qzeros, group_size, zp_bias, out, plan, bias):
    args = gemm_args(a, b_q, scales, qzeros, group_size, zp_bias, out)
    if plan is not None:
        _run_gemm(args, plan, bias)
        return
    M, K = a.shape
    nb = workspace_bytes(M, K, args[9], group_size, a.dtype, _num_cus(a.device))
    ws = stream_workspace(a.device, nb)
    _check(lib().w4a16_gemm_ws(*args[:6], _ptr(bias), *args[6:11], _ptr(ws), nb, args[11]))


NOALLOC_SCRATCH_BYTES = WORKSPACE_COUNTER_BYTES + (32 << 20)   # W4A16_NOALLOC_SCRATCH_BYTES


def gemm_noalloc(a, b_q, scales, qzeros, group_size, zp_bias, out, bias=None) -> torch.Tensor:
    """``w4a16_gemm_noalloc``: scratch from the library's fixed device array
    (no allocation); shapes checked as in ``gemm``."""
    _shapes(a, b_q, scales, qzeros, group_size)
    args = gemm_args(a, b_q, scales, qzeros, group_size, zp_bias, out)
    with torch.cuda.device(a.device):
        _check(lib().w4a16_gemm_noalloc(*args[:6], _ptr(bias), *args[6:]))
    return out


def gemm_ws(a, b_q, scales, qzeros, group_size, zp_bias, out, workspace, ws_bytes=None,
            bias=None) -> torch.Tensor:
    """``w4a16_gemm_ws`` with a caller-owned ``workspace`` (a device tensor,
    or None when the problem needs none); shapes checked as in ``gemm``."""
    _shapes(a, b_q, scales, qzeros, group_size)
    args = gemm_args(a, b_q, scales, qzeros, group_size, zp_bias, out)
    nb = (0 if workspace is None else workspace.numel() * workspace.element_size()) \
        if ws_bytes is None else ws_bytes
    with torch.cuda.device(a.device):
        _check(lib().w4a16_gemm_ws(*args[:6], _ptr(bias), *args[6:11], _ptr(workspace), nb,
                                   args[11]))
    return out


def gemm_args(a, b_q, scales, qzeros, group_size, zp_bias, out):
    """The C-ABI argument tuple of one GEMM (pointers, sizes, dtype, stream),
    for callers that launch the same problem repeatedly without re-checking
    shapes; pass it to ``launch``."""
    M, K = a.shape
    N = b_q.shape[1] * 8
    return (_ptr(a), _ptr(b_q), _ptr(scales), _ptr(qzeros), group_size, zp_bias, _ptr(out),
            M, K, N, _DTYPE_CODE[a.dtype], _stream(a.device))


def _run_gemm(args, plan, bias=None):
    L = lib()
    if bias is not None:
        _check(L.w4a16_gemm_bias(*args[:6], _ptr(bias), *args[6:]))
    elif plan is None:
        _check(L.w4a16_gemm(*args))
    else:
        _check(L.w4a16_gemm_planned(*args[:-1], ctypes.byref(plan), args[-1]))


def gemm_ws_args(a, b_q, scales, qzeros, group_size, zp_bias, out, workspace, bias=None):
    """The ``w4a16_gemm_ws`` argument tuple of one GEMM with a caller-owned
    ``workspace`` tensor (or None), for repeated launches without re-checking
    shapes; pass it to ``launch_ws``."""
    M, K = a.shape
    N = b_q.shape[1] * 8
    nb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return (_ptr(a), _ptr(b_q), _ptr(scales), _ptr(qzeros), group_size, zp_bias, _ptr(bias),
            _ptr(out), M, K, N, _DTYPE_CODE[a.dtype], _ptr(workspace), nb, _stream(a.device))


def launch_ws(args) -> None:
    """Run a tuple made by ``gemm_ws_args`` (on the stream it names)."""
    _check(lib().w4a16_gemm_ws(*args))


def launch(args) -> None:
    """Run a tuple made by ``gemm_args`` (on the stream it names)."""
    st = lib().w4a16_gemm(*args)
    if st != OK:
        raise W4A16Error(st, last_error())


def gemm_kpacked(a: torch.Tensor, w: torch.Tensor, scales: torch.Tensor,
                 zeros: torch.Tensor | None = None, group_size: int = 128, zp_bias: int = 8,
                 bias: torch.Tensor | None = None,
                 out: torch.Tensor | None = None) -> torch.Tensor:
    """``a @ dequant(w) (+ bias)`` for K-packed weights: ``w`` int32 ``[N, K/8]``
    in ExLlama nibble order (``pack_int4_kshuffle``), ``scales`` ``[N, K/G]``
    in ``a``'s dtype, ``zeros`` uint8 ``[N, K/G]`` or None (PR #40977 "RDNA
    hybrid W4A16", Impl. item 4)."""
    if a.dim() != 2 or w.dim() != 2 or scales.dim() != 2:
        raise ValueError("a, w and scales must be 2-D")
    if a.dtype not in _DTYPE_CODE or scales.dtype != a.dtype:
        raise ValueError("a and scales must both be float16 or both bfloat16")
    if w.dtype != torch.int32 or (zeros is not None and zeros.dtype != torch.uint8):
        raise ValueError("w must be int32 and zeros uint8")
    M, K = a.shape
    N = w.shape[0]
    if w.shape[1] * 8 != K:
        raise ValueError(f"w must be [N, {K // 8}], got {list(w.shape)}")
    if group_size <= 0 or K % group_size != 0:
        raise ValueError(f"K={K} is not a multiple of group size {group_size}")
    if tuple(scales.shape) != (N, K // group_size):
        raise ValueError(f"scales must be [{N}, {K // group_size}], got {list(scales.shape)}")
    if zeros is not None and tuple(zeros.shape) != (N, K // group_size):
        raise ValueError(f"zeros must be [{N}, {K // group_size}], got {list(zeros.shape)}")
    if bias is not None and (bias.dim() != 1 or bias.shape[0] != N or bias.dtype != a.dtype):
        raise ValueError(f"bias must be [{N}] in a's dtype")
    if out is None:
        out = torch.empty((M, N), dtype=a.dtype, device=a.device)
    elif tuple(out.shape) != (M, N) or out.dtype != a.dtype:
        raise ValueError("out must be [M, N] like a")
    for t in (a, w, scales, zeros, bias, out):
        if t is not None:
            if not t.is_cuda or t.device != a.device:
                raise ValueError("all tensors must be on the same GPU")
            if not t.is_contiguous():
                raise ValueError("all tensors must be contiguous")
    with torch.cuda.device(a.device):
        _check(lib().w4a16_gemm_kpacked(_ptr(a), _ptr(w), _ptr(scales), _ptr(zeros), group_size,
                                        zp_bias, _ptr(bias), _ptr(out), M, K, N,
                                        _DTYPE_CODE[a.dtype], _stream(a.device)))
    return out


def gemm_kpacked_args(a, w, scales, zeros, group_size, zp_bias, out, bias=None):
    """The C-ABI argument tuple of one K-packed GEMM, for repeated launches
    without re-checking shapes; pass it to ``launch_kpacked``."""
    M, K = a.shape
    return (_ptr(a), _ptr(w), _ptr(scales), _ptr(zeros), group_size, zp_bias, _ptr(bias),
            _ptr(out), M, K, w.shape[0], _DTYPE_CODE[a.dtype], _stream(a.device))


def launch_kpacked(args) -> None:
    """Run a tuple made by ``gemm_kpacked_args`` (on the stream it names)."""
    _check(lib().w4a16_gemm_kpacked(*args))


def dequant(b_q: torch.Tensor, scales: torch.Tensor, qzeros: torch.Tensor | None = None,
            group_size: int = 128, zp_bias: int = 8,
            out: torch.Tensor | None = None) -> torch.Tensor:
    """Dense ``[K, N]`` RNE((q - z) * s) in ``scales``' dtype (test probe)."""
    K, N = b_q.shape[0], b_q.shape[1] * 8
    dummy = torch.empty((0, K), dtype=scales.dtype, device=scales.device)
    _shapes(dummy, b_q, scales, qzeros, group_size)
    if out is None:
        out = torch.empty((K, N), dtype=scales.dtype, device=scales.device)
    L = lib()
    with torch.cuda.device(scales.device):
        _check(L.w4a16_dequant(_ptr(b_q), _ptr(scales), _ptr(qzeros), group_size, zp_bias,
                               _ptr(out), K, N, _DTYPE_CODE[scales.dtype],
                               _stream(scales.device)))
    return out


def plan(M: int, K: int, N: int, group_size: int, has_zp: bool, dtype, num_cus: int = 256,
         route: int | None = None, steps_per_wave: int = 0, decode_mode: int = -1) -> Plan:
    """The launch the selector picks, or one with the route / decode steps per
    wavefront / decode mode forced (host only)."""
    code = _DTYPE_CODE.get(dtype, dtype)
    p = Plan()
    L = lib()
    if route is None and steps_per_wave == 0 and decode_mode < 0:
        _check(L.w4a16_plan(M, K, N, group_size, int(has_zp), code, num_cus, ctypes.byref(p)))
    else:
        r = route if route is not None else (ROUTE_DECODE if M <= 16 else ROUTE_PREFILL)
        _check(L.w4a16_plan_route(M, K, N, group_size, int(has_zp), code, num_cus, r,
                                  steps_per_wave, decode_mode, ctypes.byref(p)))
    return p


def pack_int4(q) -> np.ndarray:
    """Host pack: uint8 ``[R, C]`` values 0..15 -> int32 ``[R, C/8]``."""
    if isinstance(q, torch.Tensor):
        q = q.cpu().numpy()
    q = np.asarray(q)
    if q.dtype != np.uint8 and q.size and (q.min() < 0 or q.max() > 255):
        raise W4A16Error(ERR_VALUE, "uint4 values must lie in 0..15")
    q = np.ascontiguousarray(q, dtype=np.uint8)
    if q.ndim != 2:
        raise ValueError("q must be 2-D")
    out = np.empty((q.shape[0], q.shape[1] // 8), dtype=np.int32)
    _check(lib().w4a16_pack_int4(q.ctypes.data_as(ctypes.c_void_p), q.shape[0], q.shape[1],
                                 out.ctypes.data_as(ctypes.c_void_p)))
    return out


def unpack_int4(packed) -> np.ndarray:
    """Host unpack: int32 ``[R, W]`` -> uint8 ``[R, 8W]``."""
    if isinstance(packed, torch.Tensor):
        packed = packed.cpu().numpy()
    packed = np.ascontiguousarray(packed, dtype=np.int32)
    out = np.empty((packed.shape[0], packed.shape[1] * 8), dtype=np.uint8)
    _check(lib().w4a16_unpack_int4(packed.ctypes.data_as(ctypes.c_void_p), packed.shape[0],
                                   packed.shape[1] * 8, out.ctypes.data_as(ctypes.c_void_p)))
    return out


def pack_int4_kshuffle(q_nk) -> np.ndarray:
    """Host pack: uint8 ``[N, K]`` values 0..15 -> int32 ``[N, K/8]``, K-packed
    in ExLlama nibble order."""
    if isinstance(q_nk, torch.Tensor):
        q_nk = q_nk.cpu().numpy()
    q = np.asarray(q_nk)
    if q.dtype != np.uint8 and q.size and (q.min() < 0 or q.max() > 255):
        raise W4A16Error(ERR_VALUE, "uint4 values must lie in 0..15")
    q = np.ascontiguousarray(q, dtype=np.uint8)
    if q.ndim != 2:
        raise ValueError("q must be 2-D")
    out = np.empty((q.shape[0], q.shape[1] // 8), dtype=np.int32)
    _check(lib().w4a16_pack_int4_kshuffle(q.ctypes.data_as(ctypes.c_void_p), q.shape[0],
                                          q.shape[1], out.ctypes.data_as(ctypes.c_void_p)))
    return out


def unpack_int4_kshuffle(packed) -> np.ndarray:
    """Host unpack: int32 ``[N, K/8]`` -> uint8 ``[N, K]``."""
    if isinstance(packed, torch.Tensor):
        packed = packed.cpu().numpy()
    packed = np.ascontiguousarray(packed, dtype=np.int32)
    out = np.empty((packed.shape[0], packed.shape[1] * 8), dtype=np.uint8)
    _check(lib().w4a16_unpack_int4_kshuffle(packed.ctypes.data_as(ctypes.c_void_p),
                                            packed.shape[0], packed.shape[1] * 8,
                                            out.ctypes.data_as(ctypes.c_void_p)))
    return out


def version() -> str:
    return lib().w4a16_version().decode()
