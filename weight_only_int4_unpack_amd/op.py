"""The GEMM as an opaque torch operator: ``torch.ops.w4a16.gemm``.

PR #51453 "Register the Triton W4A16 GEMM as a custom op" (Motivation and
Impl. items 1-4) puts the kernel behind a custom-op boundary so that a
graph compiler sees one call node and never traces the host-side tile
choice: the choice then runs on every call with the real runtime M, K, N
(here it runs inside the C library, ``w4a16_plan``). The pieces follow the
page:

* the operator does not write its inputs (``mutates_args=()``) and returns
  a new ``[M, 8 * b_q.shape[1]]`` tensor in ``a``'s dtype on ``a``'s device;
* a fake implementation gives that shape, dtype and device without
  computing, so tracing under fake tensors works without a GPU;
* ``gemm`` is the facade with the page's signature
  ``(a, b_q, scales, qzeros, group_size, zp_bias=8)``, plus the optional
  ``bias`` of the bias epilogue.

The page's fake checks nothing and its Risks section names that as a gap
(the output shape is taken on trust). The fake here applies the same shape
and dtype checks as the real call, so a malformed call fails while tracing.

``torch.ops.w4a16.gemm_kpacked`` does the same for weights K-packed
(``[N, K/8]`` in ExLlama order, scales and uint8 zero points ``[N, K/G]``;
PR #40977 "RDNA hybrid W4A16", Impl. items 2 and 4: the hybrid path's skinny
kernel is registered with a fake implementation for the same reason).

The real implementation is the ctypes binding (argument marshalling only);
every step of the computation runs in the library's gfx950 kernels.
"""
from __future__ import annotations

import torch

from . import w4a16 as _W

_FLOATS = (torch.float16, torch.bfloat16)


def _check_meta(a, b_q, scales, qzeros, group_size, bias):
    """Shape/dtype contract shared by the real and the fake implementation."""
    if a.dim() != 2 or b_q.dim() != 2 or scales.dim() != 2:
        raise ValueError("a, b_q and scales must be 2-D")
    if a.dtype not in _FLOATS or scales.dtype != a.dtype:
        raise ValueError("a and scales must both be float16 or both bfloat16")
    if b_q.dtype != torch.int32 or (qzeros is not None and qzeros.dtype != torch.int32):
        raise ValueError("b_q and qzeros must be int32")
    K = a.size(1)
    N = b_q.size(1) * 8
    if b_q.size(0) != K:
        raise ValueError(f"b_q has {b_q.size(0)} rows, a has K={K} columns")
    if group_size <= 0 or K % group_size != 0:
        raise ValueError(f"K={K} is not a multiple of group size {group_size}")
    if tuple(scales.shape) != (K // group_size, N):
        raise ValueError(f"scales must be [{K // group_size}, {N}]")
    if qzeros is not None and tuple(qzeros.shape) != (K // group_size, N // 8):
        raise ValueError(f"qzeros must be [{K // group_size}, {N // 8}]")
    if bias is not None and (bias.dim() != 1 or bias.size(0) != N or bias.dtype != a.dtype):
        raise ValueError(f"bias must be [{N}] in a's dtype")


@torch.library.custom_op("w4a16::gemm", mutates_args=())
def _gemm_op(a: torch.Tensor, b_q: torch.Tensor, scales: torch.Tensor,
             qzeros: torch.Tensor | None, group_size: int, zp_bias: int = 8,
             bias: torch.Tensor | None = None) -> torch.Tensor:
    _check_meta(a, b_q, scales, qzeros, group_size, bias)
    return _W.gemm(a.contiguous(), b_q.contiguous(), scales.contiguous(),
                   None if qzeros is None else qzeros.contiguous(), group_size, zp_bias,
                   bias=None if bias is None else bias.contiguous())


@_gemm_op.register_fake
def _gemm_fake(a, b_q, scales, qzeros, group_size, zp_bias=8, bias=None):
    _check_meta(a, b_q, scales, qzeros, group_size, bias)
    return torch.empty((a.size(0), b_q.size(1) * 8), dtype=a.dtype, device=a.device)


def gemm(a: torch.Tensor, b_q: torch.Tensor, scales: torch.Tensor,
         qzeros: torch.Tensor | None, group_size: int, zp_bias: int = 8,
         bias: torch.Tensor | None = None) -> torch.Tensor:
    """Facade: ``a @ dequant(b_q, scales, qzeros) (+ bias)`` through the
    opaque operator ``torch.ops.w4a16.gemm``."""
    return torch.ops.w4a16.gemm(a, b_q, scales, qzeros, group_size, zp_bias, bias)


def _check_meta_kpacked(a, w, scales, zeros, group_size, bias):
    """Shape/dtype contract of the K-packed operator (real and fake)."""
    if a.dim() != 2 or w.dim() != 2 or scales.dim() != 2:
        raise ValueError("a, w and scales must be 2-D")
    if a.dtype not in _FLOATS or scales.dtype != a.dtype:
        raise ValueError("a and scales must both be float16 or both bfloat16")
    if w.dtype != torch.int32 or (zeros is not None and zeros.dtype != torch.uint8):
        raise ValueError("w must be int32 and zeros uint8")
    K = a.size(1)
    N = w.size(0)
    if w.size(1) * 8 != K:
        raise ValueError(f"w must be [N, {K // 8}]")
    if group_size <= 0 or K % group_size != 0:
        raise ValueError(f"K={K} is not a multiple of group size {group_size}")
    if tuple(scales.shape) != (N, K // group_size):
        raise ValueError(f"scales must be [{N}, {K // group_size}]")
    if zeros is not None and tuple(zeros.shape) != (N, K // group_size):
        raise ValueError(f"zeros must be [{N}, {K // group_size}]")
    if bias is not None and (bias.dim() != 1 or bias.size(0) != N or bias.dtype != a.dtype):
        raise ValueError(f"bias must be [{N}] in a's dtype")


@torch.library.custom_op("w4a16::gemm_kpacked", mutates_args=())
def _gemm_kpacked_op(a: torch.Tensor, w: torch.Tensor, scales: torch.Tensor,
                     zeros: torch.Tensor | None, group_size: int, zp_bias: int = 8,
                     bias: torch.Tensor | None = None) -> torch.Tensor:
    _check_meta_kpacked(a, w, scales, zeros, group_size, bias)
    return _W.gemm_kpacked(a.contiguous(), w.contiguous(), scales.contiguous(),
                           None if zeros is None else zeros.contiguous(), group_size, zp_bias,
                           bias=None if bias is None else bias.contiguous())


@_gemm_kpacked_op.register_fake
def _gemm_kpacked_fake(a, w, scales, zeros, group_size, zp_bias=8, bias=None):
    _check_meta_kpacked(a, w, scales, zeros, group_size, bias)
    return torch.empty((a.size(0), w.size(0)), dtype=a.dtype, device=a.device)


def gemm_kpacked(a: torch.Tensor, w: torch.Tensor, scales: torch.Tensor,
                 zeros: torch.Tensor | None, group_size: int, zp_bias: int = 8,
                 bias: torch.Tensor | None = None) -> torch.Tensor:
    """Facade: ``a @ dequant(w) (+ bias)`` for K-packed weights through the
    opaque operator ``torch.ops.w4a16.gemm_kpacked``."""
    return torch.ops.w4a16.gemm_kpacked(a, w, scales, zeros, group_size, zp_bias, bias)
