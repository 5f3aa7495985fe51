"""Seeded synthetic inputs for the W4A16 GEMM workloads.

This module only draws random numbers; it holds none of the method's
arithmetic (no packing, no dequantisation, no product). Both the CPU oracle
and the HIP library consume what it returns, each packing the uint4 values
with its own routine.

Workloads (all on one GPU):

=============  ====  =====  =====  =====  =====  ==========
name             M     K      N      G    dtype  zero points
=============  ====  =====  =====  =====  =====  ==========
tiny             4    256    512    128   fp16   symmetric
decode_m1        1   5120  17408    128   bf16   symmetric
decode_m5        5   5120  17408    128   bf16   symmetric
k2112            8   2112   5120     64   fp16   packed
prefill       2048   5120  17408    128   bf16   symmetric
sweep_m{M}       M   4096   4096     32   fp16   packed
sweep_pc16      16   4096   4096   4096   fp16   packed
=============  ====  =====  =====  =====  =====  ==========

Distributions: activations ~ N(0, 1) drawn in fp32 and rounded to the dtype;
uint4 weights uniform on 0..15; scales uniform on [1e-3, 1e-2] drawn in fp32
and rounded to the dtype; zero points uniform on 0..15. Generator: NumPy's
PCG64 ``default_rng(seed)`` with ``seed = 1000 * family + stream`` where the
stream is 0 for activations, 1 for weights, 2 for scales and 3 for zero
points. The sweep family shares one weight set across all M, and the
activations of each M are the first M rows of one 4096-row draw.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    K: int
    N: int
    group_size: int
    dtype: str          # "fp16" or "bf16"
    has_zp: bool
    family: int         # seed family
    a_rows: int         # rows of the activation draw (sliced to M)


def _wl(name, M, K, N, G, dtype, has_zp, family, a_rows=None):
    return Workload(name, M, K, N, G, dtype, has_zp, family,
                    M if a_rows is None else a_rows)


WORKLOADS = {w.name: w for w in [
    _wl("tiny", 4, 256, 512, 128, "fp16", False, 0),
    _wl("decode_m1", 1, 5120, 17408, 128, "bf16", False, 1, a_rows=8),
    _wl("decode_m5", 5, 5120, 17408, 128, "bf16", False, 1, a_rows=8),
    _wl("k2112", 8, 2112, 5120, 64, "fp16", True, 2),
    _wl("prefill", 2048, 5120, 17408, 128, "bf16", False, 3),
    *[_wl(f"sweep_m{m}", m, 4096, 4096, 32, "fp16", True, 4, a_rows=4096)
      for m in (1, 2, 4, 5, 6, 16, 64, 256, 4096)],
    _wl("sweep_pc16", 16, 4096, 4096, 4096, "fp16", True, 5),
]}


def round_to_dtype_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """fp32 draw -> uint16 bit pattern of the nearest fp16/bf16 (torch cast)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    t = t.to(torch.float16 if dtype == "fp16" else torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def draw(M: int, K: int, N: int, group_size: int, dtype: str, has_zp: bool,
         family: int, a_rows: int | None = None) -> dict:
    """Random inputs of one problem.

    Returns a dict with ``a_bits`` uint16 ``[M, K]``, ``q`` uint8 ``[K, N]``
    (values 0..15), ``s_bits`` uint16 ``[K/G, N]`` and ``z`` uint8
    ``[K/G, N]`` or None.
    """
    a_rows = M if a_rows is None else max(a_rows, M)
    ng = K // group_size
    rng_a = np.random.default_rng(1000 * family + 0)
    rng_q = np.random.default_rng(1000 * family + 1)
    rng_s = np.random.default_rng(1000 * family + 2)
    rng_z = np.random.default_rng(1000 * family + 3)
    a32 = rng_a.standard_normal((a_rows, K), dtype=np.float32)[:M]
    q = rng_q.integers(0, 16, size=(K, N), dtype=np.uint8)
    s32 = rng_s.uniform(1e-3, 1e-2, size=(ng, N)).astype(np.float32)
    z = rng_z.integers(0, 16, size=(ng, N), dtype=np.uint8) if has_zp else None
    return {
        "a_bits": round_to_dtype_bits(a32, dtype),
        "q": q,
        "s_bits": round_to_dtype_bits(s32, dtype),
        "z": z,
    }


def draw_workload(w: Workload | str) -> dict:
    if isinstance(w, str):
        w = WORKLOADS[w]
    return draw(w.M, w.K, w.N, w.group_size, w.dtype, w.has_zp, w.family,
                a_rows=w.a_rows)


def random_bits(shape, dtype: str, seed: int, scale: float = 1.0) -> np.ndarray:
    """Normal(0, scale) values rounded to the dtype, for ad-hoc test shapes."""
    rng = np.random.default_rng(seed)
    return round_to_dtype_bits(
        (rng.standard_normal(shape) * scale).astype(np.float32), dtype)
