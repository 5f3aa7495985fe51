"""Shared test plumbing: build one problem for both the oracle and the GPU.

The uint4 values are drawn once (``synthetic``); the oracle packs them with
its own routine and the GPU side with the library's host pack, and the two
packings are checked equal before anything else.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

import oracle as O
from weight_only_int4_unpack_amd import synthetic
from weight_only_int4_unpack_amd import w4a16 as W

TORCH_DT = {"fp16": torch.float16, "bf16": torch.bfloat16}


def bits_to_dev(bits: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(TORCH_DT[dtype])
    return t.to(device)


def dev_to_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


@dataclass
class Problem:
    M: int
    K: int
    N: int
    G: int
    dtype: str
    zp_bias: int
    # oracle side (host)
    a_bits: np.ndarray
    b_q: np.ndarray
    s_bits: np.ndarray
    qz: np.ndarray | None
    # library side (device)
    a: torch.Tensor | None = None
    b_q_d: torch.Tensor | None = None
    s: torch.Tensor | None = None
    qz_d: torch.Tensor | None = None

    def oracle_gemm(self, rows=None, cols=None):
        return O.gemm(self.a_bits, self.b_q, self.s_bits, self.qz, self.G, self.zp_bias,
                      self.dtype, rows=rows, cols=cols)

    def gpu_gemm(self, plan=None, out=None):
        return W.gemm(self.a, self.b_q_d, self.s, self.qz_d, self.G, self.zp_bias,
                      out=out, plan=plan)


def make_problem(d: dict, M: int, K: int, N: int, G: int, dtype: str, zp_bias: int = 8,
                 device: str | None = "cuda") -> Problem:
    b_q = O.pack_int4(d["q"])
    qz = None if d["z"] is None else O.pack_int4(d["z"])
    p = Problem(M, K, N, G, dtype, zp_bias, d["a_bits"][:M], b_q, d["s_bits"], qz)
    if device is not None:
        lib_bq = W.pack_int4(d["q"])
        assert np.array_equal(lib_bq, b_q), "library pack differs from the oracle's"
        p.a = bits_to_dev(p.a_bits, dtype, device)
        p.b_q_d = torch.from_numpy(lib_bq).to(device)
        p.s = bits_to_dev(d["s_bits"], dtype, device)
        if d["z"] is not None:
            lib_qz = W.pack_int4(d["z"])
            assert np.array_equal(lib_qz, qz)
            p.qz_d = torch.from_numpy(lib_qz).to(device)
    return p


def random_problem(M, K, N, G, dtype, has_zp, seed, zp_bias=8, device="cuda") -> Problem:
    d = synthetic.draw(M, K, N, G, dtype, has_zp, family=500 + seed)
    return make_problem(d, M, K, N, G, dtype, zp_bias, device)


def workload_problem(name: str, device="cuda") -> Problem:
    w = synthetic.WORKLOADS[name]
    d = synthetic.draw_workload(w)
    return make_problem(d, w.M, w.K, w.N, w.group_size, w.dtype, 8, device)


def assert_within_tolerance(got_bits, want_bits, dtype, what=""):
    ok = O.within_tolerance(got_bits, want_bits, dtype)
    if not ok.all():
        idx = np.argwhere(~ok)[:5]
        g = O.to_f32(got_bits, dtype)
        w = O.to_f32(want_bits, dtype)
        detail = ", ".join(f"{tuple(i)}: got {g[tuple(i)]} want {w[tuple(i)]}" for i in idx)
        raise AssertionError(f"{what}: {int((~ok).sum())} of {ok.size} outside 2e-2 "
                             f"tolerance; first: {detail}")
