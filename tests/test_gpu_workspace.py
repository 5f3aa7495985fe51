"""GPU tests of the scratch contract (``w4a16_gemm_ws`` and the library's
per-stream workspaces), through the C ABI.

* ``w4a16_gemm_ws`` captured into a HIP graph on its first use (no
  allocation, no synchronisation inside the call; PR #51453 "Register the
  Triton W4A16 GEMM as a custom op", Code section: the operator writes no
  input so that it is safe under graph capture), replayed several times with
  eager work in between, every replay checked against the eager result and
  the oracle;
* two streams, each with its own workspace, running split-K launches at the
  same time, both checked against the oracle;
* the library's own workspace: per stream, grown without synchronising, and
  refused (WORKSPACE) rather than allocated while the stream is captured;
* the counter region is left zero by every launch.
"""
import ctypes

import numpy as np
import pytest
import torch

from weight_only_int4_unpack_amd import w4a16 as W
from helpers import assert_within_tolerance, dev_to_bits, random_problem, TORCH_DT

pytestmark = pytest.mark.gpu

# (M, K, N, G, dtype, zp): a decode split-K launch (last-arrival hand-off)
# and a prefill K-split launch (partials + reduction kernel)
SPLIT_CASES = [(5, 4096, 2048, 128, "bf16", False), (40, 4096, 1024, 32, "fp16", True)]


def _need(p):
    return W.workspace_bytes(p.M, p.K, p.N, p.G, TORCH_DT[p.dtype],
                             torch.cuda.get_device_properties(0).multi_processor_count)


def _ws_call(p, ws, out, nbytes=None):
    return W.gemm_ws(p.a, p.b_q_d, p.s, p.qz_d, p.G, 8, out, ws, nbytes)


@pytest.mark.parametrize("M,K,N,G,dtype,zp", SPLIT_CASES)
def test_gemm_ws_captured_on_first_use(M, K, N, G, dtype, zp):
    p = random_problem(M, K, N, G, dtype, zp, seed=600 + M)
    need = _need(p)
    assert need > W.WORKSPACE_COUNTER_BYTES          # the launch splits K
    want = p.oracle_gemm()
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    out = torch.empty((M, N), dtype=TORCH_DT[dtype], device="cuda")
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            _ws_call(p, ws, out)                     # first call with this workspace
    torch.cuda.synchronize()
    eager = dev_to_bits(p.gpu_gemm())
    assert_within_tolerance(eager, want, dtype, "eager")
    for r in range(4):
        out.fill_(0)
        _ = torch.randn(1 << 20, device="cuda").sum()  # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        got = dev_to_bits(out)
        assert np.array_equal(got, eager), f"replay {r}"
        assert_within_tolerance(got, want, dtype, f"replay {r}")
    assert torch.count_nonzero(ws[:W.WORKSPACE_COUNTER_BYTES]).item() == 0


def test_two_streams_own_workspaces():
    pa = random_problem(*SPLIT_CASES[0], seed=610)
    pb = random_problem(6, 4096, 2048, 64, "fp16", True, seed=611)
    wa, wb = pa.oracle_gemm(), pb.oracle_gemm()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    ws1 = torch.zeros(_need(pa), dtype=torch.uint8, device="cuda")
    ws2 = torch.zeros(_need(pb), dtype=torch.uint8, device="cuda")
    outs1 = [torch.empty((pa.M, pa.N), dtype=torch.bfloat16, device="cuda") for _ in range(6)]
    outs2 = [torch.empty((pb.M, pb.N), dtype=torch.float16, device="cuda") for _ in range(6)]
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    for i in range(6):                                # interleaved, no sync in between
        with torch.cuda.stream(s1):
            _ws_call(pa, ws1, outs1[i])
        with torch.cuda.stream(s2):
            _ws_call(pb, ws2, outs2[i])
    torch.cuda.synchronize()
    for i in range(6):
        assert_within_tolerance(dev_to_bits(outs1[i]), wa, "bf16", f"stream 1 call {i}")
        assert_within_tolerance(dev_to_bits(outs2[i]), wb, "fp16", f"stream 2 call {i}")
    for ws in (ws1, ws2):
        assert torch.count_nonzero(ws[:W.WORKSPACE_COUNTER_BYTES]).item() == 0


def test_two_streams_library_workspaces():
    # forced plans go through w4a16_gemm_planned and the library's own
    # workspace of each stream
    pa = random_problem(*SPLIT_CASES[0], seed=620)
    pb = random_problem(*SPLIT_CASES[1], seed=621)
    plans = [W.plan(q.M, q.K, q.N, q.G, q.qz is not None, TORCH_DT[q.dtype]) for q in (pa, pb)]
    assert all(pl.splits > 1 for pl in plans)
    wa, wb = pa.oracle_gemm(), pb.oracle_gemm()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    r1, r2 = [], []
    for i in range(5):
        with torch.cuda.stream(s1):
            r1.append(pa.gpu_gemm(plan=plans[0]))
        with torch.cuda.stream(s2):
            r2.append(pb.gpu_gemm(plan=plans[1]))
    torch.cuda.synchronize()
    for i in range(5):
        assert_within_tolerance(dev_to_bits(r1[i]), wa, "bf16", f"stream 1 call {i}")
        assert_within_tolerance(dev_to_bits(r2[i]), wb, "fp16", f"stream 2 call {i}")


def _hip_runtime():
    """The HIP runtime already loaded in this process (the one torch and the
    library use), found by path so that no second copy is loaded."""
    with open("/proc/self/maps") as f:
        paths = {l.split()[-1] for l in f if "libamdhip64" in l}
    assert len(paths) == 1, paths
    return ctypes.CDLL(paths.pop())


def test_library_workspace_not_grown_under_capture():
    # a stream the library has never seen (created here, not taken from
    # torch's stream pool) has no library workspace; a capture on it must not
    # allocate: the call fails with WORKSPACE and nothing is recorded
    p = random_problem(*SPLIT_CASES[0], seed=630)
    plan = W.plan(p.M, p.K, p.N, p.G, False, torch.bfloat16)
    hip = _hip_runtime()
    handle = ctypes.c_void_p()
    assert hip.hipStreamCreate(ctypes.byref(handle)) == 0
    s = torch.cuda.ExternalStream(handle.value)
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    status = None
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            try:
                p.gpu_gemm(plan=plan)
            except W.W4A16Error as e:
                status = e.status
    torch.cuda.synchronize()
    assert status == W.ERR_WORKSPACE
    # uncaptured, the same stream gets its workspace and the call succeeds
    with torch.cuda.stream(s):
        out = p.gpu_gemm(plan=plan)
    s.synchronize()
    assert_within_tolerance(dev_to_bits(out), p.oracle_gemm(), "bf16", "after capture")
    torch.cuda.synchronize()
    assert hip.hipStreamDestroy(handle) == 0


def test_binding_gemm_captured_on_first_use():
    # W.gemm (no forced plan) takes its workspace from torch's allocator, so
    # the opaque operator above it can be captured without a prior call
    p = random_problem(5, 2048, 3072, 64, "bf16", True, seed=640)
    want = p.oracle_gemm()
    out = torch.empty((p.M, p.N), dtype=torch.bfloat16, device="cuda")
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            p.gpu_gemm(out=out)
    torch.cuda.synchronize()
    for r in range(3):
        out.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        assert_within_tolerance(dev_to_bits(out), want, "bf16", f"replay {r}")
