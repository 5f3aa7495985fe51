"""CPU tests of the opaque operator ``torch.ops.w4a16.gemm`` (no kernel runs).

Mirrors the boundary test of PR #51453 "Register the Triton W4A16 GEMM as a
custom op" (Impl. item 4): under fake tensors the operator reports the output
shape, dtype and device, and a traced graph keeps it as one call node rather
than inlining the host-side logic.
"""
import pytest
import torch
from torch._subclasses.fake_tensor import FakeTensorMode
from torch.fx.experimental.proxy_tensor import make_fx

from weight_only_int4_unpack_amd import op


def _fake_inputs(M=4, K=256, N=512, G=128, dtype=torch.float16, zp=False, bias=False):
    a = torch.empty((M, K), device="cuda", dtype=dtype)
    b_q = torch.empty((K, N // 8), device="cuda", dtype=torch.int32)
    s = torch.empty((K // G, N), device="cuda", dtype=dtype)
    z = torch.empty((K // G, N // 8), device="cuda", dtype=torch.int32) if zp else None
    b = torch.empty((N,), device="cuda", dtype=dtype) if bias else None
    return a, b_q, s, z, b


def test_fake_reports_shape_dtype_device():
    with FakeTensorMode():
        a, b_q, s, _, _ = _fake_inputs()
        out = op.gemm(a, b_q, s, None, 128)
        assert tuple(out.shape) == (4, 512)
        assert out.dtype == a.dtype and out.device == a.device
        a, b_q, s, z, b = _fake_inputs(M=7, K=2112, N=5120, G=64, dtype=torch.bfloat16,
                                       zp=True, bias=True)
        out = op.gemm(a, b_q, s, z, 64, 8, b)
        assert tuple(out.shape) == (7, 5120) and out.dtype == torch.bfloat16


@pytest.mark.parametrize("zp,bias", [(False, False), (True, False), (False, True)])
def test_graph_keeps_one_call_node(zp, bias):
    with FakeTensorMode():
        a, b_q, s, z, b = _fake_inputs(zp=zp, bias=bias)
        gm = make_fx(lambda a, b_q, s, z, b: op.gemm(a, b_q, s, z, 128, 8, b))(a, b_q, s, z, b)
    calls = [n for n in gm.graph.nodes if n.op == "call_function"]
    assert [n.target for n in calls] == [torch.ops.w4a16.gemm.default]


def test_operator_writes_no_input():
    schema = torch.ops.w4a16.gemm.default._schema
    assert not schema.is_mutable
    assert all(arg.alias_info is None for arg in schema.arguments)


@pytest.mark.parametrize("bad", ["scales", "qzeros", "k_rows", "group", "dtype", "bias"])
def test_fake_rejects_malformed_calls(bad):
    with FakeTensorMode():
        a, b_q, s, z, b = _fake_inputs(zp=True, bias=True)
        G = 128
        if bad == "scales":
            s = torch.empty((3, 512), device="cuda", dtype=torch.float16)
        elif bad == "qzeros":
            z = torch.empty((2, 63), device="cuda", dtype=torch.int32)
        elif bad == "k_rows":
            b_q = torch.empty((255, 64), device="cuda", dtype=torch.int32)
        elif bad == "group":
            G = 96
        elif bad == "dtype":
            s = s.to(torch.bfloat16)
        elif bad == "bias":
            b = torch.empty((511,), device="cuda", dtype=torch.float16)
        with pytest.raises(ValueError):
            op.gemm(a, b_q, s, z, G, 8, b)


# ------------------------------------------------------------ K-packed operator
def _fake_kp(M=4, K=256, N=512, G=128, dtype=torch.float16, zp=False):
    a = torch.empty((M, K), device="cuda", dtype=dtype)
    w = torch.empty((N, K // 8), device="cuda", dtype=torch.int32)
    s = torch.empty((N, K // G), device="cuda", dtype=dtype)
    z = torch.empty((N, K // G), device="cuda", dtype=torch.uint8) if zp else None
    return a, w, s, z


def test_kpacked_fake_shape_and_one_call_node():
    with FakeTensorMode():
        a, w, s, z = _fake_kp(M=7, K=2112, N=5120, G=64, dtype=torch.bfloat16, zp=True)
        out = op.gemm_kpacked(a, w, s, z, 64)
        assert tuple(out.shape) == (7, 5120) and out.dtype == torch.bfloat16
        a, w, s, z = _fake_kp()
        gm = make_fx(lambda a, w, s: op.gemm_kpacked(a, w, s, None, 128))(a, w, s)
    calls = [n for n in gm.graph.nodes if n.op == "call_function"]
    assert [n.target for n in calls] == [torch.ops.w4a16.gemm_kpacked.default]
    assert not torch.ops.w4a16.gemm_kpacked.default._schema.is_mutable


@pytest.mark.parametrize("bad", ["w_cols", "scales", "zeros_dtype", "group"])
def test_kpacked_fake_rejects_malformed_calls(bad):
    with FakeTensorMode():
        a, w, s, z = _fake_kp(zp=True)
        G = 128
        if bad == "w_cols":
            w = torch.empty((512, 31), device="cuda", dtype=torch.int32)
        elif bad == "scales":
            s = torch.empty((2, 512), device="cuda", dtype=torch.float16)
        elif bad == "zeros_dtype":
            z = torch.empty((512, 2), device="cuda", dtype=torch.int32)
        else:
            G = 96
        with pytest.raises(ValueError):
            op.gemm_kpacked(a, w, s, z, G)
