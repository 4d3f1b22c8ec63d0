"""The torch custom ops without a GPU (CPU only): fake (meta) implementations give the
shapes the entry points produce, graph capture keeps each op as one node, and the autograd
formula of `glu` routes to the fused backward op."""
import pytest
import torch
from torch._subclasses.fake_tensor import FakeTensorMode
from torch.fx.experimental.proxy_tensor import make_fx

import glu_activation_microscaling_amd as glu
import glu_activation_microscaling_amd.torch_ops  # noqa: F401  (registers torch.ops.glu_mx)

ops = torch.ops.glu_mx


def _bf16(*shape):
    return torch.empty(shape, dtype=torch.bfloat16, device="cuda")


def test_fake_shapes_match_the_entry_points():
    M, N = 160, 96
    with FakeTensorMode():
        g, u, d = _bf16(M, N), _bf16(M, N), _bf16(M, N)
        assert ops.glu(g, u, "swiglu", "split").shape == (M, N)
        assert ops.glu(_bf16(M, 2 * N), _bf16(0), "geglu", "paired").shape == (M, N)
        da, db = ops.glu_backward(g, u, d, "swiglu", "split")
        assert da.shape == db.shape == (M, N)
        dp, e = ops.glu_backward(_bf16(M, 2 * N), _bf16(0), d, "swiglu", "paired")
        assert dp.shape == (M, 2 * N) and e.numel() == 0
        qr, qc, sr, sc = ops.glu_mxfp8(g, u, "swiglu", "split", True, True, False)
        assert (qr.shape, qc.shape, sr.shape, sc.shape) == ((M, N), (N, M), (M, N // 32), (N, M // 32))
        qr, qc, sr, sc = ops.glu_mxfp8(g, u, "swiglu", "split", True, False, True)
        assert qc.numel() == 0 and sc.numel() == 0
        assert sr.numel() == glu.mxfp8_sf_bytes(M, N, True)
        qr, qc, sr, sc = ops.glu_backward_mxfp8(g, u, d, "swiglu", True, True, True)
        assert qr.shape == (M, 2 * N) and qc.shape == (2 * N, M)
        assert sr.numel() == glu.mxfp8_sf_bytes(M, 2 * N, True)
        assert sc.numel() == glu.mxfp8_sf_bytes(2 * N, M, True)
        q, sf = ops.glu_nvfp4(_bf16(M, 2 * N), _bf16(0), "geglu", "paired", "128x4")
        assert q.shape == (M, N // 2) and sf.numel() == glu.nvfp4_sf_bytes(M, N, "128x4")
        q, sf = ops.glu_backward_nvfp4(g, u, d, "swiglu", "rowmajor")
        assert q.shape == (M, N) and sf.shape == (M, 2 * N // 16)
        a = ops.glu_amax(g, u, "swiglu", "split")
        assert a.shape == (1,) and a.dtype == torch.float32
        q, sf = ops.glu_nvfp4_gs(g, u, a, "geglu", "split", "128x4")
        assert q.dtype == torch.uint8 and sf.numel() == glu.nvfp4_sf_bytes(M, N, "128x4")
        K, u8 = 256, dict(dtype=torch.uint8, device="cuda")
        xq, xs = torch.empty((M, K), **u8), torch.empty((M, K // 32), **u8)
        wq, ws = torch.empty((2 * 128, K), **u8), torch.empty((2 * 128, K // 32), **u8)
        h = ops.glu_gemm(xq, xs, wq, ws, "geglu")
        assert h.shape == (M, 128) and h.dtype == torch.bfloat16
        q, sr = ops.glu_gemm_mxfp8(xq, xs, wq, ws, "swiglu")
        assert q.shape == (M, 128) and sr.shape == (M, 4) and q.dtype == sr.dtype == torch.uint8
        q, sf = ops.glu_gemm_nvfp4(xq, xs, wq, ws, "geglu", "128x4")
        assert q.shape == (M, 64) and sf.numel() == glu.nvfp4_sf_bytes(M, 128, "128x4")
        am = torch.empty((1,), dtype=torch.float32, device="cuda")
        q, sf = ops.glu_gemm_nvfp4_gs(xq, xs, wq, ws, am, "geglu", "rowmajor")
        assert q.shape == (M, 64) and sf.shape == (M, 8)


def test_graph_capture_keeps_each_op_whole():
    def step(g, u, d):
        h = ops.glu(g, u, "swiglu", "split")
        q = ops.glu_mxfp8(g, u, "swiglu", "split", True, True, False)
        b = ops.glu_backward_mxfp8(g, u, d, "swiglu", True, True, False)
        return h, q[0], b[2]

    with FakeTensorMode() as m:
        args = (_bf16(64, 128), _bf16(64, 128), _bf16(64, 128))
        gm = make_fx(step, tracing_mode="fake")(*args)
    targets = [n.target for n in gm.graph.nodes if n.op == "call_function"]
    names = [str(t) for t in targets]
    assert any("glu_mx.glu.default" in n for n in names)
    assert any("glu_mx.glu_mxfp8.default" in n for n in names)
    assert any("glu_mx.glu_backward_mxfp8.default" in n for n in names)


def test_autograd_routes_to_the_fused_backward():
    """On meta tensors (the fake implementations serve the meta device) the backward of glu
    is one glu_backward call, split and paired."""
    def f(g, u, dh, layout):
        g = g.detach().requires_grad_(True)
        u = u.detach().requires_grad_(True)
        h = ops.glu(g, u, "geglu", layout)
        return torch.autograd.grad(h, (g,) if layout == "paired" else (g, u), dh)

    m = dict(dtype=torch.bfloat16, device="meta")
    gm = make_fx(lambda g, u, d: f(g, u, d, "split"))(*(torch.empty(32, 64, **m) for _ in range(3)))
    names = [str(n.target) for n in gm.graph.nodes if n.op == "call_function"]
    assert any("glu_mx.glu_backward.default" in n for n in names)
    (dp,) = f(torch.empty(32, 128, **m), torch.empty(0, **m), torch.empty(32, 64, **m), "paired")
    assert dp.shape == (32, 128)
