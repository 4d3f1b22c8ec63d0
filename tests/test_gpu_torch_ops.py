"""The torch custom ops on the GPU: each equals the binding call it wraps byte for byte,
glu's autograd gives the fused backward's gradients, torch.library.opcheck accepts the
registrations, and torch.compile(fullgraph=True) (aot_eager: no generated kernels) gives
the eager results."""
import pytest
import torch

import synthetic_inputs as si
import glu_activation_microscaling_amd.torch_ops  # noqa: F401

pytestmark = pytest.mark.gpu
ops = torch.ops.glu_mx


def _operands(M, N, seed):
    return [t.cuda() for t in si.glu_operands(M, N, seed=seed, outliers=True, with_dh=True)]


def _same(a, b):
    return all(torch.equal(x.view(torch.uint8), y.view(torch.uint8)) for x, y in zip(a, b))


def test_ops_equal_the_binding(gpu):
    g, u, d = _operands(128, 256, 60)
    e = g.new_empty((0,))
    p = torch.stack([g, u], 2).reshape(128, 512).contiguous()
    assert _same([ops.glu(g, u, "swiglu", "split")], [gpu.glu_fwd(g, u)])
    assert _same([ops.glu(p, e, "geglu", "paired")], [gpu.glu_fwd(p, layout="paired", act="geglu")])
    assert _same(ops.glu_backward(g, u, d, "swiglu", "split"), gpu.glu_bwd(g, u, d))
    assert _same(ops.glu_mxfp8(g, u, "geglu", "split", True, True, True),
                 gpu.glu_fwd_mxfp8(g, u, act="geglu", rowwise=True, colwise=True, swizzled=True))
    assert _same(ops.glu_backward_mxfp8(g, u, d, "swiglu", True, True, False),
                 gpu.glu_bwd_mxfp8(g, u, d, rowwise=True, colwise=True))
    assert _same(ops.glu_nvfp4(p, e, "geglu", "paired", "128x4"),
                 gpu.glu_fwd_nvfp4(p, act="geglu", layout="paired", sf_layout="128x4"))
    assert _same(ops.glu_backward_nvfp4(g, u, d, "swiglu", "rowmajor"), gpu.glu_bwd_nvfp4(g, u, d))
    a = ops.glu_amax(p, e, "geglu", "paired")
    assert torch.equal(a, gpu.glu_amax(p, act="geglu", layout="paired"))
    assert _same(ops.glu_nvfp4_gs(p, e, a, "geglu", "paired", "rowmajor"),
                 gpu.glu_fwd_nvfp4_gs(p, amax=a, act="geglu", layout="paired"))
    mx = _mx_operands(96, 128, 256, 65)
    assert _same([ops.glu_gemm(*mx, "geglu")], [gpu.glu_gemm(*mx, act="geglu")])
    assert _same(ops.glu_gemm_mxfp8(*mx, "swiglu"), gpu.glu_gemm_mxfp8(*mx))
    assert _same(ops.glu_gemm_nvfp4(*mx, "geglu", "128x4"), gpu.glu_gemm_nvfp4(*mx, sf_layout="128x4"))
    am = torch.tensor([3.0], dtype=torch.float32, device="cuda")
    assert _same(ops.glu_gemm_nvfp4_gs(*mx, am, "geglu", "rowmajor"), gpu.glu_gemm_nvfp4_gs(*mx, amax=am))


def _mx_operands(M, N, K, seed):
    xq, xs = si.mx_operand(M, K, seed=seed, device="cuda")
    wq, ws = si.mx_operand(2 * N, K, seed=seed + 1, device="cuda")
    return xq, xs, wq, ws


@pytest.mark.parametrize("layout", ["split", "paired"])
def test_autograd_gives_the_fused_backward(gpu, layout):
    g, u, d = _operands(64, 192, 61)
    if layout == "paired":
        p = torch.stack([g, u], 2).reshape(64, 384).contiguous().requires_grad_(True)
        h = ops.glu(p, p.new_empty((0,)), "geglu", "paired")
        h.backward(d)
        want = gpu.glu_bwd(p.detach(), None, d, act="geglu", layout="paired")
        assert torch.equal(p.grad.view(torch.int16), want.view(torch.int16))
    else:
        gg, uu = g.clone().requires_grad_(True), u.clone().requires_grad_(True)
        h = ops.glu(gg, uu, "geglu", "split")
        h.backward(d)
        da, db = gpu.glu_bwd(g, u, d, act="geglu")
        assert torch.equal(gg.grad.view(torch.int16), da.view(torch.int16))
        assert torch.equal(uu.grad.view(torch.int16), db.view(torch.int16))


def test_broadcast_upstream_gradient(gpu):
    """h.sum().backward() hands over a stride-0 gradient; the autograd formula makes it a
    plain matrix for the kernel."""
    g, u, _ = _operands(32, 64, 62)
    gg = g.clone().requires_grad_(True)
    ops.glu(gg, u, "swiglu", "split").float().sum().backward()
    da, _ = gpu.glu_bwd(g, u, torch.ones_like(g))
    assert torch.equal(gg.grad.view(torch.int16), da.view(torch.int16))


def test_opcheck(gpu):
    g, u, d = _operands(64, 128, 63)
    e = g.new_empty((0,))
    torch.library.opcheck(ops.glu, (g.requires_grad_(True), u, "swiglu", "split"))
    torch.library.opcheck(ops.glu_mxfp8, (g.detach(), u, "swiglu", "split", True, True, False))
    torch.library.opcheck(ops.glu_backward_nvfp4, (g.detach(), u, d, "swiglu", "128x4"))
    torch.library.opcheck(ops.glu_amax, (g.detach(), u, "swiglu", "split"))
    torch.library.opcheck(ops.glu_nvfp4, (g.detach(), u, "geglu", "split", "rowmajor"))
    mx = _mx_operands(64, 128, 256, 66)
    torch.library.opcheck(ops.glu_gemm, (*mx, "swiglu"))
    torch.library.opcheck(ops.glu_gemm_mxfp8, (*mx, "geglu"))
    torch.library.opcheck(ops.glu_gemm_nvfp4, (*mx, "geglu", "rowmajor"))


def test_compile_fullgraph_matches_eager(gpu):
    g, u, d = _operands(128, 256, 64)

    mx = _mx_operands(128, 128, 256, 67)

    def step(g, u, d):
        h = ops.glu(g, u, "swiglu", "split")
        fq = ops.glu_mxfp8(g, u, "swiglu", "split", True, True, False)
        bq = ops.glu_backward_mxfp8(g, u, d, "swiglu", True, True, False)
        gq = ops.glu_gemm_mxfp8(*mx, "swiglu")
        return (h,) + tuple(fq) + tuple(bq) + tuple(gq)

    eager = step(g, u, d)
    compiled = torch.compile(step, fullgraph=True, backend="aot_eager")(g, u, d)
    assert _same(eager, compiled)

    def fwd(g, u):
        return ops.glu(g, u, "geglu", "split")

    grads = []
    for fn in (fwd, torch.compile(fwd, fullgraph=True, backend="aot_eager")):
        gg = g.clone().requires_grad_(True)
        h = fn(gg, u)
        h.backward(d)
        grads.append((h.detach(), gg.grad))
    assert _same(grads[0], grads[1])
