"""GPU parity of glu_fwd / glu_bwd (BF16 outputs) against the oracle, rule 2 (<= 1 BF16 ulp).

Covers every finite BF16 gate value for all four activations, the FP64 tail paths (exp
underflow of the sigmoid forms, the erf-GELU tail) and ReLU^2 at extreme exponents,
the three operand layouts (split, concatenated [gate | up], paired), strided rows, ragged
and contiguous widths, in-place backward, and the full-size GeGLU sweep (sampled rows,
compared in the launch configuration the benchmark uses).
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
from conftest import bits
from parity import check_rule2

pytestmark = pytest.mark.gpu
ACTS = [("swiglu", oracle.SWIGLU), ("geglu", oracle.GEGLU_TANH), ("geglu_erf", oracle.GEGLU_ERF),
        ("relu2", oracle.RELU2)]


def _dev(*ts):
    return [t.cuda() for t in ts]


@pytest.mark.parametrize("name,kind", ACTS)
def test_every_bf16_gate_value(gpu, name, kind):
    """gate = each of the 65280 finite BF16 values; up = dh = 1 gives act and act' directly,
    then random up and dh with outliers."""
    g = si.from_bits(si.special_bf16_values().reshape(255, 256))
    one = torch.ones_like(g)
    gd, od = _dev(g, one)
    h = gpu.glu_fwd(gd, od, act=name)
    check_rule2(bits(h), oracle.glu_fwd(kind, bits(g), bits(one)), f"{name} fwd, up=1")
    da, db = gpu.glu_bwd(gd, od, od, act=name)
    oa, ob = oracle.glu_bwd(kind, bits(g), bits(one), bits(one))
    check_rule2(bits(da), oa, f"{name} act'")
    check_rule2(bits(db), ob, f"{name} act")
    up, dh = si.normal_bf16([(255, 256)] * 2, seed=3, outliers=True)
    ud, dd = _dev(up, dh)
    h = gpu.glu_fwd(gd, ud, act=name)
    check_rule2(bits(h), oracle.glu_fwd(kind, bits(g), bits(up)), f"{name} fwd")
    da, db = gpu.glu_bwd(gd, ud, dd, act=name)
    oa, ob = oracle.glu_bwd(kind, bits(g), bits(up), bits(dh))
    check_rule2(bits(da), oa, f"{name} da")
    check_rule2(bits(db), ob, f"{name} db")


TAIL_RANGE = {oracle.SWIGLU: (-104.0, -80.0), oracle.GEGLU_TANH: (-11.0, -9.0),
              oracle.GEGLU_ERF: (-40.0, -11.0)}


@pytest.mark.parametrize("name,kind", ACTS[:3])
def test_exp_underflow_tail(gpu, name, kind):
    """Gates on both sides of the switch to the FP64 tail path (e^z below the FP32 normal
    range; Phi(x) near it for erf-GELU), with large ups."""
    lo, hi = TAIL_RANGE[kind]
    gen = torch.Generator().manual_seed(7)
    g = (torch.rand(64, 256, generator=gen) * (hi - lo) + lo).to(torch.bfloat16)
    up = (torch.randn(64, 256, generator=gen) * torch.exp2(torch.randint(-10, 60, (64, 256), generator=gen))).to(torch.bfloat16)
    dh = (torch.randn(64, 256, generator=gen) * 1000).to(torch.bfloat16)
    gd, ud, dd = _dev(g, up, dh)
    check_rule2(bits(gpu.glu_fwd(gd, ud, act=name)), oracle.glu_fwd(kind, bits(g), bits(up)), "tail fwd")
    da, db = gpu.glu_bwd(gd, ud, dd, act=name)
    oa, ob = oracle.glu_bwd(kind, bits(g), bits(up), bits(dh))
    check_rule2(bits(da), oa, "tail da")
    check_rule2(bits(db), ob, "tail db")


def test_relu2_extreme_exponents(gpu):
    """ReLU^2 where g^2 alone overflows or underflows FP32 while g^2 u (and dh u g, dh g^2)
    is in range: the kernels' FP64 products must give the correctly rounded exact value."""
    gen = torch.Generator().manual_seed(8)
    shape = (64, 256)

    def pow2(e):
        return torch.exp2(e.clamp(-125, 125).double())

    eg = torch.randint(-75, 76, shape, generator=gen)
    g = (torch.rand(shape, generator=gen, dtype=torch.float64) + 0.5) * pow2(eg)
    g = torch.where(torch.rand(shape, generator=gen) < 0.1, -g, g)
    u = torch.randn(shape, generator=gen, dtype=torch.float64) * pow2(-2 * eg + torch.randint(-4, 5, shape, generator=gen))
    d = torch.randn(shape, generator=gen, dtype=torch.float64) * pow2(-eg + torch.randint(-4, 5, shape, generator=gen))
    g, u, d = (t.to(torch.bfloat16) for t in (g, u, d))
    gd, ud, dd = _dev(g, u, d)
    check_rule2(bits(gpu.glu_fwd(gd, ud, act="relu2")), oracle.glu_fwd(oracle.RELU2, bits(g), bits(u)), "fwd")
    da, db = gpu.glu_bwd(gd, ud, dd, act="relu2")
    oa, ob = oracle.glu_bwd(oracle.RELU2, bits(g), bits(u), bits(d))
    check_rule2(bits(da), oa, "da")
    check_rule2(bits(db), ob, "db")


@pytest.mark.parametrize("name,kind", ACTS)
@pytest.mark.parametrize("M,N", [(1, 8), (3, 5), (64, 96), (37, 200), (16, 8193), (5, 4096 * 3 + 7)])
def test_split_contiguous(gpu, name, kind, M, N):
    gate, up, dh = si.glu_operands(M, N, seed=M * 7 + N, outliers=True, with_dh=True)
    gd, ud, dd = _dev(gate, up, dh)
    check_rule2(bits(gpu.glu_fwd(gd, ud, act=name)), oracle.glu_fwd(kind, bits(gate), bits(up)), "fwd")
    da, db = gpu.glu_bwd(gd, ud, dd, act=name)
    oa, ob = oracle.glu_bwd(kind, bits(gate), bits(up), bits(dh))
    check_rule2(bits(da), oa, "da")
    check_rule2(bits(db), ob, "db")


@pytest.mark.parametrize("name,kind", ACTS)
def test_layouts_and_strides(gpu, name, kind):
    M, N = 48, 200
    gate, up, dh = si.glu_operands(M, N, seed=21, outliers=True, with_dh=True)
    ref_h = oracle.glu_fwd(kind, bits(gate), bits(up))
    ref_a, ref_b = oracle.glu_bwd(kind, bits(gate), bits(up), bits(dh))
    gd, ud, dd = _dev(gate, up, dh)
    # concatenated [gate | up]
    cat = torch.cat([gd, ud], dim=1)
    h = gpu.glu_fwd(cat[:, :N], cat[:, N:], act=name)
    check_rule2(bits(h), ref_h, "concat fwd")
    out = torch.empty(M, 2 * N, dtype=torch.bfloat16, device="cuda")
    gpu.glu_bwd(cat[:, :N], cat[:, N:], dd, act=name, out=(out[:, :N], out[:, N:]))
    check_rule2(bits(out[:, :N]), ref_a, "concat da")
    check_rule2(bits(out[:, N:]), ref_b, "concat db")
    # paired (interleaved) operand and interleaved gradient
    pair = torch.stack([gd, ud], dim=2).reshape(M, 2 * N).contiguous()
    check_rule2(bits(gpu.glu_fwd(pair, layout="paired", act=name)), ref_h, "paired fwd")
    d = gpu.glu_bwd(pair, None, dd, act=name, layout="paired")
    check_rule2(bits(d[:, 0::2]), ref_a, "paired da")
    check_rule2(bits(d[:, 1::2]), ref_b, "paired db")
    # strided rows (row stride 208 = N + 8) for inputs and outputs
    wide = torch.zeros(2, M, 208, dtype=torch.bfloat16, device="cuda")
    wide[0, :, :N], wide[1, :, :N] = gd, ud
    hw = torch.zeros(M, 216, dtype=torch.bfloat16, device="cuda")
    gpu.glu_fwd(wide[0, :, :N], wide[1, :, :N], act=name, out=hw[:, :N])
    check_rule2(bits(hw[:, :N]), ref_h, "strided fwd")
    assert not torch.any(hw[:, N:].view(torch.int16)), "wrote outside the output view"


@pytest.mark.parametrize("name,kind", ACTS)
def test_bwd_in_place(gpu, name, kind):
    gate, up, dh = si.glu_operands(32, 1000, seed=31, outliers=True, with_dh=True)
    oa, ob = oracle.glu_bwd(kind, bits(gate), bits(up), bits(dh))
    gd, ud, dd = _dev(gate, up, dh)
    gpu.glu_bwd(gd, ud, dd, act=name, out=(gd, ud))
    check_rule2(bits(gd), oa, "in-place da")
    check_rule2(bits(ud), ob, "in-place db")


def test_deterministic_and_path_invariant(gpu):
    """Repeated calls are byte-identical, and the flat (contiguous) path equals the strided
    path on the same values."""
    gate, up = si.glu_operands(40, 4096, seed=41, outliers=True)
    gd, ud = _dev(gate, up)
    a = gpu.glu_fwd(gd, ud, act="geglu")
    b = gpu.glu_fwd(gd, ud, act="geglu")
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    wide = torch.empty(40, 4104, dtype=torch.bfloat16, device="cuda")
    wide[:, :4096] = gd
    wu = torch.empty_like(wide)
    wu[:, :4096] = ud
    c = gpu.glu_fwd(wide[:, :4096], wu[:, :4096], act="geglu")
    assert torch.equal(a.view(torch.int16), c.view(torch.int16))


def test_empty_is_noop(gpu):
    e = torch.empty(0, 64, dtype=torch.bfloat16, device="cuda")
    assert gpu.glu_fwd(e, e).shape == (0, 64)


@pytest.mark.parametrize("rows", [1024, 8192])
@pytest.mark.parametrize("width", [4096, 11008, 14336, 18944, 29568, 8193])
def test_geglu_sweep_full_size_sampled(gpu, rows, width):
    """The GeGLU BF16 workload at full size (device-seeded inputs), checked on sampled
    rows against the oracle; W = 8193 is the ragged contiguous case."""
    g, u, d = si.normal_bf16_device([(rows, width)] * 3, seed=rows + width)
    h = gpu.glu_fwd(g, u, act="geglu")
    da, db = gpu.glu_bwd(g, u, d, act="geglu")
    torch.cuda.synchronize()
    rng = np.random.default_rng(rows * width)
    sel = torch.tensor(sorted({0, rows - 1, *rng.integers(0, rows, 14).tolist()}), device="cuda")
    gs, us, ds = bits(g[sel]), bits(u[sel]), bits(d[sel])
    check_rule2(bits(h[sel]), oracle.glu_fwd(oracle.GEGLU_TANH, gs, us), "h")
    oa, ob = oracle.glu_bwd(oracle.GEGLU_TANH, gs, us, ds)
    check_rule2(bits(da[sel]), oa, "da")
    check_rule2(bits(db[sel]), ob, "db")
