"""Pins for the oracle's activations and GLU forward/backward (CPU only).

Independent references: mpmath at 80 significant digits using the textbook formulas
(silu = x/(1+e^-x); gelu_tanh = x/2 (1 + tanh(sqrt(2/pi)(x + 0.044715 x^3)));
gelu_erf = x/2 (1 + erf(x/sqrt 2)); relu2 = max(x, 0)^2), mpmath's numerical
differentiation for the derivatives, torch float64 functional and autograd, closed forms
at special points, the reflection identity act(-x) = act(x) - x of the three GELU/SiLU
forms, and the Mills-ratio asymptotic series for the erf-GELU tail.
"""
import math

import mpmath as mp
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import synthetic_inputs as si

mp.mp.dps = 80
ACTS = [oracle.SWIGLU, oracle.GEGLU_TANH, oracle.GEGLU_ERF, oracle.RELU2]
GELU_LIKE = [oracle.SWIGLU, oracle.GEGLU_TANH, oracle.GEGLU_ERF]   # act(x) = x * F(x), F(-x) = 1 - F(x)


def mp_act(kind, x):
    x = mp.mpf(x)
    if kind == oracle.SWIGLU:
        return x / (1 + mp.exp(-x))
    if kind == oracle.GEGLU_ERF:   # 1 + erf(x / sqrt 2) written as erfc(-x / sqrt 2)
        return x / 2 * mp.erfc(-x / mp.sqrt(2))
    if kind == oracle.RELU2:
        return x * x if x > 0 else mp.mpf(0)
    u = mp.sqrt(2 / mp.pi) * (x + mp.mpf("0.044715") * x ** 3)
    return x / 2 * (1 + mp.tanh(u))


def torch_act(kind, x):
    if kind == oracle.SWIGLU:
        return F.silu(x)
    if kind == oracle.GEGLU_TANH:
        return F.gelu(x, approximate="tanh")
    if kind == oracle.GEGLU_ERF:
        return F.gelu(x, approximate="none")
    return torch.relu(x) ** 2


def mp_act_grad(kind, x):
    return mp.diff(lambda t: mp_act(kind, t), mp.mpf(x))


SAMPLE_X = np.concatenate([
    np.linspace(-12, 12, 241),
    [-95.0, -90.0, -88.5, -87.0, -60.0, -30.0, -10.5, -10.2, -10.0, -9.9, -5.0, 30.0, 100.0, 1e-30, -1e-30, 1e-3],
])


@pytest.mark.parametrize("kind", ACTS)
def test_act_against_mpmath(kind):
    got = oracle.act(kind, SAMPLE_X)
    for x, g in zip(SAMPLE_X, got):
        ref = mp_act(kind, x)
        if abs(ref) < mp.mpf("1e-300"):   # zero, or below the binary64 range
            assert abs(g) < 1e-300
            continue
        rel = abs((mp.mpf(g) - ref) / ref)
        assert rel < 1e-13, (kind, x, g, ref)


@pytest.mark.parametrize("kind", ACTS)
def test_act_grad_against_mpmath(kind):
    xs = SAMPLE_X[np.abs(SAMPLE_X) < 40]
    if kind == oracle.RELU2:
        xs = xs[xs != 0]   # numerical differentiation straddles the kink
    got = oracle.act_grad(kind, xs)
    for x, g in zip(xs, got):
        ref = mp_act_grad(kind, x)
        assert abs(mp.mpf(g) - ref) <= 1e-13 * (abs(ref) + 1e-30) + 1e-15, (kind, x, g, ref)


def test_act_special_values():
    S, G, E, R = oracle.SWIGLU, oracle.GEGLU_TANH, oracle.GEGLU_ERF, oracle.RELU2
    # erf-GELU: Phi(1) = 0.841344746068542948..., Phi(-1) = 1 - Phi(1), phi(1) = e^{-1/2}/sqrt(2 pi)
    assert oracle.act(E, [0.0])[0] == 0.0 and oracle.act_grad(E, [0.0])[0] == 0.5
    assert abs(oracle.act(E, [1.0])[0] - 0.8413447460685429) < 1e-15
    assert abs(oracle.act(E, [-1.0])[0] + 0.15865525393145707) < 1e-15
    assert abs(oracle.act_grad(E, [1.0])[0] - (0.8413447460685429 + 0.24197072451914337)) < 1e-15
    # ReLU^2 at the kink and either side; NaN stays NaN
    assert list(oracle.act(R, [-3.0, -0.0, 0.0, 1.5, 3.0])) == [0.0, 0.0, 0.0, 2.25, 9.0]
    assert list(oracle.act_grad(R, [-3.0, 0.0, 1.5, 3.0])) == [0.0, 0.0, 3.0, 6.0]
    assert np.isnan(oracle.act(R, [np.nan])[0]) and np.isnan(oracle.act_grad(R, [np.nan])[0])
    assert oracle.act(S, [0.0])[0] == 0.0 and oracle.act(G, [0.0])[0] == 0.0
    assert oracle.act_grad(S, [0.0])[0] == 0.5 and oracle.act_grad(G, [0.0])[0] == 0.5
    assert abs(oracle.act(S, [1.0])[0] - 0.7310585786300049) < 1e-15
    assert abs(oracle.act(G, [1.0])[0] - 0.8411919906082768) < 1e-15
    assert abs(oracle.act(G, [3.0])[0] - 2.996362607918227) < 1e-14
    # silu has its minimum where silu'(x0) = 0, i.e. sigma(x0)(1 + x0(1 - sigma(x0))) = 0,
    # and there silu(x0) = x0 + 1 (closed form: sigma(x0) = -1/x0 ... x0 sigma(x0) = x0 + 1)
    x0 = float(mp.findroot(lambda t: 1 + t * (1 - 1 / (1 + mp.exp(-t))), -1.28))
    assert abs(oracle.act_grad(S, [x0])[0]) < 1e-15
    assert abs(oracle.act(S, [x0])[0] - (x0 + 1)) < 1e-15


@pytest.mark.parametrize("kind", GELU_LIKE)
def test_act_and_grad_negative_in_the_tail(kind):
    """For x below the minimum of act (x0 ~ -1.28 SiLU, ~ -0.75 GELUs) act(x) < 0 and
    act'(x) < 0 exactly, so a result that underflows must be -0, not +0 (an E4M3 code keeps
    the sign of zero)."""
    xs = [-5.0, -40.0, -200.0, -1000.0, -1e30]
    assert np.all(np.signbit(oracle.act(kind, xs)))
    assert np.all(np.signbit(oracle.act_grad(kind, xs)))
    assert np.isnan(oracle.act_grad(kind, [-np.inf])[0])


@pytest.mark.parametrize("kind", GELU_LIKE)
def test_act_reflection(kind):
    """silu(-x) = silu(x) - x, and the same for both GELUs (sigma(-z) = 1 - sigma(z),
    Phi(-x) = 1 - Phi(x))."""
    x = np.linspace(-8, 8, 1601)
    a, b = oracle.act(kind, -x), oracle.act(kind, x) - x
    assert np.allclose(a, b, rtol=1e-12, atol=1e-14)


# torch evaluates both GELUs through 1 + tanh or 1 + erf, which loses relative accuracy
# for x << 0; there the comparison stops at x = -4
_TORCH_CANCELS = (oracle.GEGLU_TANH, oracle.GEGLU_ERF)


@pytest.mark.parametrize("kind", ACTS)
def test_act_against_torch_float64(kind):
    x = torch.linspace(-20, 20, 40001, dtype=torch.float64)
    ref = torch_act(kind, x)
    got = torch.from_numpy(oracle.act(kind, x.numpy()))
    mask = x > -4 if kind in _TORCH_CANCELS else torch.ones_like(x, dtype=torch.bool)
    assert torch.allclose(got[mask], ref[mask], rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("kind", ACTS)
def test_act_grad_against_autograd(kind):
    x = torch.linspace(-20, 20, 4001, dtype=torch.float64, requires_grad=True)
    y = torch_act(kind, x)
    (g,) = torch.autograd.grad(y.sum(), x)
    got = torch.from_numpy(oracle.act_grad(kind, x.detach().numpy()))
    mask = x.detach() > -4 if kind in _TORCH_CANCELS else torch.ones(x.shape, dtype=torch.bool)
    assert torch.allclose(got[mask], g[mask], rtol=1e-12, atol=1e-14)


def test_act_grad_central_difference():
    eps = 2.0 ** -20
    x = np.linspace(-6, 6, 121)
    for kind in ACTS:
        xs = x[x != 0] if kind == oracle.RELU2 else x
        fd = (oracle.act(kind, xs + eps) - oracle.act(kind, xs - eps)) / (2 * eps)
        assert np.allclose(oracle.act_grad(kind, xs), fd, rtol=1e-8, atol=1e-9)


def test_gelu_erf_tail_mills_ratio():
    """For x << 0, Phi(x) = phi(x)/|x| (1 - 1/x^2 + 3/x^4 - 15/x^6 + ... + (-1)^k (2k-1)!!/x^2k)
    (the asymptotic series of the Mills ratio); with 20 terms at |x| >= 14 the truncation
    error is below 1e-20 relative.  Covers the range where Phi(x) is below the FP32 normal
    range."""
    for x in [-14.0, -16.0, -20.0, -25.0, -30.0, -37.0]:
        phi = math.exp(-0.5 * x * x) / math.sqrt(2 * math.pi)
        s, term = 0.0, 1.0
        for k in range(20):
            s += term
            term *= -(2 * k + 1) / (x * x)
        want_act = x * phi / abs(x) * s
        want_grad = phi / abs(x) * s + x * phi
        assert abs(oracle.act(oracle.GEGLU_ERF, [x])[0] / want_act - 1) < 1e-13, x
        assert abs(oracle.act_grad(oracle.GEGLU_ERF, [x])[0] / want_grad - 1) < 1e-12, x


def test_relu2_glu_is_exact():
    """relu2(g) * u of BF16 operands has at most 24 significant bits (BF16 values are
    m * 2^e with m < 256), so it is exact in binary64 and the oracle's BF16 output is the
    rounding of the exact rational product, computed here with Fractions."""
    from fractions import Fraction
    gate, up = si.glu_operands(32, 64, seed=21)
    gb, ub = si.to_bits(gate), si.to_bits(up)
    h = oracle.glu_fwd(oracle.RELU2, gb, ub).ravel()
    g, u = oracle.bf16_to_f64(gb).ravel(), oracle.bf16_to_f64(ub).ravel()
    for i in range(g.size):
        if g[i] <= 0:
            assert int(h[i]) & 0x7FFF == 0, i
            continue
        exact = Fraction(g[i]) ** 2 * Fraction(u[i])
        assert Fraction(float(exact)) == exact
        assert int(h[i]) == int(oracle.bf16_from_f64([float(exact)])[0]), i


# ---- GLU forward / backward ----------------------------------------------------------

def _dec(b):
    return si.from_bits(b).to(torch.float64)


def _bf16_nearest_ok(got_bits, exact):
    """got (BF16 bits) is the nearest BF16 to exact (float64 tensor) with a margin: every
    element is within half a BF16 ulp plus 1e-12 relative."""
    got = _dec(got_bits)
    ulp = torch.where(exact.abs() < 2.0 ** -126, torch.full_like(exact, 2.0 ** -133),
                      torch.exp2(torch.floor(torch.log2(exact.abs().clamp_min(2.0 ** -126)))) * 2.0 ** -7)
    return bool(((got - exact).abs() <= 0.5 * ulp * (1 + 1e-12) + 1e-300).all())


@pytest.mark.parametrize("kind", ACTS)
def test_glu_fwd_matches_float64_reference(kind):
    gate, up = si.glu_operands(64, 96, seed=11)
    h = oracle.glu_fwd(kind, si.to_bits(gate), si.to_bits(up))
    g64, u64 = gate.double(), up.double()
    assert _bf16_nearest_ok(h, torch_act(kind, g64) * u64)


@pytest.mark.parametrize("kind", ACTS)
def test_glu_bwd_matches_autograd(kind):
    gate, up, dh = si.glu_operands(48, 80, seed=12, with_dh=True)
    g64 = gate.double().requires_grad_(True)
    u64 = up.double().requires_grad_(True)
    (torch_act(kind, g64) * u64).backward(dh.double())
    da, db = oracle.glu_bwd(kind, si.to_bits(gate), si.to_bits(up), si.to_bits(dh))
    assert _bf16_nearest_ok(da, g64.grad)
    assert _bf16_nearest_ok(db, u64.grad)


@pytest.mark.parametrize("kind", ACTS)
def test_glu_bwd_identities(kind):
    """dh = 1, up = 1: da = act'(g) and db = act(g); dh = 0 gives zeros; up = 0 gives da = 0."""
    gate = si.normal_bf16([(16, 64)], seed=13)[0]
    gb = si.to_bits(gate)
    one = np.full(gb.shape, 0x3F80, np.uint16)
    zero = np.zeros(gb.shape, np.uint16)
    da, db = oracle.glu_bwd(kind, gb, one, one)
    g = gate.double().numpy()
    assert np.array_equal(da, oracle.bf16_from_f64(oracle.act_grad(kind, g)))
    assert np.array_equal(db, oracle.bf16_from_f64(oracle.act(kind, g)))
    da0, db0 = oracle.glu_bwd(kind, gb, one, zero)
    assert not np.any(da0 & 0x7FFF) and not np.any(db0 & 0x7FFF)
    da1, _ = oracle.glu_bwd(kind, gb, zero, one)
    assert not np.any(da1 & 0x7FFF)


@pytest.mark.parametrize("kind", [oracle.SWIGLU, oracle.GEGLU_TANH])
def test_glu_tail_closed_form(kind):
    """For z << 0 the logistic is e^z to 1e-30 relative, so act(x) = x e^{z} in closed
    form; with up = 1 the BF16 output is the rounding of that product (tiny but nonzero
    BF16 values)."""
    if kind == oracle.SWIGLU:
        xs = [-87.5, -90.0, -93.0, -96.0]
    else:
        xs = [-9.9, -10.0, -10.1, -10.2]
    for x in xs:
        gb = oracle.bf16_from_f64([x])
        h = oracle.glu_fwd(kind, gb.reshape(1, 1), np.array([[0x3F80]], np.uint16))
        xb = float(oracle.bf16_to_f64(gb)[0])
        zb = xb if kind == oracle.SWIGLU else 2 * math.sqrt(2 / math.pi) * (xb + 0.044715 * xb ** 3)
        want = oracle.bf16_from_f64([xb * math.exp(zb)])[0]
        assert int(h[0, 0]) == int(want) and int(want) & 0x7FFF != 0, (x, hex(h[0, 0]), hex(want))


def test_layouts_agree():
    """SPLIT, concatenated [gate | up] (SPLIT with up = gate + N, ld = 2N) and PAIRED
    (interleaved columns) are the same operands addressed three ways."""
    gate, up, dh = si.glu_operands(40, 72, seed=14, with_dh=True)
    gb, ub, db_ = si.to_bits(gate), si.to_bits(up), si.to_bits(dh)
    paired = np.empty((40, 144), np.uint16)
    paired[:, 0::2], paired[:, 1::2] = gb, ub
    for kind in ACTS:
        h_split = oracle.glu_fwd(kind, gb, ub)
        h_pair = oracle.glu_fwd(kind, paired, None, layout=oracle.PAIRED)
        assert np.array_equal(h_split, h_pair)
        da, dbb = oracle.glu_bwd(kind, gb, ub, db_)
        d = oracle.glu_bwd(kind, paired, None, db_, layout=oracle.PAIRED)
        assert np.array_equal(d[:, 0::2], da) and np.array_equal(d[:, 1::2], dbb)


def test_fwd_swaps_are_detected():
    """Guards against a transposed operand: act(up) * gate differs from act(gate) * up."""
    gate, up = si.glu_operands(8, 32, seed=15)
    a = oracle.glu_fwd(oracle.SWIGLU, si.to_bits(gate), si.to_bits(up))
    b = oracle.glu_fwd(oracle.SWIGLU, si.to_bits(up), si.to_bits(gate))
    assert not np.array_equal(a, b)


def test_row_slices_are_batch_invariant():
    gate, up = si.glu_operands(64, 64, seed=16)
    gb, ub = si.to_bits(gate), si.to_bits(up)
    full = oracle.glu_fwd(oracle.GEGLU_TANH, gb, ub)
    part = oracle.glu_fwd(oracle.GEGLU_TANH, gb[17:41], ub[17:41])
    assert np.array_equal(full[17:41], part)
