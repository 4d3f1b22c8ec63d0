"""GPU parity of the fused NVFP4 path and the NVFP4 quantizer hook against the oracle.

Rule 1: glu_quant_nvfp4_f32 equals oracle.quant_nvfp4 byte for byte on random, outlier,
tie-dense, all-BF16 and non-finite inputs, in both scale layouts; the fused kernel equals
the oracle quantizer applied to the GPU's own BF16 glu_fwd output.
Rule 3: the GeGLU NVFP4 workload ([M, 32768] interleaved, M in {784, 816, 880, 968}) end to
end against the oracle, plus the zero padding of the 128x4 scale layout.
Backward ([da | db] as one [M, 2N] NVFP4 matrix): rule 1 against the oracle quantizer on the
GPU's own glu_bwd output for every activation and both scale layouts, rule 3 end to end,
ragged widths and rows, and the binding's refusal of mis-shaped buffers.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
from conftest import bits, u8
from parity import check_rule3_nv, check_rule3_nv_gs

pytestmark = pytest.mark.gpu
SFL = [("rowmajor", oracle.SF_ROWMAJOR), ("128x4", oracle.SF_128x4)]


def _hook(gpu, x):
    xd = torch.from_numpy(x).cuda()
    for name, code in SFL:
        q, sf = gpu.glu_quant_nvfp4_f32(xd, sf_layout=name)
        oq, osf = oracle.quant_nvfp4(x, code)
        assert np.array_equal(u8(sf).ravel(), osf.ravel()), f"scales ({name})"
        assert np.array_equal(u8(q), oq), f"codes ({name})"


def test_hook_random_fp32(gpu):
    rng = np.random.default_rng(200)
    x = rng.normal(0, 1, (200, 1024))
    x[rng.random(x.shape) < 1e-3] *= 1000
    x[rng.random(x.shape) < 1e-2] *= 2.0 ** -30
    x[3, :16] = 0.0
    x[4, 16:32] = -0.0
    _hook(gpu, x.astype(np.float32))


def test_hook_every_bf16_value(gpu):
    allv = si.special_bf16_values()
    x = np.zeros(65536, np.float32)
    x[: allv.size] = si.from_bits(allv).float().numpy()
    _hook(gpu, x.reshape(256, 256))
    rng = np.random.default_rng(201)
    _hook(gpu, rng.permutation(x).reshape(512, 128))


def test_hook_ties_and_boundaries(gpu):
    """Blocks whose amax lands on 6 x an E4M3 midpoint (scale ties) and whose elements land
    on E2M1 midpoints x S (code ties), plus one FP32 ulp either side."""
    rng = np.random.default_rng(202)
    e4 = np.unique(np.abs(oracle.e4m3_to_f64(np.arange(0x7F, dtype=np.uint8))))
    nblk = 16384
    S = rng.choice(e4[1:], nblk)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0.5, 1, 1.5, 2, 3, 4, 6])
    y = (rng.choice(mids, (nblk, 15)) * S[:, None]).astype(np.float32)
    j = rng.integers(-1, 2, y.shape)
    y = np.where(j > 0, np.nextafter(y, np.float32(np.inf)), np.where(j < 0, np.nextafter(y, np.float32(0)), y))
    smid = (e4[1:] + e4[:-1]) / 2
    amax = (6.0 * rng.choice(smid, nblk)).astype(np.float32)
    ja = rng.integers(-1, 2, nblk)
    amax = np.where(ja > 0, np.nextafter(amax, np.float32(np.inf)), np.where(ja < 0, np.nextafter(amax, np.float32(0)), amax))
    x = np.concatenate([amax[:, None], y], axis=1) * rng.choice([-1, 1], (nblk, 16))
    _hook(gpu, x.astype(np.float32).reshape(1024, 256))


def test_hook_nonfinite_blocks(gpu):
    x = np.ones((8, 64), np.float32)
    x[0, 3] = np.inf
    x[5, 20] = np.nan
    x[6, 40] = -np.inf
    _hook(gpu, x)


@pytest.mark.parametrize("act,kind", [("geglu", oracle.GEGLU_TANH), ("swiglu", oracle.SWIGLU),
                                      ("geglu_erf", oracle.GEGLU_ERF), ("relu2", oracle.RELU2)])
@pytest.mark.parametrize("layout", ["paired", "split"])
def test_fused_equals_quantized_glu_fwd(gpu, act, kind, layout):
    M, H = 130, 1024
    gate, up = si.glu_operands(M, H, seed=12, outliers=True)
    gd, ud = gate.cuda(), up.cuda()
    args = (torch.stack([gd, ud], 2).reshape(M, 2 * H).contiguous(), None) if layout == "paired" else (gd, ud)
    h = gpu.glu_fwd(*args, act=act, layout=layout)
    hf = si.from_bits(bits(h)).float().numpy()
    for name, code in SFL:
        q, sf = gpu.glu_fwd_nvfp4(*args, act=act, layout=layout, sf_layout=name)
        oq, osf = oracle.quant_nvfp4(hf, code)
        assert np.array_equal(u8(q), oq) and np.array_equal(u8(sf).ravel(), osf.ravel())


@pytest.mark.parametrize("M", [784, 816, 880, 968])
def test_config_geglu_nvfp4(gpu, M):
    H = 16384
    x = si.paired_operand(M, H, seed=0)
    xb = bits(x)
    xd = x.cuda()
    h = oracle.glu_fwd(oracle.GEGLU_TANH, xb, None, layout=oracle.PAIRED)
    for name, code in SFL:
        q, sf = gpu.glu_fwd_nvfp4(xd, act="geglu", layout="paired", sf_layout=name)
        oq, osf = oracle.glu_fwd_nvfp4(oracle.GEGLU_TANH, xb, None, sf_layout=code)
        if code == oracle.SF_ROWMAJOR:
            check_rule3_nv(h, u8(q), u8(sf), oq, osf, f"M={M}")
        else:
            # same scales after unswizzling, and zero padding
            s = u8(sf)
            nb, cp = H // 16, (H // 16 + 3) // 4 * 4
            idx = np.array([[oracle.sf128x4_offset(r, c, cp) for c in range(0, nb, 97)] for r in range(0, M, 13)])
            assert np.array_equal(s[idx], osf[idx])
            rp = (M + 127) // 128 * 128
            pad = np.array([oracle.sf128x4_offset(r, c, cp) for r in range(M, rp) for c in range(0, nb, 31)], dtype=np.int64)
            if pad.size:
                assert not np.any(s[pad]), "128x4 padding rows must be zero"


ACTS = [("swiglu", oracle.SWIGLU), ("geglu", oracle.GEGLU_TANH), ("geglu_erf", oracle.GEGLU_ERF),
        ("relu2", oracle.RELU2)]


@pytest.mark.parametrize("act,kind", ACTS)
@pytest.mark.parametrize("M,N", [(130, 1024), (5, 48), (37, 2064), (4096, 96)])
def test_fused_bwd_equals_quantized_glu_bwd(gpu, act, kind, M, N):
    """Small launches take 2 column groups per lane, [4096, 96] takes 4."""
    gate, up, dh = si.glu_operands(M, N, seed=M + N + kind, outliers=True, with_dh=True)
    gd, ud, dd = gate.cuda(), up.cuda(), dh.cuda()
    da, db = gpu.glu_bwd(gd, ud, dd, act=act)
    X = si.from_bits(np.concatenate([bits(da), bits(db)], axis=1)).float().numpy()
    for name, code in SFL:
        q, sf = gpu.glu_bwd_nvfp4(gd, ud, dd, act=act, sf_layout=name)
        oq, osf = oracle.quant_nvfp4(X, code)
        assert np.array_equal(u8(sf).ravel(), osf.ravel()), f"scales ({name})"
        assert np.array_equal(u8(q), oq), f"codes ({name})"


@pytest.mark.parametrize("act,kind", ACTS)
def test_fused_tail_paths_equal_quantized_glu(gpu, act, kind):
    """Most elements on the FP64 tail path (si.tail_operands): the fused forward (paired and
    split operands) and backward equal the oracle quantizer applied to the GPU's own
    glu_fwd / glu_bwd output, in both scale layouts."""
    M, N = 130, 1024
    g, u, d = si.tail_operands(act, M, N, seed=21 + kind)
    gd, ud, dd = g.cuda(), u.cuda(), d.cuda()
    pair = torch.stack([gd, ud], 2).reshape(M, 2 * N).contiguous()
    hf = si.from_bits(bits(gpu.glu_fwd(gd, ud, act=act))).float().numpy()
    da, db = gpu.glu_bwd(gd, ud, dd, act=act)
    X = si.from_bits(np.concatenate([bits(da), bits(db)], axis=1)).float().numpy()
    for name, code in SFL:
        oq, osf = oracle.quant_nvfp4(hf, code)
        for args, layout in (((pair, None), "paired"), ((gd, ud), "split")):
            q, sf = gpu.glu_fwd_nvfp4(*args, act=act, layout=layout, sf_layout=name)
            assert np.array_equal(u8(q), oq) and np.array_equal(u8(sf).ravel(), osf.ravel()), f"fwd {layout} ({name})"
        q, sf = gpu.glu_bwd_nvfp4(gd, ud, dd, act=act, sf_layout=name)
        oq, osf = oracle.quant_nvfp4(X, code)
        assert np.array_equal(u8(sf).ravel(), osf.ravel()), f"bwd scales ({name})"
        assert np.array_equal(u8(q), oq), f"bwd codes ({name})"


@pytest.mark.parametrize("act,kind", ACTS)
def test_bwd_rule3_against_oracle(gpu, act, kind):
    M, N = 512, 4096
    gate, up, dh = si.glu_operands(M, N, seed=40 + kind, outliers=True, with_dh=True)
    gb, ub, db_ = bits(gate), bits(up), bits(dh)
    q, sf = gpu.glu_bwd_nvfp4(gate.cuda(), up.cuda(), dh.cuda(), act=act)
    oq, osf = oracle.glu_bwd_nvfp4(kind, gb, ub, db_)
    oa, ob = oracle.glu_bwd(kind, gb, ub, db_)
    check_rule3_nv(np.concatenate([oa, ob], 1), u8(q), u8(sf), oq, osf, f"{act} bwd")


def test_bwd_strided_operands(gpu):
    """gate/up rows inside a wider [gate | up] matrix, dh with a padded row stride."""
    M, N = 64, 512
    gate, up, dh = si.glu_operands(M, N, seed=44, with_dh=True)
    cat = torch.cat([gate, up], 1).cuda()
    dpad = torch.zeros(M, N + 64, dtype=torch.bfloat16, device="cuda")
    dpad[:, :N] = dh.cuda()
    q, sf = gpu.glu_bwd_nvfp4(cat[:, :N], cat[:, N:], dpad[:, :N])
    oq, osf = oracle.glu_bwd_nvfp4(oracle.SWIGLU, bits(gate), bits(up), bits(dh))
    oa, ob = oracle.glu_bwd(oracle.SWIGLU, bits(gate), bits(up), bits(dh))
    check_rule3_nv(np.concatenate([oa, ob], 1), u8(q), u8(sf), oq, osf, "strided bwd")


def test_binding_rejects_misshaped_buffers(gpu):
    """Buffers that do not match the operands raise before any launch."""
    gate, up, dh = (t.cuda() for t in si.glu_operands(32, 64, seed=45, with_dh=True))
    with pytest.raises(ValueError):
        gpu.glu_bwd_nvfp4(gate, up, dh[:16])
    q = torch.empty((32, 64), dtype=torch.uint8, device="cuda")
    sf = torch.empty((32, 8), dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError):
        gpu.glu_bwd_nvfp4(gate, up, dh, out=(q[:16], sf))
    with pytest.raises(ValueError):
        gpu.glu_bwd_nvfp4(gate, up, dh, out=(q, sf[:, :4]))
    with pytest.raises(ValueError):
        gpu.glu_fwd(gate, up, out=torch.empty((16, 64), dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ValueError):
        gpu.glu_bwd(gate, up, dh[:, :32])
    qr = torch.empty((32, 32), dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError):
        gpu.glu_fwd_mxfp8(gate, up, rowwise=True, out=(qr, torch.empty(0), torch.empty((32, 2)), torch.empty(0)))
    gpu.glu_bwd_nvfp4(gate, up, dh, out=(q, sf))   # the right shapes are accepted


def test_every_bf16_block_amax(gpu):
    """The fused path's scale decision for every normal BF16 block maximum: gate = 32 makes
    silu(32) * up round to exactly 32 * up in FP32, so up = a / 32 puts h = a at the head of
    a block, followed by 15 smaller random values (mixed signs)."""
    b = np.arange(0x0380, 0x7F80, dtype=np.uint32)   # a / 32 stays a normal BF16 number
    a = (b << 16).view(np.float32)
    rng = np.random.default_rng(46)
    n = a.size
    blocks = np.empty((n, 16), np.float32)
    blocks[:, 0] = a
    blocks[:, 1:] = a[:, None] * rng.uniform(-0.99, 0.99, (n, 15)).astype(np.float32)
    pad = (-n) % 16
    blocks = np.concatenate([blocks, np.ones((pad, 16), np.float32)])
    up = torch.from_numpy(blocks.reshape(-1, 256) / np.float32(32.0)).to(torch.bfloat16)
    gate = torch.full_like(up, 32.0)
    gd, ud = gate.cuda(), up.cuda()
    h = bits(gpu.glu_fwd(gd, ud, act="swiglu"))
    assert np.array_equal(h.reshape(-1, 16)[:n, 0], b.astype(np.uint16)), "h = a at each block head"
    hf = si.from_bits(h).float().numpy()
    for name, code in SFL:
        q, sf = gpu.glu_fwd_nvfp4(gd, ud, act="swiglu", layout="split", sf_layout=name)
        oq, osf = oracle.quant_nvfp4(hf, code)
        assert np.array_equal(u8(sf).ravel(), osf.ravel()), f"scales ({name})"
        assert np.array_equal(u8(q), oq), f"codes ({name})"


def test_bwd_four_groups_ragged_tile(gpu):
    """[4160, 8208]: 4 column groups per lane, with a second tile holding 16 live columns."""
    M, N = 4160, 8208
    g, u, d = si.normal_bf16_device([(M, N)] * 3, seed=47, outliers=True)
    da, db = gpu.glu_bwd(g, u, d)
    X = si.from_bits(np.concatenate([bits(da), bits(db)], axis=1)).float().numpy()
    for name, code in SFL:
        q, sf = gpu.glu_bwd_nvfp4(g, u, d, sf_layout=name)
        oq, osf = oracle.quant_nvfp4(X, code)
        assert np.array_equal(u8(sf).ravel(), osf.ravel()), f"scales ({name})"
        assert np.array_equal(u8(q), oq), f"codes ({name})"


# ---- two-level NVFP4 (global scale from the tensor amax) ----------------------------

@pytest.mark.parametrize("act,kind", ACTS)
@pytest.mark.parametrize("layout", ["split", "paired"])
def test_amax_and_two_level_equal_oracle_quantizer(gpu, act, kind, layout):
    """glu_amax equals the oracle's largest |h|; the two-level fused forward equals the oracle
    quantizer applied to the GPU's own BF16 forward at that amax (rule 1)."""
    M, H = 130, 2064
    gate, up = si.glu_operands(M, H, seed=51 + kind, outliers=True)
    gd, ud = gate.cuda(), up.cuda()
    args = (torch.stack([gd, ud], 2).reshape(M, 2 * H).contiguous(), None) if layout == "paired" else (gd, ud)
    a = gpu.glu_amax(*args, act=act, layout=layout)
    h = bits(gpu.glu_fwd(*args, act=act, layout=layout))
    assert float(a.item()) == oracle.glu_amax(kind, bits(gate), bits(up))
    hf = si.from_bits(h).float().numpy()
    for name, code in SFL:
        q, sf = gpu.glu_fwd_nvfp4_gs(*args, amax=a, act=act, layout=layout, sf_layout=name)
        oq, osf = oracle.quant_nvfp4_gs(hf, float(a.item()), code)
        assert np.array_equal(u8(sf).ravel(), osf.ravel()), f"scales ({name})"
        assert np.array_equal(u8(q), oq), f"codes ({name})"


@pytest.mark.parametrize("M", [784, 968])
def test_two_level_config_geglu(gpu, M):
    """The GeGLU NVFP4 workload with two-level scaling, end to end against the oracle at the
    oracle's amax (rule 3), and the GPU amax equal to the oracle's."""
    H = 16384
    x = si.paired_operand(M, H, seed=1)
    xb = bits(x)
    xd = x.cuda()
    amax = oracle.glu_amax(oracle.GEGLU_TANH, xb, None, layout=oracle.PAIRED)
    assert float(gpu.glu_amax(xd, act="geglu", layout="paired").item()) == amax
    ad = torch.tensor([amax], dtype=torch.float32, device="cuda")
    q, sf = gpu.glu_fwd_nvfp4_gs(xd, amax=ad, act="geglu", layout="paired")
    oq, osf = oracle.glu_fwd_nvfp4_gs(oracle.GEGLU_TANH, xb, None, amax=amax)
    h = oracle.glu_fwd(oracle.GEGLU_TANH, xb, None, layout=oracle.PAIRED)
    check_rule3_nv_gs(h, u8(q), u8(sf), oq, osf, oracle.nvfp4_global_scale(amax), f"two-level M={M}")


@pytest.mark.parametrize("amax", [0.0, 1e-30, 2.0 ** -100, 0.25, 3.0e38, float("inf"), float("nan")])
def test_two_level_degenerate_amax(gpu, amax):
    """Any amax, including ones far from the data's (saturating scales and codes), zero, tiny
    (capped global scale) and non-finite (global scale 1), quantizes as the oracle does."""
    M, H = 64, 512
    gate, up = si.glu_operands(M, H, seed=52, outliers=True)
    gd, ud = gate.cuda(), up.cuda()
    hf = si.from_bits(bits(gpu.glu_fwd(gd, ud, act="swiglu"))).float().numpy()
    ad = torch.tensor([amax], dtype=torch.float32, device="cuda")
    q, sf = gpu.glu_fwd_nvfp4_gs(gd, ud, amax=ad, act="swiglu", layout="split")
    oq, osf = oracle.quant_nvfp4_gs(hf, amax)
    assert np.array_equal(u8(sf), osf) and np.array_equal(u8(q), oq)


def test_amax_nan_and_empty(gpu):
    gate, up = (t.cuda() for t in si.glu_operands(32, 64, seed=53))
    gate[5, 7] = float("nan")
    assert np.isnan(gpu.glu_amax(gate, up).item())
    e = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    a = torch.full((1,), 7.0, dtype=torch.float32, device="cuda")
    assert gpu.glu_amax(e, e, out=a).item() == 0.0


def test_every_bf16_value_under_every_scale_fused(gpu):
    """Rule 1 through the fused NVFP4 forward for every BF16 value under every E4M3 block scale:
    for each positive finite E4M3 value S a set of 16-element blocks has the maximum 6 S (so
    the block scale is S) and runs through every BF16 magnitude up to 6 S with random signs.
    ReLU^2 with gate = 1 makes h = up exactly; codes and scales (both layouts) equal the
    oracle quantizer of the device's own h byte for byte."""
    rng = np.random.default_rng(91)
    mags = np.arange(1, 0x7F80, dtype=np.uint32)
    mvals = (mags << 16).view(np.float32).astype(np.float64)
    blocks = []
    for S in oracle.e4m3_to_f64(np.arange(1, 0x7F, dtype=np.uint8)):
        body = mags[mvals <= 6.0 * S]
        body = body | (rng.integers(0, 2, body.size, dtype=np.uint32) << 15)
        n = -(-body.size // 15)
        body = np.resize(body, n * 15).reshape(n, 15)
        head = np.full((n, 1), int(np.float32(6.0 * S).view(np.uint32) >> 16), np.uint32)
        blocks.append(np.concatenate([head | (rng.integers(0, 2, (n, 1), dtype=np.uint32) << 15), body], axis=1))
    X = np.concatenate(blocks).astype(np.uint16)
    pad = (-X.shape[0]) % 64
    X = np.concatenate([X, np.zeros((pad, 16), np.uint16)]).reshape(-1, 1024)
    x = si.from_bits(X).cuda()
    one = torch.ones_like(x)
    h = bits(gpu.glu_fwd(one, x, act="relu2"))
    assert np.array_equal(h, X), "h = up"
    hf = si.from_bits(X).float().numpy()
    for name, code in SFL:
        q, sf = gpu.glu_fwd_nvfp4(one, x, act="relu2", layout="split", sf_layout=name)
        oq, osf = oracle.quant_nvfp4(hf, code)
        assert np.array_equal(u8(sf).ravel(), osf.ravel()), f"scales ({name})"
        assert np.array_equal(u8(q), oq), f"codes ({name})"
