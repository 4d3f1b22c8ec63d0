"""GPU parity of the merged gate/up GEMM with MXFP4 operands and with pairwise-interleaved W.

MXFP4 operands are E2M1 codes packed two per byte (element 2j in the low nibble of byte j)
with E8M0 scales per 32-element block along K: the closest form of the packed E2M1 values of
the NVFP4 page ("feat(phyai-kernel): add Thor NVFP4 GeGLU kernel for pi0.5", Supported
contract, values row) that gfx950's block-scaled matrix instruction takes.  Interleaved W
holds the rows gate0, up0, gate1, up1, ... (the same contract's weight layout row).

Accumulation (test_matrix_core_accumulation_model_e2m1 pins it through the library): the
products of each aligned 16-element K chunk are summed, and the chunk sums reach the FP32
accumulator one at a time with FP32 rounding.  A chunk lies inside one 32-element block, so
its products share both scales; E2M1 magnitudes span 0.5 .. 6, so they have at most 4
significant bits and span at most 2^8, and the chunk sum is exact.  Hence, elementwise,
    |Y - X W^T| <= (K / 16) * 2^-23 * sum_k |x_k w_k|.
Parity is taken in the same three steps as for MXFP8 operands (the GEMM within that bound,
the GLU by rule 2 against the device's own Y, the quantizers bit-exact against the device's
own h), plus end to end against the oracle's exact h, and bitwise equality of the interleaved
and the split W (the same rows give the same products in the same order).
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
from conftest import bits, u8
from parity import check_rule2
from test_gpu_gemm import ACTS, _bf16_spacing, _bf16_value, _carried_bound
from test_gpu_gemm import _accumulation_bound as accumulation_bound_e4m3

pytestmark = pytest.mark.gpu
ROUND = 2.0 ** -23      # one FP32 rounding of a partial sum, relative to sum |p|
CHUNK = 16              # K elements per exact chunk sum added into FP32
F4 = oracle.FMT_E2M1


def _operands(M, N, K, seed):
    xq, xs = si.mxfp4_operand(M, K, seed=seed)
    wq, ws = si.mxfp4_operand(2 * N, K, seed=seed + 1)
    return xq, xs, wq, ws


def _decoded(q, s):
    """Packed E2M1 rows with E8M0 scales -> float64 values (element 2j from the low nibble)."""
    q = np.asarray(q)
    codes = np.empty((q.shape[0], 2 * q.shape[1]), np.uint8)
    codes[:, 0::2], codes[:, 1::2] = q & 0xF, q >> 4
    v = oracle.e2m1_to_f64(codes).reshape(codes.shape)
    return v * np.repeat(np.exp2(np.asarray(s, np.float64) - 127.0), 32, axis=1)


def _accumulation_bound(xq, xs, wq, ws):
    K = 2 * np.asarray(xq).shape[1]
    return (K / CHUNK) * ROUND * (np.abs(_decoded(xq, xs)) @ np.abs(_decoded(wq, ws)).T)


def _pairs(w):
    """Interleaved W as a torch tensor from [W_gate | W_up] (rows 2j, 2j + 1 = gate j, up j)."""
    return si.interleave_rows(w)


def _deinterleave_cols(y):
    """Y in W's row order (interleaved) -> [Y_gate | Y_up]."""
    return np.concatenate([y[:, 0::2], y[:, 1::2]], axis=1)


def test_matrix_core_accumulation_model_e2m1(gpu):
    """Rows of X crafted against W = ones (so Y[m, j] = sum_k x_mk): blocks meet in FP32, not
    in a fixed-point window (rows 0, 2); a block's products reach the FP32 accumulator as
    sums of aligned 16-element chunks, one FP32 addition each: after 2^28 (ulp 32) a chunk of
    16 ones is half an ulp and is lost to the tie (row 1), after 2^27 (ulp 16) it is one ulp
    and is kept (row 6), which chunks of 8 (half an ulp there) would not be; the two
    128-element halves of a 256-element step add in FP32 (row 5); plain exact blocks (rows 3,
    4)."""
    M, N, K = 8, 128, 256
    codes = np.zeros((M, K), np.uint8)
    xs = np.full((M, K // 32), 127, np.uint8)
    codes[0, 0], xs[0, 0], codes[0, 32] = 0x2, 127 + 20, 0x2         # 2^20 + 1
    codes[1, 0], xs[1, 0] = 0x2, 127 + 28                             # 2^28, then 32 ones
    codes[1, 32:64] = 0x2
    codes[2, 0], xs[2, 0], codes[2, 32] = 0x2, 127 + 24, 0xA          # 2^24 - 1
    codes[3, :] = 0x7                                                 # 256 sixes
    codes[4, 0], codes[4, 1], codes[4, 2] = 0x7, 0x7, 0xF             # 6 + 6 - 6
    codes[5, 0], xs[5, 0], codes[5, 128] = 0x2, 127 + 24, 0xA         # across the halves
    codes[6, 0], xs[6, 0] = 0x2, 127 + 27                             # 2^27, then 32 ones
    codes[6, 32:64] = 0x2
    xq = codes[:, 0::2] | (codes[:, 1::2] << 4)
    wq = np.full((2 * N, K // 2), 0x22, np.uint8)
    ws = np.full((2 * N, K // 32), 127, np.uint8)
    dev = [torch.from_numpy(a).cuda() for a in (xq, xs, wq, ws)]
    y = gpu.mx_gemm_f32(*dev, fmt="mxfp4").cpu().numpy().astype(np.float64)
    want = [2.0 ** 20 + 1, 2.0 ** 28, 2.0 ** 24 - 1, 1536.0, 6.0, 2.0 ** 24 - 1, 2.0 ** 27 + 32, 0.0]
    assert np.all(y == np.array(want)[:, None]), y[:, 0]


@pytest.mark.parametrize("M,N,K", [(256, 128, 512), (200, 128, 256), (128, 256, 2048), (37, 128, 256),
                                   (300, 256, 1280), (1, 128, 256)])
def test_gemm_within_the_accumulation_bound(gpu, M, N, K):
    ops = _operands(M, N, K, seed=M + N + K)
    y = gpu.mx_gemm_f32(*(t.cuda() for t in ops), fmt="mxfp4").cpu().numpy().astype(np.float64)
    exact = oracle.mx_gemm_nt(*(t.numpy() for t in ops), fmt=F4)
    err = np.abs(y - exact)
    bound = _accumulation_bound(*(t.numpy() for t in ops))
    assert np.all(err <= bound), f"worst {float((err / np.maximum(bound, 1e-300)).max()):.3g} of the bound"


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
def test_interleaved_w_equals_split_w_bitwise(gpu, fmt):
    """The same W rows, interleaved or as [W_gate | W_up], give identical Y, h and quantized
    outputs (the kernel loads the same rows into the same places)."""
    M, N, K = 200, 256, 512
    gen = si.mxfp4_operand if fmt == "mxfp4" else si.mx_operand
    xq, xs = (t.cuda() for t in gen(M, K, seed=31))
    wq, ws = gen(2 * N, K, seed=32)
    split = (xq, xs, wq.cuda(), ws.cuda())
    paired = (xq, xs, _pairs(wq).cuda(), _pairs(ws).cuda())
    assert not torch.equal(paired[2], split[2])
    ys = gpu.mx_gemm_f32(*split, fmt=fmt)
    yp = gpu.mx_gemm_f32(*paired, fmt=fmt, w_layout="paired")
    assert torch.equal(ys.view(torch.int32), yp.view(torch.int32))
    for act in ("swiglu", "geglu"):
        assert torch.equal(gpu.glu_gemm(*split, act=act, fmt=fmt).view(torch.int16),
                           gpu.glu_gemm(*paired, act=act, fmt=fmt, w_layout="paired").view(torch.int16))
        for a, b in zip(gpu.glu_gemm_mxfp8(*split, act=act, fmt=fmt),
                        gpu.glu_gemm_mxfp8(*paired, act=act, fmt=fmt, w_layout="paired")):
            assert torch.equal(a, b)
        for a, b in zip(gpu.glu_gemm_nvfp4(*split, act=act, fmt=fmt, sf_layout="128x4"),
                        gpu.glu_gemm_nvfp4(*paired, act=act, fmt=fmt, w_layout="paired", sf_layout="128x4")):
            assert torch.equal(a, b)
    # and against the oracle's reading of the interleaved rows, within the accumulation bound
    ops_np = [t.cpu().numpy() for t in paired]
    if fmt == "mxfp4":
        exact, bound = oracle.mx_gemm_nt(*ops_np, fmt=F4), _accumulation_bound(*ops_np)
    else:
        exact, bound = oracle.mx_gemm_nt(*ops_np), accumulation_bound_e4m3(*ops_np)
    y = yp.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(y - _deinterleave_cols(exact)) <= _deinterleave_cols(bound))


@pytest.mark.parametrize("act,kind", ACTS)
def test_glu_epilogue_and_quantizers(gpu, act, kind):
    """MXFP4 operands, interleaved W: h by rule 2 against the GLU of the device's own Y, the
    MXFP8 and NVFP4 outputs bit-exact against the oracle quantizers of the device's own h."""
    M, N, K = 160, 128, 512
    xq, xs, wq, ws = _operands(M, N, K, seed=40 + kind)
    ops = [xq.cuda(), xs.cuda(), _pairs(wq).cuda(), _pairs(ws).cuda()]
    kw = dict(fmt="mxfp4", w_layout="paired")
    y = gpu.mx_gemm_f32(*ops, **kw).cpu().numpy().astype(np.float64)
    h = gpu.glu_gemm(*ops, act=act, **kw)
    check_rule2(bits(h), oracle.bf16_from_f64(oracle.act(kind, y[:, :N]) * y[:, N:]), f"{act} MXFP4 epilogue")
    hf = si.from_bits(bits(h)).float().numpy()
    q, sc = gpu.glu_gemm_mxfp8(*ops, act=act, **kw)
    o = oracle.quant_mxfp8(hf, oracle.ROWWISE)
    assert np.array_equal(u8(sc), o[1]) and np.array_equal(u8(q), o[0])
    for sfl, osfl in (("rowmajor", oracle.SF_ROWMAJOR), ("128x4", oracle.SF_128x4)):
        qn = torch.full((M, N // 2), 0xAB, dtype=torch.uint8, device="cuda")
        sn = torch.full((gpu.nvfp4_sf_bytes(M, N, sfl),), 0xAB, dtype=torch.uint8, device="cuda")
        gpu.glu_gemm_nvfp4(*ops, act=act, sf_layout=sfl, out=(qn, sn), **kw)
        on = oracle.quant_nvfp4(hf, osfl)
        assert np.array_equal(u8(qn), on[0]) and np.array_equal(u8(sn).ravel(), np.asarray(on[1]).ravel())
    amax = torch.tensor([float(np.abs(hf).max()) * 2.0], dtype=torch.float32, device="cuda")
    qg, sg = gpu.glu_gemm_nvfp4_gs(*ops, amax=amax, act=act, **kw)
    og = oracle.quant_nvfp4_gs(hf, float(amax.item()), oracle.SF_ROWMAJOR)
    assert np.array_equal(u8(qg), og[0]) and np.array_equal(u8(sg), og[1])


@pytest.mark.parametrize("act,kind", ACTS)
@pytest.mark.parametrize("K", [256, 2048])
def test_end_to_end_against_the_exact_oracle(gpu, act, kind, K):
    """The fused h against the oracle's h from the exact binary64 GEMM of the interleaved
    MXFP4 operands: |h_device - h_oracle| <= D + 2 ulp elementwise, D the accumulation bound
    carried through the GLU (as for MXFP8 operands); most elements identical."""
    M, N = 128, 128
    xq, xs, wq, ws = _operands(M, N, K, seed=50 + K + kind)
    wp, wps = _pairs(wq), _pairs(ws)
    h = bits(gpu.glu_gemm(xq.cuda(), xs.cuda(), wp.cuda(), wps.cuda(), act=act, fmt="mxfp4", w_layout="paired"))
    ops_np = [xq.numpy(), xs.numpy(), wp.numpy(), wps.numpy()]
    ho = oracle.glu_gemm(kind, *ops_np, fmt=F4, w_layout=oracle.PAIRED)
    y = _deinterleave_cols(oracle.mx_gemm_nt(*ops_np, fmt=F4))
    B = _deinterleave_cols(_accumulation_bound(*ops_np))
    D = _carried_bound(kind, y[:, :N], y[:, N:], B[:, :N], B[:, N:])
    hd, hv = _bf16_value(h), _bf16_value(ho)
    ulp = _bf16_spacing(np.maximum(np.abs(hd), np.abs(hv)))
    err = np.abs(hd - hv)
    assert np.all(err <= D + 2 * ulp), f"worst {float(((err - 2 * ulp) / np.maximum(D, 1e-300)).max()):.3g} of the bound"
    assert float((h == ho).mean()) > 0.5


def test_nan_scales(gpu):
    """E2M1 has no NaN code; the E8M0 NaN scale 0xFF poisons its row of X (a row of Y) or its
    row of W (a gate or up column), as the oracle reads the format."""
    M, N, K = 64, 128, 256
    xq, xs, wq, ws = _operands(M, N, K, seed=93)
    xs[7, 2] = 0xFF
    ws[2 * 11, 1] = 0xFF          # interleaved: gate column 11
    ws[2 * 40 + 1, 0] = 0xFF      # up column 40
    ops = (xq, xs, wq, ws)
    y = gpu.mx_gemm_f32(*(t.cuda() for t in ops), fmt="mxfp4", w_layout="paired").cpu().numpy()
    exact = _deinterleave_cols(oracle.mx_gemm_nt(*(t.numpy() for t in ops), fmt=F4))
    assert np.array_equal(np.isnan(y), np.isnan(exact))
    assert np.isnan(exact[7]).all() and np.isnan(exact[:, [11, N + 40]]).all()


def test_nvfp4_page_contract_shape(gpu):
    """The NVFP4 page's contract shape: M = 968 tokens, K = 2048, merged 2N = 32768 (H =
    16384), interleaved W, GeGLU, NVFP4 output with global scale 1 in the 128x4 layout; here
    with MXFP4 operands.  Every NVFP4 code and scale byte (padding rows included) against the
    oracle quantizer of the device's own h; sampled rows of Y within the accumulation bound
    and of h by rule 2."""
    M, N, K = 968, 16384, 2048
    xq, xs, wq, ws = _operands(M, N, K, seed=9)
    wp, wps = _pairs(wq), _pairs(ws)
    dev = [xq.cuda(), xs.cuda(), wp.cuda(), wps.cuda()]
    kw = dict(fmt="mxfp4", w_layout="paired")
    q, sf = gpu.glu_gemm_nvfp4(*dev, act="geglu", sf_layout="128x4", **kw)
    h = bits(gpu.glu_gemm(*dev, act="geglu", **kw))
    rows = np.unique(np.r_[0, 1, 255, 256, M - 1, np.linspace(0, M - 1, 9).astype(int)])
    y = gpu.mx_gemm_f32(*dev, **kw).index_select(0, torch.as_tensor(rows, device="cuda")).cpu().numpy()
    torch.cuda.synchronize()
    on = oracle.quant_nvfp4(si.from_bits(h).float().numpy(), oracle.SF_128x4)
    assert np.array_equal(u8(q), on[0])
    assert np.array_equal(u8(sf).ravel(), np.asarray(on[1]).ravel())
    y = y.astype(np.float64)
    exact = _deinterleave_cols(oracle.mx_gemm_nt(xq.numpy()[rows], xs.numpy()[rows], wp.numpy(), wps.numpy(), fmt=F4))
    bound = _deinterleave_cols(_accumulation_bound(xq.numpy()[rows], xs.numpy()[rows], wp.numpy(), wps.numpy()))
    assert np.all(np.abs(y - exact) <= bound)
    check_rule2(h[rows], oracle.bf16_from_f64(oracle.act(oracle.GEGLU_TANH, y[:, :N]) * y[:, N:]),
                "contract-shape epilogue")
