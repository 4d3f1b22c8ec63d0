"""GPU parity of the merged gate/up MXFP8 GEMM with the GLU epilogue.

The matrix cores do not form Y = X W^T as IEEE FP32 sums.  The products of each aligned
8-element K chunk are added in a fixed-point window 14 bits wide, anchored at the chunk's
largest product (a product 2^-14 of it or smaller is dropped, whatever its sign), and the
chunk sums are added one at a time into the FP32 accumulator with FP32 rounding
(test_matrix_core_accumulation_model pins this through the library).  Hence, elementwise,
    |Y - X W^T| <= sum_chunks 8 * 2^-13 * max_chunk |x_k w_k|  +  (K / 8) * 2^-23 * sum_k |x_k w_k|
(each of a chunk's at most 7 other products loses less than 2^-13 of the largest; at most K/8
FP32 additions, each off by at most one FP32 ulp of a partial sum no larger than sum |p|).
Parity is taken in three steps:
  * the GEMM (test hook glu_mx_gemm_f32) against the oracle's exact binary64 GEMM, within
    that bound;
  * the GLU epilogue (glu_gemm) against the oracle's GLU of the device's own Y (rule 2,
    within 1 BF16 ulp);
  * the quantizing epilogues (glu_gemm_mxfp8, glu_gemm_nvfp4) against the oracle quantizers
    of the device's own h (rule 1, bit-exact).
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
from conftest import bits, u8
from parity import check_rule2

pytestmark = pytest.mark.gpu
WINDOW = 2.0 ** -13     # a chunk product's loss, relative to the chunk's largest product
ROUND = 2.0 ** -23      # one FP32 rounding of a partial sum, relative to sum |p|
ACTS = [("swiglu", oracle.SWIGLU), ("geglu", oracle.GEGLU_TANH), ("geglu_erf", oracle.GEGLU_ERF),
        ("relu2", oracle.RELU2)]


def _operands(M, N, K, seed):
    xq, xs = si.mx_operand(M, K, seed=seed)
    wq, ws = si.mx_operand(2 * N, K, seed=seed + 1)
    return xq, xs, wq, ws


_E4M3 = oracle.e4m3_to_f64(np.arange(256, dtype=np.uint8))   # the oracle's value of every code


@pytest.mark.parametrize("M,N,K", [(256, 128, 512), (200, 128, 256), (128, 256, 2048), (37, 128, 128),
                                   (96, 384, 384), (64, 128, 640), (300, 256, 1152), (1, 128, 128),
                                   (1, 256, 384)])
def test_gemm_within_the_accumulation_bound(gpu, M, N, K):
    ops = _operands(M, N, K, seed=M + N + K)
    y = gpu.mx_gemm_f32(*(t.cuda() for t in ops)).cpu().numpy().astype(np.float64)
    exact = oracle.mx_gemm_nt(*(t.numpy() for t in ops))
    err = np.abs(y - exact)
    bound = _accumulation_bound(*(t.numpy() for t in ops))
    assert np.all(err <= bound), f"worst {float((err / bound).max()):.3g} of the bound"


def _accumulation_bound(xq, xs, wq, ws):
    """The elementwise bound above, from the codes and scales of X [M, K] and W [2N, K]
    (dequantized one 8-element K chunk at a time)."""
    xq, xs, wq, ws = (np.asarray(t) for t in (xq, xs, wq, ws))
    K = xq.shape[1]
    xsc, wsc = np.exp2(xs.astype(np.float64) - 127.0), np.exp2(ws.astype(np.float64) - 127.0)
    chunk_max = np.zeros((xq.shape[0], wq.shape[0]))
    total = np.zeros_like(chunk_max)
    for c in range(0, K, 8):
        ax = np.abs(_E4M3[xq[:, c:c + 8]]) * xsc[:, c // 32, None]   # [M, 8]
        aw = np.abs(_E4M3[wq[:, c:c + 8]]) * wsc[:, c // 32, None]   # [2N, 8]
        m = np.outer(ax[:, 0], aw[:, 0])
        for k in range(1, 8):
            np.maximum(m, np.outer(ax[:, k], aw[:, k]), out=m)
        chunk_max += m
        total += ax @ aw.T
    return 8 * WINDOW * chunk_max + (K / 8) * ROUND * total


def _e4m3_code(v):
    """E4M3 code of a value the format holds exactly (the test's crafted operands)."""
    code = torch.tensor([v], dtype=torch.float32).to(torch.float8_e4m3fn)
    assert float(code.float()) == v
    return int(code.view(torch.uint8))


def test_matrix_core_accumulation_model(gpu):
    """Rows of X crafted against W = ones (so Y[m, j] = sum_k x_mk): the fixed-point chunk
    window, its independence across chunks, and FP32 accumulation of the chunk sums."""
    M, N, K = 8, 128, 128
    xq = torch.zeros((M, K), dtype=torch.uint8)
    xs = torch.full((M, K // 32), 127, dtype=torch.uint8)
    put = lambda m, k, v: xq.__setitem__((m, k), _e4m3_code(v))
    put(0, 0, 256.0); put(0, 1, 2.0 ** -5)            # 2^-13 of the largest: kept
    put(1, 0, 256.0); put(1, 1, 2.0 ** -6)            # 2^-14: dropped
    put(2, 0, 256.0); put(2, 7, -2.0 ** -6)           # dropped, not rounded down
    put(3, 0, 256.0); put(3, 8, -2.0 ** -9)           # next chunk: exact
    put(4, 0, 1.0); xs[4, 0] = 127 + 24; put(4, 32, -1.0)   # FP32 accumulation: 2^24 - 1 exact
    put(5, 0, 1.0); xs[5, 0] = 127 + 28                 # 2^28 plus 12 chunks of 8 ones:
    for k in range(32, 128):                             # each chunk sum 8 is below half an
        put(5, k, 1.0)                                   # FP32 ulp of 2^28 and is lost
    put(6, 3, 448.0); put(6, 4, 448.0); put(6, 5, -448.0)   # a plain exact chunk
    wq = torch.full((2 * N, K), _e4m3_code(1.0), dtype=torch.uint8)
    ws = torch.full((2 * N, K // 32), 127, dtype=torch.uint8)
    y = gpu.mx_gemm_f32(xq.cuda(), xs.cuda(), wq.cuda(), ws.cuda()).cpu().numpy().astype(np.float64)
    want = [256.0 + 2.0 ** -5, 256.0, 256.0, 256.0 - 2.0 ** -9, 2.0 ** 24 - 1, 2.0 ** 28, 448.0, 0.0]
    assert np.all(y == np.array(want)[:, None]), y[:, 0]


@pytest.mark.parametrize("act,kind", ACTS)
def test_glu_epilogue_and_quantizer(gpu, act, kind):
    M, N, K = 160, 128, 384
    ops = [t.cuda() for t in _operands(M, N, K, seed=70 + kind)]
    y = gpu.mx_gemm_f32(*ops).cpu().numpy().astype(np.float64)   # exact FP32 values
    h = gpu.glu_gemm(*ops, act=act)
    want = oracle.bf16_from_f64(oracle.act(kind, y[:, :N]) * y[:, N:])
    check_rule2(bits(h), want, f"{act} epilogue")
    q, sc = gpu.glu_gemm_mxfp8(*ops, act=act)
    o = oracle.quant_mxfp8(si.from_bits(bits(h)).float().numpy(), oracle.ROWWISE)
    assert np.array_equal(u8(sc), o[1]) and np.array_equal(u8(q), o[0])


def _tail_operands(act, M, N, K, seed):
    """Operands whose exact Y puts the gate half across the activation's switch to the FP64
    tail path.  X is all E4M3 1.0 (code 0x38, scale 2^0), so Y[i, j] = K * v_j * 2^e_j for a
    gate row j holding one code v_j with scale byte 127 + e_j:
      * SwiGLU: v in -[0.5, 1) (codes 0xB0..0xB7), e = 0 at K = 128: Y in -[64, 120];
      * GeGLU (tanh, erf): the same codes with e = -3: Y in -[8, 15];
      * ReLU^2: v in [0.5, 1) with e = 60 (Y^2 above the FP32 range) or e = -70 (Y^2 below
        it), every fourth row negated, and up rows scaled by 2^-20 or 2^60 so that h stays in
        range.
    Up rows: random E4M3 codes N(0, 1) * 64 with scale bytes 118..122."""
    g = torch.Generator().manual_seed(seed)
    xq = torch.full((M, K), 0x38, dtype=torch.uint8)
    xs = torch.full((M, K // 32), 127, dtype=torch.uint8)
    wq, ws = si.mx_operand(2 * N, K, seed=seed + 1)
    code = torch.randint(0, 8, (N,), generator=g, dtype=torch.uint8)
    if act == "relu2":
        big = torch.arange(N) % 2 == 0
        gate_code = 0x30 + code
        gate_code = torch.where(torch.arange(N) % 4 == 3, gate_code | 0x80, gate_code)
        gate_scale = torch.where(big, torch.tensor(127 + 60), torch.tensor(127 - 70)).to(torch.uint8)
        up_scale = torch.where(big, torch.tensor(127 - 20), torch.tensor(127 + 60)).to(torch.uint8)
        ws[N:] = up_scale[:, None]
    else:
        gate_code = 0xB0 + code
        gate_scale = torch.full((N,), 127 if act == "swiglu" else 124, dtype=torch.uint8)
    wq[:N] = gate_code[:, None]
    ws[:N] = gate_scale[:, None]
    return xq, xs, wq, ws


@pytest.mark.parametrize("act,kind", ACTS)
def test_epilogue_tail_paths(gpu, act, kind):
    """The epilogue's FP64 tail path: h within 1 BF16 ulp of the oracle's GLU of the device's
    own Y (rule 2), and the MXFP8 and NVFP4 codes equal to the oracle quantizers of the device's
    own h (rule 1)."""
    M, N, K = 64, 128, 128
    ops = [t.cuda() for t in _tail_operands(act, M, N, K, seed=300 + kind)]
    y = gpu.mx_gemm_f32(*ops).cpu().numpy().astype(np.float64)
    gate = y[:, :N]
    if act == "swiglu":
        assert (gate < -86.7).any() and (gate > -86.5).any(), "the gates straddle the switch"
    h = gpu.glu_gemm(*ops, act=act)
    want = oracle.bf16_from_f64(oracle.act(kind, gate) * y[:, N:])
    check_rule2(bits(h), want, f"{act} tail epilogue")
    hf = si.from_bits(bits(h)).float().numpy()
    q, sc = gpu.glu_gemm_mxfp8(*ops, act=act)
    o = oracle.quant_mxfp8(hf, oracle.ROWWISE)
    assert np.array_equal(u8(sc), o[1]) and np.array_equal(u8(q), o[0])
    q, sf = gpu.glu_gemm_nvfp4(*ops, act=act, sf_layout="128x4")
    o = oracle.quant_nvfp4(hf, oracle.SF_128x4)
    assert np.array_equal(u8(q), o[0]) and np.array_equal(u8(sf).ravel(), np.asarray(o[1]).ravel())


@pytest.mark.parametrize("act,kind", ACTS)
@pytest.mark.parametrize("M", [160, 300])
@pytest.mark.parametrize("sf_layout", ["rowmajor", "128x4"])
def test_nvfp4_epilogue(gpu, act, kind, M, sf_layout):
    """NVFP4 (global scale 1) of the device's own h, bit-exact; 128x4 padding rows are zero
    (the outputs start as 0xAB so that a missing write shows)."""
    N, K = 256, 256
    ops = [t.cuda() for t in _operands(M, N, K, seed=100 + M + kind)]
    h = bits(gpu.glu_gemm(*ops, act=act))
    sfl = oracle.SF_128x4 if sf_layout == "128x4" else oracle.SF_ROWMAJOR
    o = oracle.quant_nvfp4(si.from_bits(h).float().numpy(), sfl)
    q = torch.full((M, N // 2), 0xAB, dtype=torch.uint8, device="cuda")
    sf = torch.full((gpu.nvfp4_sf_bytes(M, N, sf_layout),), 0xAB, dtype=torch.uint8, device="cuda")
    gpu.glu_gemm_nvfp4(*ops, act=act, sf_layout=sf_layout, out=(q, sf))
    assert np.array_equal(u8(q), o[0])
    assert np.array_equal(u8(sf).ravel(), np.asarray(o[1]).ravel())


@pytest.mark.parametrize("sf_layout", ["rowmajor", "128x4"])
def test_two_level_nvfp4_epilogue(gpu, sf_layout):
    """Two-level NVFP4 of the device's own h, bit-exact against the oracle's, for amax values
    chosen as a delayed-scaling caller would pass them (the amax of h itself, an older and
    larger one, a smaller one that saturates blocks) and for the degenerate ones (zero,
    negative, infinite: global scale 1; tiny: the 2^100 cap)."""
    M, N, K = 160, 256, 256
    ops = [t.cuda() for t in _operands(M, N, K, seed=110)]
    h = bits(gpu.glu_gemm(*ops, act="geglu"))
    hf = si.from_bits(h).float().numpy()
    sfl = oracle.SF_128x4 if sf_layout == "128x4" else oracle.SF_ROWMAJOR
    top = float(np.abs(hf).max())
    for amax in (top, 3.0 * top, top / 16, 0.0, -1.0, float("inf"), 1e-35):
        a = torch.tensor([amax], dtype=torch.float32, device="cuda")
        q, sf = gpu.glu_gemm_nvfp4_gs(*ops, amax=a, act="geglu", sf_layout=sf_layout)
        o = oracle.quant_nvfp4_gs(hf, np.float32(amax), sfl)
        assert np.array_equal(u8(q), o[0]), amax
        assert np.array_equal(u8(sf).ravel(), np.asarray(o[1]).ravel()), amax


def test_gemm_deterministic_and_row_batch_invariant(gpu):
    M, N, K = 256, 128, 256
    xq, xs, wq, ws = (t.cuda() for t in _operands(M, N, K, seed=80))
    a = gpu.glu_gemm(xq, xs, wq, ws)
    b = gpu.glu_gemm(xq, xs, wq, ws)
    c = gpu.glu_gemm(xq[100:200].contiguous(), xs[100:200].contiguous(), wq, ws)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(a[100:200].view(torch.int16), c.view(torch.int16))


def test_gemm_zero_rows(gpu):
    """M = 0 is a valid empty product: every entry point returns empty outputs and leaves the
    caller's buffers untouched."""
    N, K = 128, 256
    _, _, wq, ws = (t.cuda() for t in _operands(4, N, K, seed=82))
    xq = torch.empty((0, K), dtype=torch.uint8, device="cuda")
    xs = torch.empty((0, K // 32), dtype=torch.uint8, device="cuda")
    assert gpu.glu_gemm(xq, xs, wq, ws).shape == (0, N)
    q, s = gpu.glu_gemm_mxfp8(xq, xs, wq, ws)
    assert q.shape == (0, N) and s.shape == (0, N // 32)
    q, s = gpu.glu_gemm_nvfp4(xq, xs, wq, ws, sf_layout="rowmajor")
    assert q.shape == (0, N // 2) and s.numel() == 0
    torch.cuda.synchronize()


# Largest |act'(x)| over the reals for the three smooth activations (SiLU: 1.0998 at x = 2.40;
# both GELUs: 1.1289 at x = 1.42 for the exact one, 1.1290 for the tanh form), rounded up.
_SLOPE = {oracle.SWIGLU: 1.10, oracle.GEGLU_TANH: 1.13, oracle.GEGLU_ERF: 1.13}


def _carried_bound(kind, y_gate, y_up, b_gate, b_up):
    """Elementwise bound on |act(Yg') Yu' - act(Yg) Yu| when |Yg' - Yg| <= b_gate and
    |Yu' - Yu| <= b_up:  L b_gate (|Yu| + b_up) + |act(Yg)| b_up, with L the largest |act'| on
    [Yg - b_gate, Yg + b_gate] (a global constant for the smooth activations; 2 (|Yg| + b_gate)
    for ReLU^2, whose derivative is 2 max(x, 0))."""
    L = 2.0 * (np.abs(y_gate) + b_gate) if kind == oracle.RELU2 else _SLOPE[kind]
    return L * b_gate * (np.abs(y_up) + b_up) + np.abs(oracle.act(kind, y_gate)) * b_up


@pytest.mark.parametrize("act,kind", ACTS)
@pytest.mark.parametrize("K", [128, 1024, 2048])
def test_gemm_end_to_end_against_the_exact_oracle(gpu, act, kind, K):
    """The fused h against the oracle's exact h (binary64 GEMM, one rounding), element by
    element.  With Y' the device's FP32 GEMM and Y the exact one, |Y' - Y| <= B (the
    accumulation bound above), carried through the GLU as D (_carried_bound).  The device h is
    within one BF16 ulp (rule 2) of bf16(act(Yg') Yu'), i.e. within 1.5 ulp of act(Yg') Yu';
    the oracle's h is within half an ulp of act(Yg) Yu.  So
        |h_device - h_oracle| <= D + 2 ulp(max(|h_device|, |h_oracle|)),
    asserted for every element; most elements are also identical."""
    M, N = 128, 128
    ops = _operands(M, N, K, seed=81 + K + kind)
    h = bits(gpu.glu_gemm(*(t.cuda() for t in ops), act=act))
    ops_np = [t.numpy() for t in ops]
    ho = oracle.glu_gemm(kind, *ops_np)
    y = oracle.mx_gemm_nt(*ops_np)
    B = _accumulation_bound(*ops_np)
    D = _carried_bound(kind, y[:, :N], y[:, N:], B[:, :N], B[:, N:])
    hd, hv = _bf16_value(h), _bf16_value(ho)
    ulp = _bf16_spacing(np.maximum(np.abs(hd), np.abs(hv)))
    err = np.abs(hd - hv)
    assert np.all(err <= D + 2 * ulp), f"worst {float(((err - 2 * ulp) / np.maximum(D, 1e-300)).max()):.3g} of the bound"
    same = float((h == ho).mean())
    assert same > 0.5, f"only {same:.3f} of h identical to the exact oracle"


def _bf16_value(b):
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _bf16_spacing(a):
    """Spacing of BF16 numbers at magnitude a (2^-133 below the normal range)."""
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return np.exp2(e - 7)


@pytest.mark.parametrize("act,kind", [ACTS[0], ACTS[2]])
def test_nan_codes_and_scales(gpu, act, kind):
    """The MX encodings' NaNs (E4M3 codes 0x7F and 0xFF, E8M0 scale byte 0xFF) make every
    product they enter NaN, as the oracle reads the formats: a NaN in X poisons a row of Y,
    a NaN in W a column.  h is NaN wherever its gate or up value is, and its MXFP8 blocks
    holding NaN get scale 0xFF and NaN codes."""
    M, N, K = 64, 128, 256
    xq, xs, wq, ws = _operands(M, N, K, seed=90)
    xq[3, 5] = 0x7F          # NaN code: row 3
    xs[7, 2] = 0xFF          # NaN scale of K block 2: row 7
    wq[11, 200] = 0xFF       # NaN code (sign set): gate column 11
    ws[N + 40, 1] = 0xFF     # NaN scale: up column 40
    ops = (xq, xs, wq, ws)
    dev = [t.cuda() for t in ops]
    y = gpu.mx_gemm_f32(*dev).cpu().numpy().astype(np.float64)
    exact = oracle.mx_gemm_nt(*(t.numpy() for t in ops))
    assert np.array_equal(np.isnan(y), np.isnan(exact))
    assert np.isnan(exact[[3, 7]]).all() and np.isnan(exact[:, [11, N + 40]]).all()
    assert np.isnan(exact).sum() == 2 * 2 * N + 2 * M - 4
    h = bits(gpu.glu_gemm(*dev, act=act))
    check_rule2(h, oracle.bf16_from_f64(oracle.act(kind, y[:, :N]) * y[:, N:]), f"{act} NaN epilogue")
    q, sc = gpu.glu_gemm_mxfp8(*dev, act=act)
    o = oracle.quant_mxfp8(si.from_bits(h).float().numpy(), oracle.ROWWISE)
    assert np.array_equal(u8(sc), o[1]) and np.array_equal(u8(q), o[0])
    assert (u8(sc)[[3, 7]] == 0xFF).all() and (u8(sc)[:, [0, 1]] == 0xFF).all()
    qn, sn = gpu.glu_gemm_nvfp4(*dev, act=act)
    on = oracle.quant_nvfp4(si.from_bits(h).float().numpy(), oracle.SF_ROWMAJOR)
    assert np.array_equal(u8(qn), on[0]) and np.array_equal(u8(sn), on[1])
    assert (u8(sn)[[3, 7]] == 0x7F).all() and (u8(sn)[:, [0, 2]] == 0x7F).all()


@pytest.mark.parametrize("M,N,K", [(968, 16384, 2048), (16384, 7168, 2048)])
def test_full_size_sampled_rows(gpu, M, N, K):
    """The bench's GEMM shapes, launched whole as the bench launches them; a sample of rows
    (first, last, and spread between) is checked in the three parity steps: the FP32 GEMM
    within the accumulation bound of the exact one, h by rule 2 against the GLU of the
    device's Y, and the MXFP8 and NVFP4 outputs bit-exact against the oracle quantizers of
    the device's h."""
    xq, xs, wq, ws = _operands(M, N, K, seed=7)
    dev = [t.cuda() for t in (xq, xs, wq, ws)]
    rows = np.unique(np.r_[0, 1, 255, 256, M - 1, np.linspace(0, M - 1, 11).astype(int)])
    ridx = torch.as_tensor(rows, device="cuda")
    y = gpu.mx_gemm_f32(*dev).index_select(0, ridx).cpu().numpy().astype(np.float64)
    h = bits(gpu.glu_gemm(*dev, act="swiglu").index_select(0, ridx))
    qm, sm = (t.index_select(0, ridx) for t in gpu.glu_gemm_mxfp8(*dev, act="swiglu"))
    qn, sn = (t.index_select(0, ridx) for t in gpu.glu_gemm_nvfp4(*dev, act="swiglu"))
    torch.cuda.synchronize()
    x_r, xs_r = xq[rows], xs[rows]
    exact = oracle.mx_gemm_nt(x_r.numpy(), xs_r.numpy(), wq.numpy(), ws.numpy())
    bound = _accumulation_bound(x_r.numpy(), xs_r.numpy(), wq.numpy(), ws.numpy())
    assert np.all(np.abs(y - exact) <= bound)
    check_rule2(h, oracle.bf16_from_f64(oracle.act(oracle.SWIGLU, y[:, :N]) * y[:, N:]), "full-size epilogue")
    hf = si.from_bits(h).float().numpy()
    om = oracle.quant_mxfp8(hf, oracle.ROWWISE)
    assert np.array_equal(u8(qm), om[0]) and np.array_equal(u8(sm), om[1])
    on = oracle.quant_nvfp4(hf, oracle.SF_ROWMAJOR)
    assert np.array_equal(u8(qn), on[0]) and np.array_equal(u8(sn), on[1])
