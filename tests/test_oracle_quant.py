"""Pins for the oracle's MXFP8 and NVFP4 quantizers (CPU only).

References independent of the oracle's own code: hand-worked blocks under tests/golden/,
brute-force nearest searches with exact rationals over every code of the target format,
the transpose identity colwise(X) = rowwise(X^T), and the 128x4 scale layout checked as a
zero-padded permutation with hand-placed entries.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synthetic_inputs as si
from conftest import parse_golden
from test_oracle_formats import E2M1, E4M3, _brute_e2m1, _brute_e4m3, _brute_rceil


def _block_rows(name):
    out = []
    for row in parse_golden(name):
        cols = [c.strip() for c in row.split("|")]
        lead = [float.fromhex(v) for v in cols[1].split(",")]
        fill = float(cols[4]) if cols[4] != "-0" else -0.0
        out.append((cols[0], lead, int(cols[2], 16), [int(c, 16) for c in cols[3].split(",")], fill))
    return out


def test_mx_golden_blocks_rowwise_and_colwise():
    for name, lead, scale, codes, fill in _block_rows("mx_block_hand.txt"):
        blk = np.full(32, fill, np.float32)
        blk[: len(lead)] = lead
        q, s, _, _ = oracle.quant_mxfp8(blk.reshape(1, 32), oracle.ROWWISE)
        rest = 0x80 if np.signbit(fill) else 0x00
        want = codes + [rest] * (32 - len(codes))
        assert int(s[0, 0]) == scale, name
        assert list(q[0]) == want, name
        # the same block standing as a column of a [32, 3] matrix
        X = np.zeros((32, 3), np.float32)
        X[:, 1] = blk
        _, _, qc, sc = oracle.quant_mxfp8(X, oracle.COLWISE)
        assert int(sc[1, 0]) == scale and list(qc[1]) == want, name


def test_nv_golden_blocks():
    for name, lead, scale, packed, fill in _block_rows("nv_block_hand.txt"):
        blk = np.full(16, fill, np.float32)
        blk[: len(lead)] = lead
        q, sf = oracle.quant_nvfp4(blk.reshape(1, 16))
        assert int(sf[0, 0]) == scale, name
        assert list(q[0][: len(packed)]) == packed, name
        assert not np.any(q[0][len(packed):]), name


def _random_matrix(M, N, seed):
    rng = np.random.default_rng(seed)
    X = rng.normal(0, 1, (M, N))
    X[rng.random((M, N)) < 0.01] *= 1000
    X[rng.random((M, N)) < 0.01] *= 1e-30
    X[:, :32][0] = 0.0  # one all-zero block
    X[1, 32:64] = -0.0
    return X.astype(np.float32)


def test_mx_rowwise_brute_force():
    X = _random_matrix(6, 96, 20)
    q, s, _, _ = oracle.quant_mxfp8(X, oracle.ROWWISE)
    for m in range(X.shape[0]):
        for b in range(X.shape[1] // 32):
            blk = X[m, 32 * b: 32 * b + 32]
            e = _brute_rceil(float(np.max(np.abs(blk))))
            assert int(s[m, b]) == e + 127
            for i, x in enumerate(blk):
                assert int(q[m, 32 * b + i]) == _brute_e4m3(float(x) * 2.0 ** -e)


def test_mx_colwise_is_rowwise_of_transpose():
    X = _random_matrix(64, 96, 21)
    qr, sr, qc, sc = oracle.quant_mxfp8(X, oracle.ROWWISE | oracle.COLWISE)
    tq, ts, _, _ = oracle.quant_mxfp8(np.ascontiguousarray(X.T), oracle.ROWWISE)
    assert np.array_equal(qc, tq) and np.array_equal(sc, ts)
    # "both" equals the two single-direction runs
    q1, s1, _, _ = oracle.quant_mxfp8(X, oracle.ROWWISE)
    _, _, q2, s2 = oracle.quant_mxfp8(X, oracle.COLWISE)
    assert np.array_equal(qr, q1) and np.array_equal(sr, s1)
    assert np.array_equal(qc, q2) and np.array_equal(sc, s2)


def test_mx_dequant_error_bound():
    """Every element dequantizes to within half an E4M3 step at the block scale (the
    code is the nearest value) and no scaled value exceeds 448."""
    X = _random_matrix(32, 256, 22)
    q, s, _, _ = oracle.quant_mxfp8(X, oracle.ROWWISE)
    dec = oracle.e4m3_to_f64(q) * np.exp2(np.repeat(s.astype(np.int64) - 127, 32, axis=1))
    scaled = np.abs(X.astype(np.float64)) * np.exp2(-(np.repeat(s.astype(np.int64) - 127, 32, axis=1)))
    assert np.all(scaled <= 448)
    err = np.abs(dec - X) * np.exp2(-(np.repeat(s.astype(np.int64) - 127, 32, axis=1)))
    step = np.where(scaled < 2.0 ** -6, 2.0 ** -9, np.exp2(np.floor(np.log2(np.maximum(scaled, 2.0 ** -6)))) / 8)
    assert np.all(err <= step / 2 + 1e-30)


def test_mx_nonfinite_block_reading():
    """Reading (parity unpinned): a block with NaN or Inf gets scale 0xFF and codes 0x7F;
    other blocks of the same row are unaffected."""
    X = np.ones((1, 96), np.float32)
    X[0, 5] = np.inf
    X[0, 40] = np.nan
    q, s, _, _ = oracle.quant_mxfp8(X, oracle.ROWWISE)
    assert list(s[0]) == [0xFF, 0xFF, 119]
    assert np.all(q[0, :64] == 0x7F) and np.all(q[0, 64:] == 0x78)  # 1.0 * 2^8 = 256


def test_nv_brute_force():
    X = _random_matrix(4, 64, 23)
    X[2, 16:32] = np.linspace(-7, 7, 16)
    q, sf = oracle.quant_nvfp4(X)
    for m in range(X.shape[0]):
        for b in range(X.shape[1] // 16):
            blk = X[m, 16 * b: 16 * b + 16]
            amax = Fraction(float(np.max(np.abs(blk))))
            sc = min(range(0x7F), key=lambda c: (abs(E4M3[c] - amax / 6), c % 2)) if amax / 6 < 448 else 0x7E
            assert int(sf[m, b]) == sc
            S = E4M3[sc]
            for i, x in enumerate(blk):
                nib = (int(q[m, 8 * b + i // 2]) >> (4 * (i % 2))) & 0xF
                if S == 0:
                    want = 0x8 if np.signbit(x) else 0
                else:
                    a = Fraction(float(abs(x))) / S
                    want = (0x8 if np.signbit(x) else 0) | (7 if a >= 6 else min(range(8), key=lambda c: (abs(E2M1[c] - a), c % 2)))
                assert nib == want, (m, b, i, float(x))


def test_nv_nonfinite_block_reading():
    X = np.ones((1, 32), np.float32)
    X[0, 3] = -np.inf
    q, sf = oracle.quant_nvfp4(X)
    assert int(sf[0, 0]) == 0x7F and not np.any(q[0, :8])
    # amax 1: 1/6 = 0.1667 lies between E4M3 0.15625 (0x22) and 0.171875 (0x23), nearer 0x23
    assert int(sf[0, 1]) == 0x23


def test_sf128x4_layout_is_zero_padded_permutation():
    for M, H in [(784, 16384), (968, 1024), (130, 80), (1, 16)]:
        nb = H // 16
        cp = (nb + 3) // 4 * 4
        rp = (M + 127) // 128 * 128
        offs = np.array([[oracle.sf128x4_offset(r, c, cp) for c in range(nb)] for r in range(min(M, 260))])
        assert len(set(offs.ravel().tolist())) == offs.size
        assert offs.min() >= 0 and offs.max() < rp * cp
    # hand-placed entries: 16 bytes per row within a 32-row group, 4 bytes per 32-row group,
    # 512 bytes per 128-row x 4-column tile, tiles of one row band laid out along columns.
    cp = 1024
    assert oracle.sf128x4_offset(0, 0, cp) == 0
    assert oracle.sf128x4_offset(0, 1, cp) == 1
    assert oracle.sf128x4_offset(0, 4, cp) == 512
    assert oracle.sf128x4_offset(1, 0, cp) == 16
    assert oracle.sf128x4_offset(32, 0, cp) == 4
    assert oracle.sf128x4_offset(96, 3, cp) == 15
    assert oracle.sf128x4_offset(31, 0, cp) == 496
    assert oracle.sf128x4_offset(128, 0, cp) == (cp // 4) * 512


def test_nv_128x4_equals_rowmajor_after_unswizzle():
    X = _random_matrix(200, 128, 24)
    q1, s1 = oracle.quant_nvfp4(X, oracle.SF_ROWMAJOR)
    q2, s2 = oracle.quant_nvfp4(X, oracle.SF_128x4)
    assert np.array_equal(q1, q2)
    nb, cp = 8, 8
    seen = np.zeros(s2.size, bool)
    for r in range(200):
        for c in range(nb):
            o = oracle.sf128x4_offset(r, c, cp)
            assert s2[o] == s1[r, c]
            seen[o] = True
    assert not np.any(s2[~seen])


def _unswizzle_check(s_swz, s_rm):
    rows, nb = s_rm.shape
    cp = (nb + 3) // 4 * 4
    assert s_swz.size == (rows + 127) // 128 * 128 * cp
    seen = np.zeros(s_swz.size, bool)
    for r in range(rows):
        for c in range(nb):
            o = oracle.sf128x4_offset(r, c, cp)
            assert s_swz[o] == s_rm[r, c]
            seen[o] = True
    assert not np.any(s_swz[~seen])  # padding rows and columns are zero


def test_mx_swizzled_scales_equal_rowmajor_after_unswizzle():
    """The 128x4 MXFP8 scale option moves the same scale bytes (the layout function is pinned
    above by hand-placed entries); codes are unchanged; padding is zero.  Shapes put partial
    128-row and 4-column groups on both scale matrices."""
    for M, N in [(160, 96), (96, 224), (32, 32)]:
        X = _random_matrix(M, N, M + N)
        rm = oracle.quant_mxfp8(X, oracle.ROWWISE | oracle.COLWISE)
        sw = oracle.quant_mxfp8(X, oracle.ROWWISE | oracle.COLWISE | oracle.SF_SWIZZLED)
        assert np.array_equal(rm[0], sw[0]) and np.array_equal(rm[2], sw[2])
        _unswizzle_check(sw[1], rm[1])
        _unswizzle_check(sw[3], rm[3])
    gate, up, dh = si.glu_operands(64, 96, seed=31, outliers=True, with_dh=True)
    gb, ub, db_ = si.to_bits(gate), si.to_bits(up), si.to_bits(dh)
    rm = oracle.glu_bwd_mxfp8(oracle.SWIGLU, gb, ub, db_, flags=3)
    sw = oracle.glu_bwd_mxfp8(oracle.SWIGLU, gb, ub, db_, flags=3 | oracle.SF_SWIZZLED)
    _unswizzle_check(sw[1], rm[1])
    _unswizzle_check(sw[3], rm[3])


def test_nv_backward_is_da_then_db():
    """The NVFP4 backward quantizes [da | db]: its left half (codes and scales) is the
    quantizer applied to da alone, its right half to db alone (16-element blocks never
    straddle the two when N % 16 == 0); the 128x4 option moves the same scale bytes."""
    M, N = 150, 80
    gate, up, dh = si.glu_operands(M, N, seed=33, outliers=True, with_dh=True)
    gb, ub, db_ = si.to_bits(gate), si.to_bits(up), si.to_bits(dh)
    for kind in (oracle.SWIGLU, oracle.GEGLU_TANH):
        q, sf = oracle.glu_bwd_nvfp4(kind, gb, ub, db_)
        assert q.shape == (M, N) and sf.shape == (M, 2 * N // 16)
        da, dbb = oracle.glu_bwd(kind, gb, ub, db_)
        qa, sa = oracle.quant_nvfp4(si.from_bits(da).float().numpy())
        qb, sb = oracle.quant_nvfp4(si.from_bits(dbb).float().numpy())
        assert np.array_equal(q[:, :N // 2], qa) and np.array_equal(q[:, N // 2:], qb)
        assert np.array_equal(sf[:, :N // 16], sa) and np.array_equal(sf[:, N // 16:], sb)
        q2, sf2 = oracle.glu_bwd_nvfp4(kind, gb, ub, db_, sf_layout=oracle.SF_128x4)
        assert np.array_equal(q, q2)
        _unswizzle_check(sf2, sf)


def test_fused_equals_glu_then_quantizer():
    gate, up, dh = si.glu_operands(64, 64, seed=25, outliers=True, with_dh=True)
    gb, ub, db_ = si.to_bits(gate), si.to_bits(up), si.to_bits(dh)
    for kind in (oracle.SWIGLU, oracle.GEGLU_TANH, oracle.GEGLU_ERF, oracle.RELU2):
        h = oracle.glu_fwd(kind, gb, ub)
        hf = si.from_bits(h).float().numpy()
        a = oracle.glu_fwd_mxfp8(kind, gb, ub, flags=3)
        b = oracle.quant_mxfp8(hf, 3)
        assert all(np.array_equal(x, y) for x, y in zip(a, b))
        da, dbb = oracle.glu_bwd(kind, gb, ub, db_)
        cat = si.from_bits(np.concatenate([da, dbb], axis=1)).float().numpy()
        a = oracle.glu_bwd_mxfp8(kind, gb, ub, db_, flags=3)
        b = oracle.quant_mxfp8(cat, 3)
        assert all(np.array_equal(x, y) for x, y in zip(a, b))
        paired = np.empty((64, 128), np.uint16)
        paired[:, 0::2], paired[:, 1::2] = gb, ub
        a = oracle.glu_fwd_nvfp4(kind, paired, None)
        b = oracle.quant_nvfp4(hf)
        assert all(np.array_equal(x, y) for x, y in zip(a, b))


# ---- two-level NVFP4 (global scale from the tensor's amax) -------------------------

def _e4m3_table():
    """Magnitudes of E4M3 codes 0..126 from the format definition (bias 7, 3 mantissa bits,
    subnormals m * 2^-9; 0x7F is NaN)."""
    return np.array([(c & 7) * 2.0 ** -9 if c >> 3 == 0 else (1 + (c & 7) / 8) * 2.0 ** ((c >> 3) - 7)
                     for c in range(0x7F)])


_E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _nearest_even(y, table):
    """Brute force: the code of the nearest magnitude, ties to the even code (saturates)."""
    d = np.abs(table - abs(float(y)))
    c = np.nonzero(d == d.min())[0]
    return int(c[0]) if c.size == 1 or c[0] % 2 == 0 else int(c[1])


def _nv_gs_block_ref(v, s):
    """The two-level reading restated with numpy FP32 operations and brute-force rounding."""
    f32 = np.float32
    v = v.astype(np.float32)
    k = f32(f32(s) / f32(6.0))
    d = f32(np.abs(v).max() * k)
    sc = _nearest_even(d, _e4m3_table())
    S = f32(_e4m3_table()[sc])
    r = f32(0.0) if S == 0 else f32(f32(s) / S)
    codes = []
    for x in v:
        y = f32(x * r)
        codes.append((8 if np.signbit(y) else 0) | _nearest_even(y, _E2M1))
    return sc, codes


def test_nv_global_scale_closed_forms():
    gs = oracle.nvfp4_global_scale
    assert gs(2688.0) == 1.0 and gs(1.0) == 2688.0 and gs(3.0) == 896.0 and gs(0.5) == 5376.0
    assert gs(0.0) == 1.0 and gs(-2.0) == 1.0 and gs(float("inf")) == 1.0 and gs(float("nan")) == 1.0
    assert gs(7.0) == float(np.float32(2688.0) / np.float32(7.0))
    assert gs(2.0 ** -90) == 2.0 ** 100 and gs(2.0 ** -120) == 2.0 ** 100      # capped
    assert gs(2.0 ** -80) == 2688.0 * 2.0 ** 80


def test_nv_gs_blocks_against_brute_force():
    """Random blocks (several magnitudes, ties planted) at the true amax, at amax x 8 (small
    scales) and at amax / 8 (saturating scales and codes)."""
    rng = np.random.default_rng(48)
    X = (rng.standard_normal((24, 64)) * np.exp2(rng.integers(-20, 20, (24, 1)))).astype(np.float32)
    X[3, :16] = np.float32(0.75) * np.arange(16, dtype=np.float32)   # multiples of a tie step
    X[5, 16:32] = 0.0
    amax = float(np.abs(X).max())
    for a in (amax, amax * 8, amax / 8, 1.0):
        q, sf = oracle.quant_nvfp4_gs(X, a)
        s = oracle.nvfp4_global_scale(a)
        codes = np.empty((24, 64), np.uint8)
        codes[:, 0::2], codes[:, 1::2] = q & 0xF, q >> 4
        for r in range(24):
            for b in range(4):
                sc, c = _nv_gs_block_ref(X[r, 16 * b:16 * b + 16], s)
                assert sf[r, b] == sc, (a, r, b)
                assert list(codes[r, 16 * b:16 * b + 16]) == c, (a, r, b)


def test_nv_gs_power_of_two_invariance_and_top_scale():
    """Scaling the data and amax by 2^j changes nothing (every step is exact in 2^j); with a
    power-of-two amax the block holding it gets the top scale 448 (code 0x7E)."""
    rng = np.random.default_rng(49)
    X = rng.standard_normal((16, 128)).astype(np.float32)
    X[0, 5] = 8.0
    X = np.clip(X, -7.9, 7.9)
    X[0, 5] = 8.0
    base = oracle.quant_nvfp4_gs(X, 8.0)
    assert base[1][0, 0] == 0x7E
    for j in (-12, -3, 5, 30):
        q, sf = oracle.quant_nvfp4_gs(X * np.float32(2.0 ** j), 8.0 * 2.0 ** j)
        assert np.array_equal(q, base[0]) and np.array_equal(sf, base[1]), j
    q, sf = oracle.quant_nvfp4_gs(X, 8.0, oracle.SF_128x4)
    assert np.array_equal(q, base[0])
    _unswizzle_check(sf, base[1])


def test_glu_amax_and_fused_gs():
    """glu_amax is the largest |h| of the BF16 forward (NaN dominates); the fused two-level
    forward is the quantizer applied to that forward."""
    gate, up = si.glu_operands(40, 96, seed=50, outliers=True)
    gb, ub = si.to_bits(gate), si.to_bits(up)
    h = oracle.bf16_to_f64(oracle.glu_fwd(oracle.GEGLU_TANH, gb, ub))
    a = oracle.glu_amax(oracle.GEGLU_TANH, gb, ub)
    assert a == np.abs(h).max()
    x = h.astype(np.float32)
    for code in (oracle.SF_ROWMAJOR, oracle.SF_128x4):
        got = oracle.glu_fwd_nvfp4_gs(oracle.GEGLU_TANH, gb, ub, amax=a, layout=oracle.SPLIT, sf_layout=code)
        want = oracle.quant_nvfp4_gs(x, a, code)
        assert all(np.array_equal(p, w) for p, w in zip(got, want))
    gb2 = gb.copy()
    gb2[7, 9] = 0x7FC0   # NaN gate
    assert np.isnan(oracle.glu_amax(oracle.GEGLU_TANH, gb2, ub))


# ---- merged gate/up MXFP8 GEMM with the GLU epilogue ----------------------------------

def _dequant_rows(q, s):
    v = oracle.e4m3_to_f64(np.asarray(q)).reshape(q.shape)
    return v * np.repeat(np.exp2(np.asarray(s, np.float64) - 127.0), 32, axis=1)


def test_mx_gemm_matches_numpy_on_dequantized_operands():
    """The oracle's loop equals numpy's matmul of the dequantized operands (a library
    routine), to binary64 summation-order error."""
    Xq, Xs = (t.numpy() for t in si.mx_operand(48, 256, seed=57))
    Wq, Ws = (t.numpy() for t in si.mx_operand(80, 256, seed=58))
    Y = oracle.mx_gemm_nt(Xq, Xs, Wq, Ws)
    ref = _dequant_rows(Xq, Xs) @ _dequant_rows(Wq, Ws).T
    assert np.allclose(Y, ref, rtol=1e-12, atol=0)


def test_mx_gemm_closed_forms():
    """E4M3 0x38 = 1, 0x40 = 2: a 32-long dot product of ones and twos is 64; each E8M0
    step of either operand's scale doubles it; blocks with different scales add."""
    one = np.full((1, 64), 0x38, np.uint8)
    two = np.full((1, 64), 0x40, np.uint8)
    s = np.array([[127, 127]], np.uint8)
    assert oracle.mx_gemm_nt(one, s, two, s)[0, 0] == 128.0
    assert oracle.mx_gemm_nt(one, np.array([[130, 127]], np.uint8), two, s)[0, 0] == 64.0 * 8 + 64.0
    assert oracle.mx_gemm_nt(one, s, two, np.array([[127, 120]], np.uint8))[0, 0] == 64.0 + 64.0 / 128


def test_glu_gemm_is_glu_of_the_gemm():
    """h = bf16(act(Y_gate) * Y_up) with W = [W_gate | W_up]; the MXFP8 form is the rowwise
    quantizer of that h."""
    Xq, Xs = (t.numpy() for t in si.mx_operand(40, 128, seed=59))
    Wq, Ws = (t.numpy() for t in si.mx_operand(2 * 96, 128, seed=60))
    Y = oracle.mx_gemm_nt(Xq, Xs, Wq, Ws)
    for kind in (oracle.SWIGLU, oracle.GEGLU_TANH):
        h = oracle.glu_gemm(kind, Xq, Xs, Wq, Ws)
        want = oracle.bf16_from_f64(oracle.act(kind, Y[:, :96]) * Y[:, 96:])
        assert np.array_equal(h, want)
        q, sc = oracle.glu_gemm_mxfp8(kind, Xq, Xs, Wq, Ws)
        o = oracle.quant_mxfp8(si.from_bits(h).float().numpy(), oracle.ROWWISE)
        assert np.array_equal(q, o[0]) and np.array_equal(sc, o[1])


def _dequant_rows_e2m1(q, s):
    """Packed E2M1 rows [R, K/2] (element 2j in the low nibble) with E8M0 scales -> float64
    [R, K], decoded one nibble at a time with the E2M1 table (pinned in test_oracle_formats)."""
    q = np.asarray(q)
    codes = np.empty((q.shape[0], 2 * q.shape[1]), np.uint8)
    codes[:, 0::2], codes[:, 1::2] = q & 0xF, q >> 4
    v = oracle.e2m1_to_f64(codes).reshape(codes.shape)
    return v * np.repeat(np.exp2(np.asarray(s, np.float64) - 127.0), 32, axis=1)


def test_mx_gemm_e2m1_matches_numpy_on_dequantized_operands():
    """MXFP4 operands: the oracle's loop equals numpy's matmul of the operands decoded nibble
    by nibble (a library routine), to binary64 summation-order error."""
    Xq, Xs = (t.numpy() for t in si.mxfp4_operand(48, 256, seed=61))
    Wq, Ws = (t.numpy() for t in si.mxfp4_operand(80, 256, seed=62))
    Y = oracle.mx_gemm_nt(Xq, Xs, Wq, Ws, fmt=oracle.FMT_E2M1)
    ref = _dequant_rows_e2m1(Xq, Xs) @ _dequant_rows_e2m1(Wq, Ws).T
    assert np.allclose(Y, ref, rtol=1e-12, atol=0)


def test_mx_gemm_e2m1_closed_forms():
    """E2M1 code 0x2 = 1 and 0x4 = 2, so byte 0x22 packs two ones and 0x44 two twos: a 32-long
    dot product of ones and twos is 64, each E8M0 step doubles it, blocks add; 0xF = -6 and
    0x7 = 6 in one byte cancel against a row of ones; one nonzero element lands in the block
    of its own K position (element 33 is the high nibble of byte 16)."""
    one, two = np.full((1, 32), 0x22, np.uint8), np.full((1, 32), 0x44, np.uint8)
    s = np.array([[127, 127]], np.uint8)
    f = oracle.FMT_E2M1
    assert oracle.mx_gemm_nt(one, s, two, s, fmt=f)[0, 0] == 128.0
    assert oracle.mx_gemm_nt(one, np.array([[130, 127]], np.uint8), two, s, fmt=f)[0, 0] == 64.0 * 8 + 64.0
    assert oracle.mx_gemm_nt(one, s, two, np.array([[127, 120]], np.uint8), fmt=f)[0, 0] == 64.0 + 64.0 / 128
    assert oracle.mx_gemm_nt(np.full((1, 32), 0x7F, np.uint8), s, one, s, fmt=f)[0, 0] == 0.0
    x = np.zeros((1, 32), np.uint8)
    x[0, 16] = 0x50                                      # element 33 = 3.0, in block 1
    assert oracle.mx_gemm_nt(x, np.array([[127, 129]], np.uint8), one, s, fmt=f)[0, 0] == 12.0


def test_glu_gemm_interleaved_w_rows():
    """[NV] Supported contract, weight layout row: W rows gate0, up0, gate1, up1, ...  The GLU
    GEMM on interleaved W equals the one on [W_gate | W_up] holding the same rows, and equals
    the GLU of Y's even (gate) and odd (up) columns; MXFP8 and MXFP4 operands."""
    for fmt, gen in ((oracle.FMT_E4M3, si.mx_operand), (oracle.FMT_E2M1, si.mxfp4_operand)):
        Xq, Xs = (t.numpy() for t in gen(24, 128, seed=63))
        Wq, Ws = gen(2 * 64, 128, seed=64)
        Wp, Wps = si.interleave_rows(Wq).numpy(), si.interleave_rows(Ws).numpy()
        Wq, Ws = Wq.numpy(), Ws.numpy()
        assert not np.array_equal(Wp, Wq)
        Yp = oracle.mx_gemm_nt(Xq, Xs, Wp, Wps, fmt=fmt)
        for kind in (oracle.SWIGLU, oracle.GEGLU_TANH):
            h = oracle.glu_gemm(kind, Xq, Xs, Wp, Wps, fmt=fmt, w_layout=oracle.PAIRED)
            assert np.array_equal(h, oracle.glu_gemm(kind, Xq, Xs, Wq, Ws, fmt=fmt))
            assert np.array_equal(h, oracle.bf16_from_f64(oracle.act(kind, Yp[:, 0::2]) * Yp[:, 1::2]))
            q, sc = oracle.glu_gemm_mxfp8(kind, Xq, Xs, Wp, Wps, fmt=fmt, w_layout=oracle.PAIRED)
            o = oracle.quant_mxfp8(si.from_bits(h).float().numpy(), oracle.ROWWISE)
            assert np.array_equal(q, o[0]) and np.array_equal(sc, o[1])


def test_two_level_at_unit_global_scale_against_single_level():
    """An amax of 2688 (448 x 6) makes the global scale exactly 1, so two-level NVFP4 meets the
    single-level quantizer, which is pinned on its own (hand-worked blocks, brute force).  Over
    every positive finite E4M3 block scale S (a block whose maximum is 6 S) and every BF16
    value x with |x| <= 6 S (both signs):
      * the block scales agree everywhere (fl(amax * fl(1/6)) decides as amax / 6 does);
      * the codes agree except at 42 (x, S) pairs (each with both signs), found in closed
        form: S a normal E4M3 value with all three mantissa bits set (1.875 * 2^k, k = -6..7)
        and |x| / S one of the E2M1 ties 1.25, 2.5, 5.  There fl(1/S) = fl(8/15) 2^-k lies
        above 1/S, so fl(x * fl(1/S)) lands one FP32 ulp above the tie and rounds to the next
        code up, where x / S itself rounds to the even code below.  (The subnormal 7 * 2^-9 has
        fl(1/S) = fl(8/7) 2^6 below 1/S and no such pair.)"""
    S_codes = np.arange(1, 0x7F, dtype=np.uint8)
    S_vals = oracle.e4m3_to_f64(S_codes)
    mags = np.arange(1, 0x7F80, dtype=np.uint32)
    mvals = (mags << 16).view(np.float32).astype(np.float64)
    rng = np.random.default_rng(77)
    blocks, predicted = [], []
    for code, S in zip(S_codes, S_vals):
        body = np.concatenate([mags[mvals <= 6.0 * S]] * 2)
        body = body | (rng.integers(0, 2, body.size, dtype=np.uint32) << 15)   # random signs
        n = -(-body.size // 15)
        body = np.resize(body, n * 15).reshape(n, 15)
        head_bits = int(np.float32(6.0 * S).view(np.uint32) >> 16)
        assert (head_bits << 16) == int(np.float32(6.0 * S).view(np.uint32))   # 6 S is a BF16 value
        head = np.full((n, 1), head_bits, np.uint32) | (rng.integers(0, 2, (n, 1), dtype=np.uint32) << 15)
        blk = np.concatenate([head, body], axis=1)
        blocks.append(blk)
        ratio = ((blk & 0x7FFF) << 16).view(np.float32).astype(np.float64) / S
        predicted.append(((code & 7) == 7) & ((code >> 3) >= 1) & np.isin(ratio, (1.25, 2.5, 5.0)))
    X = ((np.concatenate(blocks).astype(np.uint32)) << 16).view(np.float32)
    pred = np.concatenate(predicted)
    pad = (-X.shape[0]) % 8
    X = np.concatenate([X, np.zeros((pad, 16), np.float32)]).reshape(-1, 128)
    pred = np.concatenate([pred, np.zeros((pad, 16), bool)]).reshape(-1, 128)
    q1, s1 = oracle.quant_nvfp4(X)
    q2, s2 = oracle.quant_nvfp4_gs(X, np.float32(2688.0))
    assert oracle.nvfp4_global_scale(2688.0) == 1.0
    assert np.array_equal(s1, s2), "block scales"
    c1 = np.empty(X.shape, np.uint8); c1[:, 0::2], c1[:, 1::2] = q1 & 0xF, q1 >> 4
    c2 = np.empty(X.shape, np.uint8); c2[:, 0::2], c2[:, 1::2] = q2 & 0xF, q2 >> 4
    differ = c1 != c2
    assert np.array_equal(differ, pred), f"{int(differ.sum())} differing codes, {int(pred.sum())} predicted"
    sblk = np.repeat(np.asarray(s1).reshape(X.shape[0], 8), 16, axis=1)     # each element's scale code
    pairs = set(zip(((X.view(np.uint32)[pred] >> 16) & 0x7FFF).tolist(), sblk[pred].tolist()))
    assert len(pairs) == 42
    assert np.all((c2[differ] & 8) == (c1[differ] & 8)) and np.all((c2[differ] & 7) == (c1[differ] & 7) + 1)
