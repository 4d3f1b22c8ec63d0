"""Comparison rules between GPU results and the oracle (test helpers, numpy only).

Rule 1: quantized codes and scales are bit-exact when both quantizers see identical
        FP32 values (checked with plain array equality in the tests).
Rule 2: every BF16 output is within 1 BF16 ulp of the oracle's, distance measured between
        sign-magnitude-ordered bit patterns with +0 and -0 identified; NaN matches NaN.
Rule 3: end-to-end quantized outputs: >= 99.99% identical codes; in blocks whose scales
        agree, every differing code is one step from the oracle's and the oracle's BF16
        value lies within 1 BF16 ulp of the rounding boundary between the two codes; a
        block scale may differ by one step only when the oracle's block amax lies within
        1 BF16 ulp of the scale boundary; dequantized relative L2 error below 1e-3.
"""
import numpy as np

import oracle

E4M3_VAL = oracle.e4m3_to_f64(np.arange(256, dtype=np.uint8))
E2M1_VAL = oracle.e2m1_to_f64(np.arange(16, dtype=np.uint8))


def _ranks(vals):
    finite = ~np.isnan(vals)
    uniq = np.unique(vals[finite])
    rank = np.full(vals.shape, -10 ** 6, dtype=np.int64)
    rank[finite] = np.searchsorted(uniq, vals[finite])
    return rank


E4M3_RANK = _ranks(E4M3_VAL)
E2M1_RANK = _ranks(E2M1_VAL)


def bf16_to_f64(bits):
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def bf16_ulp(x):
    """Spacing of BF16 numbers at |x| (subnormal spacing 2^-133 below 2^-126)."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return np.exp2(e - 7)


def bf16_ulp_distance(a_bits, b_bits):
    a = np.asarray(a_bits, dtype=np.uint16).astype(np.int64)
    b = np.asarray(b_bits, dtype=np.uint16).astype(np.int64)

    def ordered(x):
        mag = x & 0x7FFF
        return np.where(x & 0x8000, -mag, mag)

    d = np.abs(ordered(a) - ordered(b))
    nan_a = (a & 0x7FFF) > 0x7F80
    nan_b = (b & 0x7FFF) > 0x7F80
    d = np.where(nan_a & nan_b, 0, d)
    d = np.where(nan_a ^ nan_b, 1 << 20, d)
    return d


def check_rule2(gpu_bits, orc_bits, what=""):
    d = bf16_ulp_distance(gpu_bits, orc_bits)
    worst = int(d.max()) if d.size else 0
    assert worst <= 1, f"{what}: {int((d > 1).sum())} elements beyond 1 BF16 ulp (worst {worst})"
    return dict(n=int(d.size), off_by_one=int((d == 1).sum()))


def _unpack_nibbles(q):
    q = np.asarray(q, dtype=np.uint8)
    out = np.empty(q.shape[:-1] + (q.shape[-1] * 2,), np.uint8)
    out[..., 0::2] = q & 0xF
    out[..., 1::2] = q >> 4
    return out


def _rule3(h_bits, q_g, s_g, q_o, s_o, block, val, rank, scale_val, scale_rank, scale_boundary,
           nonfinite_scale, what):
    h = bf16_to_f64(h_bits)
    R, C = h.shape
    nb = C // block
    q_g = np.asarray(q_g).reshape(R, C)
    q_o = np.asarray(q_o).reshape(R, C)
    s_g = np.asarray(s_g).reshape(R, nb).astype(np.int64)
    s_o = np.asarray(s_o).reshape(R, nb).astype(np.int64)
    exact = q_g == q_o
    frac = float(exact.mean()) if exact.size else 1.0
    assert frac >= 0.9999, f"{what}: only {frac:.6%} of codes identical"

    # non-finite blocks must agree exactly
    nf = (s_o == nonfinite_scale) | (s_g == nonfinite_scale)
    assert np.array_equal(s_g[nf], s_o[nf]), f"{what}: non-finite block scales differ"

    hb = h.reshape(R, nb, block)
    amax = np.abs(hb).max(axis=2)
    smis = (s_g != s_o) & ~nf
    for r, b in zip(*np.nonzero(smis)):
        assert abs(int(scale_rank[s_g[r, b]]) - int(scale_rank[s_o[r, b]])) == 1, \
            f"{what}: block ({r},{b}) scale {s_g[r, b]} vs {s_o[r, b]}"
        bnd = scale_boundary(s_g[r, b], s_o[r, b])
        assert abs(amax[r, b] - bnd) <= bf16_ulp(bnd), f"{what}: block ({r},{b}) scale off away from a boundary"

    # code mismatches inside blocks with agreeing, finite scales
    ok_blocks = (s_g == s_o) & ~nf
    mism = ~exact & np.repeat(ok_blocks, block, axis=1)
    rr, cc = np.nonzero(mism)
    if rr.size:
        cg, co = q_g[rr, cc], q_o[rr, cc]
        steps = np.abs(rank[cg] - rank[co])
        both_zero = (val[cg] == 0) & (val[co] == 0)
        assert np.all((steps == 1) | both_zero), f"{what}: a code differs by more than one step"
        S = scale_val(s_o[rr, cc // block])
        bnd = 0.5 * (val[cg] + val[co]) * S
        hv = h[rr, cc]
        assert np.all(np.abs(hv - bnd) <= bf16_ulp(np.maximum(np.abs(hv), np.abs(bnd))) + 1e-300), \
            f"{what}: a differing code is not at a rounding boundary"

    fin = np.repeat(~nf, block, axis=1)
    Sg = scale_val(np.repeat(s_g, block, axis=1))
    So = scale_val(np.repeat(s_o, block, axis=1))
    dg = np.where(fin, val[q_g] * Sg, 0.0)
    do = np.where(fin, val[q_o] * So, 0.0)
    den = np.linalg.norm(do)
    rel = float(np.linalg.norm(dg - do) / den) if den > 0 else float(np.linalg.norm(dg))
    assert rel < 1e-3, f"{what}: dequantized relative L2 {rel:.3g}"
    return dict(codes=int(exact.size), code_mismatch=int((~exact).sum()), scale_mismatch=int(smis.sum()),
                rel_l2=rel)


def check_rule3_mx(h_bits, q_g, s_g, q_o, s_o, what=""):
    """Blocks of 32 along the last axis of h_bits [R, C] (pass h transposed for colwise)."""
    return _rule3(h_bits, q_g, s_g, q_o, s_o, 32, E4M3_VAL, E4M3_RANK,
                  lambda s: np.exp2(np.asarray(s, dtype=np.float64) - 127.0),
                  np.arange(256, dtype=np.int64),
                  lambda a, b: 448.0 * 2.0 ** (min(int(a), int(b)) - 127),
                  0xFF, what)


def check_rule3_nv_gs(h_bits, q_g, s_g, q_o, s_o, s, what=""):
    """As check_rule3_nv for two-level scaling with global encode scale s: block scales decide
    on amax * fl(s/6), codes on x * s / S, and dequantize as code * S / s."""
    k = float(np.float32(np.float32(s) / np.float32(6.0)))
    return _rule3(h_bits, _unpack_nibbles(q_g), s_g, _unpack_nibbles(q_o), s_o, 16, E2M1_VAL, E2M1_RANK,
                  lambda c: E4M3_VAL[np.asarray(c, dtype=np.int64)] / s,
                  E4M3_RANK,
                  lambda a, b: 0.5 * (E4M3_VAL[int(a)] + E4M3_VAL[int(b)]) / k,
                  0x7F, what)


def check_rule3_nv(h_bits, q_g, s_g, q_o, s_o, what=""):
    """h_bits [M, H] BF16; q packed [M, H/2]; s row-major [M, H/16]."""
    return _rule3(h_bits, _unpack_nibbles(q_g), s_g, _unpack_nibbles(q_o), s_o, 16, E2M1_VAL, E2M1_RANK,
                  lambda s: E4M3_VAL[np.asarray(s, dtype=np.int64)],
                  E4M3_RANK,
                  lambda a, b: 3.0 * (E4M3_VAL[int(a)] + E4M3_VAL[int(b)]),
                  0x7F, what)
