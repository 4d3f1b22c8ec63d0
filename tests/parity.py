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


class Rule3:
    """Rule 3 over a tensor given in pieces (row chunks of the quantized matrix): the local
    conditions (scale and code mismatches only at rounding boundaries, non-finite blocks
    identical) are asserted per piece; the global ones (>= 99.99% identical codes, dequantized
    relative L2 below 1e-3) by finish(), over everything added."""

    def __init__(self, block, val, rank, scale_val, scale_rank, scale_boundary, nonfinite_scale, what):
        self.block, self.val, self.rank = block, val, rank
        self.scale_val, self.scale_rank, self.scale_boundary = scale_val, scale_rank, scale_boundary
        self.nonfinite_scale, self.what = nonfinite_scale, what
        self.val2 = val * val
        self.n = self.exact = self.smis = 0
        self.diff2 = self.ref2 = 0.0

    def add(self, h_bits, q_g, s_g, q_o, s_o):
        what, block, val, rank = self.what, self.block, self.val, self.rank
        h_bits = np.asarray(h_bits, dtype=np.uint16)
        R, C = h_bits.shape
        nb = C // block
        q_g = np.asarray(q_g).reshape(R, C)
        q_o = np.asarray(q_o).reshape(R, C)
        s_g = np.asarray(s_g).reshape(R, nb).astype(np.int64)
        s_o = np.asarray(s_o).reshape(R, nb).astype(np.int64)
        rr, cc = np.nonzero(q_g != q_o)          # the differing codes (few)
        self.n += q_g.size
        self.exact += q_g.size - rr.size

        # non-finite blocks must agree exactly
        nf = (s_o == self.nonfinite_scale) | (s_g == self.nonfinite_scale)
        assert np.array_equal(s_g[nf], s_o[nf]), f"{what}: non-finite block scales differ"

        smis = (s_g != s_o) & ~nf
        self.smis += int(smis.sum())
        br, bc = np.nonzero(smis)
        for r, b in zip(br, bc):
            assert abs(int(self.scale_rank[s_g[r, b]]) - int(self.scale_rank[s_o[r, b]])) == 1, \
                f"{what}: block ({r},{b}) scale {s_g[r, b]} vs {s_o[r, b]}"
            amax = np.abs(bf16_to_f64(h_bits[r, block * b:block * (b + 1)])).max()
            bnd = self.scale_boundary(s_g[r, b], s_o[r, b])
            assert abs(amax - bnd) <= bf16_ulp(bnd), f"{what}: block ({r},{b}) scale off away from a boundary"

        # code mismatches inside blocks with agreeing, finite scales: one step, at a rounding
        # boundary.  A pair of codes that both decode to zero (+0 and -0) passes the step test;
        # the boundary test then requires the oracle's value to be within one BF16 ulp of zero,
        # i.e. only the sign of a zero may differ (rule 2 identifies +0 and -0).
        fin_el = ~nf[rr, cc // block]
        ok = fin_el & ~smis[rr, cc // block]
        r1, c1 = rr[ok], cc[ok]
        if r1.size:
            cg, co = q_g[r1, c1], q_o[r1, c1]
            steps = np.abs(rank[cg] - rank[co])
            both_zero = (val[cg] == 0) & (val[co] == 0)
            assert np.all((steps == 1) | both_zero), f"{what}: a code differs by more than one step"
            S = self.scale_val(s_o[r1, c1 // block])
            bnd = 0.5 * (val[cg] + val[co]) * S
            hv = bf16_to_f64(h_bits[r1, c1])
            assert np.all(np.abs(hv - bnd) <= bf16_ulp(np.maximum(np.abs(hv), np.abs(bnd))) + 1e-300), \
                f"{what}: a differing code is not at a rounding boundary"

        # dequantized L2 over finite blocks: the reference norm block by block, the difference
        # only where a code or a scale differs (elsewhere it is zero)
        with np.errstate(over="ignore", invalid="ignore"):
            So = self.scale_val(np.where(nf, 0, s_o))
            blk2 = self.val2[q_o].reshape(R, nb, block).sum(axis=2)
            self.ref2 += float(np.sum(np.where(nf, 0.0, blk2 * So * So)))
        if br.size:                               # every element of a block whose scale differs
            cols = (block * bc[:, None] + np.arange(block)[None, :]).ravel()
            rows = np.repeat(br, block)
            rows, cols = np.concatenate([rows, rr[ok]]), np.concatenate([cols, cc[ok]])
        else:
            rows, cols = rr[ok], cc[ok]
        if rows.size:
            dg = val[q_g[rows, cols]] * self.scale_val(s_g[rows, cols // block])
            do = val[q_o[rows, cols]] * self.scale_val(s_o[rows, cols // block])
            self.diff2 += float(np.sum((dg - do) ** 2))
        return self

    def merge(self, other):
        """Folds in the counts of another accumulator of the same tensor (disjoint pieces)."""
        self.n += other.n
        self.exact += other.exact
        self.smis += other.smis
        self.diff2 += other.diff2
        self.ref2 += other.ref2
        return self

    def finish(self):
        frac = self.exact / self.n if self.n else 1.0
        assert frac >= 0.9999, f"{self.what}: only {frac:.6%} of codes identical"
        rel = (self.diff2 / self.ref2) ** 0.5 if self.ref2 > 0 else self.diff2 ** 0.5
        assert rel < 1e-3, f"{self.what}: dequantized relative L2 {rel:.3g}"
        return dict(codes=self.n, code_mismatch=self.n - self.exact, scale_mismatch=self.smis, rel_l2=rel)


def rule3_mx(what=""):
    """A Rule3 accumulator for MXFP8 (blocks of 32 along the last axis of what is added)."""
    return Rule3(32, E4M3_VAL, E4M3_RANK,
                 lambda s: np.exp2(np.asarray(s, dtype=np.float64) - 127.0),
                 np.arange(256, dtype=np.int64),
                 lambda a, b: 448.0 * 2.0 ** (min(int(a), int(b)) - 127),
                 0xFF, what)


def check_rule3_mx(h_bits, q_g, s_g, q_o, s_o, what=""):
    """Blocks of 32 along the last axis of h_bits [R, C] (pass h transposed for colwise)."""
    return rule3_mx(what).add(h_bits, q_g, s_g, q_o, s_o).finish()


def check_rule3_nv_gs(h_bits, q_g, s_g, q_o, s_o, s, what=""):
    """As check_rule3_nv for two-level scaling with global encode scale s: block scales decide
    on amax * fl(s/6), codes on x * s / S, and dequantize as code * S / s."""
    k = float(np.float32(np.float32(s) / np.float32(6.0)))
    return Rule3(16, E2M1_VAL, E2M1_RANK,
                 lambda c: E4M3_VAL[np.asarray(c, dtype=np.int64)] / s,
                 E4M3_RANK,
                 lambda a, b: 0.5 * (E4M3_VAL[int(a)] + E4M3_VAL[int(b)]) / k,
                 0x7F, what).add(h_bits, _unpack_nibbles(q_g), s_g, _unpack_nibbles(q_o), s_o).finish()


def check_rule3_nv(h_bits, q_g, s_g, q_o, s_o, what=""):
    """h_bits [M, H] BF16; q packed [M, H/2]; s row-major [M, H/16]."""
    return Rule3(16, E2M1_VAL, E2M1_RANK,
                 lambda s: E4M3_VAL[np.asarray(s, dtype=np.int64)],
                 E4M3_RANK,
                 lambda a, b: 3.0 * (E4M3_VAL[int(a)] + E4M3_VAL[int(b)]),
                 0x7F, what).add(h_bits, _unpack_nibbles(q_g), s_g, _unpack_nibbles(q_o), s_o).finish()
