"""The comparison rules themselves (CPU only): each accepts what it should and rejects a
planted mistake.  The "GPU" side here is the oracle run on slightly different inputs, or
the oracle's output with a deliberate error."""
import numpy as np
import pytest

import oracle
import synthetic_inputs as si
from parity import bf16_ulp_distance, check_rule2, check_rule3_mx, check_rule3_nv, check_rule3_nv_gs


def test_rule2_distance():
    assert bf16_ulp_distance([0x0000], [0x8000])[0] == 0          # +0 and -0 identified
    assert bf16_ulp_distance([0x3F80], [0x3F81])[0] == 1
    assert bf16_ulp_distance([0x0001], [0x8001])[0] == 2          # across zero
    assert bf16_ulp_distance([0x7FC0], [0xFFC1])[0] == 0          # NaN matches NaN
    assert bf16_ulp_distance([0x7FC0], [0x3F80])[0] > 1
    check_rule2(np.array([0x3F80, 0x4000]), np.array([0x3F81, 0x4000]))
    with pytest.raises(AssertionError):
        check_rule2(np.array([0x3F80]), np.array([0x3F82]))


def _h_and_nudged(M, N, seed):
    """Oracle BF16 h, and a copy where 1 in 2^14 elements moved by one ulp (what a GPU
    result within rule 2 may look like)."""
    gate, up = si.glu_operands(M, N, seed=seed, outliers=True)
    h = oracle.glu_fwd(oracle.SWIGLU, si.to_bits(gate), si.to_bits(up))
    rng = np.random.default_rng(seed)
    g = h.copy()
    idx = rng.choice(h.size, max(1, h.size >> 14), replace=False)
    g.ravel()[idx] = (g.ravel()[idx].astype(np.int64) + 1).astype(np.uint16)
    return h, g


def test_rule3_nv_accepts_rounding_boundary_noise_and_rejects_a_planted_code():
    h, g = _h_and_nudged(256, 1024, 54)
    hf, gf = (si.from_bits(x).float().numpy() for x in (h, g))
    oq, osf = oracle.quant_nvfp4(hf)
    gq, gsf = oracle.quant_nvfp4(gf)
    check_rule3_nv(h, gq, gsf, oq, osf, "nudged")
    bad = gq.copy()
    bad[3, 5] ^= 0x02                       # a code two steps away, mid-interval
    with pytest.raises(AssertionError):
        check_rule3_nv(h, bad, gsf, oq, osf, "planted")


def test_rule3_nv_gs_accepts_noise_and_rejects_a_planted_scale():
    h, g = _h_and_nudged(256, 1024, 55)
    hf, gf = (si.from_bits(x).float().numpy() for x in (h, g))
    amax = float(np.abs(hf).max())
    s = oracle.nvfp4_global_scale(amax)
    oq, osf = oracle.quant_nvfp4_gs(hf, amax)
    gq, gsf = oracle.quant_nvfp4_gs(gf, amax)
    check_rule3_nv_gs(h, gq, gsf, oq, osf, s, "nudged")
    bad = gsf.copy()
    bad[10, 7] = bad[10, 7] + 1              # one step, but the block amax is not at a boundary
    with pytest.raises(AssertionError):
        check_rule3_nv_gs(h, gq, bad, oq, osf, s, "planted")
    # the global-scale-1 checker does not accept two-level output as consistent
    with pytest.raises(AssertionError):
        check_rule3_nv(h, gq, gsf, oq, oracle.quant_nvfp4(hf)[1], "wrong rule")


def test_rule3_mx_accepts_noise_and_rejects_a_planted_code():
    h, g = _h_and_nudged(128, 256, 56)
    hf, gf = (si.from_bits(x).float().numpy() for x in (h, g))
    o = oracle.quant_mxfp8(hf, oracle.ROWWISE)
    q = oracle.quant_mxfp8(gf, oracle.ROWWISE)
    check_rule3_mx(h, q[0], q[1], o[0], o[1], "nudged")
    bad = q[0].copy()
    bad[7, 9] ^= 0x04
    with pytest.raises(AssertionError):
        check_rule3_mx(h, bad, q[1], o[0], o[1], "planted")
