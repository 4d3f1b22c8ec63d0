"""GPU parity of the fused MXFP8 paths and the MXFP8 quantizer hook against the oracle.

Rule 1 (bit-exact when the quantizer sees identical FP32 values):
  * glu_quant_mxfp8_f32 on random, outlier, subnormal, tie-dense, all-BF16 and non-finite
    inputs equals oracle.quant_mxfp8 byte for byte, rowwise, colwise and both;
  * the fused kernels equal the oracle quantizer applied to the GPU's own BF16 glu_fwd /
    glu_bwd output (the quantizer isolated end to end), also with most elements on the
    FP64 tail path (synthetic_inputs.tail_operands).
Rule 3 (fused GPU vs oracle end to end) on the five workload shapes, full or sampled.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
from conftest import bits, u8
from parity import check_rule2, check_rule3_mx, rule3_mx
from sweep_inputs import mxfp8_sweep_matrix

pytestmark = pytest.mark.gpu
FLAGS = [(True, False), (False, True), (True, True)]
ACTS = [("swiglu", oracle.SWIGLU), ("geglu", oracle.GEGLU_TANH), ("geglu_erf", oracle.GEGLU_ERF),
        ("relu2", oracle.RELU2)]


def _flags(row, col):
    return (oracle.ROWWISE if row else 0) | (oracle.COLWISE if col else 0)


def _hook_matches_oracle(gpu, x):
    xd = torch.from_numpy(x).cuda()
    for row, col in FLAGS:
        qr, qc, sr, sc = gpu.glu_quant_mxfp8_f32(xd, rowwise=row, colwise=col)
        o = oracle.quant_mxfp8(x, _flags(row, col))
        if row:
            assert np.array_equal(u8(sr), o[1]), "row scales"
            assert np.array_equal(u8(qr), o[0]), "row codes"
        if col:
            assert np.array_equal(u8(sc), o[3]), "col scales"
            assert np.array_equal(u8(qc), o[2]), "col codes"


def test_hook_random_fp32(gpu):
    rng = np.random.default_rng(100)
    x = rng.normal(0, 1, (256, 512))
    x[rng.random(x.shape) < 1e-3] *= 1000
    x[rng.random(x.shape) < 1e-2] *= 2.0 ** -40
    x[:32, :32] = 0.0
    x[32:64, 64:96] = -0.0
    x = x.astype(np.float32)
    x[100, 3] = np.float32(1e-42)  # FP32 subnormal
    _hook_matches_oracle(gpu, x)


def test_hook_every_bf16_value(gpu):
    allv = si.special_bf16_values()
    x = np.zeros(65536, np.float32)
    x[: allv.size] = si.from_bits(allv).float().numpy()
    _hook_matches_oracle(gpu, x.reshape(2048, 32))
    _hook_matches_oracle(gpu, np.ascontiguousarray(x.reshape(2048, 32)[::-1]))


def test_hook_ties_and_boundaries(gpu):
    """Each block: one element 448 * 2^k fixes the scale at 2^k; the others sit on E4M3
    rounding midpoints at that scale and one FP32 ulp either side."""
    rng = np.random.default_rng(101)
    vals = np.unique(np.abs(oracle.e4m3_to_f64(np.arange(0x7F, dtype=np.uint8))))
    mids = (vals[1:] + vals[:-1]) / 2
    nblk = 8192
    k = rng.integers(-120, 100, nblk)
    pick = rng.choice(mids, (nblk, 31))
    jitter = rng.integers(-1, 2, (nblk, 31))
    y = (pick * np.exp2(k)[:, None]).astype(np.float32)
    y = np.where(jitter > 0, np.nextafter(y, np.float32(np.inf)), np.where(jitter < 0, np.nextafter(y, np.float32(0)), y))
    y *= rng.choice([-1, 1], y.shape).astype(np.float32)
    first = (448.0 * np.exp2(k)).astype(np.float32)[:, None]
    x = np.concatenate([first, y], axis=1).astype(np.float32)
    _hook_matches_oracle(gpu, x.reshape(1024, 256))


def test_hook_nonfinite_blocks(gpu):
    x = np.ones((64, 128), np.float32)
    x[0, 5] = np.inf
    x[7, 40] = -np.inf
    x[40, 100] = np.nan
    x[33, 64:96] = 3.0e38
    _hook_matches_oracle(gpu, x)


def _q(h_or_x_bits, flags):
    return oracle.quant_mxfp8(si.from_bits(h_or_x_bits).float().numpy(), flags)


@pytest.mark.parametrize("name,kind", ACTS)
@pytest.mark.parametrize("layout", ["split", "concat", "paired"])
def test_fused_fwd_equals_quantized_glu_fwd(gpu, name, kind, layout):
    M, N = 128, 256
    gate, up = si.glu_operands(M, N, seed=5, outliers=True)
    gd, ud = gate.cuda(), up.cuda()
    if layout == "concat":
        cat = torch.cat([gd, ud], 1)
        args, lay = (cat[:, :N], cat[:, N:]), "split"
    elif layout == "paired":
        args, lay = (torch.stack([gd, ud], 2).reshape(M, 2 * N).contiguous(), None), "paired"
    else:
        args, lay = (gd, ud), "split"
    h = bits(gpu.glu_fwd(*args, act=name, layout=lay))
    for row, col in FLAGS:
        qr, qc, sr, sc = gpu.glu_fwd_mxfp8(*args, act=name, layout=lay, rowwise=row, colwise=col)
        o = _q(h, _flags(row, col))
        if row:
            assert np.array_equal(u8(qr), o[0]) and np.array_equal(u8(sr), o[1])
        if col:
            assert np.array_equal(u8(qc), o[2]) and np.array_equal(u8(sc), o[3])


@pytest.mark.parametrize("name,kind", ACTS)
@pytest.mark.parametrize("M,N", [(96, 160), (96, 640)])
def test_fused_bwd_equals_quantized_glu_bwd(gpu, name, kind, M, N):
    gate, up, dh = si.glu_operands(M, N, seed=6, outliers=True, with_dh=True)
    gd, ud, dd = gate.cuda(), up.cuda(), dh.cuda()
    da, db = gpu.glu_bwd(gd, ud, dd, act=name)
    X = np.concatenate([bits(da), bits(db)], axis=1)
    for row, col in FLAGS:
        qr, qc, sr, sc = gpu.glu_bwd_mxfp8(gd, ud, dd, act=name, rowwise=row, colwise=col)
        o = _q(X, _flags(row, col))
        if row:
            assert np.array_equal(u8(qr), o[0]) and np.array_equal(u8(sr), o[1])
        if col:
            assert np.array_equal(u8(qc), o[2]) and np.array_equal(u8(sc), o[3])


@pytest.mark.parametrize("name,kind", ACTS)
def test_fused_tail_paths_equal_quantized_glu(gpu, name, kind):
    """The fused kernels patch the FP64 tail results into their packed BF16 words; with most
    elements on the tail path, both directions and every scaling must still equal the oracle
    quantizer applied to the GPU's own glu_fwd / glu_bwd output (whose tails the BF16 tests
    hold to rule 2 against the oracle)."""
    M, N = 128, 256
    g, u, d = si.tail_operands(name, M, N, seed=11 + kind)
    gd, ud, dd = g.cuda(), u.cuda(), d.cuda()
    h = bits(gpu.glu_fwd(gd, ud, act=name))
    da, db = gpu.glu_bwd(gd, ud, dd, act=name)
    X = np.concatenate([bits(da), bits(db)], axis=1)
    for row, col in FLAGS:
        for what, got, ref in (("fwd", gpu.glu_fwd_mxfp8(gd, ud, act=name, rowwise=row, colwise=col), h),
                               ("bwd", gpu.glu_bwd_mxfp8(gd, ud, dd, act=name, rowwise=row, colwise=col), X)):
            qr, qc, sr, sc = got
            o = _q(ref, _flags(row, col))
            if row:
                assert np.array_equal(u8(qr), o[0]) and np.array_equal(u8(sr), o[1]), f"{what} rowwise"
            if col:
                assert np.array_equal(u8(qc), o[2]) and np.array_equal(u8(sc), o[3]), f"{what} colwise"


@pytest.mark.parametrize("layout", ["split", "paired"])
def test_rowwise_nonfinite_blocks(gpu, layout):
    """NaN and Inf operands in rowwise-only launches at a width with two 512-column pieces per
    row (the second one partial): the blocks they reach get scale 0xFF and codes 0x7F, the
    others quantize as usual; forward and backward against the oracle quantizer of the
    device's own h, da, db."""
    M, N = 64, 640
    gate, up, dh = si.glu_operands(M, N, seed=7, outliers=True, with_dh=True)
    gate[3, 5] = float("nan")
    up[10, 600] = float("inf")
    gate[40, 130] = float("-inf")
    dh[20, 100] = float("inf")
    gd, ud, dd = gate.cuda(), up.cuda(), dh.cuda()
    if layout == "paired":
        args, lay = (torch.stack([gd, ud], 2).reshape(M, 2 * N).contiguous(), None), "paired"
    else:
        args, lay = (gd, ud), "split"
    h = bits(gpu.glu_fwd(*args, layout=lay))
    qr, _, sr, _ = gpu.glu_fwd_mxfp8(*args, layout=lay, rowwise=True)
    o = _q(h, oracle.ROWWISE)
    assert (u8(sr) == 0xFF).any()
    assert np.array_equal(u8(qr), o[0]) and np.array_equal(u8(sr), o[1])
    if layout == "split":
        da, db = gpu.glu_bwd(gd, ud, dd)
        qr, _, sr, _ = gpu.glu_bwd_mxfp8(gd, ud, dd, rowwise=True)
        o = _q(np.concatenate([bits(da), bits(db)], axis=1), oracle.ROWWISE)
        assert (u8(sr) == 0xFF).any()
        assert np.array_equal(u8(qr), o[0]) and np.array_equal(u8(sr), o[1])


def test_both_equals_row_and_col(gpu):
    gate, up, dh = si.glu_operands(256, 512, seed=8, outliers=True, with_dh=True)
    gd, ud, dd = gate.cuda(), up.cuda(), dh.cuda()
    for fn, args in ((gpu.glu_fwd_mxfp8, (gd, ud)), (gpu.glu_bwd_mxfp8, (gd, ud, dd))):
        b = fn(*args, rowwise=True, colwise=True)
        r = fn(*args, rowwise=True, colwise=False)
        c = fn(*args, rowwise=False, colwise=True)
        assert torch.equal(b[0], r[0]) and torch.equal(b[2], r[2])
        assert torch.equal(b[1], c[1]) and torch.equal(b[3], c[3])


def test_ragged_rows_rowwise_and_edges(gpu):
    for M, N in [(100, 96), (1, 32), (33, 64), (7, 4096)]:
        gate, up = si.glu_operands(M, N, seed=M + N, outliers=True)
        gd, ud = gate.cuda(), up.cuda()
        qr, qc, sr, sc = gpu.glu_fwd_mxfp8(gd, ud, rowwise=True)
        assert qc.numel() == 0 and sc.numel() == 0
        o = _q(bits(gpu.glu_fwd(gd, ud)), oracle.ROWWISE)
        assert np.array_equal(u8(qr), o[0]) and np.array_equal(u8(sr), o[1])
    e = torch.empty(0, 64, dtype=torch.bfloat16, device="cuda")
    out = gpu.glu_fwd_mxfp8(e, e, rowwise=True, colwise=True)
    assert out[0].shape == (0, 64)


@pytest.mark.parametrize("M,N", [(352, 480), (160, 4128), (4224, 96)])
def test_partial_tiles_every_direction(gpu, M, N):
    """Tile edges in M and N with odd scale-row lengths (N/32, M/32 not multiples of 4), so
    the write-out takes its byte-wise scale path; fused == Q(BF16 GLU output) bit for bit."""
    gate, up, dh = si.glu_operands(M, N, seed=M * 7 + N, outliers=True, with_dh=True)
    gd, ud, dd = gate.cuda(), up.cuda(), dh.cuda()
    h = bits(gpu.glu_fwd(gd, ud, act="geglu"))
    da, db = gpu.glu_bwd(gd, ud, dd, act="geglu")
    X = np.concatenate([bits(da), bits(db)], axis=1)
    paired = torch.stack([gd, ud], 2).reshape(M, 2 * N).contiguous()
    for row, col in FLAGS:
        o = _q(h, _flags(row, col))
        for out in (gpu.glu_fwd_mxfp8(gd, ud, act="geglu", rowwise=row, colwise=col),
                    gpu.glu_fwd_mxfp8(paired, None, act="geglu", layout="paired", rowwise=row,
                                      colwise=col)):
            if row:
                assert np.array_equal(u8(out[0]), o[0]) and np.array_equal(u8(out[2]), o[1])
            if col:
                assert np.array_equal(u8(out[1]), o[2]) and np.array_equal(u8(out[3]), o[3])
        ob = _q(X, _flags(row, col))
        out = gpu.glu_bwd_mxfp8(gd, ud, dd, act="geglu", rowwise=row, colwise=col)
        if row:
            assert np.array_equal(u8(out[0]), ob[0]) and np.array_equal(u8(out[2]), ob[1])
        if col:
            assert np.array_equal(u8(out[1]), ob[2]) and np.array_equal(u8(out[3]), ob[3])


@pytest.mark.parametrize("M,N", [(352, 480), (160, 224), (256, 96), (130, 4160)])
def test_swizzled_scales_match_oracle(gpu, M, N):
    """GLU_SF_SWIZZLED: both scale matrices in the zero-padded 128x4 layout, forward, backward
    and the FP32 hook, bit for bit against the oracle (whose padding is zero; the device
    buffers start uninitialized, so every padding byte must be written).  N = 224 starts db's
    scales off a 4-column boundary and leaves padding past the last colwise tile; M = 130
    (rowwise only) pads 126 rows."""
    gate, up, dh = si.glu_operands(M, N, seed=M + 3 * N, outliers=True, with_dh=True)
    gd, ud, dd = gate.cuda(), up.cuda(), dh.cuda()
    h = bits(gpu.glu_fwd(gd, ud))
    da, db = gpu.glu_bwd(gd, ud, dd)
    X = np.concatenate([bits(da), bits(db)], axis=1)
    for row, col in FLAGS:
        if col and M % 32:
            continue
        f = _flags(row, col) | oracle.SF_SWIZZLED
        for got, want in ((gpu.glu_fwd_mxfp8(gd, ud, rowwise=row, colwise=col, swizzled=True), _q(h, f)),
                          (gpu.glu_bwd_mxfp8(gd, ud, dd, rowwise=row, colwise=col, swizzled=True), _q(X, f))):
            if row:
                assert np.array_equal(u8(got[0]), want[0]) and np.array_equal(u8(got[2]), want[1])
            if col:
                assert np.array_equal(u8(got[1]), want[2]) and np.array_equal(u8(got[3]), want[3])
    x = si.from_bits(h).float().numpy()
    f = oracle.ROWWISE | (oracle.COLWISE if M % 32 == 0 else 0) | oracle.SF_SWIZZLED
    got = gpu.glu_quant_mxfp8_f32(torch.from_numpy(x).cuda(), rowwise=True, colwise=bool(f & 2),
                                  swizzled=True)
    want = oracle.quant_mxfp8(x, f)
    assert np.array_equal(u8(got[2]), want[1])
    if f & 2:
        assert np.array_equal(u8(got[3]), want[3])


def test_row_slices_are_batch_invariant(gpu):
    gate, up = si.glu_operands(256, 256, seed=9, outliers=True)
    gd, ud = gate.cuda(), up.cuda()
    full = gpu.glu_fwd_mxfp8(gd, ud, rowwise=True, colwise=True)
    part = gpu.glu_fwd_mxfp8(gd[64:160], ud[64:160], rowwise=True, colwise=True)
    assert torch.equal(full[0][64:160], part[0]) and torch.equal(full[2][64:160], part[2])
    assert torch.equal(full[1][:, 64:160], part[1]) and torch.equal(full[3][:, 2:5], part[3])
    again = gpu.glu_fwd_mxfp8(gd, ud, rowwise=True, colwise=True)
    assert all(torch.equal(a, b) for a, b in zip(full, again))


# ---- rule 3 on the workload shapes ---------------------------------------------------

def _rule3_rows(h_bits, out, oref, what):
    qr, qc, sr, sc = out
    if qr.numel():
        check_rule3_mx(h_bits, u8(qr), u8(sr), oref[0], oref[1], what + " rowwise")
    if qc.numel():
        check_rule3_mx(np.ascontiguousarray(h_bits.T), u8(qc), u8(sc), oref[2], oref[3], what + " colwise")


def test_config_small_swiglu_fwd_rowwise(gpu):
    gate, up = si.glu_operands(128, 128, seed=0)
    gb, ub = bits(gate), bits(up)
    out = gpu.glu_fwd_mxfp8(gate.cuda(), up.cuda(), rowwise=True)
    _rule3_rows(oracle.glu_fwd(oracle.SWIGLU, gb, ub), out,
                oracle.glu_fwd_mxfp8(oracle.SWIGLU, gb, ub, flags=1), "128x128")


def test_config_mid_swiglu_fwd_bwd_both(gpu):
    gate, up, dh = si.glu_operands(4096, 2048, seed=0, with_dh=True)
    gb, ub, db_ = bits(gate), bits(up), bits(dh)
    gd, ud, dd = gate.cuda(), up.cuda(), dh.cuda()
    out = gpu.glu_fwd_mxfp8(gd, ud, rowwise=True, colwise=True)
    _rule3_rows(oracle.glu_fwd(oracle.SWIGLU, gb, ub), out,
                oracle.glu_fwd_mxfp8(oracle.SWIGLU, gb, ub, flags=3), "4096x2048 fwd")
    out = gpu.glu_bwd_mxfp8(gd, ud, dd, rowwise=True, colwise=True)
    oa, ob = oracle.glu_bwd(oracle.SWIGLU, gb, ub, db_)
    _rule3_rows(np.concatenate([oa, ob], 1), out,
                oracle.glu_bwd_mxfp8(oracle.SWIGLU, gb, ub, db_, flags=3), "4096x2048 bwd")


@pytest.mark.parametrize("name,kind", ACTS[1:])
def test_other_activations_fwd_bwd_both(gpu, name, kind):
    """Rule 3 end to end for the other activations at a shape with ragged tiles in both
    directions."""
    gate, up, dh = si.glu_operands(352, 480, seed=kind, outliers=True, with_dh=True)
    gb, ub, db_ = bits(gate), bits(up), bits(dh)
    gd, ud, dd = gate.cuda(), up.cuda(), dh.cuda()
    out = gpu.glu_fwd_mxfp8(gd, ud, act=name, rowwise=True, colwise=True)
    _rule3_rows(oracle.glu_fwd(kind, gb, ub), out,
                oracle.glu_fwd_mxfp8(kind, gb, ub, flags=3), f"{name} fwd")
    out = gpu.glu_bwd_mxfp8(gd, ud, dd, act=name, rowwise=True, colwise=True)
    oa, ob = oracle.glu_bwd(kind, gb, ub, db_)
    _rule3_rows(np.concatenate([oa, ob], 1), out,
                oracle.glu_bwd_mxfp8(kind, gb, ub, db_, flags=3), f"{name} bwd")


def _full_rule3_mx(gb, ub, db_, out, flags, what, chunk=1024):
    """Rule 3 over every output of a fused launch, against the oracle run on row chunks of the
    same inputs (db_ None: forward).  out = (q_row, q_col, s_row, s_col) as host arrays, the
    disabled direction's empty.  Chunks are checked in a small thread pool (the oracle runs
    OpenMP inside each call, numpy releases the interpreter lock)."""
    import concurrent.futures as cf
    M = gb.shape[0]
    qr, qc, sr, sc = out

    def one(r0):
        r = slice(r0, r0 + chunk)
        acc_r, acc_c = rule3_mx(what + " rowwise"), rule3_mx(what + " colwise")
        if db_ is None:
            o = oracle.glu_fwd_mxfp8(oracle.SWIGLU, gb[r], ub[r], flags=flags)
            h = oracle.glu_fwd(oracle.SWIGLU, gb[r], ub[r])
        else:
            o = oracle.glu_bwd_mxfp8(oracle.SWIGLU, gb[r], ub[r], db_[r], flags=flags)
            h = np.concatenate(oracle.glu_bwd(oracle.SWIGLU, gb[r], ub[r], db_[r]), axis=1)
        if flags & oracle.ROWWISE:
            acc_r.add(h, qr[r], sr[r], o[0], o[1])
        if flags & oracle.COLWISE:
            acc_c.add(np.ascontiguousarray(h.T), qc[:, r], sc[:, r0 // 32:(r0 + chunk) // 32], o[2], o[3])
        return acc_r, acc_c

    tot_r, tot_c = rule3_mx(what + " rowwise"), rule3_mx(what + " colwise")
    with cf.ThreadPoolExecutor(max_workers=4) as ex:
        for acc_r, acc_c in ex.map(one, range(0, M, chunk)):
            tot_r.merge(acc_r)
            tot_c.merge(acc_c)
    res = {}
    if flags & oracle.ROWWISE:
        res["rowwise"] = tot_r.finish()
    if flags & oracle.COLWISE:
        res["colwise"] = tot_c.finish()
    return res


def _host(out):
    return tuple(u8(t) for t in out)


@pytest.mark.parametrize("direction", ["fwd", "bwd"])
def test_config_large_swiglu_outliers_full(gpu, direction):
    """[16384, 7168] with 0.1% x1000 outliers, both scalings: rule 3 on every code and scale
    of the fused launch (as the benchmark launches it), forward or backward."""
    M, N = 16384, 7168
    g, u, d = si.normal_bf16_device([(M, N)] * 3, seed=0, outliers=True)
    if direction == "fwd":
        out = gpu.glu_fwd_mxfp8(g, u, rowwise=True, colwise=True)
    else:
        out = gpu.glu_bwd_mxfp8(g, u, d, rowwise=True, colwise=True)
    torch.cuda.synchronize()
    gb, ub = bits(g), bits(u)
    db_ = bits(d) if direction == "bwd" else None
    res = _full_rule3_mx(gb, ub, db_, _host(out), 3, f"{direction} 16384x7168")
    assert res["rowwise"]["codes"] == (2 if direction == "bwd" else 1) * M * N
    assert res["colwise"]["codes"] == (2 if direction == "bwd" else 1) * M * N


def test_rowwise_bwd_streaming_stores_sampled(gpu):
    """Rowwise-only backward whose codes (2 x 16384 x 8192 bytes) exceed 256 MiB, so they
    leave as non-temporal stores: sampled rows of [da | db] bit-exact against the oracle
    quantizer of the device's own BF16 gradients, and end to end (rule 3) against the
    oracle's backward."""
    M, N = 16384, 8192
    g, u, d = si.normal_bf16_device([(M, N)] * 3, seed=11, outliers=True)
    qr, _, sr, _ = gpu.glu_bwd_mxfp8(g, u, d, rowwise=True)
    da, db = gpu.glu_bwd(g, u, d)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    rows = torch.tensor(sorted({0, M - 1, *rng.integers(0, M, 24).tolist()}), device="cuda")
    o = _q(np.concatenate([bits(da[rows]), bits(db[rows])], axis=1), oracle.ROWWISE)
    assert np.array_equal(u8(qr[rows]), o[0]) and np.array_equal(u8(sr[rows]), o[1])
    gb, ub, dbits = bits(g[rows]), bits(u[rows]), bits(d[rows])
    oe = oracle.glu_bwd_mxfp8(oracle.SWIGLU, gb, ub, dbits, flags=1)
    x = np.concatenate(oracle.glu_bwd(oracle.SWIGLU, gb, ub, dbits), axis=1)
    check_rule3_mx(x, u8(qr[rows]), u8(sr[rows]), oe[0], oe[1], "bwd 16384x8192")


def test_config_xlarge_swiglu_fwd_rowwise_full(gpu):
    """[131072, 8192] with the same outlier recipe, forward rowwise: rule 3 on every code and
    scale (1.07e9 codes)."""
    M, N = 131072, 8192
    g, u = si.normal_bf16_device([(M, N)] * 2, seed=0, outliers=True)
    qr, _, sr, _ = gpu.glu_fwd_mxfp8(g, u, rowwise=True)
    torch.cuda.synchronize()
    gb, ub = bits(g), bits(u)
    del g, u
    empty = np.zeros((0, 0), np.uint8)
    res = _full_rule3_mx(gb, ub, None, (u8(qr), empty, u8(sr), empty), 1, "fwd 131072x8192", chunk=2048)
    assert res["rowwise"]["codes"] == M * N


def test_int32_bound_paired_operand_2pow31(gpu):
    """The largest legal shape of the 32-bit bound: an interleaved [131072, 16384] operand holds
    2^31 elements (4 GiB), past every 32-bit element and byte index.  glu_fwd and the rowwise
    fused forward take it whole; sampled rows, the last included, are checked against the
    oracle: h within one BF16 ulp (rule 2), the codes and scales bit-exact against the oracle
    quantizer of the device's own h (rule 1) and end to end (rule 3)."""
    M, H = 131072, 8192
    x = si.normal_bf16_device([(M, 2 * H)], seed=5)[0]
    assert x.numel() == 2 ** 31
    h = gpu.glu_fwd(x, None, layout="paired")
    qr, _, sr, _ = gpu.glu_fwd_mxfp8(x, None, layout="paired", rowwise=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(12)
    rows = torch.tensor(sorted({0, 1, M // 2, M - 2, M - 1, *rng.integers(0, M, 27).tolist()}), device="cuda")
    xr = bits(x[rows])
    gb, ub = np.ascontiguousarray(xr[:, 0::2]), np.ascontiguousarray(xr[:, 1::2])
    hb = bits(h[rows])
    check_rule2(hb, oracle.glu_fwd(oracle.SWIGLU, gb, ub), "h at 2^31 elements")
    o = _q(hb, oracle.ROWWISE)
    assert np.array_equal(u8(qr[rows]), o[0]) and np.array_equal(u8(sr[rows]), o[1])
    oe = oracle.glu_fwd_mxfp8(oracle.SWIGLU, gb, ub, flags=1)
    check_rule3_mx(oracle.glu_fwd(oracle.SWIGLU, gb, ub), u8(qr[rows]), u8(sr[rows]), oe[0], oe[1], "2^31 paired")


@pytest.mark.parametrize("transposed", [False, True])
def test_every_bf16_value_under_every_scale_fused(gpu, transposed):
    """Rule 1 through the fused kernels on the sweep matrix (every scale byte 0..247 with every
    BF16 magnitude at that scale, every BF16 number as a block maximum, zero and subnormal
    blocks): ReLU^2 with gate = 1 gives h = up exactly, and in the backward (up = 0.5)
    da = db = dh exactly, so the quantizers see the sweep values themselves.  Forward rowwise
    (the row kernel), colwise and both (the tiled kernel), backward rowwise and both; the
    transposed matrix puts the blocks in columns.  Codes and scales are compared byte for byte
    with the oracle quantizer of the device's own h, da, db, which are first checked to equal
    the sweep values."""
    X = mxfp8_sweep_matrix()
    if transposed:
        X = np.ascontiguousarray(X.T)
    x = si.from_bits(X).cuda()
    one = torch.ones_like(x)
    h = bits(gpu.glu_fwd(one, x, act="relu2"))
    assert np.array_equal(h, X), "h = up"
    xf = si.from_bits(X).float().numpy()
    for row, col in FLAGS:
        qr, qc, sr, sc = gpu.glu_fwd_mxfp8(one, x, act="relu2", rowwise=row, colwise=col)
        o = oracle.quant_mxfp8(xf, _flags(row, col))
        if row:
            assert np.array_equal(u8(sr), o[1]) and np.array_equal(u8(qr), o[0]), f"fwd rowwise ({row}, {col})"
        if col:
            assert np.array_equal(u8(sc), o[3]) and np.array_equal(u8(qc), o[2]), f"fwd colwise ({row}, {col})"
    half = torch.full_like(x, 0.5)
    da, db = gpu.glu_bwd(one, half, x, act="relu2")
    assert np.array_equal(bits(da), X) and np.array_equal(bits(db), X), "da = db = dh"
    xx = np.concatenate([xf, xf], axis=1)
    for row, col in [(True, False), (True, True)]:
        qr, qc, sr, sc = gpu.glu_bwd_mxfp8(one, half, x, act="relu2", rowwise=row, colwise=col)
        o = oracle.quant_mxfp8(xx, _flags(row, col))
        assert np.array_equal(u8(sr), o[1]) and np.array_equal(u8(qr), o[0]), f"bwd rowwise ({row}, {col})"
        if col:
            assert np.array_equal(u8(sc), o[3]) and np.array_equal(u8(qc), o[2]), "bwd colwise"
