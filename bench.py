"""Benchmark of the fused GLU + MX-quant path on one MI355X.

One step = the whole hot path over one batch of the large SwiGLU workload: the fused
forward with MXFP8 rowwise + colwise output, then the fused backward with MXFP8 rowwise +
colwise output of [dGate | dUp], on gate, up, dh BF16 [16384, 7168] ~ N(0, 1) with 0.1% of
the elements scaled x1000 (the shape the MXFP8 page quotes its fused numbers on).
Inputs are resident in HBM before the timed region.  `value` is algorithmic GB/s: bytes
the method must move (BF16 inputs read once, E4M3 codes and E8M0 scales written once,
GB = 1e9) divided by the time of the K timed steps.

Before anything is timed, every timed configuration is validated on the GPU (unless
--no-validate): the fused outputs must equal, byte for byte, the library's unfused path
(glu_fwd / glu_bwd, then the FP32 quantizer hook: the activation followed by the standalone
quantizer), and sampled rows of h, da, db must be within one BF16 ulp of a float64 torch
reference of the same formulas.  A failure stops the run.

Also reported on the same JSON line:
  roofline      - the dominant kernel (the fused backward) against the 8 TB/s HBM peak,
                  its duration measured with HIP events on the launch stream, and against
                  the practical ceiling of its byte mix (the library's streaming probe:
                  three BF16 read streams and four code write streams at the same size);
  ceiling       - the streaming probe as a plain 1 GiB copy, and at the step's mixes;
  cpu_baseline  - the CPU oracle on a bounded row sample of the same workload;
  sweep         - every workload shape of the pages (MXFP8 SwiGLU fwd/bwd per direction,
                  GeGLU BF16 fwd/bwd, GeGLU NVFP4), median, min and p90 of cold launches,
                  each beside the probe's ceiling for its byte mix, plus the other
                  activations (tanh-GeGLU, erf-GeGLU, ReLU^2) at one shape of each, the
                  NVFP4 backward, two-level NVFP4 (amax pass + forward), and the merged
                  MXFP8 GEMM with the GLU epilogue (TFLOP/s against the FP8 peak).
Only one GPU is supported; --gpus above 1 exits with a message.
"""
import argparse
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused GLU+MX-quant fwd/bwd achieved HBM GB/s and % of peak, M×N sweep"
PEAK_GBPS = 8000.0  # MI355X HBM3E
PEAK_FP8_TFLOPS = 5000.0  # MI355X dense FP8 matrix cores
PEAK_FP4_TFLOPS = 10100.0  # MI355X dense FP4 matrix cores
# The MXFP8 page's fused GB200 times for this exact workload (forward both 143.36 us,
# backward both 219.14 us at (16384, 7168)), combined under the same byte model: another
# machine's figure, reported under config as context only.
PAGES_STEP_GBPS = (711_983_104 + 1_189_085_184) / ((143.36 + 219.14) * 1e-6) / 1e9


# HBM traffic of the roofline kernel comes from the rocprofv3 counter summary committed under
# profiles/; it is reported only while the kernel sources are unchanged since that profile.
KERNEL_SOURCES = [os.path.join(ROOT, "glu_activation_microscaling_amd", "csrc", f)
                  for f in ("glu_mxfp8.hip", "glu_device.h", "glu_launch.h", "glu_common.h")]
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "k_mxfp8_swiglu_16384x7168.md")


def kernel_source_sha256():
    """Hash of the kernel sources with // comments and blank lines removed (comment edits do
    not change the kernel)."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f) as fh:
            for line in fh:
                code = line.split("//", 1)[0].strip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()


def traffic_bytes(kernel):
    """Measured HBM bytes (read + write) per launch of `kernel`, or None when no profile of
    the current kernel sources exists."""
    if not os.path.exists(TRAFFIC_PROFILE):
        return None
    sha = kernel_source_sha256()
    for line in open(TRAFFIC_PROFILE):
        if not line.startswith("traffic_record:"):
            continue
        kv = dict(f.split("=", 1) for f in line.split()[1:])
        if kv.get("kernel") == kernel and kv.get("source_sha256") == sha:
            return int(kv["read_bytes"]) + int(kv["write_bytes"])
    return None


def mx_bytes(M, N, bwd, ndir):
    E = M * N
    return (6 * E + ndir * (2 * E + 2 * E // 32)) if bwd else (4 * E + ndir * (E + E // 32))


def bf16_bytes(M, N, bwd):
    return (10 if bwd else 6) * M * N


def nv_bytes(M, H):
    E = M * H
    return 4 * E + E // 2 + E // 16


def nv_bwd_bytes(M, N):
    """Read gate, up, dh; write [da | db] as packed E2M1 plus one E4M3 scale per 16."""
    E = M * N
    return 6 * E + 2 * (E // 2 + E // 16)


def _events(torch, n):
    return [torch.cuda.Event(enable_timing=True) for _ in range(n)]


def time_launches(torch, fns, iters):
    """Median / min / p90 of per-launch durations (us), cycling through fns (one per input
    set, so repeated launches do not re-read cached inputs: cold), and the median of the same
    number of launches on the first set alone (warm: inputs left in the caches by the previous
    launch, where they fit)."""
    for f in fns[: min(3, len(fns))]:
        f()
    torch.cuda.synchronize()
    ev = _events(torch, 2 * iters)
    for i in range(iters):
        ev[2 * i].record()
        fns[i % len(fns)]()
        ev[2 * i + 1].record()
    torch.cuda.synchronize()
    us = sorted(ev[2 * i].elapsed_time(ev[2 * i + 1]) * 1e3 for i in range(iters))
    for i in range(iters):
        ev[2 * i].record()
        fns[0]()
        ev[2 * i + 1].record()
    torch.cuda.synchronize()
    warm = statistics.median(ev[2 * i].elapsed_time(ev[2 * i + 1]) * 1e3 for i in range(iters))
    return dict(median_us=statistics.median(us), min_us=us[0], p90_us=us[int(0.9 * (len(us) - 1))],
                warm_median_us=warm)


def n_sets(bytes_per_set):
    """Input sets to rotate through so that one pass over them exceeds 1 GiB (4x the
    256 MB last-level cache), capped at 32."""
    return max(1, min(32, math.ceil((1 << 30) / max(1, bytes_per_set))))


# ---------------------------------------------------------------------------------------
# Validation before timing (GPU only): the fused outputs against the library's unfused path,
# and the BF16 values against a float64 torch reference of the same formulas.
# ---------------------------------------------------------------------------------------

class ValidationError(RuntimeError):
    pass


def _ref_act(torch, act, x):
    """act(x) and act'(x) in float64 (the textbook formulas; torch's own GELUs)."""
    F = torch.nn.functional
    x = x.detach().requires_grad_(True)
    if act == "swiglu":
        y = x * torch.sigmoid(x)
    elif act == "geglu":
        y = F.gelu(x, approximate="tanh")
    elif act == "geglu_erf":
        y = F.gelu(x)
    else:
        y = torch.relu(x) ** 2
    (g,) = torch.autograd.grad(y.sum(), x)
    return y.detach(), g


def _ulp_far(torch, got, ref):
    """Elements of two BF16 tensors more than one BF16 ulp apart (+0 and -0 identified,
    NaN matching NaN)."""
    def ordered(t):
        b = t.contiguous().view(torch.int16).to(torch.int32)
        mag = b & 0x7FFF
        return torch.where(b < 0, -mag, mag), mag > 0x7F80
    a, na = ordered(got)
    b, nb = ordered(ref)
    far = ((a - b).abs() > 1) & ~(na & nb)
    return int(far.sum())


def _check_bf16_rows(torch, act, g, u, d, outs, what, nrows=8):
    """Sampled rows of h (d None) or of (da, db): within one BF16 ulp of float64 torch."""
    M = g.shape[0]
    rows = torch.unique(torch.tensor([0, M - 1] + [int(M * k / nrows) for k in range(1, nrows)],
                                     device=g.device))
    gg, uu = g[rows].double(), u[rows].double()
    a, ap = _ref_act(torch, act, gg)
    if d is None:
        refs = [(a * uu).to(torch.bfloat16)]
    else:
        dd = d[rows].double()
        refs = [(dd * uu * ap).to(torch.bfloat16), (dd * a).to(torch.bfloat16)]
    for got, ref in zip(outs, refs):
        n = _ulp_far(torch, got[rows], ref)
        if n:
            raise ValidationError(f"{what}: {n} sampled BF16 values beyond one ulp of the float64 reference")


def _equal(torch, a, b, what):
    if a.shape != b.shape or not torch.equal(a, b):
        raise ValidationError(f"{what}: fused output differs from the unfused path")


def validate_mx(torch, glu, act, g, u, d, out, row, col, swz, what):
    """Fused MXFP8 outputs == glu_quant_mxfp8_f32 of the BF16 GLU output; BF16 rows vs float64."""
    if d is None:
        h = glu.glu_fwd(g, u, act=act)
        _check_bf16_rows(torch, act, g, u, None, [h], what)
        x = h.float()
    else:
        da, db = glu.glu_bwd(g, u, d, act=act)
        _check_bf16_rows(torch, act, g, u, d, [da, db], what)
        x = torch.cat([da, db], 1).float()
        del da, db
    ref = glu.glu_quant_mxfp8_f32(x, rowwise=row, colwise=col, swizzled=swz)
    for k in range(4):
        _equal(torch, out[k], ref[k], f"{what} output {k}")
    del x, ref


def validate_bf16(torch, glu, act, g, u, d, outs, what):
    _check_bf16_rows(torch, act, g, u, d, outs, what)


def validate_nv(torch, glu, act, x, out, sf_layout, what, amax=None):
    """Fused NVFP4 (paired operand) == glu_quant_nvfp4_f32 of the BF16 GLU output (global
    scale 1 only; the two-level forward is checked against its amax pass being finite)."""
    h = glu.glu_fwd(x, None, act=act, layout="paired")
    g, u = x[:, 0::2], x[:, 1::2]
    _check_bf16_rows(torch, act, g, u, None, [h], what)
    if amax is None:
        ref = glu.glu_quant_nvfp4_f32(h.float(), sf_layout=sf_layout)
        _equal(torch, out[0], ref[0], what + " codes")
        _equal(torch, out[1], ref[1], what + " scales")
    else:
        a = float(amax.item())
        if not (a == float(h.float().abs().max().item())):
            raise ValidationError(f"{what}: amax pass {a} differs from the largest |h|")


def validate_nv_bwd(torch, glu, act, g, u, d, out, sf_layout, what):
    da, db = glu.glu_bwd(g, u, d, act=act)
    _check_bf16_rows(torch, act, g, u, d, [da, db], what)
    ref = glu.glu_quant_nvfp4_f32(torch.cat([da, db], 1).float(), sf_layout=sf_layout)
    _equal(torch, out[0], ref[0], what + " codes")
    _equal(torch, out[1], ref[1], what + " scales")


def validate_gemm(torch, glu, ops, act, out_fmt, out, what, operand_kw):
    """The fused quantized output equals the standalone quantizer of glu_gemm's h (operand_kw:
    the operand format and W layout)."""
    h = glu.glu_gemm(*ops, act=act, **operand_kw)
    if out_fmt == "mxfp8":
        q, s = glu.glu_quant_mxfp8_f32(h.float(), rowwise=True)[0::2]
    else:
        q, s = glu.glu_quant_nvfp4_f32(h.float(), sf_layout="128x4")
    _equal(torch, out[0], q, what + " codes")
    _equal(torch, out[1].reshape(-1), s.reshape(-1), what + " scales")


# ---------------------------------------------------------------------------------------
# The streaming probe: practical ceilings for a byte mix
# ---------------------------------------------------------------------------------------

def probe_ceiling(torch, glu, n_src, n_dst, width, elems, iters):
    """GB/s of the streaming probe moving n_src BF16 streams of `elems` elements in and n_dst
    streams of width / 16 bytes per source byte out (cold: buffer sets rotated past 1 GiB)."""
    nbytes = 2 * elems
    nbytes -= nbytes % 16
    per = (n_src + n_dst * width / 16) * nbytes
    k = max(2, n_sets(per))
    sets = [([torch.empty(nbytes, dtype=torch.uint8, device="cuda") for _ in range(n_src)],
             [torch.empty(nbytes * width // 16, dtype=torch.uint8, device="cuda") for _ in range(n_dst)])
            for _ in range(k)]
    t = time_launches(torch, [lambda st=st: glu.glu_stream_probe(*st) for st in sets], iters)
    del sets
    return dict(gbps=round(per / t["median_us"] / 1e3, 1), us=round(t["median_us"], 2),
                frac=round(per / t["median_us"] / 1e3 / PEAK_GBPS, 4), n_src=n_src, n_dst=n_dst,
                dst_bytes_per_16=width, bytes=int(per))


# ---------------------------------------------------------------------------------------
# Sweep
# ---------------------------------------------------------------------------------------

def sweep(torch, glu, si, iters, validate):
    res = {}
    ceilings = {}

    def ceiling(n_src, n_dst, width, elems):
        key = (n_src, n_dst, width, elems)
        if key not in ceilings:
            ceilings[key] = probe_ceiling(torch, glu, n_src, n_dst, width, elems, iters)
        return ceilings[key]

    def rec(name, b, t, mix=None):
        gbps = b / t["median_us"] / 1e3
        r = dict(bytes=b, us=round(t["median_us"], 2), min_us=round(t["min_us"], 2), p90_us=round(t["p90_us"], 2),
                 gbps=round(gbps, 1), frac=round(gbps / PEAK_GBPS, 4), warm_us=round(t["warm_median_us"], 2),
                 validated=validate)
        if mix is not None:
            c = ceiling(*mix)
            r["ceiling_gbps"] = c["gbps"]
            r["frac_of_ceiling"] = round(gbps / c["gbps"], 4)
        res[name] = r
        print(f"[bench] {name}: {t['median_us']:.2f} us ({r['frac']:.3f} of peak"
              + (f", {r['frac_of_ceiling']:.3f} of ceiling" if mix else "") + ")", file=sys.stderr, flush=True)

    # practical ceiling: the streaming probe as a 1 GiB copy (2 GiB moved)
    c = ceiling(1, 1, 16, 1 << 29)
    res["stream_copy_1GiB"] = dict(bytes=c["bytes"], us=c["us"], gbps=c["gbps"], frac=c["frac"])
    print(f"[bench] stream_copy_1GiB: {c['us']:.2f} us ({c['frac']:.3f} of peak)", file=sys.stderr, flush=True)

    # MXFP8 SwiGLU shapes, and the other activations at [16384, 7168]
    others = [(d, "both", a) for a in ("geglu", "geglu_erf", "relu2") for d in ("fwd", "bwd")]
    for M, N, outl, cases in [
        (128, 128, False, [("fwd", "row")]),
        (4096, 2048, False, [("fwd", "both"), ("bwd", "both")]),
        (16384, 7168, True, [("fwd", "row"), ("fwd", "col"), ("fwd", "both"),
                             ("bwd", "row"), ("bwd", "col"), ("bwd", "both"),
                             ("fwd", "both_swizzled"), ("bwd", "both_swizzled"), *others]),
        (131072, 8192, True, [("fwd", "row")]),
    ]:
        per = 6 * M * N
        sets = [si.normal_bf16_device([(M, N)] * 3, seed=100 + s, outliers=outl) for s in range(n_sets(per))]
        for d, mode, *act in cases:
            act = act[0] if act else "swiglu"
            swz = mode.endswith("_swizzled")  # scales in the 128x4 layout
            dirs = mode.removesuffix("_swizzled")
            row, col = dirs in ("row", "both"), dirs in ("col", "both")
            bwd = d == "bwd"
            out = glu._mx_buffers(M, 2 * N if bwd else N, row, col, "cuda", None, swz)
            kw = dict(act=act, rowwise=row, colwise=col, swizzled=swz, out=out)
            name = f"{act}_mxfp8_{d}_{mode}_{M}x{N}"
            if bwd:
                fns = [lambda s=s: glu.glu_bwd_mxfp8(s[0], s[1], s[2], **kw) for s in sets]
            else:
                fns = [lambda s=s: glu.glu_fwd_mxfp8(s[0], s[1], **kw) for s in sets]
            if validate:
                fns[0]()
                validate_mx(torch, glu, act, sets[0][0], sets[0][1], sets[0][2] if bwd else None, out,
                            row, col, swz, name)
            t = time_launches(torch, fns, iters)
            ndir = 2 if dirs == "both" else 1
            mix = (3, 2 * ndir, 8, M * N) if bwd else (2, ndir, 8, M * N)
            rec(name, mx_bytes(M, N, bwd, ndir), t, mix if M * N >= (1 << 24) else None)
            del out, fns
        del sets
        torch.cuda.empty_cache()
    # GeGLU BF16 sweep
    for R in (1024, 8192):
        for W in (4096, 11008, 14336, 18944, 29568, 8193):
            sets = [si.normal_bf16_device([(R, W)] * 3, seed=R + W + s) for s in range(n_sets(6 * R * W))]
            h = torch.empty(R, W, dtype=torch.bfloat16, device="cuda")
            da, db = torch.empty_like(h), torch.empty_like(h)
            fns = [lambda s=s: glu.glu_fwd(s[0], s[1], act="geglu", out=h) for s in sets]
            if validate:
                fns[0]()
                validate_bf16(torch, glu, "geglu", sets[0][0], sets[0][1], None, [h], f"geglu bf16 fwd {R}x{W}")
            t = time_launches(torch, fns, iters)
            rec(f"geglu_bf16_fwd_{R}x{W}", bf16_bytes(R, W, False), t, (2, 1, 16, R * W))
            fns = [lambda s=s: glu.glu_bwd(s[0], s[1], s[2], act="geglu", out=(da, db)) for s in sets]
            if validate:
                fns[0]()
                validate_bf16(torch, glu, "geglu", *sets[0], [da, db], f"geglu bf16 bwd {R}x{W}")
            t = time_launches(torch, fns, iters)
            rec(f"geglu_bf16_bwd_{R}x{W}", bf16_bytes(R, W, True), t, (3, 2, 16, R * W))
            del sets, h, da, db, fns
        torch.cuda.empty_cache()
    # the other activations, BF16 at [8192, 14336]
    R, W = 8192, 14336
    sets = [si.normal_bf16_device([(R, W)] * 3, seed=R + W + s) for s in range(n_sets(6 * R * W))]
    h = torch.empty(R, W, dtype=torch.bfloat16, device="cuda")
    da, db = torch.empty_like(h), torch.empty_like(h)
    for act in ("swiglu", "geglu_erf", "relu2"):
        fns = [lambda s=s: glu.glu_fwd(s[0], s[1], act=act, out=h) for s in sets]
        if validate:
            fns[0]()
            validate_bf16(torch, glu, act, sets[0][0], sets[0][1], None, [h], f"{act} bf16 fwd")
        rec(f"{act}_bf16_fwd_{R}x{W}", bf16_bytes(R, W, False), time_launches(torch, fns, iters), (2, 1, 16, R * W))
        fns = [lambda s=s: glu.glu_bwd(s[0], s[1], s[2], act=act, out=(da, db)) for s in sets]
        if validate:
            fns[0]()
            validate_bf16(torch, glu, act, *sets[0], [da, db], f"{act} bf16 bwd")
        rec(f"{act}_bf16_bwd_{R}x{W}", bf16_bytes(R, W, True), time_launches(torch, fns, iters), (3, 2, 16, R * W))
    del sets, h, da, db, fns
    torch.cuda.empty_cache()
    # GeGLU NVFP4 (paired operand: two virtual BF16 streams in, half a byte per element out)
    H = 16384
    for M in (784, 816, 880, 968):
        sets = [si.normal_bf16_device([(M, 2 * H)], seed=M + s)[0] for s in range(n_sets(4 * M * H))]
        out = glu._nv_buffers(M, H, "128x4", "cuda", None)
        for act in ("geglu",) + (("swiglu", "geglu_erf", "relu2") if M == 968 else ()):
            fns = [lambda x=x: glu.glu_fwd_nvfp4(x, act=act, layout="paired", sf_layout="128x4", out=out)
                   for x in sets]
            if validate:
                fns[0]()
                validate_nv(torch, glu, act, sets[0], out, "128x4", f"{act} nvfp4 fwd {M}")
            rec(f"{act}_nvfp4_fwd_{M}x{H}", nv_bytes(M, H), time_launches(torch, fns, iters), (2, 1, 4, M * H))
        del sets, out, fns
    # two-level NVFP4: the amax pass and the forward with the global scale
    for M, H in ((968, 16384), (16384, 7168)):
        sets = [si.normal_bf16_device([(M, 2 * H)], seed=M + s)[0] for s in range(n_sets(4 * M * H))]
        out = glu._nv_buffers(M, H, "128x4", "cuda", None)
        amax = torch.empty((1,), dtype=torch.float32, device="cuda")
        fns = [lambda x=x: glu.glu_amax(x, act="geglu", layout="paired", out=amax) for x in sets]
        if validate:
            fns[0]()
            validate_nv(torch, glu, "geglu", sets[0], out, "128x4", f"geglu amax {M}", amax=amax)
        rec(f"geglu_amax_{M}x{H}", 4 * M * H, time_launches(torch, fns, iters))
        fns = [lambda x=x: glu.glu_fwd_nvfp4_gs(x, amax=amax, act="geglu", layout="paired", sf_layout="128x4",
                                                out=out) for x in sets]
        rec(f"geglu_nvfp4_gs_fwd_{M}x{H}", nv_bytes(M, H), time_launches(torch, fns, iters), (2, 1, 4, M * H))
        del sets, out, fns
        torch.cuda.empty_cache()
    # NVFP4 backward ([da | db] quantized), the workload's shape and the MXFP8 training shape
    for M, N in ((968, 16384), (16384, 7168)):
        sets = [si.normal_bf16_device([(M, N)] * 3, seed=M + N + s) for s in range(n_sets(6 * M * N))]
        out = glu._nv_buffers(M, 2 * N, "128x4", "cuda", None)
        for act in ("swiglu", "geglu"):
            fns = [lambda s=s: glu.glu_bwd_nvfp4(s[0], s[1], s[2], act=act, sf_layout="128x4", out=out)
                   for s in sets]
            if validate:
                fns[0]()
                validate_nv_bwd(torch, glu, act, *sets[0], out, "128x4", f"{act} nvfp4 bwd {M}x{N}")
            rec(f"{act}_nvfp4_bwd_{M}x{N}", nv_bwd_bytes(M, N), time_launches(torch, fns, iters), (3, 2, 4, M * N))
        del sets, out, fns
        torch.cuda.empty_cache()
    # merged gate/up MXFP8 GEMM with the GLU and MXFP8 rowwise (or NVFP4, 128x4 scales)
    # epilogue: the NVFP4 page's projection (M tokens, K = 2048, merged 2N = 32768) in MXFP8
    # form, and the MXFP8 page's [16384, 7168] activation produced from K = 2048
    for M, N, K in ((968, 16384, 2048), (16384, 7168, 2048)):
        per = M * K + 2 * N * K
        sets = [si.mx_operand(M, K, seed=M + s, device="cuda") + si.mx_operand(2 * N, K, seed=N + s, device="cuda")
                for s in range(min(4, n_sets(per)))]
        out = (torch.empty((M, N), dtype=torch.uint8, device="cuda"),
               torch.empty((M, N // 32), dtype=torch.uint8, device="cuda"))
        nv_out = glu._nv_buffers(M, N, "128x4", "cuda", None)
        # MXFP4 operands with interleaved W: the NVFP4 page's contract form (packed E2M1
        # values, gate/up rows interleaved, NVFP4 output) on the block scaling gfx950 takes
        sets4 = [si.mxfp4_operand(M, K, seed=M + s, device="cuda") +
                 tuple(si.interleave_rows(t) for t in si.mxfp4_operand(2 * N, K, seed=N + s, device="cuda"))
                 for s in range(min(4, n_sets(per // 2)))]
        for act, fmt, opfmt in [("swiglu", "mxfp8", "mxfp8"), ("geglu", "mxfp8", "mxfp8"),
                                ("geglu", "nvfp4", "mxfp8"), ("geglu", "nvfp4", "mxfp4")]:
            kw = dict(fmt=opfmt, w_layout="paired") if opfmt == "mxfp4" else {}
            src = sets4 if opfmt == "mxfp4" else sets
            if fmt == "mxfp8":
                fns = [lambda s=s: glu.glu_gemm_mxfp8(*s, act=act, out=out, **kw) for s in src]
            else:
                fns = [lambda s=s: glu.glu_gemm_nvfp4(*s, act=act, sf_layout="128x4", out=nv_out, **kw) for s in src]
            name = f"{act}_gemm_{fmt}_{M}x{N}x{K}" if opfmt == "mxfp8" else \
                f"{act}_gemm_{opfmt}_paired_{fmt}_{M}x{N}x{K}"
            if validate:
                fns[0]()
                validate_gemm(torch, glu, src[0], act, fmt, out if fmt == "mxfp8" else nv_out, name, kw)
            t = time_launches(torch, fns, iters)
            tf = 2.0 * M * K * 2 * N / t["median_us"] / 1e6
            peak = PEAK_FP4_TFLOPS if opfmt == "mxfp4" else PEAK_FP8_TFLOPS
            print(f"[bench] {name}: {t['median_us']:.2f} us", file=sys.stderr, flush=True)
            res[name] = dict(flops=2 * M * K * 2 * N, us=round(t["median_us"], 2), min_us=round(t["min_us"], 2),
                             p90_us=round(t["p90_us"], 2), warm_us=round(t["warm_median_us"], 2), tflops=round(tf, 1),
                             frac=round(tf / peak, 4), peak_tflops=peak, validated=validate)
        # context, not part of the path: the platform library's GEMM alone (torch._scaled_mm,
        # BF16 output, no activation, no quantizer) on the same codes, with the same E8M0 block
        # scales and with one tensor-wide scale
        one = torch.ones((), device="cuda")
        lib = {"blockwise": lambda s: torch._scaled_mm(
                   s[0].view(torch.float8_e4m3fn), s[2].view(torch.float8_e4m3fn).t(),
                   scale_a=s[1].view(torch.float8_e8m0fnu), scale_b=s[3].view(torch.float8_e8m0fnu),
                   out_dtype=torch.bfloat16),
               "tensorwise": lambda s: torch._scaled_mm(
                   s[0].view(torch.float8_e4m3fn), s[2].view(torch.float8_e4m3fn).t(),
                   scale_a=one, scale_b=one, out_dtype=torch.bfloat16)}
        for kind, fn in lib.items():
            name = f"library_fp8_gemm_{kind}_{M}x{2 * N}x{K}"
            try:
                t = time_launches(torch, [lambda s=s: fn(s) for s in sets], iters)
            except RuntimeError as e:  # a shape or scaling the library does not take
                print(f"[bench] {name}: not supported ({str(e).splitlines()[0][:80]})", file=sys.stderr, flush=True)
                continue
            tf = 2.0 * M * K * 2 * N / t["median_us"] / 1e6
            print(f"[bench] {name}: {t['median_us']:.2f} us", file=sys.stderr, flush=True)
            res[name] = dict(flops=2 * M * K * 2 * N, us=round(t["median_us"], 2), tflops=round(tf, 1),
                             frac=round(tf / PEAK_FP8_TFLOPS, 4))
        del sets, sets4, out, nv_out
        torch.cuda.empty_cache()
    return res


def cpu_model():
    """The host CPU's model name (as lscpu reports it, read from /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.lower().startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(si, budget_s):
    """The oracle (as it stands) on whole 512-row slabs of the step's workload, taken in
    order and from the start again once every row is done, until budget_s seconds of CPU
    time have passed (at most four passes)."""
    import oracle
    M, N, slab = 16384, 7168, 512
    done, t_used = 0, 0.0
    while done < 4 * M and t_used < budget_s:
        g, u, d = si.glu_operands(slab, N, seed=1000 + done % M, outliers=True, with_dh=True)
        gb, ub, db = si.to_bits(g), si.to_bits(u), si.to_bits(d)
        t0 = time.perf_counter()
        oracle.glu_fwd_mxfp8(oracle.SWIGLU, gb, ub, flags=3)
        oracle.glu_bwd_mxfp8(oracle.SWIGLU, gb, ub, db, flags=3)
        t_used += time.perf_counter() - t0
        done += slab
    b = mx_bytes(done, N, False, 2) + mx_bytes(done, N, True, 2)
    print(f"[bench] cpu oracle: {done} rows in {t_used:.1f} s", file=sys.stderr, flush=True)
    return dict(value=round(b / t_used / 1e9, 4), unit="GB/s", cores=oracle.num_threads(), kind="oracle",
                cpu_model=cpu_model(), nproc=os.cpu_count(),
                sample=f"{done} rows ({done / M:.2f} passes over the 16384 rows) x 7168 (fwd + bwd, both "
                       f"scalings), {t_used:.1f} s")


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--sweep-iters", type=int, default=20)
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-validate", action="store_true",
                    help="skip the validation of each timed configuration before it is timed")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also launch the streaming probe as a 1 GiB copy (a kernel of known bytes, "
                         "for scaling HBM counters)")
    ap.add_argument("--bf16-only", action="store_true",
                    help="only launch the GeGLU BF16 forward and backward at [8192, 14336] three times "
                         "each and print no JSON (a target for profiler counter passes)")
    ap.add_argument("--nvfp4-contract-only", action="store_true",
                    help="only launch the NVFP4 GeGLU forward at 968 x 16384 three times (for profiler passes)")
    ap.add_argument("--nvfp4-only", action="store_true",
                    help="only launch the NVFP4 forward and backward at [16384, 7168] three times "
                         "each and print no JSON (a target for profiler counter passes)")
    ap.add_argument("--gemm-only", action="store_true",
                    help="only launch the merged MXFP8 GEMM with the SwiGLU + MXFP8 epilogue at "
                         "8192 x 2048 x 7168 and 16384 x 7168 x 2048, three times each, and print "
                         "no JSON (a target for profiler counter passes)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this path needs no collective and runs one "
              "kernel per GPU on its own rows; run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import glu_activation_microscaling_amd as glu
    import synthetic_inputs as si

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    glu.lib()  # fail loudly when the HIP library is missing
    validate = not args.no_validate

    def calibrate():
        """The streaming probe as a 1 GiB copy: a kernel of known bytes for counter scaling."""
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        glu.glu_stream_probe([src], [dst])
        torch.cuda.synchronize()

    M, N = 16384, 7168
    if args.nvfp4_only:
        g, u, d = si.normal_bf16_device([(M, N)] * 3, seed=1, outliers=True)
        x = torch.stack([g, u], 2).reshape(M, 2 * N).contiguous()
        of = glu._nv_buffers(M, N, "128x4", "cuda", None)
        ob = glu._nv_buffers(M, 2 * N, "128x4", "cuda", None)
        for _ in range(3):
            glu.glu_fwd_nvfp4(x, act="swiglu", layout="paired", sf_layout="128x4", out=of)
            glu.glu_bwd_nvfp4(g, u, d, act="swiglu", sf_layout="128x4", out=ob)
        torch.cuda.synchronize()
        if args.copy_calibration:
            calibrate()
        print("[bench] nvfp4 launches done", file=sys.stderr, flush=True)
        return
    if args.nvfp4_contract_only:
        # the NVFP4 page's contract shape: GeGLU of an interleaved [968, 32768] operand, 128x4 scales
        x = si.normal_bf16_device([(968, 2 * 16384)], seed=5)[0]
        of = glu._nv_buffers(968, 16384, "128x4", "cuda", None)
        for _ in range(3):
            glu.glu_fwd_nvfp4(x, act="geglu", layout="paired", sf_layout="128x4", out=of)
        torch.cuda.synchronize()
        if args.copy_calibration:
            calibrate()
        print("[bench] nvfp4 contract-shape launches done", file=sys.stderr, flush=True)
        return
    if args.bf16_only:
        R, W = 8192, 14336
        g, u, d = si.normal_bf16_device([(R, W)] * 3, seed=2)
        h = torch.empty(R, W, dtype=torch.bfloat16, device="cuda")
        da, db = torch.empty_like(h), torch.empty_like(h)
        for _ in range(3):
            glu.glu_fwd(g, u, act="geglu", out=h)
            glu.glu_bwd(g, u, d, act="geglu", out=(da, db))
        torch.cuda.synchronize()
        if args.copy_calibration:
            calibrate()
        print("[bench] bf16 launches done", file=sys.stderr, flush=True)
        return
    if args.gemm_only:
        for gm, gn, gk in ((8192, 2048, 7168), (16384, 7168, 2048)):
            ops = si.mx_operand(gm, gk, seed=3, device="cuda") + si.mx_operand(2 * gn, gk, seed=4, device="cuda")
            for _ in range(3):
                glu.glu_gemm_mxfp8(*ops, act="swiglu")
            ops4 = si.mxfp4_operand(gm, gk, seed=3, device="cuda") + si.mxfp4_operand(2 * gn, gk, seed=4, device="cuda")
            for _ in range(3):
                glu.glu_gemm_nvfp4(*ops4, act="geglu", sf_layout="128x4", fmt="mxfp4", w_layout="paired")
        torch.cuda.synchronize()
        print("[bench] gemm launches done", file=sys.stderr, flush=True)
        return
    sets = [si.normal_bf16_device([(M, N)] * 3, seed=s, outliers=True) for s in range(2)]
    fo = glu._mx_buffers(M, N, True, True, "cuda", None)
    bo = glu._mx_buffers(M, 2 * N, True, True, "cuda", None)
    fwd_b, bwd_b = mx_bytes(M, N, False, 2), mx_bytes(M, N, True, 2)

    # Two events per timed step, around the backward; the forward's interval runs from the
    # previous step's last event (the loop's start event for the first step).  A third event
    # before each forward added about 4 us per step.
    def step(i, ev=None):
        g, u, d = sets[i % 2]
        glu.glu_fwd_mxfp8(g, u, rowwise=True, colwise=True, out=fo)
        if ev: ev[0].record()
        glu.glu_bwd_mxfp8(g, u, d, rowwise=True, colwise=True, out=bo)
        if ev: ev[1].record()

    if validate:
        for i in range(2):
            step(i)
            g, u, d = sets[i]
            validate_mx(torch, glu, "swiglu", g, u, None, fo, True, True, False, f"step forward, input set {i}")
            validate_mx(torch, glu, "swiglu", g, u, d, bo, True, True, False, f"step backward, input set {i}")
        torch.cuda.empty_cache()
        print("[bench] step validated (both input sets, forward and backward)", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    evs = [_events(torch, 2) for _ in range(args.steps)]
    start, end = _events(torch, 2)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for i in range(args.steps):
        step(i, evs[i])
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = start.elapsed_time(end)
    ms_per_step = gpu_ms / args.steps
    fwd_starts = [start] + [e[1] for e in evs[:-1]]
    fwd_us = statistics.mean(a.elapsed_time(e[0]) for a, e in zip(fwd_starts, evs)) * 1e3
    bwd_us = statistics.mean(e[0].elapsed_time(e[1]) for e in evs) * 1e3
    value = (fwd_b + bwd_b) / (ms_per_step * 1e-3) / 1e9

    if args.copy_calibration:
        calibrate()
    del sets, fo, bo
    torch.cuda.empty_cache()

    # practical ceilings of the step's byte mixes (the streaming probe at the same size)
    ceil_copy = probe_ceiling(torch, glu, 1, 1, 16, 1 << 29, args.sweep_iters)
    ceil_bwd = probe_ceiling(torch, glu, 3, 4, 8, M * N, args.sweep_iters)
    ceil_fwd = probe_ceiling(torch, glu, 2, 2, 8, M * N, args.sweep_iters)
    achieved = bwd_b / bwd_us / 1e3
    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "swiglu_mxfp8_fwd_bwd_both_16384x7168_outliers",
            "activation": "swiglu", "M": M, "N": N, "outliers": "0.1% x1000",
            "outputs": "E4M3 codes + E8M0 RCEIL scales, rowwise 1x32 and colwise 32x1",
            "bytes_per_step": fwd_b + bwd_b, "pct_of_peak": round(100 * value / PEAK_GBPS, 1),
            "fwd_us": round(fwd_us, 2), "bwd_us": round(bwd_us, 2), "wall_s": round(wall, 3),
            "validated": validate,
            "context_pages_gb200_gbps_same_workload": round(PAGES_STEP_GBPS, 1),
            "context_ratio_to_pages_gb200": round(value / PAGES_STEP_GBPS, 3),
        },
        "roofline": {
            "bound": "hbm", "kernel": "k_mxfp8 backward, both scalings",
            "achieved": round(achieved, 1), "peak": PEAK_GBPS, "unit": "GB/s",
            "frac": round(achieved / PEAK_GBPS, 4),
            "traffic": traffic_bytes("k_mxfp8<0,0,3,1>"),
            "ceiling": ceil_bwd["gbps"], "frac_of_ceiling": round(achieved / ceil_bwd["gbps"], 4),
        },
        "ceiling": {"stream_copy_1GiB": ceil_copy, "step_fwd_mix": ceil_fwd, "step_bwd_mix": ceil_bwd},
    }
    if not args.no_sweep:
        result["sweep"] = sweep(torch, glu, si, args.sweep_iters, validate)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(si, args.cpu_budget)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
