"""Host-side tests of the C ABI (no GPU needed).

The library must load, export every function include/glu_mx.h declares, and reject every
unsupported argument before touching the device.  The glu_check_* exports run the exact
checks of the entry points; here they get fake, never-dereferenced pointers.  The entry
points themselves are only called with arguments that fail validation (they return before
any HIP call) or with M == 0 (a no-op).
"""
import ctypes
import os
import re

import pytest

import glu_activation_microscaling_amd as glu
from conftest import ROOT

OK, NULL, SHAPE, ALIGN, STRIDE, ARG, OVERLAP, UNSUP, HIP = range(9)
L = None


def setup_module(module):
    global L
    if not os.path.exists(glu.LIB_PATH):
        from glu_activation_microscaling_amd import build
        build.build()
    L = glu.lib()


def P(addr):
    return ctypes.c_void_p(addr)


A0 = 0x10000000      # fake, 16-byte aligned device addresses far apart
B0 = 0x20000000
C0 = 0x30000000
D0 = 0x40000000
E0 = 0x50000000
F0 = 0x60000000


def test_every_declared_symbol_is_exported():
    with open(os.path.join(ROOT, "include", "glu_mx.h")) as f:
        text = f.read()
    names = set(re.findall(r"\b(glu_[a-z0-9_]+)\s*\(", text))
    names -= {"glu_status"}
    assert len(names) >= 17
    for n in sorted(names):
        assert hasattr(L, n), f"missing export {n}"


def test_status_strings_and_version():
    L.glu_status_string.restype = ctypes.c_char_p
    for s in range(9):
        assert L.glu_status_string(s)
    assert L.glu_version() >= 100


def fwd(**kw):
    a = dict(act=0, layout=0, M=64, N=128, gate=A0, up=B0, ld=128, h=C0, ldh=128)
    a.update(kw)
    return L.glu_check_fwd(a["act"], a["layout"], a["M"], a["N"], P(a["gate"]), P(a["up"]), a["ld"],
                           P(a["h"]), a["ldh"])


def test_fwd_checks():
    assert fwd() == OK
    assert fwd(act=2) == OK and fwd(act=3) == OK      # erf-GELU, ReLU^2
    assert fwd(act=4) == ARG and fwd(act=-1) == ARG and fwd(layout=5) == ARG
    assert fwd(M=-1) == SHAPE and fwd(N=-3) == SHAPE
    assert fwd(M=0, gate=0, up=0, h=0) == OK and fwd(N=0, gate=0) == OK
    assert fwd(gate=0) == NULL and fwd(up=0) == NULL and fwd(h=0) == NULL
    assert fwd(layout=1, up=B0, ld=256) == ARG           # paired takes one matrix
    assert fwd(layout=1, up=0, ld=256) == OK
    assert fwd(layout=1, up=0, ld=255) == STRIDE          # ld < 2N
    assert fwd(ld=127) == STRIDE and fwd(ldh=100) == STRIDE
    assert fwd(N=8193, ld=8193, ldh=8193) == OK           # contiguous: any width
    assert fwd(N=8193, ld=8200, ldh=8193) == STRIDE       # strided rows need ld % 8 == 0
    assert fwd(N=8193, ld=8200, ldh=8200) == OK
    assert fwd(gate=A0 + 2) == ALIGN and fwd(h=C0 + 8) == ALIGN
    assert fwd(h=A0 + 64) == OVERLAP                      # h inside gate
    # [gate | up] halves of one buffer: up = gate + N, ld = 2N
    assert fwd(gate=A0, up=A0 + 2 * 128, ld=256) == OK
    # an output placed in the row gaps of a strided input is not an overlap...
    assert fwd(gate=A0, up=A0 + 2 * 128, ld=384, h=A0 + 2 * 256, ldh=384) == OK
    # ...but one that lands on input elements is
    assert fwd(gate=A0, up=A0 + 2 * 128, ld=384, h=A0 + 2 * 200, ldh=384) == OVERLAP
    assert fwd(M=1 << 62, N=1 << 20, ld=1 << 20, ldh=1 << 20) == SHAPE  # extent overflow


def bwd(**kw):
    a = dict(act=1, layout=0, M=64, N=128, gate=A0, up=B0, ld=128, dh=C0, lddh=128, da=D0, db=E0, ldo=128)
    a.update(kw)
    return L.glu_check_bwd(a["act"], a["layout"], a["M"], a["N"], P(a["gate"]), P(a["up"]), a["ld"],
                           P(a["dh"]), a["lddh"], P(a["da"]), P(a["db"]), a["ldo"])


def test_bwd_checks():
    assert bwd() == OK
    assert bwd(dh=0) == NULL and bwd(da=0) == NULL and bwd(db=0) == NULL
    assert bwd(layout=1, up=0, ld=256, db=E0, ldo=256) == ARG
    assert bwd(layout=1, up=0, ld=256, db=0, ldo=256) == OK
    assert bwd(layout=1, up=0, ld=256, db=0, ldo=128) == STRIDE
    assert bwd(da=A0, db=B0) == OK                        # in place
    assert bwd(da=A0, db=B0, ldo=136) == OVERLAP          # same buffers, other stride: not in place
    assert bwd(da=C0) == OVERLAP                          # da onto dh
    assert bwd(da=D0, db=D0 + 64) == OVERLAP              # da and db collide
    # concatenated [dGate | dUp] output: db = da + N, ld_out = 2N
    assert bwd(da=D0, db=D0 + 2 * 128, ldo=256) == OK
    assert bwd(dh=C0 + 4) == ALIGN


def mxf(**kw):
    a = dict(act=0, layout=0, M=64, N=128, gate=A0, up=B0, ld=128, flags=3, qr=C0, sr=D0, qc=E0, sc=F0)
    a.update(kw)
    return L.glu_check_fwd_mxfp8(a["act"], a["layout"], a["M"], a["N"], P(a["gate"]), P(a["up"]),
                                 a["ld"], a["flags"], P(a["qr"]), P(a["sr"]), P(a["qc"]), P(a["sc"]))


def test_fwd_mxfp8_checks():
    assert mxf() == OK
    assert mxf(flags=0) == ARG and mxf(flags=4) == ARG
    assert mxf(flags=1, qc=0, sc=0) == OK and mxf(flags=2, qr=0, sr=0) == OK
    assert mxf(flags=1) == ARG                            # colwise pointers given but disabled
    assert mxf(flags=2, qr=0) == ARG
    assert mxf(qr=0) == NULL and mxf(sc=0) == NULL
    assert mxf(N=96, ld=96) == OK and mxf(N=80, ld=80) == SHAPE
    assert mxf(M=48) == SHAPE                             # colwise needs M % 32 == 0
    assert mxf(M=48, flags=1, qc=0, sc=0) == OK           # rowwise accepts ragged M
    assert mxf(ld=132) == STRIDE
    assert mxf(sr=D0 + 1) == ALIGN
    assert mxf(qr=A0) == OVERLAP and mxf(sr=C0 + 16) == OVERLAP
    assert mxf(layout=1, up=0, ld=256) == OK and mxf(layout=1, up=0, ld=128) == STRIDE
    # row pitch limit of the MXFP8 kernels: 2^24 elements
    row = dict(M=1, flags=1, qc=0, sc=0)
    assert mxf(ld=1 << 24, **row) == OK and mxf(ld=(1 << 24) + 8, **row) == STRIDE
    # colwise output rows (M codes each) at most 2^24 bytes
    col = dict(N=32, ld=32, flags=2, qr=0, sr=0, gate=1 << 36, up=2 << 36, qc=3 << 36, sc=4 << 36)
    assert mxf(M=1 << 24, **col) == OK and mxf(M=(1 << 24) + 32, **col) == SHAPE


def mxb(**kw):
    a = dict(act=0, layout=0, M=64, N=128, gate=A0, up=B0, ld=128, dh=C0, lddh=128, flags=3,
             qr=D0, sr=E0, qc=F0, sc=0x70000000)
    a.update(kw)
    return L.glu_check_bwd_mxfp8(a["act"], a["layout"], a["M"], a["N"], P(a["gate"]), P(a["up"]),
                                 a["ld"], P(a["dh"]), a["lddh"], a["flags"], P(a["qr"]), P(a["sr"]),
                                 P(a["qc"]), P(a["sc"]))


def test_mxfp8_swizzled_scale_flag_and_sizes():
    SWZ = 4
    assert mxf(flags=3 | SWZ) == OK and mxf(flags=1 | SWZ, qc=0, sc=0) == OK
    assert mxf(flags=SWZ) == ARG and mxf(flags=8) == ARG and mxf(flags=3 | 8) == ARG
    # padded scale buffers: [M, N/32] -> ceil(M/128)*128 x ceil(N/128)*4 bytes
    f = L.glu_mxfp8_sf_bytes
    f.restype = ctypes.c_int64
    assert f(130, 224, 1) == 256 * 8 and f(130, 224, 0) == 130 * 7
    assert f(128, 128, 1) == 128 * 4 and f(1, 32, 1) == 128 * 4
    assert f(1, 33, 1) == -1 and f(-1, 32, 0) == -1 and f(1, 32, 2) == -1
    # the padded extent counts for overlap: 64 x 128 both ways, s_row takes 128 * 4 bytes
    assert mxf(flags=3 | SWZ, sr=D0, sc=D0 + 512) == OK
    assert mxf(flags=3 | SWZ, sr=D0, sc=D0 + 256) == OVERLAP
    assert mxf(flags=3, sr=D0, sc=D0 + 256) == OK  # row-major s_row is 64 * 4 bytes


def test_bwd_mxfp8_checks():
    assert mxb() == OK
    assert mxb(layout=1, up=0) == UNSUP
    assert mxb(dh=0) == NULL
    assert mxb(lddh=120) == STRIDE and mxb(lddh=132) == STRIDE
    row = dict(M=1, flags=1, qc=0, sc=0)
    assert mxb(N=1 << 23, ld=1 << 23, lddh=1 << 23, **row) == OK   # [da | db] rows: 2^24 codes
    assert mxb(N=(1 << 23) + 32, ld=(1 << 23) + 32, lddh=(1 << 23) + 32, **row) == SHAPE
    assert mxb(ld=1 << 24, lddh=1 << 24, **row) == OK
    assert mxb(ld=(1 << 24) + 8, **row) == STRIDE and mxb(lddh=(1 << 24) + 8, **row) == STRIDE
    assert mxb(qr=C0) == OVERLAP
    assert mxb(N=40, ld=40, lddh=40) == SHAPE


def nv(**kw):
    a = dict(act=1, layout=1, M=100, H=256, gate=A0, up=0, ld=512, q=C0, sf=D0, sfl=0)
    a.update(kw)
    return L.glu_check_fwd_nvfp4(a["act"], a["layout"], a["M"], a["H"], P(a["gate"]), P(a["up"]),
                                 a["ld"], P(a["q"]), P(a["sf"]), a["sfl"])


def test_fwd_nvfp4_checks():
    assert nv() == OK and nv(sfl=1) == OK
    assert nv(sfl=2) == ARG
    assert nv(H=264, ld=528) == SHAPE                     # H % 16
    assert nv(M=1, H=1 << 26, ld=1 << 27) == OK and nv(M=1, H=(1 << 26) + 16, ld=(1 << 27) + 32) == SHAPE
    assert nv(ld=516) == STRIDE and nv(ld=511) == STRIDE and nv(ld=520) == OK
    assert nv(q=0) == NULL and nv(sf=0) == NULL
    assert nv(layout=0, up=B0, ld=256) == OK
    assert nv(sf=C0 + 32) == OVERLAP
    assert L.glu_nvfp4_sf_bytes(784, 16384, 0) == 784 * 1024
    assert L.glu_nvfp4_sf_bytes(784, 16384, 1) == 896 * 1024
    assert L.glu_nvfp4_sf_bytes(968, 16384, 1) == 1024 * 1024
    assert L.glu_nvfp4_sf_bytes(1, 80, 1) == 128 * 8
    assert L.glu_nvfp4_sf_bytes(1, 81, 0) == -1


def nvb(**kw):
    a = dict(act=0, layout=0, M=100, N=256, gate=A0, up=B0, ld=256, dh=C0, lddh=256, q=D0, sf=E0, sfl=0)
    a.update(kw)
    return L.glu_check_bwd_nvfp4(a["act"], a["layout"], a["M"], a["N"], P(a["gate"]), P(a["up"]),
                                 a["ld"], P(a["dh"]), a["lddh"], P(a["q"]), P(a["sf"]), a["sfl"])


def test_bwd_nvfp4_checks():
    assert nvb() == OK and nvb(sfl=1) == OK and nvb(act=3) == OK
    assert nvb(sfl=2) == ARG and nvb(act=4) == ARG
    assert nvb(layout=1, up=0) == UNSUP
    assert nvb(M=0) == OK and nvb(N=0) == OK and nvb(M=-1) == SHAPE
    assert nvb(N=264, ld=264, lddh=264) == SHAPE                       # N % 16
    assert nvb(dh=0) == NULL and nvb(q=0) == NULL and nvb(sf=0) == NULL and nvb(up=0) == NULL
    assert nvb(lddh=248) == STRIDE and nvb(lddh=260) == STRIDE and nvb(ld=252) == STRIDE
    assert nvb(dh=C0 + 8) == ALIGN and nvb(q=D0 + 4) == ALIGN
    assert nvb(q=C0 + 64) == OVERLAP                                    # codes over dh
    assert nvb(sf=D0 + 100 * 256 - 16) == OVERLAP                       # scales over the codes' end
    assert nvb(sf=D0 + 100 * 256) == OK                                 # q is [M, N] bytes
    assert nvb(N=1 << 62, ld=1 << 62, lddh=1 << 62) == SHAPE            # 2N overflows
    assert nvb(M=1, N=1 << 26, ld=1 << 26, lddh=1 << 26) == OK
    assert nvb(M=1, N=(1 << 26) + 16, ld=(1 << 26) + 16, lddh=(1 << 26) + 16) == SHAPE


def test_amax_and_two_level_checks():
    am = L.glu_check_amax
    assert am(0, 0, 64, 128, P(A0), P(B0), 128, P(C0)) == OK
    assert am(0, 1, 64, 128, P(A0), P(0), 256, P(C0)) == OK
    assert am(0, 0, 64, 128, P(A0), P(B0), 128, P(0)) == NULL
    assert am(0, 0, 64, 128, P(A0), P(B0), 128, P(C0 + 2)) == ALIGN
    assert am(0, 0, 0, 128, P(0), P(0), 128, P(C0)) == OK        # empty: still writes 0
    assert am(0, 0, 64, 120, P(A0), P(B0), 120, P(C0)) == SHAPE   # N % 16
    assert am(0, 0, 64, 128, P(A0), P(B0), 128, P(A0 + 64)) == OVERLAP
    assert am(5, 0, 64, 128, P(A0), P(B0), 128, P(C0)) == ARG
    gs = L.glu_check_fwd_nvfp4_gs
    assert gs(1, 1, 100, 256, P(A0), P(0), 512, P(E0), P(C0), P(D0), 0) == OK
    assert gs(1, 1, 100, 256, P(A0), P(0), 512, P(0), P(C0), P(D0), 0) == NULL
    assert gs(1, 1, 100, 256, P(A0), P(0), 512, P(E0 + 1), P(C0), P(D0), 0) == ALIGN
    assert gs(1, 1, 100, 256, P(A0), P(0), 512, P(C0 + 64), P(C0), P(D0), 0) == OVERLAP
    assert gs(1, 1, 100, 264, P(A0), P(0), 528, P(E0), P(C0), P(D0), 0) == SHAPE


def test_quant_hook_checks():
    q = L.glu_check_quant_mxfp8_f32
    assert q(64, 64, P(A0), 64, 3, P(B0), P(C0), P(D0), P(E0)) == OK
    assert q(64, 64, P(A0), 66, 3, P(B0), P(C0), P(D0), P(E0)) == STRIDE
    assert q(64, 64, P(A0), 60, 3, P(B0), P(C0), P(D0), P(E0)) == STRIDE
    assert q(64, 64, P(A0), 64, 1, P(B0), P(C0), P(0), P(0)) == OK
    assert q(1, 64, P(A0), 1 << 23, 1, P(B0), P(C0), P(0), P(0)) == OK
    assert q(1, 64, P(A0), (1 << 23) + 4, 1, P(B0), P(C0), P(0), P(0)) == STRIDE
    n = L.glu_check_quant_nvfp4_f32
    assert n(64, 64, P(A0), 64, P(B0), P(C0), 0) == OK
    assert n(64, 72, P(A0), 72, P(B0), P(C0), 0) == SHAPE


def _ptrs(*addrs):
    arr = (ctypes.c_void_p * max(1, len(addrs)))(*addrs)
    return ctypes.cast(arr, ctypes.c_void_p)


def test_stream_probe_checks():
    c = L.glu_check_stream_probe
    n = 1 << 20
    assert c(2, _ptrs(A0, B0), 1, _ptrs(C0), n, 8) == OK
    assert c(3, _ptrs(A0, B0, C0), 4, _ptrs(D0, E0, F0, F0 + 0x4000000), n, 16) == OK
    assert c(0, _ptrs(A0), 1, _ptrs(C0), n, 8) == ARG
    assert c(4, _ptrs(A0, B0, C0, D0), 1, _ptrs(E0), n, 8) == ARG
    assert c(1, _ptrs(A0), 5, _ptrs(B0, C0, D0, E0, F0), n, 8) == ARG
    assert c(1, _ptrs(A0), 1, _ptrs(B0), n, 4) == OK
    assert c(1, _ptrs(A0), 1, _ptrs(B0), n, 2) == ARG
    assert c(1, _ptrs(A0), 1, _ptrs(B0), -1, 8) == SHAPE
    assert c(1, _ptrs(A0), 1, _ptrs(B0), 0, 8) == OK                 # empty: nothing inspected
    assert c(1, P(0), 1, _ptrs(B0), n, 8) == NULL
    assert c(1, _ptrs(0), 1, _ptrs(B0), n, 8) == NULL
    assert c(1, _ptrs(A0 + 8), 1, _ptrs(B0), n, 8) == ALIGN
    assert c(1, _ptrs(A0), 1, _ptrs(A0 + 16 * n - 16), n, 8) == OVERLAP   # destination on the source
    assert c(1, _ptrs(A0), 2, _ptrs(B0, B0 + 8 * n - 16), n, 8) == OVERLAP  # destinations overlap
    assert c(1, _ptrs(A0), 2, _ptrs(B0, B0 + 8 * n), n, 8) == OK           # adjacent is fine
    assert L.glu_stream_probe(1, _ptrs(A0), 1, _ptrs(A0), n, 8, P(0)) == OVERLAP


def test_gemm_checks():
    g = lambda **kw: _gemm(L.glu_check_gemm, **kw)
    assert g() == OK and g(act=3) == OK and g(act=4) == ARG
    assert g(M=0) == OK and g(M=-1) == SHAPE and g(K=0) == SHAPE
    assert g(K=96) == SHAPE and g(N=64, ldh=64) == SHAPE              # K % 128, N % 128
    assert g(xq=0) == NULL and g(ws=0) == NULL and g(h=0) == NULL
    assert g(xs=B0 + 4) == ALIGN and g(h=E0 + 2) == ALIGN and g(ldh=136) == OK
    assert g(ldh=120) == STRIDE and g(ldh=132) == ALIGN
    assert g(h=A0 + 64) == OVERLAP                                    # h over X
    # 32-bit offsets: X, W and h each below 2^31 bytes (an FP32 [M, 2N] would not be)
    assert g(M=1 << 24, K=128, ldh=128) == SHAPE
    assert g(M=1 << 22, K=128, ldh=128, h=F0 * 64) == OK
    assert g(M=1 << 22, K=128, ldh=512, h=F0 * 64) == SHAPE
    assert g(N=1 << 23, K=128, ldh=1 << 23, M=1) == SHAPE             # W is 2N x K
    q = lambda **kw: _gemm(L.glu_check_gemm_mxfp8, **kw)
    assert q() == OK and q(q=0) == NULL and q(s=E0 + 1) == ALIGN and q(act=7) == ARG
    assert q(s=D0 + 64 * 128 - 16) == OVERLAP and q(s=D0 + 64 * 128) == OK
    nv = lambda *a: L.glu_check_gemm_nvfp4(a[0], 0, 0, *a[1:])
    assert nv(0, 64, 128, 256, P(A0), P(B0), P(C0), P(A0 // 2), P(D0), P(E0), 0) == OK
    assert nv(0, 64, 128, 256, P(A0), P(B0), P(C0), P(A0 // 2), P(D0), P(E0), 1) == OK
    assert nv(0, 64, 128, 256, P(A0), P(B0), P(C0), P(A0 // 2), P(D0), P(E0), 2) == ARG
    assert nv(0, 64, 128, 256, P(A0), P(B0), P(C0), P(A0 // 2), P(0), P(E0), 0) == NULL
    assert nv(0, 64, 128, 256, P(A0), P(B0), P(C0), P(A0 // 2), P(D0), P(E0 + 8), 0) == ALIGN
    # q is [M, N/2] = 4096 bytes; the 128x4 scales of 64 rows take 128 * 8 bytes
    assert nv(0, 64, 128, 256, P(A0), P(B0), P(C0), P(A0 // 2), P(D0), P(D0 + 4096 - 16), 0) == OVERLAP
    assert nv(0, 64, 128, 256, P(A0), P(B0), P(C0), P(A0 // 2), P(D0), P(D0 + 4096), 1) == OK
    assert nv(0, 64, 128, 256, P(A0), P(B0), P(C0), P(A0 // 2), P(E0 + 1024 - 16), P(E0), 1) == OVERLAP
    assert nv(0, 64, 96, 256, P(A0), P(B0), P(C0), P(A0 // 2), P(D0), P(E0), 0) == SHAPE
    gs = L.glu_check_gemm_nvfp4_gs
    base = (0, 0, 0, 64, 128, 256, P(A0), P(B0), P(C0), P(A0 // 2))
    assert gs(*base, P(F0), P(D0), P(E0), 1) == OK
    assert gs(*base, P(0), P(D0), P(E0), 1) == NULL
    assert gs(*base, P(F0 + 2), P(D0), P(E0), 1) == ALIGN
    assert gs(*base, P(D0 + 64), P(D0), P(E0), 1) == OVERLAP          # amax inside the codes
    assert gs(*base, P(F0), P(D0), P(E0), 3) == ARG
    y = lambda **kw: _gemm(L.glu_check_mx_gemm_f32, **kw)
    assert y() == OK and y(y=0) == NULL and y(y=D0 + 4) == ALIGN
    assert y(M=1 << 20, K=128, N=256, y=F0 * 64) == SHAPE             # y is M x 2N x 4 bytes
    assert y(M=(1 << 20) - 8, K=128, N=256, y=F0 * 64) == OK


def test_gemm_operand_format_and_w_layout_checks():
    """fmt: E4M3 (one code per byte) or E2M1 (two per byte, K % 256); w_layout: split or
    interleaved rows.  E2M1 operand rows take K/2 bytes, so the extents used for the 32-bit
    bound and the overlap checks halve."""
    g = lambda **kw: _gemm(L.glu_check_gemm, **kw)
    assert g(fmt=1) == OK and g(wl=1) == OK and g(fmt=1, wl=1) == OK
    assert g(fmt=2) == ARG and g(fmt=-1) == ARG and g(wl=2) == ARG
    assert g(fmt=1, K=128) == SHAPE and g(fmt=0, K=128) == OK and g(fmt=1, K=512) == OK
    # h placed just past X: X is [64, 256] E4M3 = 16 KiB, or [64, 128] bytes = 8 KiB as E2M1
    assert g(h=A0 + 8192) == OVERLAP and g(h=A0 + 8192, fmt=1) == OK
    # W is [2N, K] elements: 2^31 bytes as E4M3 at 2N = 2^23, K = 256, half of it as E2M1
    assert g(N=1 << 22, K=256, M=1, ldh=1 << 22, h=F0 * 64) == SHAPE
    assert g(N=1 << 22, K=256, M=1, ldh=1 << 22, h=F0 * 64, fmt=1) == OK
    y = lambda **kw: _gemm(L.glu_check_mx_gemm_f32, **kw)
    assert y(fmt=1, wl=1) == OK and y(fmt=3) == ARG and y(wl=5) == ARG
    q = lambda **kw: _gemm(L.glu_check_gemm_mxfp8, **kw)
    assert q(fmt=1, wl=1) == OK and q(fmt=1, K=384) == SHAPE
    assert L.glu_check_gemm_nvfp4(0, 1, 1, 64, 128, 256, P(A0), P(B0), P(C0), P(A0 // 2), P(D0), P(E0), 1) == OK
    assert L.glu_check_gemm_nvfp4(0, 2, 1, 64, 128, 256, P(A0), P(B0), P(C0), P(A0 // 2), P(D0), P(E0), 1) == ARG


def _gemm(fn, act=0, fmt=0, wl=0, M=64, N=128, K=256, xq=A0, xs=B0, wq=C0, ws=A0 // 2, h=E0, ldh=128,
          q=D0, s=E0, y=D0):
    """Fake operands: X [M, K] at A0, its scales at B0, W [2N, K] at C0, W's scales at A0/2."""
    ops = [P(xq), P(xs), P(wq), P(ws)]
    if fn is L.glu_check_gemm:
        return fn(act, fmt, wl, M, N, K, *ops, P(h), ldh)
    if fn is L.glu_check_gemm_mxfp8:
        return fn(act, fmt, wl, M, N, K, *ops, P(q), P(s))
    return fn(fmt, wl, M, N, K, *ops, P(y))


def test_entry_points_fail_before_any_hip_call():
    """Rejected arguments and empty problems return without touching HIP, so these calls
    are safe on a machine with no GPU."""
    assert L.glu_fwd(0, 0, 4, 4, P(0), P(B0), 4, P(C0), 4, P(0)) == NULL
    assert L.glu_fwd(0, 0, 0, 4, P(0), P(0), 4, P(0), 4, P(0)) == OK
    assert L.glu_bwd(0, 0, 4, 8, P(A0), P(B0), 8, P(C0), 8, P(D0), P(E0), 4, P(0)) == STRIDE
    assert L.glu_fwd_mxfp8(0, 0, 64, 40, P(A0), P(B0), 40, 1, P(C0), P(D0), P(0), P(0), P(0)) == SHAPE
    assert L.glu_bwd_mxfp8(0, 1, 64, 64, P(A0), P(0), 128, P(C0), 64, 1, P(D0), P(E0), P(0), P(0), P(0)) == UNSUP
    assert L.glu_fwd_nvfp4(1, 1, 8, 24, P(A0), P(0), 48, P(C0), P(D0), 0, P(0)) == SHAPE
    assert L.glu_bwd_nvfp4(0, 0, 8, 24, P(A0), P(B0), 24, P(C0), 24, P(D0), P(E0), 0, P(0)) == SHAPE
    assert L.glu_bwd_nvfp4(0, 0, 0, 32, P(0), P(0), 32, P(0), 32, P(0), P(0), 0, P(0)) == OK
    assert L.glu_amax(0, 0, 4, 32, P(A0), P(B0), 32, P(0), P(0)) == NULL
    assert L.glu_fwd_nvfp4_gs(1, 1, 0, 32, P(0), P(0), 64, P(0), P(0), P(0), 0, P(0)) == OK
    assert L.glu_quant_mxfp8_f32(32, 32, P(A0), 32, 8, P(B0), P(C0), P(D0), P(E0), P(0)) == ARG
    assert L.glu_quant_nvfp4_f32(32, 32, P(A0 + 4), 32, P(B0), P(C0), 0, P(0)) == ALIGN
    assert L.glu_gemm(0, 0, 0, 8, 64, 128, P(A0), P(B0), P(C0), P(D0), P(E0), 64, P(0)) == SHAPE
    assert L.glu_gemm(0, 1, 1, 8, 128, 128, P(A0), P(B0), P(C0), P(D0), P(E0), 128, P(0)) == SHAPE
    assert L.glu_gemm_mxfp8(0, 0, 0, 0, 128, 128, P(0), P(0), P(0), P(0), P(0), P(0), P(0)) == OK
    assert L.glu_gemm_nvfp4(0, 4, 0, 8, 128, 256, P(A0), P(B0), P(C0), P(D0), P(E0), P(F0), 0, P(0)) == ARG
    assert L.glu_gemm_nvfp4_gs(0, 0, 0, 8, 128, 256, P(A0), P(B0), P(C0), P(D0), P(0), P(E0), P(F0), 0,
                               P(0)) == NULL
    assert L.glu_mx_gemm_f32(0, 0, 8, 128, 100, P(A0), P(B0), P(C0), P(D0), P(E0), P(0)) == SHAPE


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(4, 32, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        glu.glu_fwd(x, x)
    with pytest.raises(TypeError):
        glu.glu_fwd(x.float(), x.float())
