"""Python access to the CPU oracle (oracle/glu_oracle.c).

TEST INFRASTRUCTURE ONLY: tests/, the smoke check and the benchmark's CPU-baseline
leg are the only callers.  The GPU library never imports this package.

Arrays are numpy: BF16 values travel as uint16 bit patterns, codes and scales as
uint8, FP32 quantizer inputs as float32.  Every function allocates and returns its
outputs.
"""
import contextlib
import ctypes
import os

import numpy as np

from . import build as _build

SWIGLU, GEGLU_TANH, GEGLU_ERF, RELU2 = 0, 1, 2, 3
SPLIT, PAIRED = 0, 1
ROWWISE, COLWISE, SF_SWIZZLED = 1, 2, 4
SF_ROWMAJOR, SF_128x4 = 0, 1

_lib = None

_i64 = ctypes.c_int64
_int = ctypes.c_int
_p = ctypes.c_void_p


_SIGNATURES = {
    "orc_num_threads": (_int, []),
    "orc_bf16_from_f64": (ctypes.c_uint16, [ctypes.c_double]),
    "orc_bf16_to_f64": (ctypes.c_double, [ctypes.c_uint16]),
    "orc_e4m3_from_f64": (ctypes.c_uint8, [ctypes.c_double]),
    "orc_e4m3_to_f64": (ctypes.c_double, [ctypes.c_uint8]),
    "orc_e2m1_from_f64": (ctypes.c_uint8, [ctypes.c_double]),
    "orc_e2m1_to_f64": (ctypes.c_double, [ctypes.c_uint8]),
    "orc_mx_scale_exponent": (_int, [ctypes.c_double]),
    "orc_act": (ctypes.c_double, [_int, ctypes.c_double]),
    "orc_act_grad": (ctypes.c_double, [_int, ctypes.c_double]),
    "orc_sf128x4_offset": (_i64, [_i64, _i64, _i64]),
    "orc_mx_sf_bytes": (_i64, [_i64, _i64, _int]),
    "orc_glu_fwd": (None, [_int, _int, _i64, _i64, _p, _p, _i64, _p, _i64]),
    "orc_glu_bwd": (None, [_int, _int, _i64, _i64, _p, _p, _i64, _p, _i64, _p, _p, _i64]),
    "orc_quant_mxfp8": (None, [_i64, _i64, _p, _int, _p, _p, _p, _p]),
    "orc_quant_nvfp4": (None, [_i64, _i64, _p, _p, _p, _int]),
    "orc_glu_fwd_mxfp8": (_int, [_int, _int, _i64, _i64, _p, _p, _i64, _int, _p, _p, _p, _p]),
    "orc_glu_bwd_mxfp8": (_int, [_int, _i64, _i64, _p, _p, _i64, _p, _i64, _int, _p, _p, _p, _p]),
    "orc_glu_fwd_nvfp4": (_int, [_int, _int, _i64, _i64, _p, _p, _i64, _p, _p, _int]),
    "orc_glu_bwd_nvfp4": (_int, [_int, _i64, _i64, _p, _p, _i64, _p, _i64, _p, _p, _int]),
    "orc_nvfp4_global_scale": (ctypes.c_float, [ctypes.c_float]),
    "orc_quant_nvfp4_gs": (None, [_i64, _i64, _p, ctypes.c_float, _p, _p, _int]),
    "orc_glu_amax": (ctypes.c_float, [_int, _int, _i64, _i64, _p, _p, _i64, _p]),
    "orc_glu_fwd_nvfp4_gs": (_int, [_int, _int, _i64, _i64, _p, _p, _i64, ctypes.c_float, _p, _p, _int]),
    "orc_mx_gemm_nt": (None, [_int, _i64, _i64, _i64, _p, _p, _p, _p, _p]),
    "orc_glu_gemm": (_int, [_int, _int, _int, _i64, _i64, _i64, _p, _p, _p, _p, _p]),
    "orc_glu_gemm_mxfp8": (_int, [_int, _int, _int, _i64, _i64, _i64, _p, _p, _p, _p, _p, _p]),
    "orc_bf16_from_f64_array": (None, [_p, _i64, _p]),
    "orc_e4m3_from_f64_array": (None, [_p, _i64, _p]),
    "orc_e2m1_from_f64_array": (None, [_p, _i64, _p]),
    "orc_act_array": (None, [_int, _p, _i64, _p]),
    "orc_act_grad_array": (None, [_int, _p, _i64, _p]),
}


def open_library(path):
    """Loads an oracle build from `path` and declares its signatures."""
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGNATURES.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        _lib = open_library(_build.LIB)
    return _lib


@contextlib.contextmanager
def use_library(path):
    """Temporarily routes every call of this module to another oracle build (the
    mutation tests use it to run the pins against deliberately broken copies)."""
    global _lib
    saved = _load()
    _lib = open_library(path)
    try:
        yield
    finally:
        _lib = saved


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def _c(a, dtype):
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {dtype}, got {a.dtype}")
    return a


def num_threads() -> int:
    return _load().orc_num_threads()


# ---- scalar and element-wise encoders (format pins) -------------------------

def bf16_from_f64(v):
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(v.shape, np.uint16)
    _load().orc_bf16_from_f64_array(_ptr(v), v.size, _ptr(out))
    return out


def e4m3_from_f64(v):
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(v.shape, np.uint8)
    _load().orc_e4m3_from_f64_array(_ptr(v), v.size, _ptr(out))
    return out


def e2m1_from_f64(v):
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(v.shape, np.uint8)
    _load().orc_e2m1_from_f64_array(_ptr(v), v.size, _ptr(out))
    return out


def bf16_to_f64(b):
    f = _load().orc_bf16_to_f64
    return np.array([f(int(x)) for x in np.asarray(b, np.uint16).ravel()]).reshape(np.shape(b))


def e4m3_to_f64(c):
    f = _load().orc_e4m3_to_f64
    return np.array([f(int(x)) for x in np.asarray(c, np.uint8).ravel()]).reshape(np.shape(c))


def e2m1_to_f64(c):
    f = _load().orc_e2m1_to_f64
    return np.array([f(int(x)) for x in np.asarray(c, np.uint8).ravel()]).reshape(np.shape(c))


def mx_scale_exponent(amax: float) -> int:
    return _load().orc_mx_scale_exponent(float(amax))


def act(kind, x):
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty_like(x)
    _load().orc_act_array(kind, _ptr(x), x.size, _ptr(out))
    return out


def act_grad(kind, x):
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty_like(x)
    _load().orc_act_grad_array(kind, _ptr(x), x.size, _ptr(out))
    return out


def sf128x4_offset(r: int, c: int, scale_cols_padded: int) -> int:
    return _load().orc_sf128x4_offset(r, c, scale_cols_padded)


def sf128x4_bytes(M: int, H: int) -> int:
    return (M + 127) // 128 * 128 * ((H // 16 + 3) // 4 * 4)


# ---- GLU ----------------------------------------------------------------------

def _operands(layout, gate, up):
    gate = _c(gate, np.uint16)
    if layout == PAIRED:
        if up is not None:
            raise ValueError("paired layout takes one interleaved matrix")
        M, two_n = gate.shape
        return gate, None, M, two_n // 2, two_n
    up = _c(up, np.uint16)
    if up.shape != gate.shape:
        raise ValueError("gate and up differ in shape")
    M, N = gate.shape
    return gate, up, M, N, N


def glu_fwd(kind, gate, up=None, layout=SPLIT):
    """h = BF16(act(gate) * up) as uint16 [M, N]."""
    gate, up, M, N, ld = _operands(layout, gate, up)
    h = np.empty((M, N), np.uint16)
    _load().orc_glu_fwd(kind, layout, M, N, _ptr(gate), _ptr(up), ld, _ptr(h), N)
    return h


def glu_bwd(kind, gate, up, dh, layout=SPLIT):
    """SPLIT: (da, db) each [M, N].  PAIRED: one interleaved [M, 2N] gradient."""
    gate, up, M, N, ld = _operands(layout, gate, up)
    dh = _c(dh, np.uint16)
    if dh.shape != (M, N):
        raise ValueError("dh shape")
    if layout == PAIRED:
        d = np.empty((M, 2 * N), np.uint16)
        _load().orc_glu_bwd(kind, layout, M, N, _ptr(gate), None, ld, _ptr(dh), N, _ptr(d), None, 2 * N)
        return d
    da = np.empty((M, N), np.uint16)
    db = np.empty((M, N), np.uint16)
    _load().orc_glu_bwd(kind, layout, M, N, _ptr(gate), _ptr(up), ld, _ptr(dh), N, _ptr(da), _ptr(db), N)
    return da, db


def mx_sf_bytes(rows: int, nb: int, swizzled: bool) -> int:
    return _load().orc_mx_sf_bytes(rows, nb, int(bool(swizzled)))


def _mx_scales(rows, nb, swizzled):
    return np.empty(mx_sf_bytes(rows, nb, True), np.uint8) if swizzled else np.empty((rows, nb), np.uint8)


def _mx_outputs(M, N, flags):
    swz = bool(flags & SF_SWIZZLED)
    row = (np.empty((M, N), np.uint8), _mx_scales(M, N // 32, swz)) if flags & ROWWISE else (None, None)
    col = (np.empty((N, M), np.uint8), _mx_scales(N, M // 32, swz)) if flags & COLWISE else (None, None)
    return row[0], row[1], col[0], col[1]


def quant_mxfp8(x, flags=ROWWISE):
    """x float32 [M, N] -> (q_row [M,N], s_row [M,N/32], q_col [N,M], s_col [N,M/32]);
    the disabled direction comes back as None.  With SF_SWIZZLED in flags the scales are
    flat zero-padded 128x4 arrays (mx_sf_bytes)."""
    x = _c(x, np.float32)
    M, N = x.shape
    out = _mx_outputs(M, N, flags)
    _load().orc_quant_mxfp8(M, N, _ptr(x), flags, *[_ptr(o) for o in out])
    return out


def quant_nvfp4(x, sf_layout=SF_ROWMAJOR):
    """x float32 [M, H] -> (q [M, H/2] packed E2M1, sf scales)."""
    x = _c(x, np.float32)
    M, H = x.shape
    q = np.empty((M, H // 2), np.uint8)
    sf = np.empty(sf128x4_bytes(M, H) if sf_layout == SF_128x4 else (M, H // 16), np.uint8)
    _load().orc_quant_nvfp4(M, H, _ptr(x), _ptr(q), _ptr(sf), sf_layout)
    return q, sf


def glu_fwd_mxfp8(kind, gate, up=None, flags=ROWWISE, layout=SPLIT):
    gate, up, M, N, ld = _operands(layout, gate, up)
    out = _mx_outputs(M, N, flags)
    rc = _load().orc_glu_fwd_mxfp8(kind, layout, M, N, _ptr(gate), _ptr(up), ld, flags,
                                   *[_ptr(o) for o in out])
    if rc != 0:
        raise MemoryError("oracle ran out of host memory")
    return out


def glu_bwd_mxfp8(kind, gate, up, dh, flags=ROWWISE):
    gate, up, M, N, ld = _operands(SPLIT, gate, up)
    dh = _c(dh, np.uint16)
    out = _mx_outputs(M, 2 * N, flags)
    rc = _load().orc_glu_bwd_mxfp8(kind, M, N, _ptr(gate), _ptr(up), ld, _ptr(dh), N, flags,
                                   *[_ptr(o) for o in out])
    if rc != 0:
        raise MemoryError("oracle ran out of host memory")
    return out


def glu_fwd_nvfp4(kind, gate, up=None, layout=PAIRED, sf_layout=SF_ROWMAJOR):
    gate, up, M, H, ld = _operands(layout, gate, up)
    q = np.empty((M, H // 2), np.uint8)
    sf = np.empty(sf128x4_bytes(M, H) if sf_layout == SF_128x4 else (M, H // 16), np.uint8)
    rc = _load().orc_glu_fwd_nvfp4(kind, layout, M, H, _ptr(gate), _ptr(up), ld, _ptr(q), _ptr(sf), sf_layout)
    if rc != 0:
        raise MemoryError("oracle ran out of host memory")
    return q, sf


def glu_bwd_nvfp4(kind, gate, up, dh, sf_layout=SF_ROWMAJOR):
    """[da | db] ([M, 2N]) as NVFP4: q [M, N] packed E2M1, scales [M, 2N/16] or 128x4."""
    gate, up, M, N, ld = _operands(SPLIT, gate, up)
    dh = _c(dh, np.uint16)
    q = np.empty((M, N), np.uint8)
    sf = np.empty(sf128x4_bytes(M, 2 * N) if sf_layout == SF_128x4 else (M, 2 * N // 16), np.uint8)
    rc = _load().orc_glu_bwd_nvfp4(kind, M, N, _ptr(gate), _ptr(up), ld, _ptr(dh), N, _ptr(q), _ptr(sf),
                                   sf_layout)
    if rc != 0:
        raise MemoryError("oracle ran out of host memory")
    return q, sf


# ---- two-level NVFP4 (global scale from the tensor's amax) ----------------------

def nvfp4_global_scale(amax):
    return float(_load().orc_nvfp4_global_scale(float(amax)))


def quant_nvfp4_gs(x, amax, sf_layout=SF_ROWMAJOR):
    """x float32 [M, H], FP32 amax -> (q [M, H/2] packed E2M1, sf E4M3 scales)."""
    x = _c(x, np.float32)
    M, H = x.shape
    q = np.empty((M, H // 2), np.uint8)
    sf = np.empty(sf128x4_bytes(M, H) if sf_layout == SF_128x4 else (M, H // 16), np.uint8)
    _load().orc_quant_nvfp4_gs(M, H, _ptr(x), float(amax), _ptr(q), _ptr(sf), sf_layout)
    return q, sf


def glu_amax(kind, gate, up=None, layout=SPLIT):
    gate, up, M, N, ld = _operands(layout, gate, up)
    ok = ctypes.c_int(0)
    a = _load().orc_glu_amax(kind, layout, M, N, _ptr(gate), _ptr(up), ld, ctypes.byref(ok))
    if ok.value != 0:
        raise MemoryError("oracle ran out of host memory")
    return float(a)


def glu_fwd_nvfp4_gs(kind, gate, up=None, amax=None, layout=PAIRED, sf_layout=SF_ROWMAJOR):
    gate, up, M, H, ld = _operands(layout, gate, up)
    q = np.empty((M, H // 2), np.uint8)
    sf = np.empty(sf128x4_bytes(M, H) if sf_layout == SF_128x4 else (M, H // 16), np.uint8)
    rc = _load().orc_glu_fwd_nvfp4_gs(kind, layout, M, H, _ptr(gate), _ptr(up), ld, float(amax), _ptr(q),
                                      _ptr(sf), sf_layout)
    if rc != 0:
        raise MemoryError("oracle ran out of host memory")
    return q, sf


# ---- merged gate/up block-scaled GEMM with the GLU epilogue -----------------------------

FMT_E4M3, FMT_E2M1 = 0, 1   # operand codes: MXFP8 (one per byte) or MXFP4 (two per byte)


def _gemm_operands(Xq, Xs, Wq, Ws, fmt):
    Xq, Xs, Wq, Ws = (_c(a, np.uint8) for a in (Xq, Xs, Wq, Ws))
    M, rb = Xq.shape
    K = 2 * rb if fmt == FMT_E2M1 else rb
    N2 = Wq.shape[0]
    if fmt not in (FMT_E4M3, FMT_E2M1) or Wq.shape[1] != rb or Xs.shape != (M, K // 32) \
            or Ws.shape != (N2, K // 32) or K % 32:
        raise ValueError("operand shapes")
    return Xq, Xs, Wq, Ws, M, N2, K


def mx_gemm_nt(Xq, Xs, Wq, Ws, fmt=FMT_E4M3):
    """Y = X W^T in float64 from block-scaled codes (E4M3 codes [rows, K], or E2M1 codes packed
    [rows, K/2] with element 2j in the low nibble) and E8M0 scales (blocks of 32 along K).
    Y keeps W's row order."""
    Xq, Xs, Wq, Ws, M, N2, K = _gemm_operands(Xq, Xs, Wq, Ws, fmt)
    Y = np.empty((M, N2), np.float64)
    _load().orc_mx_gemm_nt(fmt, M, N2, K, _ptr(Xq), _ptr(Xs), _ptr(Wq), _ptr(Ws), _ptr(Y))
    return Y


def glu_gemm(kind, Xq, Xs, Wq, Ws, fmt=FMT_E4M3, w_layout=SPLIT):
    """BF16 bits of h = act(Y_gate) * Y_up; W = [W_gate | W_up] (SPLIT) or pairwise-interleaved
    gate/up rows (PAIRED)."""
    Xq, Xs, Wq, Ws, M, N2, K = _gemm_operands(Xq, Xs, Wq, Ws, fmt)
    h = np.empty((M, N2 // 2), np.uint16)
    if _load().orc_glu_gemm(kind, fmt, w_layout, M, N2 // 2, K, _ptr(Xq), _ptr(Xs), _ptr(Wq), _ptr(Ws),
                            _ptr(h)) != 0:
        raise MemoryError("oracle ran out of host memory")
    return h


def glu_gemm_mxfp8(kind, Xq, Xs, Wq, Ws, fmt=FMT_E4M3, w_layout=SPLIT):
    """(q_row [M, N], s_row [M, N/32]): h of glu_gemm quantized MXFP8 rowwise."""
    Xq, Xs, Wq, Ws, M, N2, K = _gemm_operands(Xq, Xs, Wq, Ws, fmt)
    N = N2 // 2
    q = np.empty((M, N), np.uint8)
    sc = np.empty((M, N // 32), np.uint8)
    if _load().orc_glu_gemm_mxfp8(kind, fmt, w_layout, M, N, K, _ptr(Xq), _ptr(Xs), _ptr(Wq), _ptr(Ws),
                                  _ptr(q), _ptr(sc)) != 0:
        raise MemoryError("oracle ran out of host memory")
    return q, sc
