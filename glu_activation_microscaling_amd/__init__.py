"""Python binding of libglu_mx.so, the MI355X (gfx950) fused GLU + microscaling library.

Argument marshalling only: every function checks dtypes and devices, takes data pointers,
strides and the current HIP stream from torch tensors, allocates outputs when none are
given, and calls the C entry point of the same name.  All computation happens in the HIP
kernels; there is no CPU or PyTorch fallback, and a missing or unloadable library raises.

Entry points (C names in include/glu_mx.h):
  glu_fwd(gate, up=None, act=..., layout=...)               -> h
  glu_bwd(gate, up, dh, act=..., layout=...)                -> (da, db) or interleaved d
  glu_fwd_mxfp8(gate, up=None, rowwise=, colwise=, ...)     -> (q_row, q_col, s_row, s_col)
  glu_bwd_mxfp8(gate, up, dh, rowwise=, colwise=, ...)      -> (q_row, q_col, s_row, s_col)
  glu_fwd_nvfp4(x, up=None, layout="paired", sf_layout=...) -> (q, sf)
  glu_bwd_nvfp4(gate, up, dh, sf_layout=...)                -> (q, sf) of [da | db]
  glu_amax(gate, up=None, layout=...)                        -> amax, float32 [1] on the GPU
  glu_fwd_nvfp4_gs(x, up=None, amax=, layout=, sf_layout=)   -> (q, sf), two-level scaling
  glu_gemm(xq, xs, wq, ws, act=, fmt=, w_layout=)            -> h of the merged block-scaled GEMM
  glu_gemm_mxfp8(xq, xs, wq, ws, act=, fmt=, w_layout=)      -> (q_row, s_row) of that h
  glu_gemm_nvfp4(..., act=, fmt=, w_layout=, sf_layout=)      -> (q, sf) of that h, NVFP4
  glu_gemm_nvfp4_gs(..., amax=, act=, fmt=, w_layout=, sf_layout=) -> (q, sf), two-level NVFP4
  mx_gemm_f32(xq, xs, wq, ws, fmt=, w_layout=)               -> the GEMM alone (test hook)
  (fmt "mxfp8": E4M3 codes, or "mxfp4": packed E2M1 codes; w_layout "split" or "paired")
  glu_quant_mxfp8_f32(x, rowwise=, colwise=)                -> (q_row, q_col, s_row, s_col)
  glu_quant_nvfp4_f32(x, sf_layout=)                        -> (q, sf)
A disabled MXFP8 direction comes back as zero-sized tensors (fixed arity), as in the
MXFP8 page's API section.  Codes and scales are uint8 tensors; BF16 data is torch.bfloat16.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libglu_mx.so")

ACT = {"swiglu": 0, "geglu": 1, "geglu_tanh": 1, "geglu_erf": 2, "relu2": 3}
LAYOUT = {"split": 0, "paired": 1}
SF_LAYOUT = {"rowmajor": 0, "128x4": 1}
GEMM_FMT = {"mxfp8": 0, "mxfp4": 1}          # operand codes: E4M3 one per byte, E2M1 two per byte
W_LAYOUT = {"split": 0, "paired": 1}         # [W_gate | W_up], or rows gate0, up0, gate1, ...
ROWWISE, COLWISE, SF_SWIZZLED = 1, 2, 4

STATUS = {
    0: "GLU_OK", 1: "GLU_ERR_NULL", 2: "GLU_ERR_SHAPE", 3: "GLU_ERR_ALIGN", 4: "GLU_ERR_STRIDE",
    5: "GLU_ERR_ARG", 6: "GLU_ERR_OVERLAP", 7: "GLU_ERR_UNSUPPORTED", 8: "GLU_ERR_HIP",
}

_i64, _int, _p = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
_SIGNATURES = {
    "glu_fwd": [_int, _int, _i64, _i64, _p, _p, _i64, _p, _i64, _p],
    "glu_bwd": [_int, _int, _i64, _i64, _p, _p, _i64, _p, _i64, _p, _p, _i64, _p],
    "glu_fwd_mxfp8": [_int, _int, _i64, _i64, _p, _p, _i64, _int, _p, _p, _p, _p, _p],
    "glu_bwd_mxfp8": [_int, _int, _i64, _i64, _p, _p, _i64, _p, _i64, _int, _p, _p, _p, _p, _p],
    "glu_fwd_nvfp4": [_int, _int, _i64, _i64, _p, _p, _i64, _p, _p, _int, _p],
    "glu_bwd_nvfp4": [_int, _int, _i64, _i64, _p, _p, _i64, _p, _i64, _p, _p, _int, _p],
    "glu_amax": [_int, _int, _i64, _i64, _p, _p, _i64, _p, _p],
    "glu_gemm": [_int, _int, _int, _i64, _i64, _i64, _p, _p, _p, _p, _p, _i64, _p],
    "glu_gemm_mxfp8": [_int, _int, _int, _i64, _i64, _i64, _p, _p, _p, _p, _p, _p, _p],
    "glu_gemm_nvfp4": [_int, _int, _int, _i64, _i64, _i64, _p, _p, _p, _p, _p, _p, _int, _p],
    "glu_gemm_nvfp4_gs": [_int, _int, _int, _i64, _i64, _i64, _p, _p, _p, _p, _p, _p, _p, _int, _p],
    "glu_mx_gemm_f32": [_int, _int, _i64, _i64, _i64, _p, _p, _p, _p, _p, _p],
    "glu_fwd_nvfp4_gs": [_int, _int, _i64, _i64, _p, _p, _i64, _p, _p, _p, _int, _p],
    "glu_quant_mxfp8_f32": [_i64, _i64, _p, _i64, _int, _p, _p, _p, _p, _p],
    "glu_quant_nvfp4_f32": [_i64, _i64, _p, _i64, _p, _p, _int, _p],
    "glu_check_fwd": [_int, _int, _i64, _i64, _p, _p, _i64, _p, _i64],
    "glu_check_bwd": [_int, _int, _i64, _i64, _p, _p, _i64, _p, _i64, _p, _p, _i64],
    "glu_check_fwd_mxfp8": [_int, _int, _i64, _i64, _p, _p, _i64, _int, _p, _p, _p, _p],
    "glu_check_bwd_mxfp8": [_int, _int, _i64, _i64, _p, _p, _i64, _p, _i64, _int, _p, _p, _p, _p],
    "glu_check_fwd_nvfp4": [_int, _int, _i64, _i64, _p, _p, _i64, _p, _p, _int],
    "glu_check_bwd_nvfp4": [_int, _int, _i64, _i64, _p, _p, _i64, _p, _i64, _p, _p, _int],
    "glu_check_amax": [_int, _int, _i64, _i64, _p, _p, _i64, _p],
    "glu_check_gemm": [_int, _int, _int, _i64, _i64, _i64, _p, _p, _p, _p, _p, _i64],
    "glu_check_gemm_mxfp8": [_int, _int, _int, _i64, _i64, _i64, _p, _p, _p, _p, _p, _p],
    "glu_check_gemm_nvfp4": [_int, _int, _int, _i64, _i64, _i64, _p, _p, _p, _p, _p, _p, _int],
    "glu_check_gemm_nvfp4_gs": [_int, _int, _int, _i64, _i64, _i64, _p, _p, _p, _p, _p, _p, _p, _int],
    "glu_check_mx_gemm_f32": [_int, _int, _i64, _i64, _i64, _p, _p, _p, _p, _p],
    "glu_check_fwd_nvfp4_gs": [_int, _int, _i64, _i64, _p, _p, _i64, _p, _p, _p, _int],
    "glu_check_quant_mxfp8_f32": [_i64, _i64, _p, _i64, _int, _p, _p, _p, _p],
    "glu_check_quant_nvfp4_f32": [_i64, _i64, _p, _i64, _p, _p, _int],
    "glu_stream_probe": [_int, _p, _int, _p, _i64, _int, _p],
    "glu_check_stream_probe": [_int, _p, _int, _p, _i64, _int],
}

_lib = None


class GluError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn}: {STATUS.get(status, status)} ({lib().glu_status_string(status).decode()})")


def lib():
    """The loaded C library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "or python glu_activation_microscaling_amd/build.py")
        L = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGNATURES.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = ctypes.c_int
        L.glu_status_string.argtypes = [ctypes.c_int]
        L.glu_status_string.restype = ctypes.c_char_p
        L.glu_nvfp4_sf_bytes.argtypes = [_i64, _i64, _int]
        L.glu_nvfp4_sf_bytes.restype = _i64
        L.glu_mxfp8_sf_bytes.argtypes = [_i64, _i64, _int]
        L.glu_mxfp8_sf_bytes.restype = _i64
        L.glu_version.restype = ctypes.c_int
        _lib = L
    return _lib


def _call(fn, *args):
    st = getattr(lib(), fn)(*args)
    if st != 0:
        raise GluError(fn, st)


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None and t.numel() > 0 else None


def _rowmajor(t, name, dtype):
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dim() != 2 or (t.size(1) > 1 and t.stride(1) != 1):
        raise ValueError(f"{name} must be a 2-D tensor with unit column stride (no silent copies)")
    return t.size(0), t.size(1), t.stride(0)


def _shaped(t, name, M, N):
    """A BF16 [M, N] operand or output with unit column stride; returns its row stride."""
    Mt, Nt, ld = _rowmajor(t, name, torch.bfloat16)
    if (Mt, Nt) != (M, N):
        raise ValueError(f"{name} must be [{M}, {N}], got [{Mt}, {Nt}]")
    return ld


def _byte_buffer(t, name, numel):
    """A caller-supplied code or scale buffer: contiguous uint8 on the GPU, numel bytes."""
    if t.dtype != torch.uint8:
        raise TypeError(f"{name} must be torch.uint8, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() != numel:
        raise ValueError(f"{name} must hold {numel} bytes, got {t.numel()}")


def _dh(dh, M, N):
    return _shaped(dh, "dh", M, N)


def _operands(gate, up, layout):
    M, C, ld = _rowmajor(gate, "gate", torch.bfloat16)
    if layout == "paired":
        if up is not None:
            raise ValueError("the paired layout takes one interleaved matrix")
        if C % 2:
            raise ValueError("the paired matrix needs an even number of columns")
        return M, C // 2, ld
    if up is None:
        raise ValueError("the split layout needs gate and up")
    Mu, Cu, ldu = _rowmajor(up, "up", torch.bfloat16)
    if (Mu, Cu) != (M, C):
        raise ValueError("gate and up differ in shape")
    if ldu != ld and M > 1:
        raise ValueError("gate and up must share a row stride")
    return M, C, ld


def glu_fwd(gate, up=None, *, act="swiglu", layout="split", out=None):
    """h = bf16(act(gate) * up), [M, N]."""
    M, N, ld = _operands(gate, up, layout)
    h = out if out is not None else torch.empty((M, N), dtype=torch.bfloat16, device=gate.device)
    ldh = _shaped(h, "out", M, N)
    _call("glu_fwd", ACT[act], LAYOUT[layout], M, N, _ptr(gate), _ptr(up), ld, _ptr(h), ldh,
          _stream(gate))
    return h


def glu_bwd(gate, up, dh, *, act="swiglu", layout="split", out=None):
    """Split: (da, db) each [M, N].  Paired: one interleaved [M, 2N] gradient.
    out: (da, db) for split or a single tensor for paired; may alias (gate, up) in place."""
    M, N, ld = _operands(gate, up, layout)
    lddh = _dh(dh, M, N)
    dev = gate.device
    if layout == "paired":
        d = out if out is not None else torch.empty((M, 2 * N), dtype=torch.bfloat16, device=dev)
        ldo = _shaped(d, "out", M, 2 * N)
        _call("glu_bwd", ACT[act], 1, M, N, _ptr(gate), None, ld, _ptr(dh), lddh, _ptr(d), None,
              ldo, _stream(gate))
        return d
    if out is None:
        out = (torch.empty((M, N), dtype=torch.bfloat16, device=dev),
               torch.empty((M, N), dtype=torch.bfloat16, device=dev))
    da, db = out
    ldo = _shaped(da, "da", M, N)
    ldb = _shaped(db, "db", M, N)
    if ldb != ldo and M > 1:
        raise ValueError("da and db must share a row stride")
    _call("glu_bwd", ACT[act], 0, M, N, _ptr(gate), _ptr(up), ld, _ptr(dh), lddh, _ptr(da),
          _ptr(db), ldo, _stream(gate))
    return da, db


def mxfp8_sf_bytes(rows, cols, swizzled=False):
    """Bytes of an MXFP8 scale buffer for a quantized [rows, cols] matrix."""
    return lib().glu_mxfp8_sf_bytes(rows, cols, int(bool(swizzled)))


def _mx_buffers(M, C, rowwise, colwise, dev, out, swizzled=False):
    def sbytes(rows, cols):
        return mxfp8_sf_bytes(rows, cols, True) if swizzled else rows * (cols // 32)

    if out is not None:
        q_row, q_col, s_row, s_col = out
        if rowwise:
            _byte_buffer(q_row, "q_row", M * C)
            _byte_buffer(s_row, "s_row", sbytes(M, C))
        if colwise:
            _byte_buffer(q_col, "q_col", C * M)
            _byte_buffer(s_col, "s_col", sbytes(C, M))
        return out
    u8 = dict(dtype=torch.uint8, device=dev)
    z = torch.empty((0,), **u8)

    def scales(rows, cols):
        if swizzled:
            return torch.empty((mxfp8_sf_bytes(rows, cols, True),), **u8)
        return torch.empty((rows, cols // 32), **u8)

    q_row = torch.empty((M, C), **u8) if rowwise else z
    s_row = scales(M, C) if rowwise else z
    q_col = torch.empty((C, M), **u8) if colwise else z
    s_col = scales(C, M) if colwise else z
    return q_row, q_col, s_row, s_col


def _flags(rowwise, colwise, swizzled=False):
    f = (ROWWISE if rowwise else 0) | (COLWISE if colwise else 0)
    if f == 0:
        raise ValueError("enable rowwise, colwise or both")
    return f | (SF_SWIZZLED if swizzled else 0)


def glu_fwd_mxfp8(gate, up=None, *, act="swiglu", layout="split", rowwise=True, colwise=False,
                  swizzled=False, out=None):
    """Fused forward + MXFP8: (q_row [M,N], q_col [N,M], s_row [M,N/32], s_col [N,M/32]);
    swizzled=True gives both scale matrices as flat zero-padded 128x4 buffers."""
    M, N, ld = _operands(gate, up, layout)
    f = _flags(rowwise, colwise, swizzled)
    q_row, q_col, s_row, s_col = _mx_buffers(M, N, rowwise, colwise, gate.device, out, swizzled)
    _call("glu_fwd_mxfp8", ACT[act], LAYOUT[layout], M, N, _ptr(gate), _ptr(up), ld, f,
          _ptr(q_row), _ptr(s_row), _ptr(q_col), _ptr(s_col), _stream(gate))
    return q_row, q_col, s_row, s_col


def glu_bwd_mxfp8(gate, up, dh, *, act="swiglu", rowwise=True, colwise=False, swizzled=False,
                  out=None):
    """Fused backward + MXFP8 of [da | db] ([M, 2N]): (q_row [M,2N], q_col [2N,M],
    s_row [M,2N/32], s_col [2N,M/32]); swizzled=True as for glu_fwd_mxfp8."""
    M, N, ld = _operands(gate, up, "split")
    lddh = _dh(dh, M, N)
    f = _flags(rowwise, colwise, swizzled)
    q_row, q_col, s_row, s_col = _mx_buffers(M, 2 * N, rowwise, colwise, gate.device, out, swizzled)
    _call("glu_bwd_mxfp8", ACT[act], 0, M, N, _ptr(gate), _ptr(up), ld, _ptr(dh), lddh, f,
          _ptr(q_row), _ptr(s_row), _ptr(q_col), _ptr(s_col), _stream(gate))
    return q_row, q_col, s_row, s_col


def nvfp4_sf_bytes(M, H, sf_layout="rowmajor"):
    return lib().glu_nvfp4_sf_bytes(M, H, SF_LAYOUT[sf_layout])


def _nv_buffers(M, H, sf_layout, dev, out):
    if out is not None:
        _byte_buffer(out[0], "q", M * (H // 2))
        _byte_buffer(out[1], "sf", nvfp4_sf_bytes(M, H, sf_layout))
        return out
    q = torch.empty((M, H // 2), dtype=torch.uint8, device=dev)
    if sf_layout == "rowmajor":
        sf = torch.empty((M, H // 16), dtype=torch.uint8, device=dev)
    else:
        sf = torch.empty((nvfp4_sf_bytes(M, H, sf_layout),), dtype=torch.uint8, device=dev)
    return q, sf


def glu_fwd_nvfp4(x, up=None, *, act="geglu", layout="paired", sf_layout="rowmajor", out=None):
    """Fused forward + NVFP4 (global scale 1): (q [M, H/2] packed E2M1, sf scales)."""
    M, H, ld = _operands(x, up, layout)
    q, sf = _nv_buffers(M, H, sf_layout, x.device, out)
    _call("glu_fwd_nvfp4", ACT[act], LAYOUT[layout], M, H, _ptr(x), _ptr(up), ld, _ptr(q), _ptr(sf),
          SF_LAYOUT[sf_layout], _stream(x))
    return q, sf


def glu_amax(gate, up=None, *, act="swiglu", layout="split", out=None):
    """Largest |h| of h = bf16(act(gate) * up), as a float32 [1] GPU tensor (no host sync)."""
    M, N, ld = _operands(gate, up, layout)
    a = out if out is not None else torch.empty((1,), dtype=torch.float32, device=gate.device)
    if a.dtype != torch.float32 or not a.is_cuda or a.numel() < 1:
        raise ValueError("out must be a float32 GPU tensor with at least one element")
    _call("glu_amax", ACT[act], LAYOUT[layout], M, N, _ptr(gate), _ptr(up), ld, _ptr(a), _stream(gate))
    return a


def glu_fwd_nvfp4_gs(x, up=None, *, amax, act="geglu", layout="paired", sf_layout="rowmajor", out=None):
    """Fused forward + two-level NVFP4: global encode scale from the float32 GPU tensor amax
    (its first element, e.g. glu_amax's output): (q [M, H/2] packed E2M1, sf scales)."""
    M, H, ld = _operands(x, up, layout)
    if amax.dtype != torch.float32 or not amax.is_cuda or amax.numel() < 1:
        raise ValueError("amax must be a float32 GPU tensor")
    q, sf = _nv_buffers(M, H, sf_layout, x.device, out)
    _call("glu_fwd_nvfp4_gs", ACT[act], LAYOUT[layout], M, H, _ptr(x), _ptr(up), ld, _ptr(amax), _ptr(q),
          _ptr(sf), SF_LAYOUT[sf_layout], _stream(x))
    return q, sf


def _gemm_operands(xq, xs, wq, ws, fmt):
    """Block-scaled operands of the merged gate/up GEMM, contiguous uint8 on the GPU: codes
    xq [M, K] and wq [2N, K] (mxfp8), or packed xq [M, K/2] and wq [2N, K/2] (mxfp4), and
    E8M0 scales xs [M, K/32], ws [2N, K/32]; returns (fmt code, M, N, K)."""
    if fmt not in GEMM_FMT:
        raise ValueError(f"fmt must be one of {sorted(GEMM_FMT)}")
    for t, name in ((xq, "xq"), (xs, "xs"), (wq, "wq"), (ws, "ws")):
        if t.dtype != torch.uint8 or not t.is_cuda or t.dim() != 2 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous 2-D torch.uint8 GPU tensor")
    M, rb = xq.shape
    K = 2 * rb if fmt == "mxfp4" else rb
    N2 = wq.shape[0]
    if wq.shape[1] != rb or tuple(xs.shape) != (M, K // 32) or tuple(ws.shape) != (N2, K // 32) or N2 % 2:
        raise ValueError("operand shapes: xq [M, K], xs [M, K/32], wq [2N, K], ws [2N, K/32] "
                         "(codes [rows, K/2] bytes for mxfp4)")
    return GEMM_FMT[fmt], M, N2 // 2, K


def glu_gemm(xq, xs, wq, ws, *, act="swiglu", fmt="mxfp8", w_layout="split", out=None):
    """h = bf16(act(Y_gate) * Y_up), Y = X W^T of block-scaled operands: [M, N].  W's rows are
    [W_gate | W_up] (split) or gate0, up0, gate1, up1, ... (paired)."""
    f, M, N, K = _gemm_operands(xq, xs, wq, ws, fmt)
    h = out if out is not None else torch.empty((M, N), dtype=torch.bfloat16, device=xq.device)
    ldh = _shaped(h, "out", M, N)
    _call("glu_gemm", ACT[act], f, W_LAYOUT[w_layout], M, N, K, _ptr(xq), _ptr(xs), _ptr(wq), _ptr(ws),
          _ptr(h), ldh, _stream(xq))
    return h


def glu_gemm_mxfp8(xq, xs, wq, ws, *, act="swiglu", fmt="mxfp8", w_layout="split", out=None):
    """The same h quantized MXFP8 rowwise: (q_row [M, N], s_row [M, N/32])."""
    f, M, N, K = _gemm_operands(xq, xs, wq, ws, fmt)
    if out is not None:
        q, sc = out
        _byte_buffer(q, "q_row", M * N)
        _byte_buffer(sc, "s_row", M * (N // 32))
    else:
        q = torch.empty((M, N), dtype=torch.uint8, device=xq.device)
        sc = torch.empty((M, N // 32), dtype=torch.uint8, device=xq.device)
    _call("glu_gemm_mxfp8", ACT[act], f, W_LAYOUT[w_layout], M, N, K, _ptr(xq), _ptr(xs), _ptr(wq), _ptr(ws),
          _ptr(q), _ptr(sc), _stream(xq))
    return q, sc


def glu_gemm_nvfp4(xq, xs, wq, ws, *, act="geglu", fmt="mxfp8", w_layout="split", sf_layout="rowmajor",
                   out=None):
    """The same h quantized NVFP4, global scale 1: (q [M, N/2] packed E2M1, sf scales)."""
    f, M, N, K = _gemm_operands(xq, xs, wq, ws, fmt)
    q, sf = _nv_buffers(M, N, sf_layout, xq.device, out)
    _call("glu_gemm_nvfp4", ACT[act], f, W_LAYOUT[w_layout], M, N, K, _ptr(xq), _ptr(xs), _ptr(wq), _ptr(ws),
          _ptr(q), _ptr(sf), SF_LAYOUT[sf_layout], _stream(xq))
    return q, sf


def glu_gemm_nvfp4_gs(xq, xs, wq, ws, *, amax, act="geglu", fmt="mxfp8", w_layout="split",
                      sf_layout="rowmajor", out=None):
    """The same h quantized two-level NVFP4, the global scale from `amax` (a float32 [1] GPU
    tensor, e.g. kept from an earlier step): (q [M, N/2] packed E2M1, sf scales)."""
    f, M, N, K = _gemm_operands(xq, xs, wq, ws, fmt)
    if amax.dtype != torch.float32 or not amax.is_cuda or amax.numel() != 1:
        raise ValueError("amax must be a float32 GPU tensor with one element")
    q, sf = _nv_buffers(M, N, sf_layout, xq.device, out)
    _call("glu_gemm_nvfp4_gs", ACT[act], f, W_LAYOUT[w_layout], M, N, K, _ptr(xq), _ptr(xs), _ptr(wq),
          _ptr(ws), _ptr(amax), _ptr(q), _ptr(sf), SF_LAYOUT[sf_layout], _stream(xq))
    return q, sf


def mx_gemm_f32(xq, xs, wq, ws, *, fmt="mxfp8", w_layout="split", out=None):
    """Test hook: the merged GEMM's FP32 result as the fused kernels form it, [M, 2N] =
    [Y_gate | Y_up] whatever w_layout."""
    f, M, N, K = _gemm_operands(xq, xs, wq, ws, fmt)
    y = out if out is not None else torch.empty((M, 2 * N), dtype=torch.float32, device=xq.device)
    if y.dtype != torch.float32 or not y.is_cuda or not y.is_contiguous() or tuple(y.shape) != (M, 2 * N):
        raise ValueError(f"out must be a contiguous float32 [{M}, {2 * N}] GPU tensor")
    _call("glu_mx_gemm_f32", f, W_LAYOUT[w_layout], M, N, K, _ptr(xq), _ptr(xs), _ptr(wq), _ptr(ws), _ptr(y),
          _stream(xq))
    return y


def glu_bwd_nvfp4(gate, up, dh, *, act="swiglu", sf_layout="rowmajor", out=None):
    """Fused backward + NVFP4 (global scale 1) of [da | db] ([M, 2N]): (q [M, N] packed E2M1,
    sf scales of [M, 2N/16])."""
    M, N, ld = _operands(gate, up, "split")
    lddh = _dh(dh, M, N)
    q, sf = _nv_buffers(M, 2 * N, sf_layout, gate.device, out)
    _call("glu_bwd_nvfp4", ACT[act], 0, M, N, _ptr(gate), _ptr(up), ld, _ptr(dh), lddh, _ptr(q),
          _ptr(sf), SF_LAYOUT[sf_layout], _stream(gate))
    return q, sf


def glu_quant_mxfp8_f32(x, *, rowwise=True, colwise=False, swizzled=False, out=None):
    """The MXFP8 quantizer alone on an FP32 [M, N] matrix."""
    M, N, ld = _rowmajor(x, "x", torch.float32)
    f = _flags(rowwise, colwise, swizzled)
    q_row, q_col, s_row, s_col = _mx_buffers(M, N, rowwise, colwise, x.device, out, swizzled)
    _call("glu_quant_mxfp8_f32", M, N, _ptr(x), ld, f, _ptr(q_row), _ptr(s_row), _ptr(q_col),
          _ptr(s_col), _stream(x))
    return q_row, q_col, s_row, s_col


def glu_quant_nvfp4_f32(x, *, sf_layout="rowmajor", out=None):
    """The NVFP4 quantizer alone on an FP32 [M, H] matrix."""
    M, H, ld = _rowmajor(x, "x", torch.float32)
    q, sf = _nv_buffers(M, H, sf_layout, x.device, out)
    _call("glu_quant_nvfp4_f32", M, H, _ptr(x), ld, _ptr(q), _ptr(sf), SF_LAYOUT[sf_layout], _stream(x))
    return q, sf


def glu_stream_probe(srcs, dsts):
    """The streaming probe (a measurement hook): each of the 1..3 uint8 GPU tensors in srcs
    (n bytes each, n % 16 == 0) is read once and each of the 1..4 uint8 tensors in dsts
    (n, n / 2 or n / 4 bytes each, all the same) written once, as glu_mx.h describes."""
    n = srcs[0].numel()
    for t in (*srcs, *dsts):
        if t.dtype != torch.uint8 or not t.is_cuda or not t.is_contiguous():
            raise ValueError("stream probe buffers are contiguous uint8 GPU tensors")
    if n % 16 or any(t.numel() != n for t in srcs) or len({t.numel() for t in dsts}) != 1:
        raise ValueError("sources of equal size (a multiple of 16 bytes), destinations of equal size")
    width = dsts[0].numel() * 16 // n if n else 16
    if width not in (4, 8, 16) or dsts[0].numel() * 16 != width * n:
        raise ValueError("destinations hold 4, 8 or 16 bytes per 16 source bytes")
    src = (ctypes.c_void_p * 3)(*[t.data_ptr() for t in srcs])
    dst = (ctypes.c_void_p * 4)(*[t.data_ptr() for t in dsts])
    _call("glu_stream_probe", len(srcs), ctypes.cast(src, ctypes.c_void_p), len(dsts),
          ctypes.cast(dst, ctypes.c_void_p), n // 16, width, _stream(srcs[0]))

