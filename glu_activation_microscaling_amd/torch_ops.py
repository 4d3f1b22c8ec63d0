"""torch custom ops over the library's entry points (framework integration).

The "Add swiglu + MXFP8 fused CuTe DSL kernel" page (API) exposes its kernel as a torch op
that torch.compile keeps whole; these ops do the same for the MI355X kernels:

  torch.ops.glu_mx.glu(gate, up, act, layout)                          -> h
  torch.ops.glu_mx.glu_backward(gate, up, dh, act, layout)             -> (da, db) or (d, empty)
  torch.ops.glu_mx.glu_mxfp8(gate, up, act, layout, rowwise, colwise, swizzled)
                                                                       -> (q_row, q_col, s_row, s_col)
  torch.ops.glu_mx.glu_backward_mxfp8(gate, up, dh, act, rowwise, colwise, swizzled)
                                                                       -> (q_row, q_col, s_row, s_col)
  torch.ops.glu_mx.glu_nvfp4(x, up, act, layout, sf_layout)            -> (q, sf)
  torch.ops.glu_mx.glu_backward_nvfp4(gate, up, dh, act, sf_layout)    -> (q, sf)
  torch.ops.glu_mx.glu_amax(gate, up, act, layout)                     -> amax [1]
  torch.ops.glu_mx.glu_nvfp4_gs(x, up, amax, act, layout, sf_layout)   -> (q, sf)
  torch.ops.glu_mx.glu_gemm(xq, xs, wq, ws, act, fmt, w_layout)        -> h
  torch.ops.glu_mx.glu_gemm_mxfp8(xq, xs, wq, ws, act, fmt, w_layout)  -> (q_row, s_row)
  torch.ops.glu_mx.glu_gemm_nvfp4(xq, xs, wq, ws, act, sf_layout, fmt, w_layout) -> (q, sf)
  torch.ops.glu_mx.glu_gemm_nvfp4_gs(xq, xs, wq, ws, amax, act, sf_layout, fmt, w_layout) -> (q, sf)

Each real implementation is the binding function of the same name (argument marshalling;
the HIP kernels compute everything).  Each fake implementation gives the output shapes and
dtypes without touching a GPU, so FakeTensor tracing and torch.compile(fullgraph=True)
capture the ops as single graph nodes.  `glu` is differentiable: its backward is the
`glu_backward` op (the fused BF16 backward kernel).  The quantized ops are not
differentiable.  In the split layout `up` is the second operand; in the paired layout pass
an empty `up` (a 0-element tensor), since a custom op cannot take None for a tensor that
other layouts need.
"""
from typing import Tuple

import torch
from torch import Tensor

from . import (glu_amax as _amax, glu_bwd as _bwd, glu_bwd_mxfp8 as _bwd_mx,
               glu_bwd_nvfp4 as _bwd_nv, glu_fwd as _fwd, glu_fwd_mxfp8 as _fwd_mx,
               glu_fwd_nvfp4 as _fwd_nv, glu_fwd_nvfp4_gs as _fwd_nv_gs, glu_gemm as _gemm,
               glu_gemm_mxfp8 as _gemm_mx, glu_gemm_nvfp4 as _gemm_nv,
               glu_gemm_nvfp4_gs as _gemm_nv_gs)

_LIB = "glu_mx"


def _up(up, layout):
    return None if layout == "paired" else up


def _width(gate, layout):
    """Per-half width N of the GLU output."""
    return gate.shape[1] // 2 if layout == "paired" else gate.shape[1]


def _mx_scale_shape(rows, cols, swizzled):
    if swizzled:
        return ((rows + 127) // 128 * 128 * ((cols // 32 + 3) // 4 * 4),)
    return (rows, cols // 32)


def _nv_scale_shape(rows, cols, sf_layout):
    if sf_layout == "128x4":
        return ((rows + 127) // 128 * 128 * ((cols // 16 + 3) // 4 * 4),)
    return (rows, cols // 16)


def _mx_fake(ref, rows, cols, rowwise, colwise, swizzled):
    u8 = dict(dtype=torch.uint8, device=ref.device)
    z = torch.empty((0,), **u8)
    return (torch.empty((rows, cols), **u8) if rowwise else z,
            torch.empty((cols, rows), **u8) if colwise else z,
            torch.empty(_mx_scale_shape(rows, cols, swizzled), **u8) if rowwise else z,
            torch.empty(_mx_scale_shape(cols, rows, swizzled), **u8) if colwise else z)


# ---- BF16 GLU, differentiable -------------------------------------------------------

@torch.library.custom_op(f"{_LIB}::glu", mutates_args=())
def glu(gate: Tensor, up: Tensor, act: str = "swiglu", layout: str = "split") -> Tensor:
    return _fwd(gate, _up(up, layout), act=act, layout=layout)


@glu.register_fake
def _(gate, up, act="swiglu", layout="split"):
    return gate.new_empty((gate.shape[0], _width(gate, layout)))


@torch.library.custom_op(f"{_LIB}::glu_backward", mutates_args=())
def glu_backward(gate: Tensor, up: Tensor, dh: Tensor, act: str = "swiglu",
                 layout: str = "split") -> Tuple[Tensor, Tensor]:
    """Split: (da, db).  Paired: (the interleaved gradient of the paired operand, empty)."""
    if layout == "paired":
        return _bwd(gate, None, dh, act=act, layout="paired"), gate.new_empty((0,))
    return _bwd(gate, up, dh, act=act)


@glu_backward.register_fake
def _(gate, up, dh, act="swiglu", layout="split"):
    if layout == "paired":
        return gate.new_empty(gate.shape), gate.new_empty((0,))
    return gate.new_empty(gate.shape), up.new_empty(up.shape)


def _glu_setup(ctx, inputs, output):
    gate, up, act, layout = inputs
    ctx.save_for_backward(gate, up)
    ctx.act, ctx.layout = act, layout


def _glu_grad(ctx, dh):
    gate, up = ctx.saved_tensors
    # the binding takes unit-stride rows; autograd may hand over a broadcast gradient
    d0, d1 = glu_backward(gate, up, dh.contiguous(), ctx.act, ctx.layout)
    if ctx.layout == "paired":
        return d0, None, None, None
    return d0, d1, None, None


glu.register_autograd(_glu_grad, setup_context=_glu_setup)


# ---- fused MXFP8 --------------------------------------------------------------------

@torch.library.custom_op(f"{_LIB}::glu_mxfp8", mutates_args=())
def glu_mxfp8(gate: Tensor, up: Tensor, act: str = "swiglu", layout: str = "split",
              rowwise: bool = True, colwise: bool = False,
              swizzled: bool = False) -> Tuple[Tensor, Tensor, Tensor, Tensor]:
    return _fwd_mx(gate, _up(up, layout), act=act, layout=layout, rowwise=rowwise,
                   colwise=colwise, swizzled=swizzled)


@glu_mxfp8.register_fake
def _(gate, up, act="swiglu", layout="split", rowwise=True, colwise=False, swizzled=False):
    return _mx_fake(gate, gate.shape[0], _width(gate, layout), rowwise, colwise, swizzled)


@torch.library.custom_op(f"{_LIB}::glu_backward_mxfp8", mutates_args=())
def glu_backward_mxfp8(gate: Tensor, up: Tensor, dh: Tensor, act: str = "swiglu",
                       rowwise: bool = True, colwise: bool = False,
                       swizzled: bool = False) -> Tuple[Tensor, Tensor, Tensor, Tensor]:
    return _bwd_mx(gate, up, dh, act=act, rowwise=rowwise, colwise=colwise, swizzled=swizzled)


@glu_backward_mxfp8.register_fake
def _(gate, up, dh, act="swiglu", rowwise=True, colwise=False, swizzled=False):
    return _mx_fake(gate, gate.shape[0], 2 * gate.shape[1], rowwise, colwise, swizzled)


# ---- fused NVFP4 --------------------------------------------------------------------

@torch.library.custom_op(f"{_LIB}::glu_nvfp4", mutates_args=())
def glu_nvfp4(x: Tensor, up: Tensor, act: str = "geglu", layout: str = "paired",
              sf_layout: str = "rowmajor") -> Tuple[Tensor, Tensor]:
    return _fwd_nv(x, _up(up, layout), act=act, layout=layout, sf_layout=sf_layout)


@glu_nvfp4.register_fake
def _(x, up, act="geglu", layout="paired", sf_layout="rowmajor"):
    M, H = x.shape[0], _width(x, layout)
    return (x.new_empty((M, H // 2), dtype=torch.uint8),
            x.new_empty(_nv_scale_shape(M, H, sf_layout), dtype=torch.uint8))


@torch.library.custom_op(f"{_LIB}::glu_backward_nvfp4", mutates_args=())
def glu_backward_nvfp4(gate: Tensor, up: Tensor, dh: Tensor, act: str = "swiglu",
                       sf_layout: str = "rowmajor") -> Tuple[Tensor, Tensor]:
    return _bwd_nv(gate, up, dh, act=act, sf_layout=sf_layout)


@glu_backward_nvfp4.register_fake
def _(gate, up, dh, act="swiglu", sf_layout="rowmajor"):
    M, N = gate.shape
    return (gate.new_empty((M, N), dtype=torch.uint8),
            gate.new_empty(_nv_scale_shape(M, 2 * N, sf_layout), dtype=torch.uint8))


@torch.library.custom_op(f"{_LIB}::glu_amax", mutates_args=())
def glu_amax(gate: Tensor, up: Tensor, act: str = "swiglu", layout: str = "split") -> Tensor:
    return _amax(gate, _up(up, layout), act=act, layout=layout)


@glu_amax.register_fake
def _(gate, up, act="swiglu", layout="split"):
    return gate.new_empty((1,), dtype=torch.float32)


@torch.library.custom_op(f"{_LIB}::glu_nvfp4_gs", mutates_args=())
def glu_nvfp4_gs(x: Tensor, up: Tensor, amax: Tensor, act: str = "geglu", layout: str = "paired",
                 sf_layout: str = "rowmajor") -> Tuple[Tensor, Tensor]:
    return _fwd_nv_gs(x, _up(up, layout), amax=amax, act=act, layout=layout, sf_layout=sf_layout)


@glu_nvfp4_gs.register_fake
def _(x, up, amax, act="geglu", layout="paired", sf_layout="rowmajor"):
    M, H = x.shape[0], _width(x, layout)
    return (x.new_empty((M, H // 2), dtype=torch.uint8),
            x.new_empty(_nv_scale_shape(M, H, sf_layout), dtype=torch.uint8))


# ---- merged gate/up block-scaled GEMM with the GLU epilogue ---------------------------
# xq [M, K] codes (fmt "mxfp8": E4M3, one per byte; "mxfp4": E2M1, [M, K/2] packed), xs [M, K/32]
# E8M0 scales, wq [2N, K] (rows [W_gate | W_up], or gate0, up0, ... with w_layout "paired"),
# ws [2N, K/32]

@torch.library.custom_op(f"{_LIB}::glu_gemm", mutates_args=())
def glu_gemm(xq: Tensor, xs: Tensor, wq: Tensor, ws: Tensor, act: str = "swiglu", fmt: str = "mxfp8",
             w_layout: str = "split") -> Tensor:
    return _gemm(xq, xs, wq, ws, act=act, fmt=fmt, w_layout=w_layout)


@glu_gemm.register_fake
def _(xq, xs, wq, ws, act="swiglu", fmt="mxfp8", w_layout="split"):
    return xq.new_empty((xq.shape[0], wq.shape[0] // 2), dtype=torch.bfloat16)


@torch.library.custom_op(f"{_LIB}::glu_gemm_mxfp8", mutates_args=())
def glu_gemm_mxfp8(xq: Tensor, xs: Tensor, wq: Tensor, ws: Tensor, act: str = "swiglu",
                   fmt: str = "mxfp8", w_layout: str = "split") -> Tuple[Tensor, Tensor]:
    return _gemm_mx(xq, xs, wq, ws, act=act, fmt=fmt, w_layout=w_layout)


@glu_gemm_mxfp8.register_fake
def _(xq, xs, wq, ws, act="swiglu", fmt="mxfp8", w_layout="split"):
    M, N = xq.shape[0], wq.shape[0] // 2
    return xq.new_empty((M, N), dtype=torch.uint8), xq.new_empty((M, N // 32), dtype=torch.uint8)


@torch.library.custom_op(f"{_LIB}::glu_gemm_nvfp4", mutates_args=())
def glu_gemm_nvfp4(xq: Tensor, xs: Tensor, wq: Tensor, ws: Tensor, act: str = "geglu",
                   sf_layout: str = "rowmajor", fmt: str = "mxfp8",
                   w_layout: str = "split") -> Tuple[Tensor, Tensor]:
    return _gemm_nv(xq, xs, wq, ws, act=act, sf_layout=sf_layout, fmt=fmt, w_layout=w_layout)


@glu_gemm_nvfp4.register_fake
def _(xq, xs, wq, ws, act="geglu", sf_layout="rowmajor", fmt="mxfp8", w_layout="split"):
    M, N = xq.shape[0], wq.shape[0] // 2
    return (xq.new_empty((M, N // 2), dtype=torch.uint8),
            xq.new_empty(_nv_scale_shape(M, N, sf_layout), dtype=torch.uint8))


@torch.library.custom_op(f"{_LIB}::glu_gemm_nvfp4_gs", mutates_args=())
def glu_gemm_nvfp4_gs(xq: Tensor, xs: Tensor, wq: Tensor, ws: Tensor, amax: Tensor,
                      act: str = "geglu", sf_layout: str = "rowmajor", fmt: str = "mxfp8",
                      w_layout: str = "split") -> Tuple[Tensor, Tensor]:
    return _gemm_nv_gs(xq, xs, wq, ws, amax=amax, act=act, sf_layout=sf_layout, fmt=fmt, w_layout=w_layout)


@glu_gemm_nvfp4_gs.register_fake
def _(xq, xs, wq, ws, amax, act="geglu", sf_layout="rowmajor", fmt="mxfp8", w_layout="split"):
    M, N = xq.shape[0], wq.shape[0] // 2
    return (xq.new_empty((M, N // 2), dtype=torch.uint8),
            xq.new_empty(_nv_scale_shape(M, N, sf_layout), dtype=torch.uint8))
