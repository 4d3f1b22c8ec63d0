"""Every byte of every quantized output is written by the kernels, whatever the buffer held.

Each entry point runs twice on the same inputs, into caller buffers filled first with 0x00
and then with 0xFF; the results must be identical.  A byte the kernels leave unwritten (a
padding row or column of the 128x4 scale layout, the last partial tile, the byte scales of
a backward whose [dGate | dUp] halves do not start on a 4-block boundary) keeps the fill
and differs between the two runs.  The other GPU tests compare the outputs with the oracle.
"""
import pytest
import torch

import synthetic_inputs as si

pytestmark = pytest.mark.gpu


def _filled_twice(run, shapes):
    """run(out) into buffers of the given byte counts, filled with 0x00 then 0xFF."""
    got = []
    for fill in (0x00, 0xFF):
        out = [torch.full((n,), fill, dtype=torch.uint8, device="cuda") for n in shapes]
        run(out)
        torch.cuda.synchronize()
        got.append([o.cpu() for o in out])
    for i, (a, b) in enumerate(zip(*got)):
        assert torch.equal(a, b), f"output {i}: {int((a != b).sum())} bytes not written"


def _operands(M, N, seed, with_dh=False):
    ops = si.glu_operands(M, N, seed=seed, outliers=True, with_dh=with_dh)
    return [t.cuda() for t in ops]


@pytest.mark.parametrize("sf_layout", ["rowmajor", "128x4"])
@pytest.mark.parametrize("M,H", [(1, 512), (130, 528), (968, 1024), (37, 2064)])
def test_nvfp4_fwd(gpu, sf_layout, M, H):
    g, u = _operands(M, H, seed=M + H)
    x = torch.stack([g, u], 2).reshape(M, 2 * H).contiguous()
    shapes = [M * H // 2, gpu.nvfp4_sf_bytes(M, H, sf_layout)]
    _filled_twice(lambda out: gpu.glu_fwd_nvfp4(x, act="geglu", layout="paired", sf_layout=sf_layout,
                                                out=(out[0].view(M, H // 2), out[1])), shapes)
    _filled_twice(lambda out: gpu.glu_fwd_nvfp4(g, u, act="swiglu", layout="split", sf_layout=sf_layout,
                                                out=(out[0].view(M, H // 2), out[1])), shapes)


@pytest.mark.parametrize("sf_layout", ["rowmajor", "128x4"])
@pytest.mark.parametrize("M,H", [(1, 512), (130, 528)])
def test_nvfp4_two_level_fwd(gpu, sf_layout, M, H):
    g, u = _operands(M, H, seed=7 + M)
    amax = gpu.glu_amax(g, u, act="geglu")
    shapes = [M * H // 2, gpu.nvfp4_sf_bytes(M, H, sf_layout)]
    _filled_twice(lambda out: gpu.glu_fwd_nvfp4_gs(g, u, amax=amax, act="geglu", layout="split",
                                                   sf_layout=sf_layout, out=(out[0].view(M, H // 2), out[1])),
                  shapes)


@pytest.mark.parametrize("sf_layout", ["rowmajor", "128x4"])
@pytest.mark.parametrize("M,N", [(5, 48), (1, 512), (130, 1024), (37, 2064)])
def test_nvfp4_bwd(gpu, sf_layout, M, N):
    g, u, d = _operands(M, N, seed=11 + N, with_dh=True)
    shapes = [M * N, gpu.nvfp4_sf_bytes(M, 2 * N, sf_layout)]
    _filled_twice(lambda out: gpu.glu_bwd_nvfp4(g, u, d, act="swiglu", sf_layout=sf_layout,
                                                out=(out[0].view(M, N), out[1])), shapes)


@pytest.mark.parametrize("sf_layout", ["rowmajor", "128x4"])
@pytest.mark.parametrize("M,H", [(3, 32), (130, 528)])
def test_nvfp4_quantizer_hook(gpu, sf_layout, M, H):
    x = torch.randn(M, H, generator=torch.Generator().manual_seed(M * H), dtype=torch.float32).cuda()
    shapes = [M * H // 2, gpu.nvfp4_sf_bytes(M, H, sf_layout)]
    _filled_twice(lambda out: gpu.glu_quant_nvfp4_f32(x, sf_layout=sf_layout,
                                                      out=(out[0].view(M, H // 2), out[1])), shapes)


def _mx_shapes(gpu, M, C, swizzled):
    def sbytes(rows, cols):
        return gpu.mxfp8_sf_bytes(rows, cols, True) if swizzled else rows * (cols // 32)
    return [M * C, C * M, sbytes(M, C), sbytes(C, M)]


def _mx_out(out, M, C, swizzled):
    q_row, q_col, s_row, s_col = out
    if swizzled:
        return q_row.view(M, C), q_col.view(C, M), s_row, s_col
    return q_row.view(M, C), q_col.view(C, M), s_row.view(M, C // 32), s_col.view(C, M // 32)


@pytest.mark.parametrize("swizzled", [False, True])
@pytest.mark.parametrize("M,N", [(352, 480), (160, 224), (96, 160)])
def test_mxfp8_fwd_and_bwd_both(gpu, swizzled, M, N):
    g, u, d = _operands(M, N, seed=3 + M, with_dh=True)
    _filled_twice(lambda out: gpu.glu_fwd_mxfp8(g, u, act="swiglu", rowwise=True, colwise=True,
                                                swizzled=swizzled, out=_mx_out(out, M, N, swizzled)),
                  _mx_shapes(gpu, M, N, swizzled))
    _filled_twice(lambda out: gpu.glu_bwd_mxfp8(g, u, d, act="swiglu", rowwise=True, colwise=True,
                                                swizzled=swizzled, out=_mx_out(out, M, 2 * N, swizzled)),
                  _mx_shapes(gpu, M, 2 * N, swizzled))
