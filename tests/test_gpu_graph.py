"""The entry points under HIP graph capture.

The library launches kernels on the caller's stream and allocates, synchronizes and frees
nothing, so a sequence of its calls can be captured into a graph ([MX] API: the fused op is
graph-capturable).  Every output is allocated before the capture; the graph is replayed
several times, with eager launches and synchronizations between the replays and the outputs
overwritten in between, and every replay is compared byte for byte with the eager results.
No capture records a memset: the amax pass clears its output with a kernel of its own.
"""
import pytest
import torch

import synthetic_inputs as si

pytestmark = pytest.mark.gpu


def _same(a, b):
    return all(torch.equal(x.view(torch.uint8), y.view(torch.uint8)) for x, y in zip(a, b))


def test_replays_equal_eager(gpu):
    M, N, K = 256, 256, 512
    g, u, d = (t.cuda() for t in si.glu_operands(M, N, seed=120, outliers=True, with_dh=True))
    x = torch.stack([g, u], 2).reshape(M, 2 * N).contiguous()
    mx = si.mx_operand(M, K, seed=121, device="cuda") + si.mx_operand(2 * N, K, seed=122, device="cuda")

    h = torch.empty_like(g)
    da, db = torch.empty_like(g), torch.empty_like(g)
    fq = gpu._mx_buffers(M, N, True, True, "cuda", None)
    bq = gpu._mx_buffers(M, 2 * N, True, True, "cuda", None)
    nq = gpu._nv_buffers(M, N, "128x4", "cuda", None)
    amax = torch.empty((1,), dtype=torch.float32, device="cuda")
    gq = gpu._nv_buffers(M, N, "rowmajor", "cuda", None)
    mq = (torch.empty((M, N), dtype=torch.uint8, device="cuda"),
          torch.empty((M, N // 32), dtype=torch.uint8, device="cuda"))
    outs = [h, da, db, *fq, *bq, *nq, amax, *gq, *mq]

    def step():
        gpu.glu_fwd(g, u, act="swiglu", out=h)
        gpu.glu_bwd(g, u, d, act="swiglu", out=(da, db))
        gpu.glu_fwd_mxfp8(g, u, act="swiglu", rowwise=True, colwise=True, out=fq)
        gpu.glu_bwd_mxfp8(g, u, d, act="swiglu", rowwise=True, colwise=True, out=bq)
        gpu.glu_fwd_nvfp4(x, act="geglu", layout="paired", sf_layout="128x4", out=nq)
        gpu.glu_amax(x, act="geglu", layout="paired", out=amax)
        gpu.glu_fwd_nvfp4_gs(x, amax=amax, act="geglu", layout="paired", out=gq)
        gpu.glu_gemm_mxfp8(*mx, act="swiglu", out=mq)

    step()
    torch.cuda.synchronize()
    eager = [t.clone() for t in outs]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                     # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    for replay in range(4):
        for t in outs:
            t.view(torch.uint8).fill_(0xAB)        # eager work between the replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert _same(outs, eager), f"replay {replay} differs from the eager results"
