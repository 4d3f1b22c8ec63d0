"""Exhaustive host checks of arithmetic shortcuts that the kernels take (CPU only).

Each test restates a kernel's shortcut in numpy (FP32 arithmetic is IEEE in both places)
and checks it, over its whole input domain, against the oracle's definition.
"""
import numpy as np

import oracle


def test_nvfp4_scale_of_bf16_amax():
    """NVFP4 block scale for a BF16-valued block maximum: the FP32 product amax * fl(1/6),
    clamped to 448, rounds (E4M3, nearest even) to the same code as amax / 6 does, for every
    positive finite BF16 amax.  The kernels then let the hardware E4M3 convert decide it."""
    b = np.arange(1, 0x7F80, dtype=np.uint32)
    amax = (b << 16).view(np.float32)
    y = np.minimum((amax * np.float32(1.0 / 6.0)).astype(np.float32), np.float32(448.0))
    got = oracle.e4m3_from_f64(y.astype(np.float64))
    want = oracle.e4m3_from_f64(amax.astype(np.float64) / 6.0)
    assert np.array_equal(got, want)


def test_e2m1_code_of_bf16_rounded_quotient():
    """NVFP4 codes in the fused kernels: for a BF16 value x and a block scale S (every positive
    finite E4M3 value), the kernels form y = x * R with R the hardware reciprocal of S (within
    one FP32 ulp of 1/S), round y to BF16 (nearest even) and let the hardware E2M1 convert
    decide.  For every non-negative finite BF16 x, every S, and R = fl(1/S) and its two FP32
    neighbours, that code equals the code of the exact quotient x / S (the sign is carried by
    x; the E2M1 grid is symmetric)."""
    import torch
    b = np.arange(0, 0x7F80, dtype=np.uint32)
    x = (b << 16).view(np.float32)
    S = oracle.e4m3_to_f64(np.arange(1, 0x7F, dtype=np.uint8)).astype(np.float32)
    want = oracle.e2m1_from_f64((x[:, None].astype(np.float64) / S[None, :].astype(np.float64)).ravel())
    R0 = (np.float32(1.0) / S).astype(np.float32)
    for d in (-1, 0, 1):
        R = (R0.view(np.int32) + d).view(np.float32)
        with np.errstate(over="ignore"):
            y = (x[:, None] * R[None, :]).astype(np.float32)
        yb = torch.from_numpy(y).to(torch.bfloat16).float().numpy()     # nearest even
        got = oracle.e2m1_from_f64(yb.astype(np.float64).ravel())
        assert np.array_equal(got, want), f"R offset {d}: {int((got != want).sum())} codes differ"
