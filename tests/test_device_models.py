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
