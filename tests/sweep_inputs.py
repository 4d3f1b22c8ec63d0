"""Deterministic sweep inputs for the exhaustive quantizer tests (no arithmetic of the method:
bit patterns only, chosen so that every value and scale regime occurs)."""
import numpy as np
import torch


def mxfp8_sweep_matrix():
    """BF16 bits of a [R, 256] matrix of 32-element blocks (R a multiple of 128) covering:
      * every scale byte 0..247 (e = -127..120): a block's maximum is pinned at 448 * 2^e
        (for e = 120 at the largest BF16, which still needs that scale), at a random position,
        and its 31 other elements run through every BF16 magnitude from 2^(e-12) up to the
        maximum, with random signs: every E4M3 rounding midpoint and its BF16 neighbours at
        that scale, the subnormal E4M3 codes, and values that round to zero;
      * every finite positive BF16 number as a block maximum (the RCEIL decision at every
        boundary), the other 31 elements smaller, with random signs;
      * an all-zero block, an all -0 block, and blocks of BF16 subnormals only."""
    rng = np.random.default_rng(2024)
    mags = np.arange(1, 0x7F80, dtype=np.uint32)                 # every finite positive BF16
    vals = (mags << 16).view(np.float32).astype(np.float64)
    blocks = []
    for e in range(-127, 121):
        top = 448.0 * 2.0 ** e
        amax_bits = 0x7F7F if e == 120 else int(np.searchsorted(vals, top) + 1)   # bits of 448 * 2^e
        assert e == 120 or vals[amax_bits - 1] == top
        pick = mags[(vals >= 2.0 ** (e - 12)) & (mags < amax_bits)]
        pick = np.concatenate([pick, pick])                       # both signs of each
        pick = rng.permutation(pick)
        n = -(-pick.size // 31)
        body = np.resize(pick, n * 31).reshape(n, 31)
        body = body | (rng.integers(0, 2, body.shape, dtype=np.uint32) << 15)
        head = np.full((n, 1), amax_bits, np.uint32) | (rng.integers(0, 2, (n, 1), dtype=np.uint32) << 15)
        blk = np.concatenate([head, body], axis=1)
        pos = rng.integers(0, 32, n)
        blk[np.arange(n), 0], blk[np.arange(n), pos] = blk[np.arange(n), pos], blk[np.arange(n), 0].copy()
        blocks.append(blk)
    # every BF16 magnitude as a block maximum, the rest uniformly smaller (as BF16)
    n = mags.size
    rest = (vals[:, None] * rng.uniform(-0.999, 0.999, (n, 31))).astype(np.float32)
    rest_bits = torch.from_numpy(rest).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    blk = np.concatenate([mags[:, None], rest_bits.astype(np.uint32)], axis=1)
    blocks.append(blk)
    special = np.zeros((4, 32), np.uint32)
    special[1] = 0x8000                                             # -0
    special[2] = rng.integers(1, 0x80, 32)                          # positive subnormals
    special[3] = rng.integers(1, 0x80, 32) | 0x8000                 # negative subnormals
    blocks.append(special)
    allb = np.concatenate(blocks).astype(np.uint16)
    rows = -(-allb.shape[0] // 8)
    rows = -(-rows // 128) * 128
    out = np.zeros((rows * 8, 32), np.uint16)
    out[: allb.shape[0]] = allb
    return out.reshape(rows, 256)
