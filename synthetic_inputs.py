"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds no arithmetic of the method: it only draws random tensors.  Every
draw uses a CPU torch.Generator, so the same seed gives the same bits on any machine.

Workloads (shapes and value distributions of the pages' benchmarks):
  * swiglu_small  : gate, up BF16 [128, 128] ~ N(0, 1).
  * swiglu_mid    : gate, up, dh BF16 [4096, 2048] ~ N(0, 1).
  * swiglu_large  : gate, up, dh BF16 [16384, 7168] ~ N(0, 1) with 0.1% of the
                    elements of each tensor multiplied by 1000, and the rowwise-only
                    forward case [131072, 8192] with the same recipe.
  * geglu_bf16    : gate, up, dh BF16 [R, W] ~ N(0, 1), R in {1024, 8192},
                    W in {4096, 11008, 14336, 18944, 29568, 8193}.
  * geglu_nvfp4   : one BF16 [M, 32768] ~ N(0, 1) matrix, columns interleaved
                    gate0, up0, gate1, up1, ... for M in {784, 816, 880, 968}.
  * mx_operand    : an MXFP8 GEMM operand [rows, K]: E4M3 codes of N(0, 1) * 64 draws
                    (torch's float8_e4m3fn cast, clamped to +-448) and E8M0 block scales
                    (one per 32 along K) drawn uniformly from 2^-9 .. 2^-5, the range a
                    block of N(0, 1) data quantized to E4M3 takes.
  * mxfp4_operand : an MXFP4 GEMM operand: E2M1 codes [rows, K] packed two per byte
                    (element 2j in the low nibble), each code's magnitude drawn from the
                    eight E2M1 magnitudes with the frequencies a block of N(0, 1) data
                    scaled to a block maximum of 6 puts on them, a uniform sign, and E8M0
                    block scales drawn uniformly from 2^-5 .. 2^-1.
  * tail_operands : gate, up, dh BF16 [M, N] that send most elements down the kernels'
                    FP64 tail path: gates uniform over a range that straddles the switch
                    (SwiGLU -104 .. -78, tanh-GeGLU -11 .. -9, erf-GeGLU -40 .. -11) with
                    N(0, 1) * 2^k ups (k uniform in -10 .. 59) and N(0, 1) * 1000 dh; for
                    ReLU^2, gates of magnitude 2^e (e uniform in -75 .. 75, 10% negative)
                    with ups near 2^-2e and dh near 2^-e, so g^2 or dh g leaves the FP32
                    normal range while the results stay in it.
Draw order within one call: gate, up, dh (then the outlier masks, in the same order).
"""
import numpy as np
import torch

OUTLIER_FRACTION = 1e-3
OUTLIER_FACTOR = 1000.0


def _bits(t: torch.Tensor) -> np.ndarray:
    """BF16 tensor -> numpy uint16 bit patterns (a view, no arithmetic)."""
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def normal_bf16(shapes, seed=0, outliers=False):
    """Draws len(shapes) BF16 tensors ~ N(0,1) in order; with outliers=True each tensor
    has an independent Bernoulli(OUTLIER_FRACTION) mask of elements scaled by
    OUTLIER_FACTOR before the BF16 rounding.  Returns torch bfloat16 CPU tensors."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    ts = [torch.randn(s, generator=g, dtype=torch.float32) for s in shapes]
    if outliers:
        for t in ts:
            mask = torch.rand(t.shape, generator=g) < OUTLIER_FRACTION
            t[mask] *= OUTLIER_FACTOR
    return [t.to(torch.bfloat16) for t in ts]


def glu_operands(M, N, seed=0, outliers=False, with_dh=False):
    """gate, up (and dh) BF16 [M, N] as torch CPU tensors."""
    n = 3 if with_dh else 2
    return normal_bf16([(M, N)] * n, seed=seed, outliers=outliers)


# gate ranges of tail_operands that straddle the switch to the FP64 tail path
TAIL_GATE_RANGE = {"swiglu": (-104.0, -78.0), "geglu": (-11.0, -9.0), "geglu_erf": (-40.0, -11.0)}


def tail_operands(act, M, N, seed=0):
    """gate, up, dh BF16 [M, N] CPU tensors for the tail path of activation `act`
    ("swiglu", "geglu", "geglu_erf" or "relu2"); see the module docstring."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    shape = (M, N)
    if act == "relu2":
        def pow2(e):
            return torch.exp2(e.clamp(-125, 125).double())
        eg = torch.randint(-75, 76, shape, generator=g)
        gate = (torch.rand(shape, generator=g, dtype=torch.float64) + 0.5) * pow2(eg)
        gate = torch.where(torch.rand(shape, generator=g) < 0.1, -gate, gate)
        up = torch.randn(shape, generator=g, dtype=torch.float64) * pow2(-2 * eg + torch.randint(-4, 5, shape, generator=g))
        dh = torch.randn(shape, generator=g, dtype=torch.float64) * pow2(-eg + torch.randint(-4, 5, shape, generator=g))
    else:
        lo, hi = TAIL_GATE_RANGE[act]
        gate = torch.rand(shape, generator=g, dtype=torch.float64) * (hi - lo) + lo
        up = torch.randn(shape, generator=g, dtype=torch.float64) * torch.exp2(
            torch.randint(-10, 60, shape, generator=g).double())
        dh = torch.randn(shape, generator=g, dtype=torch.float64) * 1000
    return [t.to(torch.bfloat16) for t in (gate, up, dh)]


def paired_operand(M, H, seed=0):
    """One BF16 [M, 2H] matrix ~ N(0,1); column 2j is gate_j, column 2j+1 is up_j."""
    return normal_bf16([(M, 2 * H)], seed=seed)[0]


def special_bf16_values():
    """Every finite BF16 bit pattern (both signs), as a uint16 numpy array."""
    allb = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    mag = allb & 0x7FFF
    return allb[mag < 0x7F80]


def to_bits(t: torch.Tensor) -> np.ndarray:
    return _bits(t)


def from_bits(b: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16)


WORKLOADS = {
    "swiglu_small": dict(M=128, N=128),
    "swiglu_mid": dict(M=4096, N=2048),
    "swiglu_large": dict(M=16384, N=7168),
    "swiglu_xlarge_fwd_row": dict(M=131072, N=8192),
    "geglu_rows": (1024, 8192),
    "geglu_widths": (4096, 11008, 14336, 18944, 29568, 8193),
    "geglu_nvfp4_rows": (784, 816, 880, 968),
    "geglu_nvfp4_hidden": 16384,
}


def normal_bf16_device(shapes, seed=0, device="cuda", outliers=False):
    """Like normal_bf16 but drawn on the device with a seeded device generator (for the
    full-size workloads, where drawing gigabytes on the host would dominate).  The bits
    differ from the host draw of the same seed but are reproducible on any MI355X."""
    g = torch.Generator(device=device).manual_seed(seed)
    out = []
    for s in shapes:
        t = torch.randn(s, generator=g, device=device, dtype=torch.float32)
        if outliers:
            mask = torch.rand(s, generator=g, device=device) < OUTLIER_FRACTION
            t = torch.where(mask, t * OUTLIER_FACTOR, t)
        out.append(t.to(torch.bfloat16))
        del t
    return out


def mx_operand(rows, K, seed=0, device="cpu"):
    """(codes uint8 [rows, K], scales uint8 [rows, K / 32]) as torch tensors: E4M3 codes of
    N(0, 1) * 64 draws (torch's float8_e4m3fn cast of the clamped draw) and E8M0 scale bytes
    drawn uniformly from 118 .. 122 (2^-9 .. 2^-5).  Drawn on the host generator, then
    moved."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    v = (torch.randn((rows, K), generator=g, dtype=torch.float32) * 64.0).clamp(-448.0, 448.0)
    codes = v.to(torch.float8_e4m3fn).view(torch.uint8)
    scales = torch.randint(118, 123, (rows, K // 32), generator=g, dtype=torch.uint8)
    return codes.to(device), scales.to(device)


# Frequencies of the E2M1 magnitude codes 0..7 (0, 0.5, 1, 1.5, 2, 3, 4, 6) for N(0, 1) blocks
# of 32 scaled so that the block maximum sits near 6 (a fixed table: the draw itself does no
# rounding).
_E2M1_MAG_FREQ = (0.10, 0.20, 0.19, 0.16, 0.13, 0.13, 0.06, 0.03)


def mxfp4_operand(rows, K, seed=0, device="cpu"):
    """(packed E2M1 codes uint8 [rows, K / 2], E8M0 scales uint8 [rows, K / 32]) as torch
    tensors: per element a magnitude code drawn with _E2M1_MAG_FREQ and a uniform sign bit,
    two codes per byte with element 2j in the low nibble; scale bytes uniform in 122 .. 126
    (2^-5 .. 2^-1).  Drawn on the host generator, then moved."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    mag = torch.multinomial(torch.tensor(_E2M1_MAG_FREQ), rows * K, replacement=True, generator=g)
    sign = torch.randint(0, 2, (rows * K,), generator=g)
    codes = (mag | (sign << 3)).to(torch.uint8).reshape(rows, K // 2, 2)
    packed = codes[:, :, 0] | (codes[:, :, 1] << 4)
    scales = torch.randint(122, 127, (rows, K // 32), generator=g, dtype=torch.uint8)
    return packed.contiguous().to(device), scales.to(device)


def interleave_rows(w):
    """[2N, ...] = [gate rows | up rows] -> pairwise-interleaved rows gate0, up0, gate1, up1,
    ... (a permutation)."""
    n = w.shape[0] // 2
    return torch.stack([w[:n], w[n:]], dim=1).reshape(w.shape).contiguous()
