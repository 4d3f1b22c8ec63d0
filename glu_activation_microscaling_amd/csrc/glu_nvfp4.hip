// Fused GLU + NVFP4 quantization with global scale 1 ("feat(phyai-kernel): add Thor NVFP4
// GeGLU kernel for pi0.5", Summary: GeGLU fold and compact NVFP4 store; Supported contract:
// E2M1 values, E4M3 scales in the 128x4 layout, pairwise-interleaved gate/up columns), and
// the FP32 quantizer hook running the same quantize-and-store stage.
//
// Work decomposition (wave64): a workgroup of 4 waves covers 2048 consecutive outputs of one
// row; each lane computes 8 consecutive outputs (one 32-byte load of interleaved gate/up
// pairs, or 16 bytes each of gate and up).  A 16-element block is a lane pair, so the block
// amax is one DPP quad_perm exchange.  Each lane stores its 8 E2M1 codes as one 4-byte word
// (a wave writes 256 contiguous bytes); the even lane of a pair stores the scale byte.
// With the 128x4 layout the grid also covers the padding rows up to a multiple of 128, and
// the lane holding the last block of a row zero-fills the padding scale columns.
#include "glu_device.h"
#include "glu_launch.h"

namespace glu {
namespace {

constexpr int NV_THREADS = 256;
constexpr int64_t NV_TILE = 2048;  // outputs per workgroup and group
#ifndef GLU_NV_GROUPS              // build-time override, for measurements
#define GLU_NV_GROUPS 1
#endif
constexpr int NV_GROUPS = GLU_NV_GROUPS;  // groups of 8 outputs per lane

// Build-time tuning (fixed defaults; alternatives are compiled only to measure them):
//   GLU_NV_NT_LOADS / GLU_NV_NT_STORES: non-temporal (streaming) loads / code stores.
#ifndef GLU_NV_NT_LOADS
#define GLU_NV_NT_LOADS 0
#endif
#ifndef GLU_NV_NT_STORES
#define GLU_NV_NT_STORES 0
#endif

typedef unsigned int nu32x4 __attribute__((ext_vector_type(4)));

struct Words4 {
  uint32_t w[4];
};
__device__ __forceinline__ Words4 ld16(const void* p) {
  nu32x4 v;
  if constexpr (GLU_NV_NT_LOADS) v = __builtin_nontemporal_load(reinterpret_cast<const nu32x4*>(p));
  else v = *reinterpret_cast<const nu32x4*>(p);
  return Words4{{v.x, v.y, v.z, v.w}};
}
__device__ __forceinline__ void st4(uint8_t* p, uint32_t w) {
  if constexpr (GLU_NV_NT_STORES) __builtin_nontemporal_store(w, reinterpret_cast<uint32_t*>(p));
  else *reinterpret_cast<uint32_t*>(p) = w;
}

// Raw operand words of a lane's 8 outputs: interleaved (gate, up) pairs, gate and up
// vectors, or FP32 values.
struct Raw8 {
  Words4 A, B;
};

template <int LAYOUT, bool F32>
__device__ __forceinline__ Raw8 load_raw(const NvArgs& a, int64_t row, int64_t j) {
  if constexpr (F32) {
    const float* p = static_cast<const float*>(a.src) + row * a.ld_in + j;
    return Raw8{ld16(p), ld16(p + 4)};
  } else if constexpr (LAYOUT == PAIRED) {
    const uint16_t* p = static_cast<const uint16_t*>(a.src) + row * a.ld_in + 2 * j;
    return Raw8{ld16(p), ld16(p + 8)};
  } else {
    return Raw8{ld16(static_cast<const uint16_t*>(a.src) + row * a.ld_in + j),
                ld16(a.up + row * a.ld_in + j)};
  }
}

// The lane's 8 values to quantize: the FP32 inputs, or the GLU outputs rounded to BF16.
template <int ACT, int LAYOUT, bool F32>
__device__ __forceinline__ void values(const Raw8& r, float v[8]) {
  if constexpr (F32) {
#pragma unroll
    for (int k = 0; k < 4; k++) {
      v[k] = __uint_as_float(r.A.w[k]);
      v[4 + k] = __uint_as_float(r.B.w[k]);
    }
  } else {
    float g[8], u[8];
    if constexpr (LAYOUT == PAIRED) {
#pragma unroll
      for (int k = 0; k < 4; k++) {
        g[k] = bf_lo(r.A.w[k]);
        u[k] = bf_hi(r.A.w[k]);
        g[4 + k] = bf_lo(r.B.w[k]);
        u[4 + k] = bf_hi(r.B.w[k]);
      }
    } else {
#pragma unroll
      for (int k = 0; k < 4; k++) {
        g[2 * k] = bf_lo(r.A.w[k]);
        g[2 * k + 1] = bf_hi(r.A.w[k]);
        u[2 * k] = bf_lo(r.B.w[k]);
        u[2 * k + 1] = bf_hi(r.B.w[k]);
      }
    }
    bool tail = false;
#pragma unroll
    for (int k = 0; k < 8; k++) v[k] = glu_fwd_elem<ACT>(g[k], u[k], tail);
    if (tail) {
#pragma unroll
      for (int k = 0; k < 8; k++)
        if (fwd_tail_needed<ACT>(g[k], u[k])) v[k] = glu_fwd_tail<ACT>(g[k], u[k]);
    }
#pragma unroll
    for (int k = 0; k < 4; k++) {
      const uint32_t p = pack_bf16(v[2 * k], v[2 * k + 1]);
      v[2 * k] = bf_lo(p);
      v[2 * k + 1] = bf_hi(p);
    }
  }
}

// A workgroup covers NV_GROUPS * 2048 consecutive outputs of one row: lane l takes 8 outputs
// at l * 8 + g * 2048 for each group g, and issues the loads of all its groups first.
template <int ACT, int LAYOUT, int SFL, bool F32>
__global__ __launch_bounds__(NV_THREADS) void k_nvfp4(NvArgs a, int64_t tiles_per_row,
                                                      int64_t ntiles, int64_t scale_cols,
                                                      int64_t scale_cols_padded) {
  const int lane = threadIdx.x & 63;
  for (int64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
    const int64_t row = t / tiles_per_row;
    const int64_t j0 = (t - row * tiles_per_row) * (NV_TILE * NV_GROUPS) + (int64_t)threadIdx.x * 8;
    Raw8 raw[NV_GROUPS];
#pragma unroll
    for (int gi = 0; gi < NV_GROUPS; gi++) {
      const int64_t j = j0 + gi * NV_TILE;
      if (j < a.H && row < a.M) raw[gi] = load_raw<LAYOUT, F32>(a, row, j);
    }
#pragma unroll
    for (int gi = 0; gi < NV_GROUPS; gi++) {
      const int64_t j = j0 + gi * NV_TILE;
      const bool in_row = j < a.H;  // pairs of lanes agree (H % 16 == 0)
      const bool live = in_row && row < a.M;
      float v[8];
      if (live) {
        values<ACT, LAYOUT, F32>(raw[gi], v);
      } else {
#pragma unroll
        for (int k = 0; k < 8; k++) v[k] = 0.0f;
      }

      // block amax over the lane pair (all lanes take part in the exchange)
      uint32_t m = __float_as_uint(v[0]) & 0x7fffffffu;
#pragma unroll
      for (int k = 1; k < 8; k++) m = umax(m, __float_as_uint(v[k]) & 0x7fffffffu);
      m = umax(m, dpp<DPP_XOR1>(m));

      const bool nonfinite = m >= 0x7f800000u;
      const uint32_t sc = nonfinite ? 0x7fu : nv_scale_code(__uint_as_float(m));

      if (live) {
        uint32_t word = 0;
        const float S = e4m3_value(nonfinite ? 0u : sc);
        if constexpr (F32) {
          // any FP32 value: exact threshold comparisons
          const E2m1Thresholds T = e2m1_thresholds(S);
#pragma unroll
          for (int k = 0; k < 8; k++) word |= e2m1_code(v[k], T) << (4 * k);
        } else {
          // BF16 values: scaled operand + hardware convert
          const float R = S > 0.0f ? __builtin_amdgcn_rcpf(S) : 0.0f;
          word = fp4x2<0>(word, e2m1_operand(v[0], R), e2m1_operand(v[1], R));
          word = fp4x2<1>(word, e2m1_operand(v[2], R), e2m1_operand(v[3], R));
          word = fp4x2<2>(word, e2m1_operand(v[4], R), e2m1_operand(v[5], R));
          word = fp4x2<3>(word, e2m1_operand(v[6], R), e2m1_operand(v[7], R));
        }
        if (nonfinite) word = 0;
        st4(a.q + row * (a.H / 2) + j / 2, word);
      }
      if (in_row && (lane & 1) == 0) {
        const int64_t blk = j / 16;
        const uint8_t byte = row < a.M ? (uint8_t)sc : (uint8_t)0;  // padding rows hold 0
        if constexpr (SFL == SF_ROWMAJOR) {
          a.sf[row * scale_cols + blk] = byte;
        } else {
          a.sf[sf128x4_offset(row, blk, scale_cols_padded)] = byte;
          if (blk == scale_cols - 1)
            for (int64_t c = scale_cols; c < scale_cols_padded; c++)
              a.sf[sf128x4_offset(row, c, scale_cols_padded)] = 0;
        }
      }
    }
  }
}

template <int ACT, int LAYOUT, bool F32>
hipError_t launch(const NvArgs& a, hipStream_t s) {
  const int64_t nb = a.H / 16;
  const int64_t cp = (nb + 3) / 4 * 4;
  const int64_t rows = a.sf_layout == SF_128x4 ? (a.M + 127) / 128 * 128 : a.M;
  const int64_t tpr = (a.H + NV_TILE * NV_GROUPS - 1) / (NV_TILE * NV_GROUPS);
  const int64_t ntiles = rows * tpr;
  const dim3 grid(grid_for(ntiles, (int64_t)1 << 20)), block(NV_THREADS);
  if (a.sf_layout == SF_128x4)
    return launch_kernel(k_nvfp4<ACT, LAYOUT, SF_128x4, F32>, grid, block, s, a, tpr, ntiles, nb, cp);
  return launch_kernel(k_nvfp4<ACT, LAYOUT, SF_ROWMAJOR, F32>, grid, block, s, a, tpr, ntiles, nb, cp);
}

}  // namespace

hipError_t launch_glu_fwd_nvfp4(const NvArgs& a, hipStream_t s) {
  return with_act(a.act, [&](auto A) {
    constexpr int ACT = decltype(A)::value;
    return a.layout == PAIRED ? launch<ACT, PAIRED, false>(a, s) : launch<ACT, SPLIT, false>(a, s);
  });
}

hipError_t launch_quant_nvfp4_f32(const NvArgs& a, hipStream_t s) {
  return launch<SWIGLU, SPLIT, true>(a, s);
}

}  // namespace glu
