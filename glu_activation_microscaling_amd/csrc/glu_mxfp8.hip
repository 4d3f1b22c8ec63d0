// Fused GLU + MXFP8 quantization, forward and backward, rowwise / colwise / both from one
// read of the inputs ("Add swiglu + MXFP8 fused CuTe DSL kernel", Summary and API), and
// the FP32 quantizer hook that runs the same quantize-and-store stage on given values.
//
// Work decomposition (wave64):
//   workgroup = 4 waves = a 64-row x 128-column tile; wave w covers rows 32*(w&1) and
//   columns 64*(w>>1) of it, i.e. one 32-row colwise block row and two 32-column rowwise
//   blocks per row.  Lane = lr + 8*lc owns rows 4lr..4lr+3 and columns 8lc..8lc+7 of the
//   wave tile: 16-byte loads per row and per operand, 32 elements per lane.
//   Rowwise amax of a 32-column block spans the 4 lanes lc = 4b..4b+3 (lane bits 3, 4):
//   DPP row_ror:8 then ds_swizzle xor 16.  Colwise amax of a 32-row block spans the
//   8 lanes lr = 0..7 (lane bits 0..2) after an in-lane max over 4 rows: DPP quad_perm
//   xor 1, xor 2, then row_half_mirror.  No LDS is needed: each lane already holds 4
//   consecutive rows of every column it owns, so colwise codes leave as 4-byte stores into
//   the transposed [N, M] output and rowwise codes as 8-byte stores.
//   Tiles are dealt to the 8 XCDs in contiguous runs along M (workgroups go to XCDs
//   round-robin by id), so the transposed colwise lines and their scale bytes, which
//   neighbouring tiles along M share, are assembled in one XCD's L2.
#include "glu_device.h"
#include "glu_launch.h"

namespace glu {
namespace {

constexpr int MX_THREADS = 256;
constexpr int TILE_M = 64, TILE_N = 128;
enum { MODE_FWD = 0, MODE_BWD = 1, MODE_F32 = 2 };

struct MxOut {
  uint8_t* q_row;
  uint8_t* s_row;
  uint8_t* q_col;
  uint8_t* s_col;
  int64_t M;    // rows of the quantized matrix
  int64_t ldq;  // columns of the quantized matrix (N forward, 2N backward)
};

// Quantizes the lane's 4x8 values (rows r0 + 4lr + i, columns col + c of the quantized
// matrix) and stores codes and scales.  All 64 lanes must call it together.
template <int FLAGS>
__device__ __forceinline__ void mx_quant_store(const float (&v)[4][8], const MxOut& o,
                                               int64_t r0, int64_t col, int lr, int lc,
                                               bool col_ok) {
  uint32_t ab[4][8];
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int c = 0; c < 8; c++) ab[i][c] = __float_as_uint(v[i][c]) & 0x7fffffffu;

  if constexpr ((FLAGS & ROWWISE) != 0) {
    uint32_t packed = 0;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      uint32_t m = ab[i][0];
#pragma unroll
      for (int c = 1; c < 8; c++) m = umax(m, ab[i][c]);
      m = umax(m, dpp<DPP_ROW_ROR8>(m));
      m = umax(m, swz_xor16(m));
      const bool nonfinite = m >= 0x7f800000u;
      const uint32_t b = nonfinite ? 0xffu : mx_scale_byte(m);
      const float P = mx_inv_scale(nonfinite ? 0u : b);
      packed |= b << (8 * i);
      const int64_t row = r0 + 4 * lr + i;
      if (col_ok && row < o.M) {
        uint32_t w0 = e4m3x4(v[i][0] * P, v[i][1] * P, v[i][2] * P, v[i][3] * P);
        uint32_t w1 = e4m3x4(v[i][4] * P, v[i][5] * P, v[i][6] * P, v[i][7] * P);
        if (nonfinite) w0 = w1 = 0x7f7f7f7fu;
        *reinterpret_cast<uint2*>(o.q_row + row * o.ldq + col) = make_uint2(w0, w1);
      }
    }
    // lane lc = 4b + i stores the scale of row 4lr + i in block b
    const int i = lc & 3;
    const int64_t row = r0 + 4 * lr + i;
    if (col_ok && row < o.M)
      o.s_row[row * (o.ldq / 32) + (col - 8 * i) / 32] = (uint8_t)(packed >> (8 * i));
  }

  if constexpr ((FLAGS & COLWISE) != 0) {
    uint32_t packed0 = 0, packed1 = 0;
#pragma unroll
    for (int c = 0; c < 8; c++) {
      uint32_t m = umax(umax(ab[0][c], ab[1][c]), umax(ab[2][c], ab[3][c]));
      m = umax(m, dpp<DPP_XOR1>(m));
      m = umax(m, dpp<DPP_XOR2>(m));
      m = umax(m, dpp<DPP_HALF_MIRROR>(m));
      const bool nonfinite = m >= 0x7f800000u;
      const uint32_t b = nonfinite ? 0xffu : mx_scale_byte(m);
      const float P = mx_inv_scale(nonfinite ? 0u : b);
      if (c < 4) packed0 |= b << (8 * c); else packed1 |= b << (8 * (c - 4));
      if (col_ok) {
        uint32_t w = e4m3x4(v[0][c] * P, v[1][c] * P, v[2][c] * P, v[3][c] * P);
        if (nonfinite) w = 0x7f7f7f7fu;
        *reinterpret_cast<uint32_t*>(o.q_col + (col + c) * o.M + r0 + 4 * lr) = w;
      }
    }
    // lane lr stores the scale of column 8lc + lr of this 32-row block
    if (col_ok) {
      const uint32_t w = lr < 4 ? packed0 : packed1;
      o.s_col[(col + lr) * (o.M / 32) + r0 / 32] = (uint8_t)(w >> (8 * (lr & 3)));
    }
  }
}

struct Words4 {
  uint32_t w[4];
};
__device__ __forceinline__ Words4 ld16(const void* p) {
  uint4 v = *reinterpret_cast<const uint4*>(p);
  return Words4{{v.x, v.y, v.z, v.w}};
}

// Gate and up of 8 consecutive outputs (BF16 widened exactly).
template <int LAYOUT>
__device__ __forceinline__ void load_gu(const uint16_t* gate, const uint16_t* up, int64_t ld,
                                        int64_t row, int64_t col, float g[8], float u[8]) {
  if constexpr (LAYOUT == SPLIT) {
    Words4 G = ld16(gate + row * ld + col), U = ld16(up + row * ld + col);
#pragma unroll
    for (int k = 0; k < 4; k++) {
      g[2 * k] = bf_lo(G.w[k]);
      g[2 * k + 1] = bf_hi(G.w[k]);
      u[2 * k] = bf_lo(U.w[k]);
      u[2 * k + 1] = bf_hi(U.w[k]);
    }
  } else {
    const uint16_t* p = gate + row * ld + 2 * col;
    Words4 A = ld16(p), B = ld16(p + 8);
#pragma unroll
    for (int k = 0; k < 4; k++) {
      g[k] = bf_lo(A.w[k]);
      u[k] = bf_hi(A.w[k]);
      g[4 + k] = bf_lo(B.w[k]);
      u[4 + k] = bf_hi(B.w[k]);
    }
  }
}

template <int ACT, int LAYOUT, int FLAGS, int MODE>
__global__ __launch_bounds__(MX_THREADS) void k_mxfp8(MxArgs a, int64_t tiles_m, int64_t ntiles,
                                                      int64_t per_xcd) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int lr = lane & 7, lc = lane >> 3;
  const int64_t b = blockIdx.x;
  const int64_t t = (b & 7) * per_xcd + (b >> 3);
  if (t >= ntiles) return;
  const int64_t tm = t % tiles_m, tn = t / tiles_m;
  const int64_t r0 = tm * TILE_M + 32 * (w & 1);
  const int64_t cw = tn * TILE_N + 64 * (w >> 1);
  if (r0 >= a.M || cw >= a.N) return;  // wave-uniform
  const int64_t col = cw + 8 * lc;
  const bool col_ok = col < a.N;

  if constexpr (MODE == MODE_FWD || MODE == MODE_F32) {
    float v[4][8];
    if constexpr (MODE == MODE_F32) {
      const float* x = static_cast<const float*>(a.src);
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int64_t row = r0 + 4 * lr + i;
        if (col_ok && row < a.M) {
          const float* p = x + row * a.ld_in + col;
          Words4 A = ld16(p), B = ld16(p + 4);
#pragma unroll
          for (int k = 0; k < 4; k++) {
            v[i][k] = __uint_as_float(A.w[k]);
            v[i][4 + k] = __uint_as_float(B.w[k]);
          }
        } else {
#pragma unroll
          for (int c = 0; c < 8; c++) v[i][c] = 0.0f;
        }
      }
    } else {
      const uint16_t* gate = static_cast<const uint16_t*>(a.src);
      float g[4][8], u[4][8];
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int64_t row = r0 + 4 * lr + i;
        if (col_ok && row < a.M) {
          load_gu<LAYOUT>(gate, a.up, a.ld_in, row, col, g[i], u[i]);
        } else {
#pragma unroll
          for (int c = 0; c < 8; c++) g[i][c] = u[i][c] = 0.0f;
        }
      }
      float zmin = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; i++)
#pragma unroll
        for (int c = 0; c < 8; c++) v[i][c] = glu_fwd_elem<ACT>(g[i][c], u[i][c], zmin);
      if (zmin < TAIL_ZL2) {
#pragma unroll
        for (int i = 0; i < 4; i++)
#pragma unroll
          for (int c = 0; c < 8; c++)
            if (zl2<ACT>(g[i][c]) < TAIL_ZL2) v[i][c] = glu_fwd_tail<ACT>(g[i][c], u[i][c]);
      }
#pragma unroll
      for (int i = 0; i < 4; i++)
#pragma unroll
        for (int c = 0; c < 8; c++) v[i][c] = round_bf16(v[i][c]);
    }
    const MxOut o{a.q_row, a.s_row, a.q_col, a.s_col, a.M, a.N};
    mx_quant_store<FLAGS>(v, o, r0, col, lr, lc, col_ok);
  } else {
    const uint16_t* gate = static_cast<const uint16_t*>(a.src);
    float va[4][8], vb[4][8];
    {
      float g[4][8], u[4][8], d[4][8];
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int64_t row = r0 + 4 * lr + i;
        if (col_ok && row < a.M) {
          load_gu<SPLIT>(gate, a.up, a.ld_in, row, col, g[i], u[i]);
          Words4 D = ld16(a.dh + row * a.ld_dh + col);
#pragma unroll
          for (int k = 0; k < 4; k++) {
            d[i][2 * k] = bf_lo(D.w[k]);
            d[i][2 * k + 1] = bf_hi(D.w[k]);
          }
        } else {
#pragma unroll
          for (int c = 0; c < 8; c++) g[i][c] = u[i][c] = d[i][c] = 0.0f;
        }
      }
      float zmin = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; i++)
#pragma unroll
        for (int c = 0; c < 8; c++) glu_bwd_elem<ACT>(g[i][c], u[i][c], d[i][c], va[i][c], vb[i][c], zmin);
      if (zmin < TAIL_ZL2) {
#pragma unroll
        for (int i = 0; i < 4; i++)
#pragma unroll
          for (int c = 0; c < 8; c++)
            if (zl2<ACT>(g[i][c]) < TAIL_ZL2) glu_bwd_tail<ACT>(g[i][c], u[i][c], d[i][c], va[i][c], vb[i][c]);
      }
#pragma unroll
      for (int i = 0; i < 4; i++)
#pragma unroll
        for (int c = 0; c < 8; c++) {
          va[i][c] = round_bf16(va[i][c]);
          vb[i][c] = round_bf16(vb[i][c]);
        }
    }
    const MxOut o{a.q_row, a.s_row, a.q_col, a.s_col, a.M, 2 * a.N};
    mx_quant_store<FLAGS>(va, o, r0, col, lr, lc, col_ok);
    mx_quant_store<FLAGS>(vb, o, r0, a.N + col, lr, lc, col_ok);
  }
}

template <int ACT, int LAYOUT, int FLAGS, int MODE>
hipError_t launch(const MxArgs& a, hipStream_t s) {
  const int64_t tiles_m = (a.M + TILE_M - 1) / TILE_M;
  const int64_t tiles_n = (a.N + TILE_N - 1) / TILE_N;
  const int64_t ntiles = tiles_m * tiles_n;
  const int64_t per_xcd = (ntiles + 7) / 8;
  const dim3 grid((unsigned)(8 * per_xcd)), block(MX_THREADS);
  return launch_kernel(k_mxfp8<ACT, LAYOUT, FLAGS, MODE>, grid, block, s, a, tiles_m, ntiles,
                       per_xcd);
}

template <int ACT, int LAYOUT, int MODE>
hipError_t by_flags(const MxArgs& a, hipStream_t s) {
  switch (a.flags) {
    case ROWWISE: return launch<ACT, LAYOUT, ROWWISE, MODE>(a, s);
    case COLWISE: return launch<ACT, LAYOUT, COLWISE, MODE>(a, s);
    default: return launch<ACT, LAYOUT, ROWWISE | COLWISE, MODE>(a, s);
  }
}

}  // namespace

hipError_t launch_glu_fwd_mxfp8(const MxArgs& a, hipStream_t s) {
  if (a.act == SWIGLU)
    return a.layout == SPLIT ? by_flags<SWIGLU, SPLIT, MODE_FWD>(a, s)
                             : by_flags<SWIGLU, PAIRED, MODE_FWD>(a, s);
  return a.layout == SPLIT ? by_flags<GEGLU_TANH, SPLIT, MODE_FWD>(a, s)
                           : by_flags<GEGLU_TANH, PAIRED, MODE_FWD>(a, s);
}

hipError_t launch_glu_bwd_mxfp8(const MxArgs& a, hipStream_t s) {
  return a.act == SWIGLU ? by_flags<SWIGLU, SPLIT, MODE_BWD>(a, s)
                         : by_flags<GEGLU_TANH, SPLIT, MODE_BWD>(a, s);
}

hipError_t launch_quant_mxfp8_f32(const MxArgs& a, hipStream_t s) {
  return by_flags<SWIGLU, SPLIT, MODE_F32>(a, s);
}

}  // namespace glu
