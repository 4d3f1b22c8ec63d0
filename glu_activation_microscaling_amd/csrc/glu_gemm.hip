// Merged gate/up MXFP8 GEMM with the GLU as its epilogue (and optionally the MXFP8 rowwise
// quantizer after it): "feat(phyai-kernel): add Thor NVFP4 GeGLU kernel for pi0.5" (Summary:
// the GeGLU fold follows the merged gate/up GEMM), in the MXFP8 form of "Add swiglu + MXFP8
// fused CuTe DSL kernel" (Performance: the fused-w13 MoE composite under an MXFP8 recipe;
// API: a fused w13 projection packs [gate | up]).  The pre-activation never reaches memory.
//
//   Y = X W^T, X [M, K] E4M3 with E8M0 scales [M, K/32], W = [W_gate | W_up] [2N, K] with
//   scales [2N, K/32] (blocks of 32 along K, K contiguous); h = bf16(act(Y_gate) * Y_up).
//
// Matrix cores: v_mfma_scale_f32_16x16x128_f8f6f4 (FP8 E4M3 operands, E8M0 block scales).
// Its operand layout, established on the device: lane l = 16 g + r (g = l / 16) holds row r
// of the 16-row operand and the 16-byte K chunks g and g + 4 of the 128-byte K step; its
// scale byte covers K block g (chunks 2g, 2g + 1).  The 16x16 result: lane l holds rows
// 4 g + i, i = 0..3, of column r.  The instruction does not add products as IEEE FP32
// values: the products of each aligned 8-element K chunk are summed in a 14-bit fixed-point
// window anchored at the chunk's largest product (bits below it are dropped, whatever the
// sign), and the chunk sums are added to the FP32 accumulator one at a time with FP32
// rounding.
//
// Work decomposition: a workgroup of 4 waves owns 128 rows x 128 output columns, i.e. 128 gate
// and 128 up rows of W; each wave a 64 x 64 quarter, holding the gate and up accumulators of
// the same (row, column) positions (4 x 4 tiles of 16 x 16 each, in the accumulation
// registers), so the GLU is applied in registers.  Operands are read straight into the
// matrix-core layout with 16-byte raw buffer loads (rows past M read zeros), two K steps of
// 128 in flight: one step's loads are issued before the previous step's products.
#include "glu_device.h"
#include "glu_launch.h"

namespace glu {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int GM_THREADS = 256;
#ifndef GLU_GEMM_WN                                   // build-time override, for measurements
#define GLU_GEMM_WN 4
#endif
constexpr int WM = 4, WN = GLU_GEMM_WN;               // 16x16 tiles per wave: rows, columns
constexpr int GM_BM = 2 * 16 * WM, GM_BN = 2 * 16 * WN, GM_BK = 128;  // workgroup tile, K step
static_assert(WN % 2 == 0, "an MXFP8 block is two 16-column tiles");

enum { GEMM_H = 0, GEMM_MXFP8 = 1, GEMM_F32 = 2 };

// One lane's 32 bytes of a 16-row operand slice at K step k0: chunks g and g + 4.
__device__ __forceinline__ v8i frag(__amdgpu_buffer_rsrc_t r, uint32_t row_off, bool ok,
                                    uint32_t k0, uint32_t g) {
  const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(r, ok ? row_off + k0 + 16u * g : kOob, 0, 0);
  const u32x4 b = __builtin_amdgcn_raw_buffer_load_b128(r, ok ? row_off + k0 + 64u + 16u * g : kOob, 0, 0);
  return (v8i){(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
}

// The lane's scale byte: block g of the K step, from the row's 4 scale bytes of the step.
__device__ __forceinline__ int scale_of(__amdgpu_buffer_rsrc_t r, uint32_t srow_off, bool ok,
                                        uint32_t kb0, uint32_t g) {
  const uint32_t w = __builtin_amdgcn_raw_buffer_load_b32(r, ok ? srow_off + kb0 : kOob, 0, 0);
  return (int)((w >> (8u * g)) & 0xffu);
}

template <int ACT, int OUT>
__global__ __launch_bounds__(GM_THREADS) void k_glu_gemm(GemmArgs a, uint32_t tiles_n) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t g = (uint32_t)lane >> 4, r = (uint32_t)lane & 15u;
  const uint32_t tm = blockIdx.x / tiles_n, tn = blockIdx.x - tm * tiles_n;
  const uint32_t row0 = tm * GM_BM + (wave >> 1) * (16 * WM);  // the wave's first row
  const uint32_t col0 = tn * GM_BN + (wave & 1) * (16 * WN);   // its first output column
  const uint32_t K = (uint32_t)a.K, KB = K / 32u, N = (uint32_t)a.N;

  const auto rx = rsrc(a.xq), rxs = rsrc(a.xs), rw = rsrc(a.wq), rws = rsrc(a.ws);
  uint32_t xo[WM], xso[WM];
  bool xok[WM];
#pragma unroll
  for (int i = 0; i < WM; i++) {
    const uint32_t row = row0 + 16u * i + r;
    xok[i] = row < (uint32_t)a.M;
    xo[i] = row * K;
    xso[i] = row * KB;
  }
  uint32_t wo[2][WN], wso[2][WN];  // [gate, up][tile]: W rows col0 + 16 j + r and N + ...
#pragma unroll
  for (int h = 0; h < 2; h++)
#pragma unroll
    for (int j = 0; j < WN; j++) {
      const uint32_t wrow = h * N + col0 + 16u * j + r;
      wo[h][j] = wrow * K;
      wso[h][j] = wrow * KB;
    }

  v4f acc[2][WM][WN];
#pragma unroll
  for (int h = 0; h < 2; h++)
#pragma unroll
    for (int i = 0; i < WM; i++)
#pragma unroll
      for (int j = 0; j < WN; j++) acc[h][i][j] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};

  // Operand fragments of one K step (the lane's part of the matrix-core layout).
  struct Step {
    v8i xa[WM], wb[2][WN];
    int xs[WM], ws[2][WN];
  };
  // Loads of the K step at k0; past K every load reads zeros (and zero scales), which add
  // nothing, so the two-step loop below needs no tail.
  auto load = [&](Step& st, uint32_t k0) {
    const bool in = k0 < K;
    const uint32_t kb0 = k0 / 32u;
#pragma unroll
    for (int i = 0; i < WM; i++) {
      st.xa[i] = frag(rx, xo[i], xok[i] && in, k0, g);
      st.xs[i] = scale_of(rxs, xso[i], xok[i] && in, kb0, g);
    }
#pragma unroll
    for (int h = 0; h < 2; h++)
#pragma unroll
      for (int j = 0; j < WN; j++) {
        st.wb[h][j] = frag(rw, wo[h][j], in, k0, g);
        st.ws[h][j] = scale_of(rws, wso[h][j], in, kb0, g);
      }
  };
  auto mma = [&](const Step& st) {
#pragma unroll
    for (int h = 0; h < 2; h++)
#pragma unroll
      for (int i = 0; i < WM; i++)
#pragma unroll
        for (int j = 0; j < WN; j++)
          acc[h][i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              st.xa[i], st.wb[h][j], acc[h][i][j], 0, 0, 0, st.xs[i], 0, st.ws[h][j]);
  };
  // Two register buffers: the loads of one K step are in flight while the other's products
  // issue.
  Step s0, s1;
  load(s0, 0);
  for (uint32_t k0 = 0; k0 < K; k0 += 2 * GM_BK) {
    load(s1, k0 + GM_BK);
    mma(s0);
    load(s0, k0 + 2 * GM_BK);
    mma(s1);
  }

  // Epilogue.  acc[h][i][j][e] is Y at row row0 + 16 i + 4 g + e, column col0 + 16 j + r of
  // the gate (h = 0) or up (h = 1) half.
  if constexpr (OUT == GEMM_F32) {
    // test hook: the pre-activation itself, [M, 2N] FP32
    const auto ry = rsrc(a.y);
#pragma unroll
    for (int h = 0; h < 2; h++)
#pragma unroll
      for (int i = 0; i < WM; i++)
#pragma unroll
        for (int j = 0; j < WN; j++)
#pragma unroll
          for (int e = 0; e < 4; e++) {
            const uint32_t row = row0 + 16u * i + 4u * g + (uint32_t)e;
            const uint32_t col = h * N + col0 + 16u * j + r;
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[h][i][j][e]), ry,
                                                  row < (uint32_t)a.M ? 4u * (row * 2u * N + col) : kOob, 0, 0);
          }
  } else {
    // h = bf16(act(gate) * up); the tail path covers gates whose activation leaves FP32
    uint32_t hb[WM][WN][4];
#pragma unroll
    for (int i = 0; i < WM; i++)
#pragma unroll
      for (int j = 0; j < WN; j++)
#pragma unroll
        for (int e = 0; e < 4; e++) {
          const float gv = acc[0][i][j][e], uv = acc[1][i][j][e];
          float hv = glu_fwd_fast<ACT>(gv, uv);
          if (fwd_tail_needed<ACT>(gv, uv)) hv = glu_fwd_tail<ACT>(gv, uv);
          hb[i][j][e] = bf16_rne(hv);
        }
    if constexpr (OUT == GEMM_H) {
      const auto rh = rsrc(a.h);
#pragma unroll
      for (int i = 0; i < WM; i++)
#pragma unroll
        for (int j = 0; j < WN; j++)
#pragma unroll
          for (int e = 0; e < 4; e++) {
            const uint32_t row = row0 + 16u * i + 4u * g + (uint32_t)e;
            const uint32_t col = col0 + 16u * j + r;
            __builtin_amdgcn_raw_buffer_store_b16((uint16_t)hb[i][j][e], rh,
                                                  row < (uint32_t)a.M ? 2u * (row * (uint32_t)a.ld_h + col) : kOob, 0, 0);
          }
    } else {
      // MXFP8 rowwise: the wave's columns of a row form WN / 2 blocks of 32 (tiles 2b and
      // 2b + 1); a row's values sit in the 16 lanes of one DPP row (columns r and 16 + r)
      const auto rq = rsrc(a.q_row), rs = rsrc(a.s_row);
      const uint32_t NB = N / 32u;
#pragma unroll
      for (int i = 0; i < WM; i++)
#pragma unroll
        for (int e = 0; e < 4; e++) {
          const uint32_t row = row0 + 16u * i + 4u * g + (uint32_t)e;
          const bool ok = row < (uint32_t)a.M;
#pragma unroll
          for (int b = 0; b < WN / 2; b++) {
            uint32_t m = umax(hb[i][2 * b][e] & 0x7fffu, hb[i][2 * b + 1][e] & 0x7fffu);
            m = umax(m, dpp<DPP_XOR1>(m));
            m = umax(m, dpp<DPP_XOR2>(m));
            m = umax(m, dpp<0x124>(m));  // row_ror:4
            m = umax(m, dpp<DPP_ROW_ROR8>(m));
            const bool nonfinite = m >= 0x7f80u;
            const uint32_t sb = nonfinite ? 0xffu : mx_scale_byte(m << 16);
            const float inv = nonfinite ? 1.0f : mx_inv_scale(sb);
#pragma unroll
            for (int t = 0; t < 2; t++) {
              const int j = 2 * b + t;
              const uint32_t code = nonfinite
                  ? 0x7fu
                  : fp8x2<false>(0u, __uint_as_float(hb[i][j][e] << 16) * inv, 0.0f) & 0xffu;
              __builtin_amdgcn_raw_buffer_store_b8((uint8_t)code, rq, ok ? row * N + col0 + 16u * j + r : kOob, 0, 0);
            }
            __builtin_amdgcn_raw_buffer_store_b8((uint8_t)sb, rs,
                                                 ok && r == 0 ? row * NB + (col0 + 32u * b) / 32u : kOob, 0, 0);
          }
        }
    }
  }
}

template <int OUT>
hipError_t launch(const GemmArgs& a, hipStream_t s) {
  const uint32_t tiles_m = (uint32_t)((a.M + GM_BM - 1) / GM_BM), tiles_n = (uint32_t)(a.N / GM_BN);
  const dim3 grid(tiles_m * tiles_n), block(GM_THREADS);
  if constexpr (OUT == GEMM_F32) {
    return launch_kernel(k_glu_gemm<SWIGLU, GEMM_F32>, grid, block, s, a, tiles_n);
  } else {
    return with_act(a.act, [&](auto A) {
      constexpr int ACT = decltype(A)::value;
      return launch_kernel(k_glu_gemm<ACT, OUT>, grid, block, s, a, tiles_n);
    });
  }
}

}  // namespace

hipError_t launch_glu_gemm(const GemmArgs& a, hipStream_t s) { return launch<GEMM_H>(a, s); }
hipError_t launch_glu_gemm_mxfp8(const GemmArgs& a, hipStream_t s) { return launch<GEMM_MXFP8>(a, s); }
hipError_t launch_mx_gemm_f32(const GemmArgs& a, hipStream_t s) { return launch<GEMM_F32>(a, s); }

}  // namespace glu
