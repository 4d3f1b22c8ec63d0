// Internal interface between the C-ABI layer (api.cpp) and the kernel translation units.
// Arguments arrive here already validated; launchers only pick a template instance and
// a grid, and return the HIP launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>
#include <type_traits>

#include "glu_common.h"

namespace glu {

struct BF16Args {
  int act, layout;
  int64_t M, N;
  const uint16_t* gate;
  const uint16_t* up;
  int64_t ld_in;
  const uint16_t* dh;  // backward only
  int64_t ld_dh;
  uint16_t* out0;      // h (forward) or da (backward)
  uint16_t* out1;      // db (backward, split layout)
  int64_t ld_out;
  bool flat;           // operands contiguous: treat as one row of M*N elements
};

struct MxArgs {
  int act, layout, flags;
  int64_t M, N;              // per-half shape; the quantized matrix is [M, N] (fwd) or [M, 2N] (bwd)
  const void* src;           // gate (BF16) or x (FP32, quantizer hook)
  const uint16_t* up;
  int64_t ld_in;
  const uint16_t* dh;
  int64_t ld_dh;
  uint8_t* q_row;
  uint8_t* s_row;
  uint8_t* q_col;
  uint8_t* s_col;
};

struct NvArgs {
  int act, layout, sf_layout;
  int64_t M, H;              // operand shape; the quantized matrix is [M, H] (fwd) or [M, 2H] (bwd)
  const void* src;           // gate (BF16) or x (FP32, quantizer hook)
  const uint16_t* up;
  int64_t ld_in;
  uint8_t* q;
  uint8_t* sf;
  const uint16_t* dh;        // backward only
  int64_t ld_dh;
  const float* amax;         // two-level forward: the tensor amax (device memory)
  float* amax_out;           // amax pass: where it goes (device memory)
};

struct GemmArgs {
  int act;
  int fmt;                   // FMT_E4M3 (a code per byte) or FMT_E2M1 (two codes per byte)
  int w_layout;              // SPLIT: W = [W_gate | W_up]; PAIRED: rows gate0, up0, gate1, ...
  int64_t M, N, K;           // X [M, K], W [2N, K] elements; the output has N columns
  const uint8_t* xq;         // codes [M, K] (E2M1: [M, K/2] bytes)
  const uint8_t* xs;         // E8M0 scales [M, K/32]
  const uint8_t* wq;         // codes [2N, K] (E2M1: [2N, K/2] bytes), rows in w_layout
  const uint8_t* ws;         // scales [2N, K/32], rows in w_layout
  uint16_t* h;               // BF16 h [M, N], row stride ld_h
  int64_t ld_h;
  uint8_t* q_row;            // MXFP8 rowwise codes [M, N] (NVFP4: packed E2M1 [M, N/2])
  uint8_t* s_row;            // scales [M, N/32] (NVFP4: E4M3, row-major or 128x4)
  float* y;                  // test hook: the pre-activation [M, 2N] = [Y_gate | Y_up]
  const float* amax = nullptr;  // two-level NVFP4: the amax the global scale comes from
};

struct StreamArgs {          // streaming probe (validated: 1..3 sources, 1..4 destinations)
  int n_src, n_dst, dst_bytes;  // dst_bytes: 4, 8 or 16 per source vector
  int64_t n_vec;                // 16-byte vectors per source
  const void* src[3];
  void* dst[4];
};

hipError_t launch_glu_fwd_bf16(const BF16Args& a, hipStream_t s);
hipError_t launch_glu_bwd_bf16(const BF16Args& a, hipStream_t s);
hipError_t launch_glu_fwd_mxfp8(const MxArgs& a, hipStream_t s);
hipError_t launch_glu_bwd_mxfp8(const MxArgs& a, hipStream_t s);
hipError_t launch_quant_mxfp8_f32(const MxArgs& a, hipStream_t s);
hipError_t launch_glu_fwd_nvfp4(const NvArgs& a, hipStream_t s);
hipError_t launch_glu_bwd_nvfp4(const NvArgs& a, hipStream_t s);
hipError_t launch_glu_fwd_nvfp4_gs(const NvArgs& a, hipStream_t s);
hipError_t launch_glu_amax(const NvArgs& a, hipStream_t s);
hipError_t launch_glu_gemm(const GemmArgs& a, hipStream_t s);
hipError_t launch_glu_gemm_mxfp8(const GemmArgs& a, hipStream_t s);
hipError_t launch_mx_gemm_f32(const GemmArgs& a, hipStream_t s);
// NVFP4 epilogue: codes into q_row ([M, N/2] packed E2M1), E4M3 scales into s_row
hipError_t launch_glu_gemm_nvfp4(const GemmArgs& a, int sf_layout, bool two_level, hipStream_t s);
hipError_t launch_quant_nvfp4_f32(const NvArgs& a, hipStream_t s);
hipError_t launch_stream_probe(const StreamArgs& a, hipStream_t s);

// Launches kernel k and returns the launch status of this call alone (the HIP error
// state left by earlier, unrelated calls is not consulted).
template <typename... KArgs, typename... Ts>
hipError_t launch_kernel_shm(void (*k)(KArgs...), dim3 grid, dim3 block, size_t shm,
                             hipStream_t s, Ts&&... ts) {
  std::tuple<KArgs...> args(static_cast<KArgs>(ts)...);
  return std::apply(
      [&](auto&... xs) {
        void* argv[] = {(void*)&xs...};
        return hipLaunchKernel((const void*)k, grid, block, argv, shm, s);
      },
      args);
}

template <typename... KArgs, typename... Ts>
hipError_t launch_kernel(void (*k)(KArgs...), dim3 grid, dim3 block, hipStream_t s,
                         Ts&&... ts) {
  return launch_kernel_shm(k, grid, block, 0, s, static_cast<Ts&&>(ts)...);
}

// Calls f(std::integral_constant<int, ACT>) for the run-time activation code (validated by
// the caller), so a launcher names each template instance once for every activation.
template <typename F>
hipError_t with_act(int act, F&& f) {
  switch (act) {
    case SWIGLU: return f(std::integral_constant<int, SWIGLU>{});
    case GEGLU_TANH: return f(std::integral_constant<int, GEGLU_TANH>{});
    case GEGLU_ERF: return f(std::integral_constant<int, GEGLU_ERF>{});
    default: return f(std::integral_constant<int, RELU2>{});
  }
}

// Workgroups of a grid-stride launch over `units` work items: enough waves to fill the
// chip several times over, never more than the work.
inline unsigned grid_for(int64_t units, int64_t cap) {
  if (units < 1) return 1;
  return (unsigned)(units < cap ? units : cap);
}

// Grid of a launch over `rows` rows of `tiles_per_row` tiles each: x walks the tiles of a row,
// y the rows, each dimension with a grid-stride loop past its cap, so kernels find their tile
// without dividing.  At most `cap` workgroups in all (x first).
inline dim3 grid_2d(int64_t tiles_per_row, int64_t rows, int64_t cap = (int64_t)1 << 26) {
  int64_t x = tiles_per_row < 1 ? 1 : (tiles_per_row < ((int64_t)1 << 20) ? tiles_per_row : (int64_t)1 << 20);
  if (x > cap) x = cap;
  int64_t y = rows < 1 ? 1 : (rows < 65535 ? rows : 65535);
  if (x * y > cap) y = cap / x;
  return dim3((unsigned)x, (unsigned)y);
}

}  // namespace glu
