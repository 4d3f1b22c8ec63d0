// GLU forward / backward with BF16 outputs ("perf: tile wide GeGLU rows on SM103",
// Summary and Testing Done: forward, da and db; "Add swiglu + MXFP8 fused CuTe DSL
// kernel", API: [gate | up] input and [dGate | dUp] output).
//
// A purely element-wise, HBM-bound pass: each thread moves 16-byte vectors of 8 elements
// (gate, up and dh loads, h or da/db stores), computes in FP32 and rounds once to BF16.
// Contiguous operands are processed as a single flat row, so any width (8193 included)
// runs the vector path everywhere except for the last < 8 elements.
#include <type_traits>

#include "glu_device.h"
#include "glu_launch.h"

namespace glu {
namespace {

// 256 threads per workgroup.  128, 512 and 1024 moved single launches by up to 5% either way
// with no size better everywhere (same-box A/B over the twenty GeGLU launches of [1024 | 8192,
// 4096 .. 29568], cold inputs); [8192, 4096] forward 36.7 us against 36.8 - 37.5.
constexpr int BF_THREADS = 256;
template <int VEC>  // 16-byte vectors per operand per thread
constexpr int64_t bf_chunk() { return (int64_t)BF_THREADS * VEC * 8; }  // elements per tile

// Loads are non-temporal (streaming): [8192, 14336] GeGLU forward 122 vs 130 us, backward 193
// vs 206 us against ordinary loads.
// Per launch, by the bytes it writes against the 256 MiB last-level cache, and by direction
// (same-box A/B with cold inputs, GeGLU, us):
//   stores: non-temporal above 256 MiB, ordinary below (the cache absorbs them).  Above:
//     forward [8192, 18944] 149.6 vs 156.7 ordinary, [8192, 29568] 228.7 vs 239.3; backward
//     [8192, 11008] 149.7 vs 157.0, [8192, 29568] 394.1 vs 408.3.  Below, non-temporal stores
//     cost 5% (forward [8192, 14336] 114.9 vs 109.0).  The choice is a template parameter: a
//     run-time branch between the two stores of one value to one address is merged into a
//     single ordinary store, which drops the non-temporal hint.
//   16-byte vectors per operand per thread: one, except two for a backward above 512 MiB.
//     up to 256 MiB, one vs two:  [1024, 29568] forward 33.9 vs 38.5, backward 50.4 vs 55.7;
//                                 [8192, 4096] 36.9 vs 40.1 and 57.1 vs 60.2;
//                                 [8192, 14336] forward 107.9 vs 118.3;
//     above, one vs two:          forward [8192, 18944] 149.0 vs 152.6, [8192, 29568] 231.6
//                                 vs 233.2; backward [8192, 11008] (361 MB) 146.9 vs 149.7,
//                                 [8192, 14336] 194.3 vs 194.8, [8192, 18944] (621 MB) 256.8
//                                 vs 253.2, [8192, 29568] 400.5 vs 396.1.
constexpr int64_t kBf16NtStoreBytes = 256ll << 20;
constexpr int64_t kBf16TwoVecBwdBytes = 512ll << 20;

typedef unsigned int bu32x4 __attribute__((ext_vector_type(4)));

struct Uint4 {
  uint32_t w[4];
};

__device__ __forceinline__ Uint4 ld16(const uint16_t* p) {
  bu32x4 v;
  v = __builtin_nontemporal_load(reinterpret_cast<const bu32x4*>(p));
  return Uint4{{v.x, v.y, v.z, v.w}};
}
template <bool NT>
__device__ __forceinline__ void st16(uint16_t* p, uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  const bu32x4 v = {a, b, c, d};
  if constexpr (NT) __builtin_nontemporal_store(v, reinterpret_cast<bu32x4*>(p));
  else *reinterpret_cast<bu32x4*>(p) = v;
}
__device__ __forceinline__ float ld_bf(const uint16_t* p) {
  return __uint_as_float((uint32_t)*p << 16);
}

// Eight (gate, up) pairs starting at output column j of a row; `in` points at the row.
template <int LAYOUT>
__device__ __forceinline__ void load8(const uint16_t* gate_row, const uint16_t* up_row,
                                      int64_t j, float g[8], float u[8]) {
  if constexpr (LAYOUT == SPLIT) {
    Uint4 G = ld16(gate_row + j), U = ld16(up_row + j);
#pragma unroll
    for (int k = 0; k < 4; k++) {
      g[2 * k] = bf_lo(G.w[k]);
      g[2 * k + 1] = bf_hi(G.w[k]);
      u[2 * k] = bf_lo(U.w[k]);
      u[2 * k + 1] = bf_hi(U.w[k]);
    }
  } else {
    Uint4 A = ld16(gate_row + 2 * j), B = ld16(gate_row + 2 * j + 8);
#pragma unroll
    for (int k = 0; k < 4; k++) {
      g[k] = bf_lo(A.w[k]);
      u[k] = bf_hi(A.w[k]);
      g[4 + k] = bf_lo(B.w[k]);
      u[4 + k] = bf_hi(B.w[k]);
    }
  }
}

template <int LAYOUT>
__device__ __forceinline__ void load1(const uint16_t* gate_row, const uint16_t* up_row,
                                      int64_t j, float& g, float& u) {
  if constexpr (LAYOUT == SPLIT) {
    g = ld_bf(gate_row + j);
    u = ld_bf(up_row + j);
  } else {
    g = ld_bf(gate_row + 2 * j);
    u = ld_bf(gate_row + 2 * j + 1);
  }
}

template <int ACT, int LAYOUT, int BF_VEC, bool NT>
__global__ __launch_bounds__(BF_THREADS) void k_glu_fwd_bf16(BF16Args a, int64_t cols,
                                                             int64_t tiles_per_row, int64_t rows) {
  for (int64_t row = blockIdx.y; row < rows; row += gridDim.y)
  for (int64_t tc = blockIdx.x; tc < tiles_per_row; tc += gridDim.x) {
    const int64_t j0 = tc * bf_chunk<BF_VEC>();
    const uint16_t* grow = a.gate + row * a.ld_in;
    const uint16_t* urow = (LAYOUT == SPLIT) ? a.up + row * a.ld_in : nullptr;
    uint16_t* hrow = a.out0 + row * a.ld_out;

    float g[BF_VEC][8], u[BF_VEC][8];
#pragma unroll
    for (int v = 0; v < BF_VEC; v++) {
      const int64_t j = j0 + ((int64_t)v * BF_THREADS + threadIdx.x) * 8;
      if (j + 8 <= cols) load8<LAYOUT>(grow, urow, j, g[v], u[v]);
    }
#pragma unroll
    for (int v = 0; v < BF_VEC; v++) {
      const int64_t j = j0 + ((int64_t)v * BF_THREADS + threadIdx.x) * 8;
      if (j + 8 <= cols) {
        float h[8];
        bool tail = false;
#pragma unroll
        for (int k = 0; k < 8; k++) h[k] = glu_fwd_elem<ACT>(g[v][k], u[v][k], tail);
        if (tail) {
#pragma unroll
          for (int k = 0; k < 8; k++)
            if (fwd_tail_needed<ACT>(g[v][k], u[v][k])) h[k] = glu_fwd_tail<ACT>(g[v][k], u[v][k]);
        }
        st16<NT>(hrow + j, pack_bf16(h[0], h[1]), pack_bf16(h[2], h[3]), pack_bf16(h[4], h[5]),
             pack_bf16(h[6], h[7]));
      } else if (j < cols) {
        for (int64_t jj = j; jj < cols; jj++) {
          float gg, uu;
          bool tail = false;
          load1<LAYOUT>(grow, urow, jj, gg, uu);
          float h = glu_fwd_elem<ACT>(gg, uu, tail);
          if (tail) h = glu_fwd_tail<ACT>(gg, uu);
          hrow[jj] = (uint16_t)bf16_rne(h);
        }
      }
    }
  }
}

template <int ACT, int LAYOUT, int BF_VEC, bool NT>
__global__ __launch_bounds__(BF_THREADS) void k_glu_bwd_bf16(BF16Args a, int64_t cols,
                                                             int64_t tiles_per_row, int64_t rows) {
  for (int64_t row = blockIdx.y; row < rows; row += gridDim.y)
  for (int64_t tc = blockIdx.x; tc < tiles_per_row; tc += gridDim.x) {
    const int64_t j0 = tc * bf_chunk<BF_VEC>();
    const uint16_t* grow = a.gate + row * a.ld_in;
    const uint16_t* urow = (LAYOUT == SPLIT) ? a.up + row * a.ld_in : nullptr;
    const uint16_t* drow = a.dh + row * a.ld_dh;
    uint16_t* arow = a.out0 + row * a.ld_out;
    uint16_t* brow = (LAYOUT == SPLIT) ? a.out1 + row * a.ld_out : nullptr;

    float g[BF_VEC][8], u[BF_VEC][8], d[BF_VEC][8];
#pragma unroll
    for (int v = 0; v < BF_VEC; v++) {
      const int64_t j = j0 + ((int64_t)v * BF_THREADS + threadIdx.x) * 8;
      if (j + 8 <= cols) {
        load8<LAYOUT>(grow, urow, j, g[v], u[v]);
        Uint4 D = ld16(drow + j);
#pragma unroll
        for (int k = 0; k < 4; k++) {
          d[v][2 * k] = bf_lo(D.w[k]);
          d[v][2 * k + 1] = bf_hi(D.w[k]);
        }
      }
    }
#pragma unroll
    for (int v = 0; v < BF_VEC; v++) {
      const int64_t j = j0 + ((int64_t)v * BF_THREADS + threadIdx.x) * 8;
      if (j + 8 <= cols) {
        float da[8], db[8];
        bool tail = false;
#pragma unroll
        for (int k = 0; k < 8; k++) glu_bwd_elem<ACT>(g[v][k], u[v][k], d[v][k], da[k], db[k], tail);
        if (tail) {
#pragma unroll
          for (int k = 0; k < 8; k++)
            if (bwd_tail_needed<ACT>(g[v][k], u[v][k], d[v][k]))
              glu_bwd_tail<ACT>(g[v][k], u[v][k], d[v][k], da[k], db[k]);
        }
        if constexpr (LAYOUT == SPLIT) {
          st16<NT>(arow + j, pack_bf16(da[0], da[1]), pack_bf16(da[2], da[3]), pack_bf16(da[4], da[5]),
               pack_bf16(da[6], da[7]));
          st16<NT>(brow + j, pack_bf16(db[0], db[1]), pack_bf16(db[2], db[3]), pack_bf16(db[4], db[5]),
               pack_bf16(db[6], db[7]));
        } else {
          st16<NT>(arow + 2 * j, pack_bf16(da[0], db[0]), pack_bf16(da[1], db[1]), pack_bf16(da[2], db[2]),
               pack_bf16(da[3], db[3]));
          st16<NT>(arow + 2 * j + 8, pack_bf16(da[4], db[4]), pack_bf16(da[5], db[5]),
               pack_bf16(da[6], db[6]), pack_bf16(da[7], db[7]));
        }
      } else if (j < cols) {
        for (int64_t jj = j; jj < cols; jj++) {
          float gg, uu, da, db;
          bool tail = false;
          load1<LAYOUT>(grow, urow, jj, gg, uu);
          float dd = ld_bf(drow + jj);
          glu_bwd_elem<ACT>(gg, uu, dd, da, db, tail);
          if (tail) glu_bwd_tail<ACT>(gg, uu, dd, da, db);
          if constexpr (LAYOUT == SPLIT) {
            arow[jj] = (uint16_t)bf16_rne(da);
            brow[jj] = (uint16_t)bf16_rne(db);
          } else {
            arow[2 * jj] = (uint16_t)bf16_rne(da);
            arow[2 * jj + 1] = (uint16_t)bf16_rne(db);
          }
        }
      }
    }
  }
}

template <bool BWD, int ACT, int LAYOUT>
hipError_t launch(const BF16Args& a, hipStream_t s) {
  const int64_t rows = a.flat ? 1 : a.M;
  const int64_t cols = a.flat ? a.M * a.N : a.N;
  const int64_t written = (BWD ? 2 : 1) * 2 * a.M * a.N;
  auto go = [&](auto V, auto NTC) {
    constexpr int VEC = decltype(V)::value;
    constexpr bool NT = decltype(NTC)::value;
    const int64_t tpr = (cols + bf_chunk<VEC>() - 1) / bf_chunk<VEC>();
    const dim3 grid = grid_2d(tpr, rows), block(BF_THREADS);
    if constexpr (BWD)
      return launch_kernel(k_glu_bwd_bf16<ACT, LAYOUT, VEC, NT>, grid, block, s, a, cols, tpr, rows);
    else
      return launch_kernel(k_glu_fwd_bf16<ACT, LAYOUT, VEC, NT>, grid, block, s, a, cols, tpr, rows);
  };
  if (written <= kBf16NtStoreBytes) return go(std::integral_constant<int, 1>{}, std::false_type{});
  if constexpr (BWD)
    if (written > kBf16TwoVecBwdBytes) return go(std::integral_constant<int, 2>{}, std::true_type{});
  return go(std::integral_constant<int, 1>{}, std::true_type{});
}

template <bool BWD>
hipError_t dispatch(const BF16Args& a, hipStream_t s) {
  return with_act(a.act, [&](auto A) {
    constexpr int ACT = decltype(A)::value;
    return a.layout == SPLIT ? launch<BWD, ACT, SPLIT>(a, s) : launch<BWD, ACT, PAIRED>(a, s);
  });
}

}  // namespace

hipError_t launch_glu_fwd_bf16(const BF16Args& a, hipStream_t s) { return dispatch<false>(a, s); }
hipError_t launch_glu_bwd_bf16(const BF16Args& a, hipStream_t s) { return dispatch<true>(a, s); }

}  // namespace glu
