// Fused GLU + NVFP4 quantization with global scale 1 ("feat(phyai-kernel): add Thor NVFP4
// GeGLU kernel for pi0.5", Summary: GeGLU fold and compact NVFP4 store; Supported contract:
// E2M1 values, E4M3 scales in the 128x4 layout, pairwise-interleaved gate/up columns), and
// the FP32 quantizer hook running the same quantize-and-store stage.
//
// The backward quantizes [dGate | dUp] the same way (a reading: no page defines an NVFP4
// backward; the placement is that of the MXFP8 backward, "Add swiglu + MXFP8 fused CuTe DSL
// kernel", API).
//
// Work decomposition (wave64): a workgroup is one wave and covers 512 consecutive operand
// columns of one row; each lane takes 8 consecutive columns (one 32-byte load of interleaved
// gate/up pairs, or 16 bytes each of gate and up, and of dh in the backward).  A 16-element block is a lane pair, so the block
// amax is one DPP quad_perm exchange.  Each lane stores its 8 E2M1 codes as one 4-byte word
// (a wave writes 256 contiguous bytes).  With the 128x4 layout the four scales of a lane
// octet (4 consecutive blocks) leave as one 4-byte word; the grid also covers the padding
// rows up to a multiple of 128, which get zero scales.
//
// The row is uniform in a workgroup, so every row-dependent address is formed once on the
// scalar unit as a buffer descriptor base; lanes add 32-bit offsets, and a lane outside the
// matrix passes kOob (loads return zeros, stores are dropped), so every path issues the same
// memory instructions.  The host keeps the quantized width at most 2^26 columns, so every
// lane offset stays below 2^28 bytes.
#include "glu_device.h"
#include "glu_launch.h"

namespace glu {
namespace {

// Quantizing kernels: a workgroup is one wave and a lane takes one group of 8 columns, so a
// workgroup covers 512 operand columns of one row.  That divides every multiple of 512
// exactly, where 256-thread workgroups with 2 (forward) or 4 (backward) groups per lane left
// an eighth of the lanes idle at widths of 7168 columns.  Same-box A/B, cold inputs, us:
//   forward  [16384, 7168] GeGLU 112.9 -> 97.1; [968, 16384] 17.0 -> 16.4; [784, 16384]
//            14.8 -> 14.2;
//   backward [16384, 7168] SwiGLU 155.7 -> 139.5, GeGLU 152.8 -> 141.0; [968, 16384] 24.6 ->
//            23.8 (all bit-identical).  128 threads with one group was within 2% of it, and
//            better only at [16384, 7168] forward (95.4); two groups per lane were slower.
constexpr int NV_THREADS = 64;
constexpr int64_t NV_TILE = 8 * NV_THREADS;  // operand columns per workgroup
// The amax pass keeps 256-thread workgroups with two groups per lane (its grid is capped).
constexpr int AMAX_THREADS = 256, AMAX_GROUPS = 2;
constexpr int64_t AMAX_TILE = 8 * AMAX_THREADS;  // operand columns per workgroup and group
// Workgroups of the amax pass (each folds its maximum in with one atomic): a capped grid took
// the pass from 97 to 88 us at [16384, 7168] and from 38 to 23 us at [968, 16384] against one
// workgroup per tile, where fewer same-address atomics matter more than parallelism.  With
// the next row prefetched, 512 beat 1024 (968 rows 24.7 -> 20.9 us, 784 rows 24.7 -> 18.6,
// [16384, 7168] 88.4 -> 85.5); 2048 took 40 us at 968 rows, 256 and 384 were slower than 512.
constexpr int64_t kAmaxWorkgroups = 512;

enum { NV_FWD = 0, NV_BWD = 1, NV_F32 = 2, NV_FWD_GS = 3 };


struct Words4 {
  uint32_t w[4];
};
// Non-temporal operand loads for the backward only: same-box A/B with cold inputs, SwiGLU
// backward [16384, 7168] 156.5 vs 166.2 us; GeGLU forward 122.8 vs 110.6 us there and 19.6 vs
// 19.0 us at [968, 16384] (slower).
template <bool BWD>
constexpr bool nv_nt_loads() { return BWD; }
template <bool NT>
__device__ __forceinline__ Words4 bld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, NT ? 2 : 0);
  return Words4{{x.x, x.y, x.z, x.w}};
}

// Raw operand words of a lane's 8 columns: interleaved (gate, up) pairs (A, B), gate and up
// vectors (A, B) and dh (C) in the backward, or FP32 values (A, B).
struct Raw8 {
  Words4 A, B, C;
};

// Row-dependent descriptors of one tile row.
struct RowIn {
  __amdgpu_buffer_rsrc_t a, b, d;
};

template <int LAYOUT, int MODE>
__device__ __forceinline__ RowIn row_in(const NvArgs& a, int64_t row) {
  RowIn r;
  if constexpr (MODE == NV_F32) {
    r.a = rsrc(static_cast<const float*>(a.src) + row * a.ld_in);
  } else {
    r.a = rsrc(static_cast<const uint16_t*>(a.src) + row * a.ld_in);
    if constexpr (LAYOUT == SPLIT) r.b = rsrc(a.up + row * a.ld_in);
    if constexpr (MODE == NV_BWD) r.d = rsrc(a.dh + row * a.ld_dh);
  }
  return r;
}

// Loads of column j (every lane issues them; off-matrix lanes pass kOob).
template <int LAYOUT, int MODE>
__device__ __forceinline__ Raw8 load_raw(const RowIn& r, uint32_t j, bool live) {
  Raw8 x;
  if constexpr (MODE == NV_F32 || LAYOUT == PAIRED) {  // 32 contiguous bytes per lane
    const uint32_t off = live ? 4u * j : kOob;
    x.A = bld16<nv_nt_loads<MODE == NV_BWD>()>(r.a, off);
    x.B = bld16<nv_nt_loads<MODE == NV_BWD>()>(r.a, live ? off + 16u : kOob);
  } else {
    const uint32_t off = live ? 2u * j : kOob;
    x.A = bld16<nv_nt_loads<MODE == NV_BWD>()>(r.a, off);
    x.B = bld16<nv_nt_loads<MODE == NV_BWD>()>(r.b, off);
    if constexpr (MODE == NV_BWD) x.C = bld16<nv_nt_loads<MODE == NV_BWD>()>(r.d, off);
  }
  return x;
}

// Largest raw gate bit pattern (unsigned 16-bit) of the lane's 8 gates, the argument of
// tail_possible: paired words hold (gate, up) with the gate in the low half.
template <int LAYOUT>
__device__ __forceinline__ uint32_t gate_max16(const Raw8& r) {
  if constexpr (LAYOUT == PAIRED) {
    uint32_t m = pkmax(pkmax(pkmax(r.A.w[0], r.A.w[1]), pkmax(r.A.w[2], r.A.w[3])),
                       pkmax(pkmax(r.B.w[0], r.B.w[1]), pkmax(r.B.w[2], r.B.w[3])));
    return lo16(m);
  } else {
    const uint32_t m = pkmax(pkmax(r.A.w[0], r.A.w[1]), pkmax(r.A.w[2], r.A.w[3]));
    return umax(lo16(m), hi16(m));
  }
}

// The lane's GLU results as packed BF16 pairs (4 words = 8 columns): h (forward), or da in
// p and db in q (backward).
template <int ACT, int LAYOUT, int MODE>
__device__ __forceinline__ void glu_values(const Raw8& r, uint32_t p[4], uint32_t q[4]) {
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
  if constexpr (tail_from_gate_bits<ACT>()) tail = tail_possible<ACT>(gate_max16<LAYOUT>(r));
  if constexpr (MODE == NV_BWD) {
    float d[8], da[8], db[8];
#pragma unroll
    for (int k = 0; k < 4; k++) {
      d[2 * k] = bf_lo(r.C.w[k]);
      d[2 * k + 1] = bf_hi(r.C.w[k]);
    }
#pragma unroll
    for (int k = 0; k < 8; k++) {
      glu_bwd_fast<ACT>(g[k], u[k], d[k], da[k], db[k]);
      if constexpr (!tail_from_gate_bits<ACT>()) tail |= bwd_tail_needed<ACT>(g[k], u[k], d[k]);
    }
    if (tail) {  // rare: some element may need the FP64 tail path
#pragma unroll
      for (int k = 0; k < 8; k++)
        if (bwd_tail_needed<ACT>(g[k], u[k], d[k])) glu_bwd_tail<ACT>(g[k], u[k], d[k], da[k], db[k]);
    }
#pragma unroll
    for (int k = 0; k < 4; k++) {
      p[k] = pack_bf16(da[2 * k], da[2 * k + 1]);
      q[k] = pack_bf16(db[2 * k], db[2 * k + 1]);
    }
  } else {
    float h[8];
#pragma unroll
    for (int k = 0; k < 8; k++) {
      h[k] = glu_fwd_fast<ACT>(g[k], u[k]);
      if constexpr (!tail_from_gate_bits<ACT>()) tail |= fwd_tail_needed<ACT>(g[k], u[k]);
    }
    if (tail) {  // rare: some element may need the FP64 tail path
#pragma unroll
      for (int k = 0; k < 8; k++)
        if (fwd_tail_needed<ACT>(g[k], u[k])) h[k] = glu_fwd_tail<ACT>(g[k], u[k]);
    }
#pragma unroll
    for (int k = 0; k < 4; k++) p[k] = pack_bf16(h[2 * k], h[2 * k + 1]);
  }
}

// Output geometry of the quantized matrix: codes are q_pitch bytes per row, scales
// scale_cols per row (scale_cols_padded in the 128x4 layout).
struct NvOut {
  int64_t q_pitch, scale_cols, scale_cols_padded;
};

// Scale and code descriptors of one output row.  128x4: the row's scales sit at
// base + (c / 4) * 512 + c % 4 from base = ((row / 128) * (Cp / 4)) * 512 + (row % 32) * 16 +
// ((row % 128) / 32) * 4.
template <int SFL>
__device__ __forceinline__ void row_out(const NvArgs& a, const NvOut& o, int64_t row,
                                        __amdgpu_buffer_rsrc_t& qr, __amdgpu_buffer_rsrc_t& sr) {
  qr = rsrc(a.q + row * o.q_pitch);
  if constexpr (SFL == SF_ROWMAJOR)
    sr = rsrc(a.sf + row * o.scale_cols);
  else
    sr = rsrc(a.sf + (row >> 7) * (o.scale_cols_padded >> 2) * 512 + (row & 31) * 16 +
              ((row & 127) >> 5) * 4);
}

template <int N>
__device__ __forceinline__ uint32_t row_shl(uint32_t v) {
  // lane i of a 16-lane row reads lane i + N; lanes without a source read 0
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x100 + N, 0xf, 0xf, true);
}

// Block scale, codes and stores for the lane's 8 BF16 results (packed in p) at output column
// jq.  Every lane of the wave calls it (the block amax is a lane-pair exchange, the 128x4
// scale word a lane-octet gather).  WORD_SCALES: 128x4 scales leave as 4-byte words (needs
// jq's block index to be a multiple of 4 at every lane octet, true when the column offset of
// this part is a multiple of 64).
template <int SFL, bool WORD_SCALES, bool GS = false>
__device__ __forceinline__ void quant_store_bf16(const uint32_t p[4], __amdgpu_buffer_rsrc_t qr,
                                                 __amdgpu_buffer_rsrc_t sr, uint32_t jq,
                                                 bool in_row, bool live, int lane,
                                                 uint32_t scale_cols, uint32_t scale_cols_padded,
                                                 const GlobalScale& gs = GlobalScale{}) {
  const uint32_t M = 0x7fff7fffu;
  const uint32_t m2 = pkmax(pkmax(p[0] & M, p[1] & M), pkmax(p[2] & M, p[3] & M));
  uint32_t m = umax(lo16(m2), hi16(m2));
  m = umax(m, dpp<DPP_XOR1>(m));  // BF16 magnitude bits of the block amax
  const bool nonfinite = m >= 0x7f80u;
  uint32_t word = 0, sc;
  if constexpr (GS) {
    // two-level: E4M3(fl(bamax * k)), saturating at 448; codes E2M1(fl(x * fl(s / S)))
    const float d = __builtin_fminf(__uint_as_float(m << 16) * gs.k, 448.0f);
    sc = nonfinite ? 0x7fu : (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(d, 0.0f, 0, false) & 0xffu;
    const float S = e4m3_value(nonfinite ? 0u : sc);
    const float r = S > 0.0f ? gs.s / S : 0.0f;  // IEEE division
    // |x * r| beyond 8 saturates to 6 either way; the clamp keeps the convert's input finite
    auto y = [&](float x) { return __builtin_amdgcn_fmed3f(x * r, -8.0f, 8.0f); };
    word = fp4x2<0>(word, y(bf_lo(p[0])), y(bf_hi(p[0])));
    word = fp4x2<1>(word, y(bf_lo(p[1])), y(bf_hi(p[1])));
    word = fp4x2<2>(word, y(bf_lo(p[2])), y(bf_hi(p[2])));
    word = fp4x2<3>(word, y(bf_lo(p[3])), y(bf_hi(p[3])));
  } else {
    sc = nonfinite ? 0x7fu : nv_scale_code_bf16(__uint_as_float(m << 16));
    const float S = e4m3_value(nonfinite ? 0u : sc);
    const float R = S > 0.0f ? __builtin_amdgcn_rcpf(S) : 0.0f;
    word = fp4x2_of_quotients<0>(word, bf_lo(p[0]), bf_hi(p[0]), R);
    word = fp4x2_of_quotients<1>(word, bf_lo(p[1]), bf_hi(p[1]), R);
    word = fp4x2_of_quotients<2>(word, bf_lo(p[2]), bf_hi(p[2]), R);
    word = fp4x2_of_quotients<3>(word, bf_lo(p[3]), bf_hi(p[3]), R);
  }
  if (nonfinite) word = 0;
  __builtin_amdgcn_raw_buffer_store_b32(word, qr, live ? jq / 2 : kOob, 0, 0);

  const uint32_t blk = jq / 16;
  const uint32_t byte = live ? sc : 0u;  // padding rows and columns hold 0
  if constexpr (SFL == SF_128x4 && WORD_SCALES) {
    // lane 8k + 2i holds block 4k' + i of the octet: gather the four into lane 8k
    uint32_t w = byte | (row_shl<2>(byte) << 8);
    w |= row_shl<4>(w) << 16;
    // only octets that start inside this part write (in the backward, the da part's octets
    // past column H would otherwise land on db's scales); an octet reaching past the last
    // block fills padding columns with zeros
    const bool lead = (lane & 7) == 0 && in_row;
    __builtin_amdgcn_raw_buffer_store_b32(w, sr, lead ? (blk >> 2) * 512u : kOob, 0, 0);
  } else {
    const bool even = (lane & 1) == 0 && in_row;
    if constexpr (SFL == SF_ROWMAJOR) {
      __builtin_amdgcn_raw_buffer_store_b8((uint8_t)byte, sr, even ? blk : kOob, 0, 0);
    } else {
      __builtin_amdgcn_raw_buffer_store_b8((uint8_t)byte, sr, even ? (blk >> 2) * 512u + (blk & 3) : kOob, 0, 0);
      // the lane holding the last block zero-fills the padding scale columns
      if (even && blk == scale_cols - 1)
        for (uint32_t c = scale_cols; c < scale_cols_padded; c++)
          __builtin_amdgcn_raw_buffer_store_b8((uint8_t)0, sr, (c >> 2) * 512u + (c & 3), 0, 0);
    }
  }
}

// FP32 hook: any FP32 value, exact scale decision and threshold comparisons; byte scales.
template <int SFL>
__device__ __forceinline__ void quant_store_f32(const float v[8], __amdgpu_buffer_rsrc_t qr,
                                                __amdgpu_buffer_rsrc_t sr, uint32_t jq,
                                                bool in_row, bool live, int lane,
                                                uint32_t scale_cols, uint32_t scale_cols_padded) {
  uint32_t m = __float_as_uint(v[0]) & 0x7fffffffu;
#pragma unroll
  for (int k = 1; k < 8; k++) m = umax(m, __float_as_uint(v[k]) & 0x7fffffffu);
  m = umax(m, dpp<DPP_XOR1>(m));
  const bool nonfinite = m >= 0x7f800000u;
  const uint32_t sc = nonfinite ? 0x7fu : nv_scale_code(__uint_as_float(m));
  const E2m1Thresholds T = e2m1_thresholds(e4m3_value(nonfinite ? 0u : sc));
  uint32_t word = 0;
#pragma unroll
  for (int k = 0; k < 8; k++) word |= e2m1_code(v[k], T) << (4 * k);
  if (nonfinite) word = 0;
  __builtin_amdgcn_raw_buffer_store_b32(word, qr, live ? jq / 2 : kOob, 0, 0);
  const uint32_t blk = jq / 16;
  const uint32_t byte = live ? sc : 0u;
  const bool even = (lane & 1) == 0 && in_row;
  if constexpr (SFL == SF_ROWMAJOR) {
    __builtin_amdgcn_raw_buffer_store_b8((uint8_t)byte, sr, even ? blk : kOob, 0, 0);
  } else {
    __builtin_amdgcn_raw_buffer_store_b8((uint8_t)byte, sr, even ? (blk >> 2) * 512u + (blk & 3) : kOob, 0, 0);
    if (even && blk == scale_cols - 1)
      for (uint32_t c = scale_cols; c < scale_cols_padded; c++)
        __builtin_amdgcn_raw_buffer_store_b8((uint8_t)0, sr, (c >> 2) * 512u + (c & 3), 0, 0);
  }
}

// A workgroup covers NV_TILE consecutive operand columns of one row (a.H wide): lane l takes
// the 8 columns at l * 8.  Forward: the quantized matrix is h, [M, H].  Backward: it is
// [da | db], [M, 2H]; the lane's da results go to column j, its db results to column H + j.
// WORD_SCALES as for quant_store_bf16 (the backward needs H % 64 == 0 for it).
template <int ACT, int LAYOUT, int SFL, int MODE, bool WORD_SCALES>
__global__ __launch_bounds__(NV_THREADS) void k_nvfp4(NvArgs a, int64_t tiles_per_row,
                                                      int64_t rows, NvOut o) {
  const int lane = threadIdx.x & 63;
  const uint32_t H = (uint32_t)a.H;
  const uint32_t nb = (uint32_t)o.scale_cols, cp = (uint32_t)o.scale_cols_padded;
  for (int64_t row = blockIdx.y; row < rows; row += gridDim.y)
  for (int64_t tc = blockIdx.x; tc < tiles_per_row; tc += gridDim.x) {
    const uint32_t j = (uint32_t)tc * (uint32_t)NV_TILE + threadIdx.x * 8u;
    const bool row_ok = row < a.M;
    const RowIn in = row_in<LAYOUT, MODE>(a, row_ok ? row : 0);
    const Raw8 raw = load_raw<LAYOUT, MODE>(in, j, j < H && row_ok);
    // Two-level: the amax is loaded after the operand loads are issued (the scheduling barrier
    // keeps it and the global scale's divisions below them), so its latency overlaps theirs.
    // Loaded first, it held the operand loads back by a whole memory latency.  Same-box A/B,
    // cold inputs, GeGLU, us: [968, 16384] 18.8 -> 17.3, [784, 16384] 16.4 -> 15.2,
    // [16384, 7168] 101.6 -> 95.6 (bit-identical); a scalar load of the amax, which the
    // compiler hoists with the divisions above the loop, was slower (19.3, 16.9, 104.7).
    GlobalScale gs;
    if constexpr (MODE == NV_FWD_GS) {
      __builtin_amdgcn_sched_barrier(0);
      gs = global_scale(*a.amax);
    }
    __amdgpu_buffer_rsrc_t qr, sr;
    row_out<SFL>(a, o, row, qr, sr);
    {
      const bool in_row = j < H;  // pairs (octets) of lanes agree: H % 16 == 0
      const bool live = in_row && row_ok;
      if constexpr (MODE == NV_F32) {
        float v[8];
#pragma unroll
        for (int k = 0; k < 4; k++) {
          v[k] = __uint_as_float(raw.A.w[k]);
          v[4 + k] = __uint_as_float(raw.B.w[k]);
        }
        quant_store_f32<SFL>(v, qr, sr, j, in_row, live, lane, nb, cp);
      } else if constexpr (MODE == NV_FWD_GS) {
        uint32_t p[4] = {0u, 0u, 0u, 0u}, q[4];
        if (row_ok) glu_values<ACT, LAYOUT, NV_FWD>(raw, p, q);
        quant_store_bf16<SFL, WORD_SCALES, true>(p, qr, sr, j, in_row, live, lane, nb, cp, gs);
      } else {
        // rows past M (the 128x4 layout's padding rows) only store zero scales: the
        // activation is skipped there (row_ok is uniform in the workgroup)
        uint32_t p[4] = {0u, 0u, 0u, 0u}, q[4] = {0u, 0u, 0u, 0u};
        if (row_ok) glu_values<ACT, LAYOUT, MODE>(raw, p, q);
        // backward: with H % 64 != 0 the last da octet would reach into db's blocks
        quant_store_bf16<SFL, WORD_SCALES>(p, qr, sr, j, in_row, live, lane, nb, cp);
        if constexpr (MODE == NV_BWD)
          quant_store_bf16<SFL, WORD_SCALES>(q, qr, sr, H + j, in_row, live, lane, nb, cp);
      }
    }
  }
}

template <int ACT, int LAYOUT, int MODE>
hipError_t launch(const NvArgs& a, hipStream_t s) {
  const int64_t width = MODE == NV_BWD ? 2 * a.H : a.H;  // of the quantized matrix
  const int64_t nb = width / 16;
  const NvOut o{width / 2, nb, (nb + 3) / 4 * 4};
  const int64_t rows = a.sf_layout == SF_128x4 ? (a.M + 127) / 128 * 128 : a.M;
  const int64_t tpr = (a.H + NV_TILE - 1) / NV_TILE;
  const dim3 grid = grid_2d(tpr, rows), block(NV_THREADS);
  const bool word = MODE != NV_BWD || a.H % 64 == 0;  // db's blocks start on a 4-block boundary
  if (a.sf_layout == SF_128x4) {
    if (word) return launch_kernel(k_nvfp4<ACT, LAYOUT, SF_128x4, MODE, true>, grid, block, s, a, tpr, rows, o);
    return launch_kernel(k_nvfp4<ACT, LAYOUT, SF_128x4, MODE, false>, grid, block, s, a, tpr, rows, o);
  }
  return launch_kernel(k_nvfp4<ACT, LAYOUT, SF_ROWMAJOR, MODE, true>, grid, block, s, a, tpr, rows, o);
}

// Amax pass of two-level NVFP4: the largest |h| over the matrix, h = bf16(act(gate) * up)
// (NaN if some h is NaN), as FP32 bits in *a.amax_out.  A capped grid of 256-thread
// workgroups (2 groups of 8 columns per lane) covers the operand: each takes a column tile
// and walks its rows in a grid stride with the next row's loads in flight, keeping a running
// maximum of BF16 magnitude bits (NaN patterns order above Inf), reduces it over the
// workgroup, and folds it into the output with at most one unsigned atomic max per workgroup; k_zero_u32 clears the output first (on
// the same stream).  Non-negative FP32 values order like their bit patterns.
__global__ void k_zero_u32(uint32_t* p) {
  if (threadIdx.x == 0 && blockIdx.x == 0) *p = 0u;
}

template <int ACT, int LAYOUT>
__global__ __launch_bounds__(AMAX_THREADS) void k_glu_amax(NvArgs a, int64_t tiles_per_row) {
  constexpr int G = AMAX_GROUPS;
  const uint32_t H = (uint32_t)a.H;
  uint32_t m = 0;
  for (int64_t tc = blockIdx.x; tc < tiles_per_row; tc += gridDim.x) {
    const uint32_t j0 = (uint32_t)tc * (uint32_t)(AMAX_TILE * G) + threadIdx.x * 8u;
    // lanes past the row, and rows past M, read zeros (every activation gives h = 0 for them)
    auto load_row = [&](int64_t row, Raw8 (&raw)[G]) {
      const bool ok = row < a.M;
      const RowIn in = row_in<LAYOUT, NV_FWD>(a, ok ? row : 0);
#pragma unroll
      for (int gi = 0; gi < G; gi++) {
        const uint32_t j = j0 + gi * (uint32_t)AMAX_TILE;
        raw[gi] = load_raw<LAYOUT, NV_FWD>(in, j, j < H && ok);
      }
    };
    // the workgroup walks its rows with the next row's operands already in flight
    Raw8 cur[G];
    load_row(blockIdx.y, cur);
    for (int64_t row = blockIdx.y; row < a.M; row += gridDim.y) {
      Raw8 nxt[G];
      load_row(row + gridDim.y, nxt);
#pragma unroll
      for (int gi = 0; gi < G; gi++) {
        uint32_t p[4], q[4];
        glu_values<ACT, LAYOUT, NV_FWD>(cur[gi], p, q);
        const uint32_t M = 0x7fff7fffu;
        const uint32_t m2 = pkmax(pkmax(p[0] & M, p[1] & M), pkmax(p[2] & M, p[3] & M));
        m = umax(m, umax(lo16(m2), hi16(m2)));
      }
#pragma unroll
      for (int gi = 0; gi < G; gi++) cur[gi] = nxt[gi];
    }
  }
#pragma unroll
  for (int k = 32; k >= 1; k >>= 1) m = umax(m, (uint32_t)__shfl_xor((int)m, k));
  __shared__ uint32_t wave_max[AMAX_THREADS / 64];
  if ((threadIdx.x & 63) == 0) wave_max[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t w = wave_max[0];
#pragma unroll
    for (int i = 1; i < AMAX_THREADS / 64; i++) w = umax(w, wave_max[i]);
    // the running value only grows, so a workgroup whose maximum is not above it skips the
    // atomic (an older, smaller value read here only costs a redundant atomic)
    unsigned int* out = reinterpret_cast<unsigned int*>(a.amax_out);
    if ((w << 16) > __hip_atomic_load(out, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
      atomicMax(out, w << 16);
  }
}

}  // namespace

hipError_t launch_glu_amax(const NvArgs& a, hipStream_t s) {
  hipError_t e = launch_kernel(k_zero_u32, dim3(1), dim3(64), s, reinterpret_cast<uint32_t*>(a.amax_out));
  if (e != hipSuccess || a.M == 0 || a.H == 0) return e;
  const int64_t tpr = (a.H + AMAX_TILE * AMAX_GROUPS - 1) / (AMAX_TILE * AMAX_GROUPS);
  const dim3 grid = grid_2d(tpr, a.M, kAmaxWorkgroups), block(AMAX_THREADS);
  return with_act(a.act, [&](auto A) {
    constexpr int ACT = decltype(A)::value;
    return a.layout == PAIRED ? launch_kernel(k_glu_amax<ACT, PAIRED>, grid, block, s, a, tpr)
                              : launch_kernel(k_glu_amax<ACT, SPLIT>, grid, block, s, a, tpr);
  });
}

hipError_t launch_glu_fwd_nvfp4_gs(const NvArgs& a, hipStream_t s) {
  return with_act(a.act, [&](auto A) {
    constexpr int ACT = decltype(A)::value;
    return a.layout == PAIRED ? launch<ACT, PAIRED, NV_FWD_GS>(a, s) : launch<ACT, SPLIT, NV_FWD_GS>(a, s);
  });
}

hipError_t launch_glu_fwd_nvfp4(const NvArgs& a, hipStream_t s) {
  return with_act(a.act, [&](auto A) {
    constexpr int ACT = decltype(A)::value;
    return a.layout == PAIRED ? launch<ACT, PAIRED, NV_FWD>(a, s) : launch<ACT, SPLIT, NV_FWD>(a, s);
  });
}

hipError_t launch_glu_bwd_nvfp4(const NvArgs& a, hipStream_t s) {
  return with_act(a.act, [&](auto A) {
    constexpr int ACT = decltype(A)::value;
    return launch<ACT, SPLIT, NV_BWD>(a, s);
  });
}

hipError_t launch_quant_nvfp4_f32(const NvArgs& a, hipStream_t s) {
  return launch<SWIGLU, SPLIT, NV_F32>(a, s);
}

}  // namespace glu
