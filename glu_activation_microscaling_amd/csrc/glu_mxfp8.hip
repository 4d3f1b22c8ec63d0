// Fused GLU + MXFP8 quantization, forward and backward, rowwise / colwise / both from one
// read of the inputs ("Add swiglu + MXFP8 fused CuTe DSL kernel", Summary and API), and
// the FP32 quantizer hook that runs the same block rules on given FP32 values.
//
// Work decomposition (wave64):
//   A workgroup owns a TM x TN = 128 x 128 tile of the quantized matrix (of each of da and db
//   in the backward) with WGM x WGN = 4 x 2 waves.  A wave covers 32 rows x 64 columns: one
//   32-row colwise block row and two 32-column rowwise blocks per row.  Lane = lr + 8*lc owns
//   rows 4lr..4lr+3 and columns 8lc..8lc+7 of the wave's piece: 16-byte loads per row and per
//   operand, 32 elements per lane, kept after the activation as 16 packed BF16 pairs.
//   Rowwise amax of a 32-column block spans the 4 lanes lc = 4b..4b+3 (lane bits 3, 4):
//   DPP row_ror:8 then ds_swizzle xor 16.  Colwise amax of a 32-row block spans the 8
//   lanes lr = 0..7 (lane bits 0..2) after an in-lane max over 4 rows: DPP quad_perm xor 1,
//   xor 2, then row_half_mirror.  Maxima are taken on packed 16-bit magnitudes (two
//   columns, or two rows, per instruction).
//   Codes and scales are staged in LDS and leave, after one workgroup barrier, as 16-byte
//   stores that fill whole 128-byte lines: a tile row of rowwise codes and a tile column of
//   colwise codes are 128 bytes each, and the scales of a tile row (column) are one 4-byte
//   word.  Straight from the registers the same data would leave as 32-byte (colwise) and
//   64-byte (rowwise) pieces and single scale bytes: several times more L2 write requests,
//   which measured as the limit once enough tiles run concurrently to keep HBM busy.
//   Tiles are dealt to the 8 XCDs in contiguous runs along M (workgroups go to XCDs
//   round-robin by id), so neighbouring tiles along M, which share the transposed colwise
//   output's scale words, run on one XCD at about the same time.
#include "glu_device.h"
#include "glu_launch.h"

namespace glu {
namespace {

// Build-time tuning (fixed defaults; alternatives are compiled only to measure them):
//   GLU_MX_NT_LOADS: non-temporal (streaming) operand loads.
//   GLU_MX_NT_STORES: -1 per kernel (below); 0 / 1 non-temporal code stores off / on.
#ifndef GLU_MX_NT_LOADS
#define GLU_MX_NT_LOADS 1
#endif
#ifndef GLU_MX_NT_STORES
#define GLU_MX_NT_STORES -1
#endif
//   GLU_MX_TILE_ORDER: -1 per direction (below), else the order 0, 1 or 2 for every kernel.
#ifndef GLU_MX_TILE_ORDER
#define GLU_MX_TILE_ORDER -1
#endif

enum { MODE_FWD = 0, MODE_BWD = 1, MODE_F32 = 2 };

constexpr int WGM = 4, WGN = 2;                 // waves per workgroup along M and N
constexpr int TM = 32 * WGM, TN = 64 * WGN;     // quantized tile per workgroup
constexpr int NTHREADS = 64 * WGM * WGN;
static_assert(TM == 128 && TN == 128, "the LDS swizzles and 4-byte scale words assume 128 x 128");

// Non-temporal code stores: measured faster only for the backward quantized both ways
// (234 vs 267 us at [16384, 7168] in the blocked tile order); slower for the forward both
// ways (138 vs 126 us).
template <int MODE, int FLAGS>
constexpr bool nt_stores() {
  return GLU_MX_NT_STORES < 0 ? MODE == MODE_BWD && FLAGS == (ROWWISE | COLWISE)
                               : GLU_MX_NT_STORES == 1;
}

// Order of the tiles; each XCD takes a contiguous run of it.
//   0 (colwise only): along M first, so consecutive tiles continue the same rows of the
//     transposed [N, M] output and fill its scale rows word after word.
//   1 (rowwise only): along N first, so consecutive tiles continue the same input and output
//     rows and fill the rowwise scale rows word after word (about 3% faster at [16384, 7168]).
//   2 (both): strips of 8 tile columns; in a strip, blocks of 8 x 8 tiles going down M; in a
//     block, along M first.  The 8 tiles of a block that share rows (columns) write their
//     4-byte rowwise (colwise) scale words into one 32-byte sector within the same window of
//     concurrent tiles, so both scale streams leave L2 as whole sectors (orders 0 and 1 leave
//     one of them as single words: 6% slower at [16384, 7168]).
#ifndef GLU_MX_ORDER_BLOCK  // build-time override of the block size, for measurements
#define GLU_MX_ORDER_BLOCK 8
#endif
constexpr int kOrderBlock = GLU_MX_ORDER_BLOCK;  // 4: 252, 8: 234, 16: 238 us backward both

template <int FLAGS>
constexpr int tile_order() {
  return GLU_MX_TILE_ORDER >= 0 ? GLU_MX_TILE_ORDER
                                : FLAGS == ROWWISE ? 1 : FLAGS == COLWISE ? 0 : 2;
}

template <int ORDER>
__device__ __forceinline__ void tile_of(uint32_t t, uint32_t tiles_m, uint32_t tiles_n,
                                        uint32_t& tm, uint32_t& tn) {
  if constexpr (ORDER == 0) {
    tn = t / tiles_m;
    tm = t - tn * tiles_m;
  } else if constexpr (ORDER == 1) {
    tm = t / tiles_n;
    tn = t - tm * tiles_n;
  } else {
    constexpr uint32_t B = kOrderBlock;
    const uint32_t strip = tiles_m * B;  // tiles per full strip
    const uint32_t bj = t / strip, u = t - bj * strip;
    const uint32_t w = tiles_n - bj * B < B ? tiles_n - bj * B : B;  // strip width
    const uint32_t bi = u / (B * w), v = u - bi * B * w;
    const uint32_t h = tiles_m - bi * B < B ? tiles_m - bi * B : B;  // block height
    const uint32_t j = v / h;
    tm = bi * B + (v - j * h);
    tn = bj * B + j;
  }
}

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));


typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ u16x2 as_u16x2(uint32_t w) { return __builtin_bit_cast(u16x2, w); }
__device__ __forceinline__ uint32_t as_u32(u16x2 v) { return __builtin_bit_cast(uint32_t, v); }
__device__ __forceinline__ uint32_t pkmax(uint32_t a, uint32_t b) {
  return as_u32(__builtin_elementwise_max(as_u16x2(a), as_u16x2(b)));
}
// Packed E8M0 RCEIL scale bytes from packed BF16 magnitudes A = E << 7 | m of finite block
// maxima: e + 127 = E - 8 + (m > 0x60), i.e. ((A + 0x1F) >> 7) - 8 saturated at 0.
__device__ __forceinline__ uint32_t pk_scale_bytes(uint32_t A) {
  const u16x2 t = (as_u16x2(A) + (u16x2){0x1f, 0x1f}) >> (u16x2){7, 7};
  return as_u32(__builtin_elementwise_sub_sat(t, (u16x2){8, 8}));
}
__device__ __forceinline__ uint32_t lo16(uint32_t w) { return w & 0xffffu; }
__device__ __forceinline__ uint32_t hi16(uint32_t w) { return w >> 16; }
// (a.lo, b.lo) and (a.hi, b.hi) as packed pairs
__device__ __forceinline__ uint32_t pair_lo(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x05040100u); }
__device__ __forceinline__ uint32_t pair_hi(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x07060302u); }

// Raw operand words of 8 consecutive outputs: SPLIT gives gate and up words (each a BF16
// pair of adjacent columns); PAIRED gives 8 words, each a (gate, up) BF16 pair.
template <int LAYOUT>
struct GU {
  uint32_t a[LAYOUT == SPLIT ? 4 : 8];
  uint32_t b[LAYOUT == SPLIT ? 4 : 1];
};

template <int LAYOUT>
__device__ __forceinline__ void unpack_gu(const GU<LAYOUT>& r, float g[8], float u[8]) {
  if constexpr (LAYOUT == SPLIT) {
#pragma unroll
    for (int k = 0; k < 4; k++) {
      g[2 * k] = bf_lo(r.a[k]);
      g[2 * k + 1] = bf_hi(r.a[k]);
      u[2 * k] = bf_lo(r.b[k]);
      u[2 * k + 1] = bf_hi(r.b[k]);
    }
  } else {
#pragma unroll
    for (int k = 0; k < 8; k++) {
      g[k] = bf_lo(r.a[k]);
      u[k] = bf_hi(r.a[k]);
    }
  }
}

// Operands are read with raw buffer loads through a descriptor whose base is the first byte
// of a wave's piece (a wave-uniform address).  A lane whose element is outside the matrix
// passes kOob as its offset; the hardware's range check turns that load into zeros, so every
// path through a tile issues the same loads, with no branch and no select.  Row pitches are
// limited (by the host checks) so that 32 rows of offsets stay below kOob.
constexpr uint32_t kOob = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base) {
  // gfx9 descriptor word 3: 32-bit data format, raw (stride 0) addressing
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)(kOob - 1),
                                           0x00020000);
}

__device__ __forceinline__ void bld16(uint32_t (&w)[4], __amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, GLU_MX_NT_LOADS ? 2 : 0);
  w[0] = x.x; w[1] = x.y; w[2] = x.z; w[3] = x.w;
}

// Raw operands of one lane's 4x8 elements of a tile.
template <int LAYOUT, int MODE>
struct TileOps {
  GU<MODE == MODE_BWD ? SPLIT : LAYOUT> in[4];  // gate/up words (forward, backward)
  uint32_t d[MODE == MODE_BWD ? 4 : 1][4];      // dh words (backward)
  uint32_t x[MODE == MODE_F32 ? 4 : 1][8];      // FP32 bits (quantizer hook)
};

// Where one wave's 32 x 64 piece of a tile lies.
struct TileGeom {
  int64_t r0, cw;  // first row and column of the piece (wave-uniform)
  int64_t col;     // this lane's first column
  bool col_ok;     // this lane's 8 columns are inside
};

// Issues the loads of the lane's 4 x 8 operands of a piece (4 consecutive rows, 8 columns).
template <int LAYOUT, int MODE>
__device__ __forceinline__ void load_ops(TileOps<LAYOUT, MODE>& o, const MxArgs& a,
                                         const TileGeom& g, int lr, int lc) {
  const int64_t left = a.M - g.r0;
  const int rows = left < 0 ? 0 : (left > 32 ? 32 : (int)left);  // rows of the piece inside
  bool ok[4];
#pragma unroll
  for (int i = 0; i < 4; i++) ok[i] = g.col_ok && 4 * lr + i < rows;
  if constexpr (MODE == MODE_F32) {
    const uint32_t ld = (uint32_t)a.ld_in * 4u;
    const auto r = rsrc(static_cast<const float*>(a.src) + g.r0 * a.ld_in + g.cw);
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const uint32_t off = (uint32_t)(4 * lr + i) * ld + 32u * lc;
      uint32_t w0[4], w1[4];
      bld16(w0, r, ok[i] ? off : kOob);
      bld16(w1, r, ok[i] ? off + 16u : kOob);
#pragma unroll
      for (int k = 0; k < 4; k++) {
        o.x[i][k] = w0[k];
        o.x[i][4 + k] = w1[k];
      }
    }
  } else {
    constexpr int L = MODE == MODE_BWD ? SPLIT : LAYOUT;
    const uint32_t ld = (uint32_t)a.ld_in * 2u;
    const uint16_t* gate = static_cast<const uint16_t*>(a.src);
    if constexpr (L == SPLIT) {
      const int64_t base = g.r0 * a.ld_in + g.cw;
      const auto rg = rsrc(gate + base), ru = rsrc(a.up + base);
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const uint32_t off = ok[i] ? (uint32_t)(4 * lr + i) * ld + 16u * lc : kOob;
        bld16(o.in[i].a, rg, off);
        bld16(o.in[i].b, ru, off);
      }
    } else {
      const auto rg = rsrc(gate + g.r0 * a.ld_in + 2 * g.cw);
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const uint32_t off = (uint32_t)(4 * lr + i) * ld + 32u * lc;
        uint32_t w0[4], w1[4];
        bld16(w0, rg, ok[i] ? off : kOob);
        bld16(w1, rg, ok[i] ? off + 16u : kOob);
#pragma unroll
        for (int k = 0; k < 4; k++) {
          o.in[i].a[k] = w0[k];
          o.in[i].a[4 + k] = w1[k];
        }
      }
    }
    if constexpr (MODE == MODE_BWD) {
      const uint32_t ldd = (uint32_t)a.ld_dh * 2u;
      const auto rd = rsrc(a.dh + g.r0 * a.ld_dh + g.cw);
#pragma unroll
      for (int i = 0; i < 4; i++)
        bld16(o.d[i], rd, ok[i] ? (uint32_t)(4 * lr + i) * ldd + 16u * lc : kOob);
    }
  }
}

// A tile's results before quantization: BF16 words (forward: h; backward: da, db) or the
// FP32 input of the quantizer hook.
template <int MODE>
struct TileVals {
  uint32_t h[MODE == MODE_BWD ? 2 : 1][4][4];
  float v[MODE == MODE_F32 ? 4 : 1][8];
};

template <int ACT, int LAYOUT, int MODE>
__device__ __forceinline__ void compute(TileVals<MODE>& r, const TileOps<LAYOUT, MODE>& o) {
  if constexpr (MODE == MODE_F32) {
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
      for (int c = 0; c < 8; c++) r.v[i][c] = __uint_as_float(o.x[i][c]);
  } else if constexpr (MODE == MODE_FWD) {
#pragma unroll
    for (int i = 0; i < 4; i++) {
      float gg[8], u[8], h[8], zmin = 0.0f;
      unpack_gu<LAYOUT>(o.in[i], gg, u);
#pragma unroll
      for (int c = 0; c < 8; c++) h[c] = glu_fwd_elem<ACT>(gg[c], u[c], zmin);
      if (zmin < TAIL_ZL2) {  // rare: e^z below the FP32 normal range
#pragma unroll
        for (int c = 0; c < 8; c++)
          if (zl2<ACT>(gg[c]) < TAIL_ZL2) h[c] = glu_fwd_tail<ACT>(gg[c], u[c]);
      }
#pragma unroll
      for (int k = 0; k < 4; k++) r.h[0][i][k] = pack_bf16(h[2 * k], h[2 * k + 1]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; i++) {
      float gg[8], u[8], d[8], da[8], db[8], zmin = 0.0f;
      unpack_gu<SPLIT>(o.in[i], gg, u);
#pragma unroll
      for (int c = 0; c < 8; c++) {
        d[c] = (c & 1) ? bf_hi(o.d[i][c >> 1]) : bf_lo(o.d[i][c >> 1]);
        glu_bwd_elem<ACT>(gg[c], u[c], d[c], da[c], db[c], zmin);
      }
      if (zmin < TAIL_ZL2) {  // rare: e^z below the FP32 normal range
#pragma unroll
        for (int c = 0; c < 8; c++)
          if (zl2<ACT>(gg[c]) < TAIL_ZL2) glu_bwd_tail<ACT>(gg[c], u[c], d[c], da[c], db[c]);
      }
#pragma unroll
      for (int k = 0; k < 4; k++) {
        r.h[0][i][k] = pack_bf16(da[2 * k], da[2 * k + 1]);
        r.h[1][i][k] = pack_bf16(db[2 * k], db[2 * k + 1]);
      }
    }
  }
}

// LDS staging of one quantized part (the tile of h, or of da or db):
//   rq  rowwise codes [TM][TN], row-major;      rs  rowwise scales [TM][TN/32];
//   cq  colwise codes [TN][TM], column-major;   cs  colwise scales [TN][TM/32].
// The 16-byte segments of each code row (rq) and column (cq) are XOR-swizzled, by
// (row / 4) % 8 and (column / 8) % 8, so that the staging writes of a wave (8 rows 4 apart,
// or 8 columns 8 apart, at the same offset) and the 16-byte reads of the write-out fall in
// different banks.
template <int FLAGS>
struct Stage {
  static constexpr int RQ = (FLAGS & ROWWISE) ? TM * TN : 0;
  static constexpr int CQ = (FLAGS & COLWISE) ? TN * TM : 0;
  static constexpr int RS = (FLAGS & ROWWISE) ? TM * (TN / 32) : 0;
  static constexpr int CS = (FLAGS & COLWISE) ? TN * (TM / 32) : 0;
  static constexpr int BYTES = RQ + CQ + RS + CS;
  uint8_t* rq;
  uint8_t* cq;
  uint8_t* rs;
  uint8_t* cs;
  __device__ explicit Stage(uint8_t* base)
      : rq(base), cq(base + RQ), rs(base + RQ + CQ), cs(base + RQ + CQ + RS) {}
};

// Byte offsets in rq of (row, col) and in cq of (col, row), within a 16-byte segment.
__device__ __forceinline__ int rq_at(int row, int col) {
  return row * TN + 16 * ((col >> 4) ^ ((row >> 2) & 7)) + (col & 15);
}
__device__ __forceinline__ int cq_at(int col, int row) {
  return col * TM + 16 * ((row >> 4) ^ ((col >> 3) & 7)) + (row & 15);
}

__device__ __forceinline__ void lds_st8(uint8_t* p, uint32_t w0, uint32_t w1) {
  *reinterpret_cast<u32x2*>(p) = (u32x2){w0, w1};
}
__device__ __forceinline__ void lds_st4(uint8_t* p, uint32_t w) { *reinterpret_cast<uint32_t*>(p) = w; }

// Quantizes the lane's 4x8 BF16 values H[i][k] = (columns 2k, 2k+1 of tile row row0 + i),
// tile columns col..col+7 (row0 = 32wm + 4lr, col = 64wn + 8lc), into the LDS stage.  All
// 64 lanes of the wave take part (cross-lane maxima).  Elements outside the matrix were
// loaded as zeros: they form blocks of their own (N and, when colwise, M are multiples of
// 32), quantize to zero codes and are never written out.
template <int FLAGS>
__device__ __forceinline__ void stage_bf16(const uint32_t (&H)[4][4], const Stage<FLAGS>& st,
                                           int row0, int col, int lr, int lc) {
  uint32_t A[4][4];
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int k = 0; k < 4; k++) A[i][k] = H[i][k] & 0x7fff7fffu;

  uint32_t R01 = 0, R23 = 0;  // row block maxima, rows (0,1) and (2,3) packed
  uint32_t C[4] = {0, 0, 0, 0};  // column block maxima, columns (2k, 2k+1) packed
  if constexpr ((FLAGS & ROWWISE) != 0) {
    uint32_t m[4];
#pragma unroll
    for (int i = 0; i < 4; i++) m[i] = pkmax(pkmax(A[i][0], A[i][1]), pkmax(A[i][2], A[i][3]));
    R01 = pkmax(pair_lo(m[0], m[1]), pair_hi(m[0], m[1]));
    R23 = pkmax(pair_lo(m[2], m[3]), pair_hi(m[2], m[3]));
    R01 = pkmax(R01, dpp<DPP_ROW_ROR8>(R01));
    R23 = pkmax(R23, dpp<DPP_ROW_ROR8>(R23));
    R01 = pkmax(R01, swz_xor16(R01));
    R23 = pkmax(R23, swz_xor16(R23));
  }
  if constexpr ((FLAGS & COLWISE) != 0) {
#pragma unroll
    for (int k = 0; k < 4; k++) {
      uint32_t c = pkmax(pkmax(A[0][k], A[1][k]), pkmax(A[2][k], A[3][k]));
      c = pkmax(c, dpp<DPP_XOR1>(c));
      c = pkmax(c, dpp<DPP_XOR2>(c));
      C[k] = pkmax(c, dpp<DPP_HALF_MIRROR>(c));
    }
  }
  // any non-finite block among those this lane touches? (rare: patched after the fast path)
  const uint32_t all = pkmax(pkmax(R01, R23), pkmax(pkmax(C[0], C[1]), pkmax(C[2], C[3])));
  const bool nonfinite = umax(lo16(all), hi16(all)) >= 0x7f80u;

  if constexpr ((FLAGS & ROWWISE) != 0) {
    const uint32_t S01 = pk_scale_bytes(R01), S23 = pk_scale_bytes(R23);
    const uint32_t sb[4] = {lo16(S01), hi16(S01), lo16(S23), hi16(S23)};
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const float sc = e8m0_value(sb[i]);
      uint32_t w0 = fp8x2_scaled<false>(0u, H[i][0], sc);
      w0 = fp8x2_scaled<true>(w0, H[i][1], sc);
      uint32_t w1 = fp8x2_scaled<false>(0u, H[i][2], sc);
      w1 = fp8x2_scaled<true>(w1, H[i][3], sc);
      lds_st8(st.rq + rq_at(row0 + i, col), w0, w1);
    }
    // lane lc = 4b + i stages the scale of row 4lr + i in the wave's block b
    const int i = lc & 3;
    const uint32_t w = i < 2 ? S01 : S23;
    st.rs[(row0 + i) * (TN / 32) + ((col - 8 * i) >> 5)] = (uint8_t)((i & 1) ? hi16(w) : lo16(w));
  }
  if constexpr ((FLAGS & COLWISE) != 0) {
    uint32_t S[4];
#pragma unroll
    for (int k = 0; k < 4; k++) S[k] = pk_scale_bytes(C[k]);
#pragma unroll
    for (int k = 0; k < 4; k++) {
      const float s0 = e8m0_value(lo16(S[k])), s1 = e8m0_value(hi16(S[k]));
      // column 2k: rows (0,1) from the low halves, rows (2,3) likewise
      uint32_t w0 = fp8x2_scaled<false>(0u, pair_lo(H[0][k], H[1][k]), s0);
      w0 = fp8x2_scaled<true>(w0, pair_lo(H[2][k], H[3][k]), s0);
      uint32_t w1 = fp8x2_scaled<false>(0u, pair_hi(H[0][k], H[1][k]), s1);
      w1 = fp8x2_scaled<true>(w1, pair_hi(H[2][k], H[3][k]), s1);
      lds_st4(st.cq + cq_at(col + 2 * k, row0), w0);
      lds_st4(st.cq + cq_at(col + 2 * k + 1, row0), w1);
    }
    // lane lr stages the scale of column 8lc + lr of this 32-row block
    const uint32_t w = (lr >> 1) == 0 ? S[0] : (lr >> 1) == 1 ? S[1] : (lr >> 1) == 2 ? S[2] : S[3];
    st.cs[(col + lr) * (TM / 32) + (row0 >> 5)] = (uint8_t)((lr & 1) ? hi16(w) : lo16(w));
  }

  if (nonfinite) {
    // a block holding NaN or Inf: scale 0xFF, every code 0x7F (overwrites the fast path; each
    // lane patches only what it staged itself, so program order suffices)
    if constexpr ((FLAGS & ROWWISE) != 0) {
      const uint32_t rm[4] = {lo16(R01), hi16(R01), lo16(R23), hi16(R23)};
#pragma unroll
      for (int i = 0; i < 4; i++) {
        if (rm[i] >= 0x7f80u) {
          lds_st8(st.rq + rq_at(row0 + i, col), 0x7f7f7f7fu, 0x7f7f7f7fu);
          if ((lc & 3) == i) st.rs[(row0 + i) * (TN / 32) + ((col - 8 * i) >> 5)] = 0xff;
        }
      }
    }
    if constexpr ((FLAGS & COLWISE) != 0) {
#pragma unroll
      for (int c = 0; c < 8; c++) {
        const uint32_t cm = (c & 1) ? hi16(C[c >> 1]) : lo16(C[c >> 1]);
        if (cm >= 0x7f80u) {
          lds_st4(st.cq + cq_at(col + c, row0), 0x7f7f7f7fu);
          if (lr == c) st.cs[(col + c) * (TM / 32) + (row0 >> 5)] = 0xff;
        }
      }
    }
  }
}

// The same rules on FP32 values (quantizer hook): magnitudes compared as FP32 bits, the
// scaled value x * 2^-e computed exactly in FP32, then v_cvt_pk_fp8_f32.
template <int FLAGS>
__device__ __forceinline__ void stage_f32(const float (&v)[4][8], const Stage<FLAGS>& st,
                                          int row0, int col, int lr, int lc) {
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
      uint32_t w0 = fp8x2<false>(0u, v[i][0] * P, v[i][1] * P);
      w0 = fp8x2<true>(w0, v[i][2] * P, v[i][3] * P);
      uint32_t w1 = fp8x2<false>(0u, v[i][4] * P, v[i][5] * P);
      w1 = fp8x2<true>(w1, v[i][6] * P, v[i][7] * P);
      if (nonfinite) w0 = w1 = 0x7f7f7f7fu;
      lds_st8(st.rq + rq_at(row0 + i, col), w0, w1);
    }
    const int i = lc & 3;
    st.rs[(row0 + i) * (TN / 32) + ((col - 8 * i) >> 5)] = (uint8_t)(packed >> (8 * i));
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
      uint32_t w = fp8x2<false>(0u, v[0][c] * P, v[1][c] * P);
      w = fp8x2<true>(w, v[2][c] * P, v[3][c] * P);
      if (nonfinite) w = 0x7f7f7f7fu;
      lds_st4(st.cq + cq_at(col + c, row0), w);
    }
    const uint32_t w = lr < 4 ? packed0 : packed1;
    st.cs[(col + lr) * (TM / 32) + (row0 >> 5)] = (uint8_t)(w >> (8 * (lr & 3)));
  }
}

template <bool NT>
__device__ __forceinline__ void st16(uint8_t* p, u32x4 v) {
  if constexpr (NT) __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
  else *reinterpret_cast<u32x4*>(p) = v;
}

// Writes a staged part to global memory: the part is the [M, N] matrix at column offset
// `coloff` of the quantized matrix, whose rows hold ldq codes; the tile starts at (r0, c0).
// Rows >= M and columns >= N are skipped, in whole 16-byte segments (N and, when colwise,
// M are multiples of 32).  Scale words are written whole where the 4 bytes are in range and
// 4-byte aligned, else byte by byte.
template <int FLAGS, bool NT>
__device__ __forceinline__ void write_out(const Stage<FLAGS>& st, const MxArgs& a, int64_t r0,
                                          int64_t c0, int64_t coloff, int64_t ldq, int tid) {
  const int64_t M = a.M, N = a.N;
  if constexpr ((FLAGS & ROWWISE) != 0) {
    constexpr int SEGS = TN / 16;
#pragma unroll
    for (int k = tid; k < TM * SEGS; k += NTHREADS) {
      const int row = k / SEGS, seg = k % SEGS;
      if (r0 + row < M && c0 + 16 * seg < N) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(st.rq + row * TN + 16 * (seg ^ ((row >> 2) & 7)));
        st16<NT>(a.q_row + (r0 + row) * ldq + coloff + c0 + 16 * seg, v);
      }
    }
    const int64_t nb = ldq / 32;
    const bool whole = nb % 4 == 0 && (coloff / 32) % 4 == 0 && c0 + TN <= N;
    for (int row = tid; row < TM; row += NTHREADS) {
      if (r0 + row < M) {
        uint8_t* dst = a.s_row + (r0 + row) * nb + (coloff + c0) / 32;
        const uint8_t* src = st.rs + row * (TN / 32);
        if (whole) {
          *reinterpret_cast<uint32_t*>(dst) = *reinterpret_cast<const uint32_t*>(src);
        } else {
          for (int b = 0; b < TN / 32; b++)
            if (c0 + 32 * b < N) dst[b] = src[b];
        }
      }
    }
  }
  if constexpr ((FLAGS & COLWISE) != 0) {
    constexpr int SEGS = TM / 16;
#pragma unroll
    for (int k = tid; k < TN * SEGS; k += NTHREADS) {
      const int col = k / SEGS, seg = k % SEGS;
      if (c0 + col < N && r0 + 16 * seg < M) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(st.cq + col * TM + 16 * (seg ^ ((col >> 3) & 7)));
        st16<NT>(a.q_col + (coloff + c0 + col) * M + r0 + 16 * seg, v);
      }
    }
    const int64_t nb = M / 32;
    const bool whole = nb % 4 == 0 && r0 + TM <= M;
    for (int col = tid; col < TN; col += NTHREADS) {
      if (c0 + col < N) {
        uint8_t* dst = a.s_col + (coloff + c0 + col) * nb + r0 / 32;
        const uint8_t* src = st.cs + col * (TM / 32);
        if (whole) {
          *reinterpret_cast<uint32_t*>(dst) = *reinterpret_cast<const uint32_t*>(src);
        } else {
          for (int b = 0; b < TM / 32; b++)
            if (r0 + 32 * b < M) dst[b] = src[b];
        }
      }
    }
  }
}

// One workgroup per tile.  Workgroup id b runs on XCD b % 8 (workgroups are dealt to the
// XCDs round-robin); XCD x takes tiles x * per_xcd + b / 8 of the tile order.
template <int ACT, int LAYOUT, int FLAGS, int MODE>
__global__ __launch_bounds__(NTHREADS) void k_mxfp8(MxArgs a, uint32_t tiles_m, uint32_t tiles_n,
                                                    uint32_t ntiles, uint32_t per_xcd) {
  constexpr int PARTS = MODE == MODE_BWD ? 2 : 1;
  __shared__ __attribute__((aligned(16))) uint8_t lds[PARTS * Stage<FLAGS>::BYTES];
  const uint32_t t = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (t >= ntiles) return;  // the whole workgroup
  uint32_t tm, tn;
  tile_of<tile_order<FLAGS>()>(t, tiles_m, tiles_n, tm, tn);
  const int64_t r0 = (int64_t)tm * TM, c0 = (int64_t)tn * TN;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
  const int wm = w % WGM, wn = w / WGM;
  const int lr = lane & 7, lc = lane >> 3;

  TileGeom g;
  g.r0 = r0 + 32 * wm;
  g.cw = c0 + 64 * wn;
  g.col = g.cw + 8 * lc;
  g.col_ok = g.col < a.N;
  TileOps<LAYOUT, MODE> o;
  load_ops<LAYOUT, MODE>(o, a, g, lr, lc);
  TileVals<MODE> R;
  compute<ACT, LAYOUT, MODE>(R, o);

  const int row0 = 32 * wm + 4 * lr, col = 64 * wn + 8 * lc;
  if constexpr (MODE == MODE_F32) {
    stage_f32<FLAGS>(R.v, Stage<FLAGS>(lds), row0, col, lr, lc);
  } else {
    stage_bf16<FLAGS>(R.h[0], Stage<FLAGS>(lds), row0, col, lr, lc);
    if constexpr (MODE == MODE_BWD)
      stage_bf16<FLAGS>(R.h[1], Stage<FLAGS>(lds + Stage<FLAGS>::BYTES), row0, col, lr, lc);
  }
  __syncthreads();
  const int64_t ldq = PARTS * a.N;
  constexpr bool NT = nt_stores<MODE, FLAGS>();
  write_out<FLAGS, NT>(Stage<FLAGS>(lds), a, r0, c0, 0, ldq, tid);
  if constexpr (MODE == MODE_BWD)
    write_out<FLAGS, NT>(Stage<FLAGS>(lds + Stage<FLAGS>::BYTES), a, r0, c0, a.N, ldq, tid);
}

template <int ACT, int LAYOUT, int FLAGS, int MODE>
hipError_t launch(const MxArgs& a, hipStream_t s) {
  const int64_t tiles_m = (a.M + TM - 1) / TM, tiles_n = (a.N + TN - 1) / TN;
  const int64_t ntiles = tiles_m * tiles_n, per_xcd = (ntiles + 7) / 8;
  return launch_kernel(k_mxfp8<ACT, LAYOUT, FLAGS, MODE>, dim3((unsigned)(8 * per_xcd)),
                       dim3(NTHREADS), s, a, (uint32_t)tiles_m, (uint32_t)tiles_n, (uint32_t)ntiles,
                       (uint32_t)per_xcd);
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
