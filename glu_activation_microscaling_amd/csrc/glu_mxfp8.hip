// Fused GLU + MXFP8 quantization, forward and backward, rowwise / colwise / both from one
// read of the inputs ("Add swiglu + MXFP8 fused CuTe DSL kernel", Summary and API), and
// the FP32 quantizer hook that runs the same block rules on given FP32 values.
//
// Work decomposition (wave64):
//   A wave covers 32 rows x 64 columns: one 32-row colwise block row and two 32-column
//   rowwise blocks per row.  Lane = lr + 8*lc owns rows 4lr..4lr+3 and columns 8lc..8lc+7:
//   16-byte loads per row and per operand, 32 elements per lane, kept after the activation
//   as 16 packed BF16 pairs.  A workgroup stacks WGM x WGN waves (the launch shape per
//   direction is set in WgShape below).
//   Rowwise amax of a 32-column block spans the 4 lanes lc = 4b..4b+3 (lane bits 3, 4):
//   DPP row_ror:8 then ds_swizzle xor 16.  Colwise amax of a 32-row block spans the 8
//   lanes lr = 0..7 (lane bits 0..2) after an in-lane max over 4 rows: DPP quad_perm xor 1,
//   xor 2, then row_half_mirror.  Maxima are taken on packed 16-bit magnitudes (two
//   columns, or two rows, per instruction).  No LDS is needed: each lane already holds 4
//   consecutive rows of every column it owns, so colwise codes leave as 4-byte stores into
//   the transposed [N, M] output and rowwise codes as 8-byte stores.
//   Tiles are dealt to the 8 XCDs in contiguous runs along M (workgroups go to XCDs
//   round-robin by id), so the transposed colwise lines and their scale bytes, which
//   neighbouring tiles along M share, are assembled in one XCD's L2.
#include "glu_device.h"
#include "glu_launch.h"

namespace glu {
namespace {

// Launch shape per direction: waves per workgroup along M and N (each wave covers 32 rows x
// 64 columns) and LDS bytes reserved per workgroup.  The LDS is not used by the kernel; the
// reservation (more than half of a CU's 160 KiB) keeps one workgroup per CU.  Chosen from
// interleaved measurements on MI355X at [16384, 7168]: rowwise-only forward output is
// fastest with 64 x 128 tiles at full occupancy; whenever colwise codes are written or two
// matrices are quantized (backward), 64 x 256 tiles with one workgroup per CU are fastest
// (fewer concurrent tile streams: 146 vs 176 us forward both, 258 vs 360 us backward both).
template <int MODE, int FLAGS>
struct WgShape {
#if defined(GLU_MX_WG_M) && defined(GLU_MX_WG_N)  // build-time override, for measurements
  static constexpr int M = GLU_MX_WG_M;
  static constexpr int N = GLU_MX_WG_N;
  static constexpr int LDS = GLU_MX_LDS_BYTES;
#else
  static constexpr bool ROW_FWD = MODE == 0 && FLAGS == 1;
  static constexpr int M = 2;
  static constexpr int N = ROW_FWD ? 2 : 4;
  static constexpr int LDS = ROW_FWD ? 0 : 86016;
#endif
};

// Build-time tuning (fixed defaults; alternatives are compiled only to measure them):
//   GLU_MX_TILE_ORDER 0: each XCD takes a contiguous run of tiles in M-fastest order;
//                     1: each XCD takes a contiguous run of tiles in N-fastest order;
//                     2: tiles in workgroup-id order, N fastest (no XCD remapping).
//   GLU_MX_NT_LOADS / GLU_MX_NT_STORES: non-temporal (streaming) operand loads / code stores.
#ifndef GLU_MX_TILE_ORDER
#define GLU_MX_TILE_ORDER 0
#endif
#ifndef GLU_MX_NT_LOADS
#define GLU_MX_NT_LOADS 1
#endif
#ifndef GLU_MX_NT_STORES
#define GLU_MX_NT_STORES 0
#endif
//   GLU_MX_WG_M, GLU_MX_WG_N, GLU_MX_LDS_BYTES: launch shape for every direction (below).
#ifndef GLU_MX_LDS_BYTES
#define GLU_MX_LDS_BYTES 0
#endif

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void st_code(uint32_t* p, uint32_t v) {
  if constexpr (GLU_MX_NT_STORES) __builtin_nontemporal_store(v, p);
  else *p = v;
}
__device__ __forceinline__ void st_code(uint2* p, uint2 v) {
  const u32x2 x = {v.x, v.y};
  if constexpr (GLU_MX_NT_STORES) __builtin_nontemporal_store(x, reinterpret_cast<u32x2*>(p));
  else *reinterpret_cast<u32x2*>(p) = x;
}
enum { MODE_FWD = 0, MODE_BWD = 1, MODE_F32 = 2 };

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

struct MxOut {
  uint8_t* q_row;
  uint8_t* s_row;
  uint8_t* q_col;
  uint8_t* s_col;
  int64_t M;    // rows of the quantized matrix
  int64_t ldq;  // columns of the quantized matrix (N forward, 2N backward)
};

// Quantizes the lane's 4x8 BF16 values H[i][k] = (columns 2k, 2k+1 of row r0 + 4lr + i),
// columns starting at `col` of the quantized matrix, and stores codes and scales.  All 64
// lanes must call it together.  FULL: the wave's 32 rows and 64 columns are all in range
// (no per-row or per-column guards); otherwise rows >= M and columns >= the matrix width
// are skipped.
template <int FLAGS, bool FULL>
__device__ __forceinline__ void mx_store_bf16(const uint32_t (&H)[4][4], const MxOut& o,
                                              int64_t r0, int64_t col, int lr, int lc,
                                              bool col_ok) {
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
  // any non-finite block among those this lane touches? (rare: handled after the stores)
  const uint32_t all = pkmax(pkmax(R01, R23), pkmax(pkmax(C[0], C[1]), pkmax(C[2], C[3])));
  const bool nonfinite = umax(lo16(all), hi16(all)) >= 0x7f80u;

  const int64_t row0 = r0 + 4 * lr;
  const int64_t nb_row = o.ldq / 32, nb_col = o.M / 32;
  const bool lane_ok = FULL || col_ok;
  if constexpr ((FLAGS & ROWWISE) != 0) {
    const uint32_t S01 = pk_scale_bytes(R01), S23 = pk_scale_bytes(R23);
    const uint32_t sb[4] = {lo16(S01), hi16(S01), lo16(S23), hi16(S23)};
    uint8_t* q = o.q_row + row0 * o.ldq + col;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      if (FULL || (col_ok && row0 + i < o.M)) {
        const float sc = e8m0_value(sb[i]);
        uint32_t w0 = fp8x2_scaled<false>(0u, H[i][0], sc);
        w0 = fp8x2_scaled<true>(w0, H[i][1], sc);
        uint32_t w1 = fp8x2_scaled<false>(0u, H[i][2], sc);
        w1 = fp8x2_scaled<true>(w1, H[i][3], sc);
        st_code(reinterpret_cast<uint2*>(q), make_uint2(w0, w1));
      }
      q += o.ldq;
    }
    // lane lc = 4b + i stores the scale of row 4lr + i in block b
    const int i = lc & 3;
    if (FULL || (col_ok && row0 + i < o.M)) {
      const uint32_t w = i < 2 ? S01 : S23;
      o.s_row[(row0 + i) * nb_row + ((col - 8 * i) >> 5)] = (uint8_t)((i & 1) ? hi16(w) : lo16(w));
    }
  }
  if constexpr ((FLAGS & COLWISE) != 0) {
    uint32_t S[4];
#pragma unroll
    for (int k = 0; k < 4; k++) S[k] = pk_scale_bytes(C[k]);
    if (lane_ok) {
      uint8_t* q = o.q_col + col * o.M + row0;
#pragma unroll
      for (int k = 0; k < 4; k++) {
        const float s0 = e8m0_value(lo16(S[k])), s1 = e8m0_value(hi16(S[k]));
        // column 2k: rows (0,1) from the low halves, rows (2,3) likewise
        uint32_t w0 = fp8x2_scaled<false>(0u, pair_lo(H[0][k], H[1][k]), s0);
        w0 = fp8x2_scaled<true>(w0, pair_lo(H[2][k], H[3][k]), s0);
        uint32_t w1 = fp8x2_scaled<false>(0u, pair_hi(H[0][k], H[1][k]), s1);
        w1 = fp8x2_scaled<true>(w1, pair_hi(H[2][k], H[3][k]), s1);
        st_code(reinterpret_cast<uint32_t*>(q), w0);
        st_code(reinterpret_cast<uint32_t*>(q + o.M), w1);
        q += 2 * o.M;
      }
      // lane lr stores the scale of column 8lc + lr of this 32-row block
      const uint32_t w = (lr >> 1) == 0 ? S[0] : (lr >> 1) == 1 ? S[1] : (lr >> 1) == 2 ? S[2] : S[3];
      o.s_col[(col + lr) * nb_col + (r0 >> 5)] = (uint8_t)((lr & 1) ? hi16(w) : lo16(w));
    }
  }

  if (nonfinite) {
    // a block holding NaN or Inf: scale 0xFF, every code 0x7F (overwrites the fast path)
    if constexpr ((FLAGS & ROWWISE) != 0) {
      const uint32_t rm[4] = {lo16(R01), hi16(R01), lo16(R23), hi16(R23)};
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int64_t row = row0 + i;
        if (col_ok && row < o.M && rm[i] >= 0x7f80u) {
          *reinterpret_cast<uint2*>(o.q_row + row * o.ldq + col) = make_uint2(0x7f7f7f7fu, 0x7f7f7f7fu);
          if ((lc & 3) == i) o.s_row[row * nb_row + ((col - 8 * i) >> 5)] = 0xff;
        }
      }
    }
    if constexpr ((FLAGS & COLWISE) != 0) {
      if (col_ok) {
#pragma unroll
        for (int c = 0; c < 8; c++) {
          const uint32_t cm = (c & 1) ? hi16(C[c >> 1]) : lo16(C[c >> 1]);
          if (cm >= 0x7f80u) {
            *reinterpret_cast<uint32_t*>(o.q_col + (col + c) * o.M + row0) = 0x7f7f7f7fu;
            if (lr == c) o.s_col[(col + c) * nb_col + (r0 >> 5)] = 0xff;
          }
        }
      }
    }
  }
}

// The same rules on FP32 values (quantizer hook): magnitudes compared as FP32 bits, the
// scaled value x * 2^-e computed exactly in FP32, then v_cvt_pk_fp8_f32.
template <int FLAGS>
__device__ __forceinline__ void mx_store_f32(const float (&v)[4][8], const MxOut& o, int64_t r0,
                                             int64_t col, int lr, int lc, bool col_ok) {
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
        uint32_t w0 = fp8x2<false>(0u, v[i][0] * P, v[i][1] * P);
        w0 = fp8x2<true>(w0, v[i][2] * P, v[i][3] * P);
        uint32_t w1 = fp8x2<false>(0u, v[i][4] * P, v[i][5] * P);
        w1 = fp8x2<true>(w1, v[i][6] * P, v[i][7] * P);
        if (nonfinite) w0 = w1 = 0x7f7f7f7fu;
        *reinterpret_cast<uint2*>(o.q_row + row * o.ldq + col) = make_uint2(w0, w1);
      }
    }
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
        uint32_t w = fp8x2<false>(0u, v[0][c] * P, v[1][c] * P);
        w = fp8x2<true>(w, v[2][c] * P, v[3][c] * P);
        if (nonfinite) w = 0x7f7f7f7fu;
        *reinterpret_cast<uint32_t*>(o.q_col + (col + c) * o.M + r0 + 4 * lr) = w;
      }
    }
    if (col_ok) {
      const uint32_t w = lr < 4 ? packed0 : packed1;
      o.s_col[(col + lr) * (o.M / 32) + r0 / 32] = (uint8_t)(w >> (8 * (lr & 3)));
    }
  }
}

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

// 16 bytes at p, or zeros when !ok (a value select, so the operands stay in registers).
__device__ __forceinline__ uint4 ld16_if(const void* p, bool ok) {
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (ok) {
    u32x4 x;
    if constexpr (GLU_MX_NT_LOADS) x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    else x = *reinterpret_cast<const u32x4*>(p);
    v = make_uint4(x.x, x.y, x.z, x.w);
  }
  return v;
}

// Loads the lane's 4 rows of operands.  FULL: every row and column in range.
template <int LAYOUT, bool FULL>
__device__ __forceinline__ void load_rows(GU<LAYOUT> (&in)[4], const uint16_t* gate,
                                          const uint16_t* up, int64_t ld, int64_t row0,
                                          int64_t col, int64_t M, bool col_ok) {
  const int64_t off = row0 * ld + (LAYOUT == PAIRED ? 2 * col : col);
  const uint16_t* g = gate + off;
  const uint16_t* u = LAYOUT == SPLIT ? up + off : nullptr;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const bool ok = FULL || (col_ok && row0 + i < M);
    if constexpr (LAYOUT == SPLIT) {
      const uint4 G = ld16_if(g, ok), U = ld16_if(u, ok);
      in[i].a[0] = G.x; in[i].a[1] = G.y; in[i].a[2] = G.z; in[i].a[3] = G.w;
      in[i].b[0] = U.x; in[i].b[1] = U.y; in[i].b[2] = U.z; in[i].b[3] = U.w;
      u += ld;
    } else {
      const uint4 A = ld16_if(g, ok), B = ld16_if(g + 8, ok);
      in[i].a[0] = A.x; in[i].a[1] = A.y; in[i].a[2] = A.z; in[i].a[3] = A.w;
      in[i].a[4] = B.x; in[i].a[5] = B.y; in[i].a[6] = B.z; in[i].a[7] = B.w;
    }
    g += ld;
  }
}

template <int ACT, int LAYOUT, int FLAGS, int MODE, bool FULL>
__device__ __forceinline__ void mx_tile(const MxArgs& a, int64_t r0, int64_t col, int lr, int lc,
                                        bool col_ok) {
  const int64_t row0 = r0 + 4 * lr;
  if constexpr (MODE == MODE_F32) {
    float v[4][8];
    const float* x = static_cast<const float*>(a.src) + row0 * a.ld_in + col;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const bool ok = FULL || (col_ok && row0 + i < a.M);
      const uint4 A = ld16_if(x, ok), B = ld16_if(x + 4, ok);
      v[i][0] = __uint_as_float(A.x); v[i][1] = __uint_as_float(A.y);
      v[i][2] = __uint_as_float(A.z); v[i][3] = __uint_as_float(A.w);
      v[i][4] = __uint_as_float(B.x); v[i][5] = __uint_as_float(B.y);
      v[i][6] = __uint_as_float(B.z); v[i][7] = __uint_as_float(B.w);
      x += a.ld_in;
    }
    const MxOut o{a.q_row, a.s_row, a.q_col, a.s_col, a.M, a.N};
    mx_store_f32<FLAGS>(v, o, r0, col, lr, lc, col_ok);
  } else if constexpr (MODE == MODE_FWD) {
    GU<LAYOUT> in[4];
    load_rows<LAYOUT, FULL>(in, static_cast<const uint16_t*>(a.src), a.up, a.ld_in, row0, col, a.M,
                            col_ok);
    uint32_t H[4][4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      float g[8], u[8], h[8], zmin = 0.0f;
      unpack_gu<LAYOUT>(in[i], g, u);
#pragma unroll
      for (int c = 0; c < 8; c++) h[c] = glu_fwd_elem<ACT>(g[c], u[c], zmin);
      if (zmin < TAIL_ZL2) {  // rare: e^z below the FP32 normal range
#pragma unroll
        for (int c = 0; c < 8; c++)
          if (zl2<ACT>(g[c]) < TAIL_ZL2) h[c] = glu_fwd_tail<ACT>(g[c], u[c]);
      }
#pragma unroll
      for (int k = 0; k < 4; k++) H[i][k] = pack_bf16(h[2 * k], h[2 * k + 1]);
    }
    const MxOut o{a.q_row, a.s_row, a.q_col, a.s_col, a.M, a.N};
    mx_store_bf16<FLAGS, FULL>(H, o, r0, col, lr, lc, col_ok);
  } else {
    GU<SPLIT> in[4];
    load_rows<SPLIT, FULL>(in, static_cast<const uint16_t*>(a.src), a.up, a.ld_in, row0, col, a.M,
                           col_ok);
    uint32_t D[4][4];
    const uint16_t* dp = a.dh + row0 * a.ld_dh + col;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const uint4 d = ld16_if(dp, FULL || (col_ok && row0 + i < a.M));
      D[i][0] = d.x; D[i][1] = d.y; D[i][2] = d.z; D[i][3] = d.w;
      dp += a.ld_dh;
    }
    uint32_t HA[4][4], HB[4][4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      float g[8], u[8], d[8], da[8], db[8], zmin = 0.0f;
      unpack_gu<SPLIT>(in[i], g, u);
#pragma unroll
      for (int c = 0; c < 8; c++) {
        d[c] = (c & 1) ? bf_hi(D[i][c >> 1]) : bf_lo(D[i][c >> 1]);
        glu_bwd_elem<ACT>(g[c], u[c], d[c], da[c], db[c], zmin);
      }
      if (zmin < TAIL_ZL2) {  // rare: e^z below the FP32 normal range
#pragma unroll
        for (int c = 0; c < 8; c++)
          if (zl2<ACT>(g[c]) < TAIL_ZL2) glu_bwd_tail<ACT>(g[c], u[c], d[c], da[c], db[c]);
      }
#pragma unroll
      for (int k = 0; k < 4; k++) {
        HA[i][k] = pack_bf16(da[2 * k], da[2 * k + 1]);
        HB[i][k] = pack_bf16(db[2 * k], db[2 * k + 1]);
      }
    }
    const MxOut o{a.q_row, a.s_row, a.q_col, a.s_col, a.M, 2 * a.N};
    mx_store_bf16<FLAGS, FULL>(HA, o, r0, col, lr, lc, col_ok);
    mx_store_bf16<FLAGS, FULL>(HB, o, r0, a.N + col, lr, lc, col_ok);
  }
}

template <int ACT, int LAYOUT, int FLAGS, int MODE, int WGM, int WGN>
__global__ __launch_bounds__(64 * WGM * WGN) void k_mxfp8(MxArgs a, uint32_t tiles_m,
                                                          uint32_t ntiles, uint32_t per_xcd) {
  constexpr int TILE_M = 32 * WGM, TILE_N = 64 * WGN;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int lr = lane & 7, lc = lane >> 3;
  const uint32_t b = blockIdx.x;
  const uint32_t t = GLU_MX_TILE_ORDER == 2 ? b : (b & 7) * per_xcd + (b >> 3);
  if (t >= ntiles) return;
  uint32_t tm, tn;
  if constexpr (GLU_MX_TILE_ORDER == 0) {
    tn = t / tiles_m;
    tm = t - tn * tiles_m;
  } else {
    const uint32_t tiles_n = ntiles / tiles_m;
    tm = t / tiles_n;
    tn = t - tm * tiles_n;
  }
  const int64_t r0 = (int64_t)tm * TILE_M + 32 * (w % WGM);
  const int64_t cw = (int64_t)tn * TILE_N + 64 * (w / WGM);
  if (r0 >= a.M || cw >= a.N) return;  // wave-uniform
  const int64_t col = cw + 8 * lc;
  const bool col_ok = col < a.N;
  if (r0 + 32 <= a.M && cw + 64 <= a.N)  // wave-uniform
    mx_tile<ACT, LAYOUT, FLAGS, MODE, true>(a, r0, col, lr, lc, col_ok);
  else
    mx_tile<ACT, LAYOUT, FLAGS, MODE, false>(a, r0, col, lr, lc, col_ok);
}

template <int ACT, int LAYOUT, int FLAGS, int MODE>
hipError_t launch(const MxArgs& a, hipStream_t s) {
  constexpr int WGM = WgShape<MODE, FLAGS>::M, WGN = WgShape<MODE, FLAGS>::N;
  constexpr int TILE_M = 32 * WGM, TILE_N = 64 * WGN;
  const int64_t tiles_m = (a.M + TILE_M - 1) / TILE_M;
  const int64_t tiles_n = (a.N + TILE_N - 1) / TILE_N;
  const int64_t ntiles = tiles_m * tiles_n;
  const int64_t per_xcd = (ntiles + 7) / 8;
  const dim3 grid((unsigned)(8 * per_xcd)), block(64 * WGM * WGN);
  constexpr int LDS = WgShape<MODE, FLAGS>::LDS;
  auto k = k_mxfp8<ACT, LAYOUT, FLAGS, MODE, WGM, WGN>;
  if constexpr (LDS > 65536) {
    const hipError_t e =
        hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, LDS);
    if (e != hipSuccess) return e;
  }
  return launch_kernel_shm(k, grid, block, LDS, s, a, (uint32_t)tiles_m, (uint32_t)ntiles,
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
