// Fused GLU + MXFP8 quantization, forward and backward, rowwise / colwise / both from one
// read of the inputs ("Add swiglu + MXFP8 fused CuTe DSL kernel", Summary and API), and
// the FP32 quantizer hook that runs the same block rules on given FP32 values.
//
// Work decomposition (wave64):
//   A workgroup owns a TM x TN tile of the quantized matrix (of each of da and db in the
//   backward): 128 x 128 with 4 x 2 waves, or, when only rowwise codes are written, a band
//   of 32 rows 512 (forward) or 256 (backward) columns wide with 1 x 8 or 1 x 4 waves.  A
//   wave covers 32 rows x 64 columns: one 32-row colwise block row and
//   two 32-column rowwise blocks per row.  Lane = lr + 8*lc owns rows 4lr..4lr+3 and columns
//   8lc..8lc+7 of the wave's piece: 16-byte loads per row and per operand, 32 elements per
//   lane, kept after the activation as 16 packed BF16 pairs.
//   Rowwise amax of a 32-column block spans the 4 lanes lc = 4b..4b+3 (lane bits 3, 4):
//   DPP row_ror:8 then ds_swizzle xor 16.  Colwise amax of a 32-row block spans the 8
//   lanes lr = 0..7 (lane bits 0..2) after an in-lane max over 4 rows: DPP quad_perm xor 1,
//   xor 2, then row_half_mirror.  Maxima are taken on packed 16-bit magnitudes (two
//   columns, or two rows, per instruction).
//   Codes and scales are staged in LDS and leave, after one workgroup barrier, as 16-byte
//   stores that fill whole 128-byte lines (the backward stages da, writes it out, then
//   stages db in the same LDS): a tile row of rowwise codes and a tile column of
//   colwise codes are 128 bytes each (colwise output always uses 128-row tiles), and the
//   scales of a tile row (column) are one 4-byte word.  Straight from the registers the same
//   data would leave as 32-byte (colwise) and 64-byte (rowwise) pieces and single scale
//   bytes: several times more L2 write requests, which measured as the limit once enough
//   tiles run concurrently to keep HBM busy.
//   Straight from the registers, 32- and 64-byte pieces also measured 20-60% slower than
//   whole lines in a skeleton with the same loads and no arithmetic.
//   Tiles follow an order chosen per direction (below); a launch that writes scale words of
//   both directions gives each XCD a contiguous run of it, so tiles that share scale sectors
//   run on one XCD at about the same time.
//   Rowwise-only launches with row-major scales and N % 128 == 0 go to a second kernel,
//   k_mxfp8_row, which needs no LDS: one row per wave, one 16-byte load per operand per lane
//   (further below).
#include "glu_device.h"
#include "glu_launch.h"

namespace glu {
namespace {

enum { MODE_FWD = 0, MODE_BWD = 1, MODE_F32 = 2 };

// Tile of the quantized matrix per workgroup: WM x WN waves, each covering 32 x 64 elements.
// Every code line leaves as 128 bytes: rowwise codes need TN = 128, colwise codes TM = 128.
template <int WM_, int WN_>
struct Tile {
  static constexpr int WM = WM_, WN = WN_;
  static constexpr int TM = 32 * WM, TN = 64 * WN;
  static constexpr int NTHREADS = 64 * WM * WN;
  static constexpr int RSEG = TN / 16, CSEG = TM / 16;  // 16-byte segments per code line
  // order-2 block: the tiles of a block that share rows (columns) fill one 32-byte sector of
  // rowwise (colwise) scale words, TN / 32 (TM / 32) bytes per tile
  static constexpr int BM = 32 / (TM / 32), BN = 32 / (TN / 32);
  static_assert(TM >= 32 && TM <= 128 && TN >= 128 && TN <= 1024 && NTHREADS <= 1024,
                "shapes the swizzles and scale words fit");
};

// Tile per kernel, from interleaved measurements at [16384, 7168].  Rowwise only (the launches
// k_mxfp8_row does not take): a band of 32 rows, 512 columns wide in the forward (102 vs 110 us
// with 64 x 128; 984 vs 1043 us at [131072, 8192]) and 256 wide in the backward (158 vs 169
// us), so each workgroup reads and writes long runs of its rows.  With colwise output,
// 128 x 128 (128 x 64 and 128 x 256 were slower).
template <int FLAGS, int MODE>
using TileOf = Tile<FLAGS == ROWWISE ? 1 : 4, FLAGS == ROWWISE ? (MODE == MODE_BWD ? 4 : 8) : 2>;

// Where a launch's code stores go, and how its workgroups map to tiles; both are uniform
// kernel arguments chosen per launch from measurements (SwiGLU, cold inputs, us).
//   Non-temporal code stores.  Ordinary stores are absorbed by the 256 MB last-level cache
//   and drain after the kernel while the codes fit there:
//     tiled kernel, [16384, 7168]: forward both (235 MB) 126.2 ordinary vs 137.0
//     non-temporal, backward both (470 MB) 234 vs 267 the other way, backward rowwise
//     (235 MB, k_mxfp8_row) 146.7 vs 152.4, [131072, 8192] forward both (2.1 GB) 1368 vs 1211;
//   so the size decides, at 256 MiB.  Two launches stream their codes whatever the size:
//     forward rowwise (k_mxfp8_row): [16384, 7168] 95.7 non-temporal vs 101.8 ordinary,
//     [131072, 8192] 843.6 vs 857.2;
//     forward colwise only: [16384, 7168] 105.1 vs 107.0.
//   Tile mapping.  Workgroups are dealt to the XCDs round-robin by id.  Consecutive ids on
//   consecutive positions of the tile order keep the whole chip on one region of the
//   operands, as a streaming copy does, which is faster for pure streams; a contiguous run of
//   the order per XCD instead keeps the tiles that share scale words on one L2, which the
//   launches writing rowwise and colwise scale words together need:
//     forward colwise only, [16384, 7168]: 105.1 round-robin vs 109.8 per-XCD runs;
//     forward both: 127.7 per-XCD runs vs 134.0; backward both 229.2 vs 234.6.
//   With 128x4 scales a rowwise-only tile writes whole scale lines of its own, and
//   round-robin is faster there: forward 99.0 vs 102.3, backward 150.4 vs 155.6; launches
//   with both scalings keep per-XCD runs (forward 123.7 vs 128.4 round-robin, backward
//   223.9 vs 226.0).
constexpr int64_t kNtStoreBytes = 256ll << 20;
struct LaunchPolicy {
  uint32_t nt;        // non-temporal code stores
  uint32_t xcd_runs;  // each XCD takes a contiguous run of the tile (unit) order
};
// row_kernel: the launch goes to k_mxfp8_row (rowwise only, further below); swizzled: the
// scales are written in the 128x4 layout.
LaunchPolicy launch_policy(int flags, int mode, int64_t code_bytes, bool row_kernel, bool swizzled) {
  const bool streamed = mode == MODE_FWD && (row_kernel || (flags & (ROWWISE | COLWISE)) == COLWISE);
  LaunchPolicy p;
  p.nt = streamed || code_bytes > kNtStoreBytes;
  p.xcd_runs = !streamed && !(swizzled && (flags & (ROWWISE | COLWISE)) == ROWWISE);
  return p;
}

// Order of the tiles:
//   0 (colwise only): along M first, so consecutive tiles continue the same rows of the
//     transposed [N, M] output and fill its scale rows word after word.
//   1 (rowwise only): along N first, so consecutive tiles continue the same input and output
//     rows and fill the rowwise scale rows word after word (about 3% faster at [16384, 7168]).
//   2 (both): strips of BN tile columns; in a strip, blocks of BM x BN tiles going down M; in
//     a block, along M first.  The tiles of a block that share rows (columns) write their
//     rowwise (colwise) scale words into one 32-byte sector within the same window of
//     concurrent tiles, so both scale streams leave L2 as whole sectors (orders 0 and 1 leave
//     one of them as single words: 6% slower at [16384, 7168]; blocks of 4 x 4 or 16 x 16
//     128 x 128 tiles were 8% and 2% slower than 8 x 8).
// One tile per workgroup: a workgroup that prefetched its next tile during the write-out was
// slower (forward both 179 vs 128 us, backward both 288 vs 227 us at [16384, 7168]).
template <int FLAGS>
constexpr int tile_order() {
  return FLAGS == ROWWISE ? 1 : FLAGS == COLWISE ? 0 : 2;
}

template <class T, int ORDER>
__device__ __forceinline__ void tile_of(uint32_t t, uint32_t tiles_m, uint32_t tiles_n,
                                        uint32_t& tm, uint32_t& tn) {
  if constexpr (ORDER == 0) {
    tn = t / tiles_m;
    tm = t - tn * tiles_m;
  } else if constexpr (ORDER == 1) {
    tm = t / tiles_n;
    tn = t - tm * tiles_n;
  } else {
    constexpr uint32_t BM = T::BM, BN = T::BN;
    const uint32_t strip = tiles_m * BN;  // tiles per full strip
    const uint32_t bj = t / strip, u = t - bj * strip;
    const uint32_t w = tiles_n - bj * BN < BN ? tiles_n - bj * BN : BN;  // strip width
    const uint32_t bi = u / (BM * w), v = u - bi * BM * w;
    const uint32_t h = tiles_m - bi * BM < BM ? tiles_m - bi * BM : BM;  // block height
    const uint32_t j = v / h;
    tm = bi * BM + (v - j * h);
    tn = bj * BN + j;
  }
}

// Packed E8M0 RCEIL scale bytes from packed BF16 magnitudes A = E << 7 | m of finite block
// maxima: e + 127 = E - 8 + (m > 0x60), i.e. ((A + 0x1F) >> 7) - 8 saturated at 0.
__device__ __forceinline__ uint32_t pk_scale_bytes(uint32_t A) {
  const u16x2 t = (as_u16x2(A) + (u16x2){0x1f, 0x1f}) >> (u16x2){7, 7};
  return as_u32(__builtin_elementwise_sub_sat(t, (u16x2){8, 8}));
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

// Operands are read with raw buffer loads through a descriptor whose base is the first byte
// of a wave's piece (a wave-uniform address).  A lane whose element is outside the matrix
// passes kOob as its offset; the hardware's range check turns that load into zeros, so every
// path through a tile issues the same loads, with no branch and no select.  Row pitches are
// limited (by the host checks) so that 32 rows of offsets stay below kOob.

__device__ __forceinline__ void bld16(uint32_t (&w)[4], __amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2);  // non-temporal
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

// Largest raw gate bit pattern of the lane's operands, as an unsigned 16-bit number (the
// argument of tail_possible).
template <int LAYOUT>
__device__ __forceinline__ uint32_t gate_max16(const GU<LAYOUT> (&in)[4]) {
  uint32_t m = in[0].a[0];
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int k = 0; k < (LAYOUT == SPLIT ? 4 : 8); k++)
      if (i || k) m = pkmax(m, in[i].a[k]);
  return LAYOUT == SPLIT ? umax(lo16(m), hi16(m)) : lo16(m);  // paired: gate is the low half
}

template <int ACT, int LAYOUT, int MODE>
__device__ __forceinline__ void compute(TileVals<MODE>& r, const TileOps<LAYOUT, MODE>& o) {
  if constexpr (MODE == MODE_F32) {
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
      for (int c = 0; c < 8; c++) r.v[i][c] = __uint_as_float(o.x[i][c]);
  } else if constexpr (MODE == MODE_FWD) {
    bool tail = false;
    if constexpr (tail_from_gate_bits<ACT>()) tail = tail_possible<ACT>(gate_max16<LAYOUT>(o.in));
#pragma unroll
    for (int i = 0; i < 4; i++) {
      float gg[8], u[8], h[8];
      unpack_gu<LAYOUT>(o.in[i], gg, u);
#pragma unroll
      for (int c = 0; c < 8; c++) {
        h[c] = glu_fwd_fast<ACT>(gg[c], u[c]);
        if constexpr (!tail_from_gate_bits<ACT>()) tail |= fwd_tail_needed<ACT>(gg[c], u[c]);
      }
      if (tail) {  // rare: some element may need the FP64 tail path
#pragma unroll
        for (int c = 0; c < 8; c++)
          if (fwd_tail_needed<ACT>(gg[c], u[c])) h[c] = glu_fwd_tail<ACT>(gg[c], u[c]);
      }
#pragma unroll
      for (int k = 0; k < 4; k++) r.h[0][i][k] = pack_bf16(h[2 * k], h[2 * k + 1]);
    }
  } else {
    // Each row is packed to BF16 right after its fast path, and the rare tail elements then
    // overwrite their halves of the packed words (recomputed from the raw operand words), so
    // no FP32 result outlives its row.  The empty asm keeps the compiler from sinking the
    // packs of db past da's staging (it would hold 32 FP32 values instead of 16 words), and
    // the scheduling barriers keep the halves and rows in order.  SwiGLU at [16384, 7168]:
    // 102 -> 83 VGPRs and 228 -> 226 us (both), 100 -> 80 VGPRs and 174 -> 167 us (colwise
    // only); without the barriers the same VGPRs and 232 and 170 us.
    bool tail = false;
    if constexpr (tail_from_gate_bits<ACT>()) tail = tail_possible<ACT>(gate_max16<SPLIT>(o.in));
#pragma unroll
    for (int i = 0; i < 4; i++) {
      float gg[8], u[8], d[8], da[8], db[8];
      unpack_gu<SPLIT>(o.in[i], gg, u);
      bool rt = tail;
#pragma unroll
      for (int half = 0; half < 2; half++) {  // 4 elements, then their 2 packed words
#pragma unroll
        for (int c = 4 * half; c < 4 * half + 4; c++) {
          d[c] = (c & 1) ? bf_hi(o.d[i][c >> 1]) : bf_lo(o.d[i][c >> 1]);
          glu_bwd_fast<ACT>(gg[c], u[c], d[c], da[c], db[c]);
          if constexpr (!tail_from_gate_bits<ACT>()) rt |= bwd_tail_needed<ACT>(gg[c], u[c], d[c]);
        }
#pragma unroll
        for (int k = 2 * half; k < 2 * half + 2; k++) {
          r.h[0][i][k] = pack_bf16(da[2 * k], da[2 * k + 1]);
          r.h[1][i][k] = pack_bf16(db[2 * k], db[2 * k + 1]);
          asm volatile("" : "+v"(r.h[0][i][k]), "+v"(r.h[1][i][k]));
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (rt) {  // rare: some element may need the FP64 tail path
#pragma unroll
        for (int c = 0; c < 8; c++) {
          const int k = c >> 1;
          const float g1 = (c & 1) ? bf_hi(o.in[i].a[k]) : bf_lo(o.in[i].a[k]);
          const float u1 = (c & 1) ? bf_hi(o.in[i].b[k]) : bf_lo(o.in[i].b[k]);
          const float d1 = (c & 1) ? bf_hi(o.d[i][k]) : bf_lo(o.d[i][k]);
          if (bwd_tail_needed<ACT>(g1, u1, d1)) {
            float ta, tb;
            glu_bwd_tail<ACT>(g1, u1, d1, ta, tb);
            const uint32_t keep = (c & 1) ? 0x0000ffffu : 0xffff0000u;  // the other element's half
            r.h[0][i][k] = (r.h[0][i][k] & keep) | (pack_bf16(ta, ta) & ~keep);
            r.h[1][i][k] = (r.h[1][i][k] & keep) | (pack_bf16(tb, tb) & ~keep);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// LDS staging of one quantized part (the tile of h, or of da or db):
//   rq  rowwise codes [TM][TN], row-major;      rs  rowwise scales [TM][TN/32];
//   cq  colwise codes [TN][TM], column-major;   cs  colwise scales [TN][TM/32].
// The 16-byte segments of each code row (rq) and column (cq) are XOR-swizzled, by row / 4
// and column / 8 modulo the segments per line, so that the staging writes of a wave (8 rows 4 apart,
// or 8 columns 8 apart, at the same offset) and the 16-byte reads of the write-out fall in
// different banks.
template <class T, int FLAGS>
struct Stage {
  static constexpr int RQ = (FLAGS & ROWWISE) ? T::TM * T::TN : 0;
  static constexpr int CQ = (FLAGS & COLWISE) ? T::TN * T::TM : 0;
  static constexpr int RS = (FLAGS & ROWWISE) ? T::TM * (T::TN / 32) : 0;
  static constexpr int CS = (FLAGS & COLWISE) ? T::TN * (T::TM / 32) : 0;
  static constexpr int BYTES = RQ + CQ + RS + CS;
  uint8_t* rq;
  uint8_t* cq;
  uint8_t* rs;
  uint8_t* cs;
  __device__ explicit Stage(uint8_t* base)
      : rq(base), cq(base + RQ), rs(base + RQ + CQ), cs(base + RQ + CQ + RS) {}
};

// Byte offsets in rq of (row, col) and in cq of (col, row), within a 16-byte segment.
template <class T>
__device__ __forceinline__ int rq_at(int row, int col) {
  return row * T::TN + 16 * ((col >> 4) ^ ((row >> 2) & (T::RSEG - 1))) + (col & 15);
}
template <class T>
__device__ __forceinline__ int cq_at(int col, int row) {
  return col * T::TM + 16 * ((row >> 4) ^ ((col >> 3) & (T::CSEG - 1))) + (row & 15);
}

__device__ __forceinline__ void lds_st8(uint8_t* p, uint32_t w0, uint32_t w1) {
  *reinterpret_cast<u32x2*>(p) = (u32x2){w0, w1};
}
__device__ __forceinline__ void lds_st4(uint8_t* p, uint32_t w) { *reinterpret_cast<uint32_t*>(p) = w; }

// A[i][k] = H[i][k] with the sign bits cleared (packed BF16 magnitudes).
template <class T, int FLAGS>
__device__ __forceinline__ void stage_rows(const uint32_t (&H)[4][4], const uint32_t (&A)[4][4],
                                          const Stage<T, FLAGS>& st, int row0, int col, int lc) {
  uint32_t m[4];
#pragma unroll
  for (int i = 0; i < 4; i++) m[i] = pkmax(pkmax(A[i][0], A[i][1]), pkmax(A[i][2], A[i][3]));
  uint32_t R01 = pkmax(pair_lo(m[0], m[1]), pair_hi(m[0], m[1]));  // rows (0,1) packed
  uint32_t R23 = pkmax(pair_lo(m[2], m[3]), pair_hi(m[2], m[3]));  // rows (2,3) packed
  R01 = pkmax(R01, dpp<DPP_ROW_ROR8>(R01));
  R23 = pkmax(R23, dpp<DPP_ROW_ROR8>(R23));
  R01 = pkmax(R01, swz_xor16(R01));
  R23 = pkmax(R23, swz_xor16(R23));

  const uint32_t S01 = pk_scale_bytes(R01), S23 = pk_scale_bytes(R23);
  const uint32_t sb[4] = {lo16(S01), hi16(S01), lo16(S23), hi16(S23)};
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const float sc = e8m0_value(sb[i]);
    uint32_t w0 = fp8x2_scaled<false>(0u, H[i][0], sc);
    w0 = fp8x2_scaled<true>(w0, H[i][1], sc);
    uint32_t w1 = fp8x2_scaled<false>(0u, H[i][2], sc);
    w1 = fp8x2_scaled<true>(w1, H[i][3], sc);
    lds_st8(st.rq + rq_at<T>(row0 + i, col), w0, w1);
  }
  // lane lc = 4b + i stages the scale of row 4lr + i in the wave's block b
  const int i = lc & 3;
  const uint32_t w = i < 2 ? S01 : S23;
  st.rs[(row0 + i) * (T::TN / 32) + ((col - 8 * i) >> 5)] = (uint8_t)((i & 1) ? hi16(w) : lo16(w));

  const uint32_t rm = pkmax(R01, R23);
  if (umax(lo16(rm), hi16(rm)) >= 0x7f80u) {
    // a block holding NaN or Inf: scale 0xFF, every code 0x7F (overwrites the fast path; each
    // lane patches only what it staged itself, so program order suffices)
    const uint32_t rmax[4] = {lo16(R01), hi16(R01), lo16(R23), hi16(R23)};
#pragma unroll
    for (int r = 0; r < 4; r++) {
      if (rmax[r] >= 0x7f80u) {
        lds_st8(st.rq + rq_at<T>(row0 + r, col), 0x7f7f7f7fu, 0x7f7f7f7fu);
        if ((lc & 3) == r) st.rs[(row0 + r) * (T::TN / 32) + ((col - 8 * r) >> 5)] = 0xff;
      }
    }
  }
}

template <class T, int FLAGS>
__device__ __forceinline__ void stage_cols(const uint32_t (&H)[4][4], const uint32_t (&A)[4][4],
                                          const Stage<T, FLAGS>& st, int row0, int col, int lr) {
  uint32_t C[4];  // column block maxima, columns (2k, 2k+1) packed
#pragma unroll
  for (int k = 0; k < 4; k++) {
    uint32_t c = pkmax(pkmax(A[0][k], A[1][k]), pkmax(A[2][k], A[3][k]));
    c = pkmax(c, dpp<DPP_XOR1>(c));
    c = pkmax(c, dpp<DPP_XOR2>(c));
    C[k] = pkmax(c, dpp<DPP_HALF_MIRROR>(c));
  }
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
    lds_st4(st.cq + cq_at<T>(col + 2 * k, row0), w0);
    lds_st4(st.cq + cq_at<T>(col + 2 * k + 1, row0), w1);
  }
  // lane lr stages the scale of column 8lc + lr of this 32-row block
  const uint32_t w = (lr >> 1) == 0 ? S[0] : (lr >> 1) == 1 ? S[1] : (lr >> 1) == 2 ? S[2] : S[3];
  st.cs[(col + lr) * (T::TM / 32) + (row0 >> 5)] = (uint8_t)((lr & 1) ? hi16(w) : lo16(w));

  const uint32_t cm = pkmax(pkmax(C[0], C[1]), pkmax(C[2], C[3]));
  if (umax(lo16(cm), hi16(cm)) >= 0x7f80u) {
    // a block holding NaN or Inf: scale 0xFF, every code 0x7F (as for the rows)
#pragma unroll
    for (int c = 0; c < 8; c++) {
      const uint32_t cmax = (c & 1) ? hi16(C[c >> 1]) : lo16(C[c >> 1]);
      if (cmax >= 0x7f80u) {
        lds_st4(st.cq + cq_at<T>(col + c, row0), 0x7f7f7f7fu);
        if (lr == c) st.cs[(col + c) * (T::TM / 32) + (row0 >> 5)] = 0xff;
      }
    }
  }
}

// Quantizes the lane's 4x8 BF16 values H[i][k] = (columns 2k, 2k+1 of tile row row0 + i),
// tile columns col..col+7 (row0 = 32wm + 4lr, col = 64wn + 8lc), into the LDS stage.  All
// 64 lanes of the wave take part (cross-lane maxima).  Elements outside the matrix were
// loaded as zeros: they form blocks of their own (N and, when colwise, M are multiples of
// 32), quantize to zero codes and are never written out.
template <class T, int FLAGS>
__device__ __forceinline__ void stage_bf16(const uint32_t (&H)[4][4], const Stage<T, FLAGS>& st,
                                           int row0, int col, int lr, int lc) {
  uint32_t A[4][4];
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int k = 0; k < 4; k++) A[i][k] = H[i][k] & 0x7fff7fffu;
  if constexpr ((FLAGS & ROWWISE) != 0) stage_rows<T, FLAGS>(H, A, st, row0, col, lc);
  if constexpr ((FLAGS & COLWISE) != 0) stage_cols<T, FLAGS>(H, A, st, row0, col, lr);
}

// The same rules on FP32 values (quantizer hook): magnitudes compared as FP32 bits, the
// scaled value x * 2^-e computed exactly in FP32, then v_cvt_pk_fp8_f32.
template <class T, int FLAGS>
__device__ __forceinline__ void stage_f32(const float (&v)[4][8], const Stage<T, FLAGS>& st,
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
      lds_st8(st.rq + rq_at<T>(row0 + i, col), w0, w1);
    }
    const int i = lc & 3;
    st.rs[(row0 + i) * (T::TN / 32) + ((col - 8 * i) >> 5)] = (uint8_t)(packed >> (8 * i));
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
      lds_st4(st.cq + cq_at<T>(col + c, row0), w);
    }
    const uint32_t w = lr < 4 ? packed0 : packed1;
    st.cs[(col + lr) * (T::TM / 32) + (row0 >> 5)] = (uint8_t)(w >> (8 * (lr & 3)));
  }
}

// Scale words in the zero-padded 128x4 layout (GLU_SF_SWIZZLED).  The scale matrix of a
// direction is [rows, nb] (rowwise: [M, ldq/32]; colwise: [ldq, M/32]), padded to
// Rp = ceil(rows/128)*128 and Cp = ceil(nb/4)*4; scale (r, c) sits at sf128x4_offset(r, c, Cp).
// A tile's 4 consecutive blocks of one row (or column) of the quantized matrix are one aligned
// 4-byte group there.  Offsets are taken from the start of the tile's first 128-row band of the
// scale matrix, so they stay small.  Padding bytes are written as zeros: blocks outside the
// matrix were staged as zero scales, and the launch adds tiles where the padding reaches past
// the last tile (see launch).  In the backward, a run of da's last scale columns that would
// reach into db's is written byte by byte, only da's bytes, and so are db's runs when its
// first scale column is not a multiple of 4.
template <class T, int FLAGS>
__device__ __forceinline__ void write_row_scales_128x4(const Stage<T, FLAGS>& st, const MxArgs& a,
                                                       int64_t r0, int64_t c0, int64_t coloff,
                                                       int64_t ldq, int tid) {
  constexpr int TM = T::TM, NB = T::TN / 32;
  const int64_t nbt = ldq / 32, cp = (nbt + 3) / 4 * 4, rp = (a.M + 127) / 128 * 128;
  const int64_t part_end = (coloff + a.N) / 32;  // blocks of this part end here
  const bool last = coloff + a.N == ldq;          // padding columns follow this part
  const int64_t band0 = r0 / 128 * (cp / 4) * 512;
  const auto sout = rsrc(a.s_row + band0);
  const int row = tid < TM ? tid : 0;
  const int64_t gr = r0 + row;
  const bool row_ok = tid < TM && gr < rp;
  // db's first block is 4-aligned only when N % 128 == 0; a misaligned run of 4 blocks spans
  // two groups of the layout, so it goes byte by byte
  const bool aligned = ((coloff / 32) & 3) == 0;
#pragma unroll
  for (int g = 0; g < NB / 4; g++) {
    const int64_t b = (coloff + c0) / 32 + 4 * g;
    const uint8_t* src = st.rs + row * NB + 4 * g;
    if (aligned && (b + 4 <= part_end || (last && b < cp))) {
      const uint32_t off = (uint32_t)(sf128x4_offset(gr, b, cp) - band0);
      __builtin_amdgcn_raw_buffer_store_b32(*reinterpret_cast<const uint32_t*>(src), sout,
                                            row_ok ? off : kOob, 0, 0);
    } else {
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const int64_t bj = b + j;
        const bool ok = row_ok && (bj < part_end || (last && bj < cp));
        const uint32_t off = (uint32_t)(sf128x4_offset(gr, bj, cp) - band0);
        __builtin_amdgcn_raw_buffer_store_b8(src[j], sout, ok ? off : kOob, 0, 0);
      }
    }
  }
}

template <class T, int FLAGS>
__device__ __forceinline__ void write_col_scales_128x4(const Stage<T, FLAGS>& st, const MxArgs& a,
                                                       int64_t r0, int64_t c0, int64_t coloff,
                                                       int64_t ldq, int tid) {
  constexpr int TN = T::TN;
  static_assert(T::TM == 128, "one 4-byte group of colwise scales per tile column");
  const int64_t cp = (a.M / 32 + 3) / 4 * 4, rp = (ldq + 127) / 128 * 128;
  const bool last = coloff + a.N == ldq;
  const int64_t band0 = (coloff + c0) / 128 * (cp / 4) * 512;
  const auto sout = rsrc(a.s_col + band0);
  const int col = tid < TN ? tid : 0;
  const int64_t gc = coloff + c0 + col;  // row of the colwise scale matrix
  const bool ok = tid < TN && (c0 + col < a.N || (last && gc < rp));
  const uint32_t off = (uint32_t)(sf128x4_offset(gc, r0 / 32, cp) - band0);
  __builtin_amdgcn_raw_buffer_store_b32(*reinterpret_cast<const uint32_t*>(st.cs + col * 4), sout,
                                        ok ? off : kOob, 0, 0);
}

// Writes a staged part to global memory: the part is the [M, N] matrix at column offset
// `coloff` of the quantized matrix, whose rows hold ldq codes; the tile starts at (r0, c0).
// Stores are raw buffer stores through descriptors based at the tile's first byte (scalar
// address arithmetic), with 32-bit lane offsets; a store outside the matrix gets kOob as its
// offset and the hardware's range check drops it.  Rows >= M and columns >= N fall out in
// whole 16-byte segments (N and, when colwise, M are multiples of 32).  The host checks keep
// 128 rows of either output's pitch below kOob.  Scale words are written whole where they are
// 4-byte aligned and in range, else byte by byte.
template <class T, int FLAGS, bool NT>
__device__ __forceinline__ void write_rows(const Stage<T, FLAGS>& st, const MxArgs& a, int64_t r0,
                                          int64_t c0, int64_t coloff, int64_t ldq, int tid,
                                          bool swz) {
  constexpr int AUX = NT ? 2 : 0;
  const int64_t M = a.M, N = a.N;
  constexpr int TM = T::TM, TN = T::TN, NTHREADS = T::NTHREADS, RSEG = T::RSEG, CSEG = T::CSEG;
  const int rows = M - r0 < TM ? (int)(M - r0) : TM;  // rows of the tile inside the part
  const int cols = N - c0 < TN ? (int)(N - c0) : TN;  // columns of the tile inside the part
  // thread -> (line, 16-byte segment) of a code line; two lines per thread
  static_assert(TM * RSEG == 2 * NTHREADS && TN * CSEG == 2 * NTHREADS, "two lines per thread");
  if constexpr ((FLAGS & ROWWISE) != 0) {
    const auto out = rsrc(a.q_row + r0 * ldq + coloff + c0);
    const uint32_t pitch = (uint32_t)ldq;
    const int line = tid / RSEG, seg = tid % RSEG;
    const bool seg_ok = 16 * seg < cols;
#pragma unroll
    for (int i = 0; i < 2; i++) {
      const int row = line + (NTHREADS / RSEG) * i;
      const u32x4 v = *reinterpret_cast<const u32x4*>(st.rq + row * TN + 16 * (seg ^ ((row >> 2) & (RSEG - 1))));
      const uint32_t off = seg_ok && row < rows ? (uint32_t)row * pitch + 16u * seg : kOob;
      __builtin_amdgcn_raw_buffer_store_b128(v, out, off, 0, AUX);
    }
    if (swz) {
      write_row_scales_128x4<T, FLAGS>(st, a, r0, c0, coloff, ldq, tid);
      return;
    }
    // scale words: thread `row` < TM writes the TN/32 scales of tile row `row`
    const int64_t nb = ldq / 32;
    const auto sout = rsrc(a.s_row + r0 * nb + (coloff + c0) / 32);
    const int row = tid < TM ? tid : 0;
    const bool row_ok = tid < TM && row < rows;
    const uint32_t base = (uint32_t)row * (uint32_t)nb;
    constexpr int NB = TN / 32;  // scale bytes per tile row
    const bool whole = nb % NB == 0 && (coloff / 32) % NB == 0 && cols == TN;
    if (whole) {
      const uint8_t* src = st.rs + row * NB;
      const uint32_t o = row_ok ? base : kOob;
      if constexpr (NB == 4) {
        __builtin_amdgcn_raw_buffer_store_b32(*reinterpret_cast<const uint32_t*>(src), sout, o, 0, 0);
      } else if constexpr (NB == 8) {
        __builtin_amdgcn_raw_buffer_store_b64(*reinterpret_cast<const u32x2*>(src), sout, o, 0, 0);
      } else {
#pragma unroll
        for (int h = 0; h < NB / 16; h++)
          __builtin_amdgcn_raw_buffer_store_b128(*reinterpret_cast<const u32x4*>(src + 16 * h), sout,
                                                 row_ok ? base + 16 * h : kOob, 0, 0);
      }
    } else {
#pragma unroll
      for (int b = 0; b < NB; b++)
        __builtin_amdgcn_raw_buffer_store_b8(st.rs[row * NB + b], sout,
                                             row_ok && 32 * b < cols ? base + b : kOob, 0, 0);
    }
  }
}

template <class T, int FLAGS, bool NT>
__device__ __forceinline__ void write_cols(const Stage<T, FLAGS>& st, const MxArgs& a, int64_t r0,
                                          int64_t c0, int64_t coloff, int64_t ldq, int tid,
                                          bool swz) {
  constexpr int AUX = NT ? 2 : 0;
  const int64_t M = a.M, N = a.N;
  constexpr int TM = T::TM, TN = T::TN, NTHREADS = T::NTHREADS, RSEG = T::RSEG, CSEG = T::CSEG;
  const int rows = M - r0 < TM ? (int)(M - r0) : TM;  // rows of the tile inside the part
  const int cols = N - c0 < TN ? (int)(N - c0) : TN;  // columns of the tile inside the part
  // thread -> (line, 16-byte segment) of a code line; two lines per thread
  static_assert(TM * RSEG == 2 * NTHREADS && TN * CSEG == 2 * NTHREADS, "two lines per thread");
  if constexpr ((FLAGS & COLWISE) != 0) {
    static_assert(TM == 128, "colwise code lines and scale words are 128 rows long");
    const auto out = rsrc(a.q_col + (coloff + c0) * M + r0);
    const uint32_t pitch = (uint32_t)M;
    const int line = tid / CSEG, seg = tid % CSEG;
    const bool seg_ok = 16 * seg < rows;
#pragma unroll
    for (int i = 0; i < 2; i++) {
      const int col = line + (NTHREADS / CSEG) * i;
      const u32x4 v = *reinterpret_cast<const u32x4*>(st.cq + col * TM + 16 * (seg ^ ((col >> 3) & (CSEG - 1))));
      const uint32_t off = seg_ok && col < cols ? (uint32_t)col * pitch + 16u * seg : kOob;
      __builtin_amdgcn_raw_buffer_store_b128(v, out, off, 0, AUX);
    }
    // scale words: thread `col` < TN writes the TM/32 scales of tile column `col`
    if (swz) {
      write_col_scales_128x4<T, FLAGS>(st, a, r0, c0, coloff, ldq, tid);
      return;
    }
    const int64_t nb = M / 32;
    const auto sout = rsrc(a.s_col + (coloff + c0) * nb + r0 / 32);
    const int col = tid < TN ? tid : 0;
    const bool col_ok = tid < TN && col < cols;
    const uint32_t base = (uint32_t)col * (uint32_t)nb;
    const bool whole = nb % 4 == 0 && rows == TM;
    if (whole) {
      const uint32_t w = *reinterpret_cast<const uint32_t*>(st.cs + col * (TM / 32));
      __builtin_amdgcn_raw_buffer_store_b32(w, sout, col_ok ? base : kOob, 0, 0);
    } else {
#pragma unroll
      for (int b = 0; b < TM / 32; b++)
        __builtin_amdgcn_raw_buffer_store_b8(st.cs[col * (TM / 32) + b], sout,
                                             col_ok && 32 * b < rows ? base + b : kOob, 0, 0);
    }
  }
}

template <class T, int FLAGS, bool NT>
__device__ __forceinline__ void write_out(const Stage<T, FLAGS>& st, const MxArgs& a, int64_t r0,
                                          int64_t c0, int64_t coloff, int64_t ldq, int tid) {
  const bool swz = (a.flags & SF_SWIZZLED) != 0;
  write_rows<T, FLAGS, NT>(st, a, r0, c0, coloff, ldq, tid, swz);
  write_cols<T, FLAGS, NT>(st, a, r0, c0, coloff, ldq, tid, swz);
}

// The wave's piece of tile (r0, c0).
__device__ __forceinline__ TileGeom wave_geom(const MxArgs& a, int64_t r0, int64_t c0, int wm,
                                              int wn, int lc) {
  TileGeom g;
  g.r0 = r0 + 32 * wm;
  g.cw = c0 + 64 * wn;
  g.col = g.cw + 8 * lc;
  g.col_ok = g.col < a.N;
  return g;
}

// A workgroup owns one tile of the tile order.  Workgroup id b runs on XCD b % 8 (workgroups
// are dealt to the XCDs round-robin).  With xcd_runs, XCD x owns positions
// [x * per_xcd, (x + 1) * per_xcd) of the order and workgroup b takes x * per_xcd + b / 8;
// otherwise workgroup b takes position b.
template <int ACT, int LAYOUT, int FLAGS, int MODE>
__global__ __launch_bounds__((TileOf<FLAGS, MODE>::NTHREADS)) void k_mxfp8(
    MxArgs a, uint32_t tiles_m, uint32_t tiles_n, uint32_t ntiles, uint32_t per_xcd, LaunchPolicy pol) {
  using T = TileOf<FLAGS, MODE>;
  using St = Stage<T, FLAGS>;
  constexpr int TM = T::TM, TN = T::TN;
  constexpr int PARTS = MODE == MODE_BWD ? 2 : 1;
  __shared__ __attribute__((aligned(16))) uint8_t lds[St::BYTES];
  uint32_t t = blockIdx.x;
  if (pol.xcd_runs != 0u) {
    const uint32_t xcd = blockIdx.x & 7;
    t = xcd * per_xcd + (blockIdx.x >> 3);
    if (t >= xcd * per_xcd + per_xcd) return;  // the whole workgroup
  }
  if (t >= ntiles) return;  // the whole workgroup
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
  const int wm = w % T::WM, wn = w / T::WM;
  const int lr = lane & 7, lc = lane >> 3;
  const int row0 = 32 * wm + 4 * lr, col = 64 * wn + 8 * lc;
  const int64_t ldq = PARTS * a.N;

  uint32_t tm, tn;
  tile_of<T, tile_order<FLAGS>()>(t, tiles_m, tiles_n, tm, tn);
  const int64_t r0 = (int64_t)tm * TM, c0 = (int64_t)tn * TN;
  // one store form per launch (pol.nt is uniform): both are instantiated, a scalar branch picks
  auto write_part = [&](const St& S, int64_t coloff) {
    if (pol.nt != 0u) write_out<T, FLAGS, true>(S, a, r0, c0, coloff, ldq, tid);
    else write_out<T, FLAGS, false>(S, a, r0, c0, coloff, ldq, tid);
  };
  TileOps<LAYOUT, MODE> o;
  load_ops<LAYOUT, MODE>(o, a, wave_geom(a, r0, c0, wm, wn, lc), lr, lc);
  TileVals<MODE> R;
  compute<ACT, LAYOUT, MODE>(R, o);
  const St A(lds);
  if constexpr (MODE == MODE_BWD) {
    // da and db pass through one stage in turn: backward both [16384, 7168] 227 vs 229 us
    // against a second stage that takes db while da is written out, at half the LDS
    stage_bf16<T, FLAGS>(R.h[0], A, row0, col, lr, lc);
    __syncthreads();
    write_part(A, 0);
    __syncthreads();
    stage_bf16<T, FLAGS>(R.h[1], A, row0, col, lr, lc);
    __syncthreads();
    write_part(A, a.N);
  } else {
    if constexpr (MODE == MODE_F32) stage_f32<T, FLAGS>(R.v, A, row0, col, lr, lc);
    else stage_bf16<T, FLAGS>(R.h[0], A, row0, col, lr, lc);
    __syncthreads();
    write_part(A, 0);
  }
}

// Rowwise-only launches without LDS (forward, and the backward's [da | db]).  A wave owns one
// row and 512 columns of it (a unit); lane l holds columns 8l..8l+7, so a 32-column block is
// the lane quad 4b..4b+3 (amax over two DPP steps), its 32 codes are the 8-byte stores of those
// 4 lanes, and 16 lanes together store one whole 128-byte line straight from their registers.
// One 16-byte load per operand per lane: the simplest streaming shape measured fastest for
// these byte mixes.  Units run along the rows, mapped to workgroups as the launch policy says
// (round-robin over the XCDs in the forward, per-XCD runs in the backward).  The arithmetic is
// that of the tiled kernel (the same device functions, the same NaN/Inf block rule), so the
// two produce identical bytes.
// Measured against the tiled kernel (us, SwiGLU, one box):
//   forward rowwise   [16384, 7168] 103.6 -> 101.1   [131072, 8192] 893.9 -> 855.5
//   backward rowwise  [16384, 7168] 157.5 -> 148.2   [65536, 8192]  728.7 -> 691.7
//                     [4096, 2048]   17.5 -> 16.4    [8192, 8192]    99.7 -> 93.8
constexpr int RF_WAVES = 4;    // waves per workgroup, one unit each
constexpr int RF_COLS = 512;   // columns per unit

// Quantizes the lane's 8 BF16 values H (columns 2k, 2k+1 in word k) of one part and stores
// its codes at byte 8 lane of rq and the unit's scales at rs: lane 4b holds block b's byte,
// and lane 16k gathers blocks 4k..4k+3 into one word (aligned, as N % 128 == 0).
__device__ __forceinline__ void row_quant_store(const uint32_t (&H)[4], __amdgpu_buffer_rsrc_t rq,
                                                __amdgpu_buffer_rsrc_t rs, uint32_t lane, bool ok,
                                                uint32_t nt) {
  uint32_t m = pkmax(pkmax(H[0] & 0x7fff7fffu, H[1] & 0x7fff7fffu), pkmax(H[2] & 0x7fff7fffu, H[3] & 0x7fff7fffu));
  m = umax(lo16(m), hi16(m));
  m = umax(m, dpp<DPP_XOR1>(m));
  m = umax(m, dpp<DPP_XOR2>(m));
  uint32_t sb = lo16(pk_scale_bytes(m));
  const float sc = e8m0_value(sb);
  uint32_t w0 = fp8x2_scaled<false>(0u, H[0], sc);
  w0 = fp8x2_scaled<true>(w0, H[1], sc);
  uint32_t w1 = fp8x2_scaled<false>(0u, H[2], sc);
  w1 = fp8x2_scaled<true>(w1, H[3], sc);
  if (m >= 0x7f80u) {  // a block holding NaN or Inf: scale 0xFF, every code 0x7F
    w0 = w1 = 0x7f7f7f7fu;
    sb = 0xffu;
  }
  const uint32_t qo = ok ? 8u * lane : kOob;
  if (nt != 0u) __builtin_amdgcn_raw_buffer_store_b64((u32x2){w0, w1}, rq, qo, 0, 2);
  else __builtin_amdgcn_raw_buffer_store_b64((u32x2){w0, w1}, rq, qo, 0, 0);
  const uint32_t s1 = __shfl_down(sb, 4, 16), s2 = __shfl_down(sb, 8, 16), s3 = __shfl_down(sb, 12, 16);
  const uint32_t word = sb | (s1 << 8) | (s2 << 16) | (s3 << 24);
  __builtin_amdgcn_raw_buffer_store_b32(word, rs, ok && (lane & 15u) == 0u ? lane / 4u : kOob, 0, 0);
}

template <int ACT, int LAYOUT, int MODE>
__global__ __launch_bounds__(64 * RF_WAVES) void k_mxfp8_row(MxArgs a, uint32_t segs, uint32_t units,
                                                             uint32_t wg_per_xcd, LaunchPolicy pol) {
  static_assert(MODE == MODE_FWD || LAYOUT == SPLIT, "the backward takes split operands");
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t wg = pol.xcd_runs != 0u ? (blockIdx.x & 7u) * wg_per_xcd + (blockIdx.x >> 3) : blockIdx.x;
  const uint32_t unit = wg * RF_WAVES + w;
  if (unit >= units) return;  // the whole wave; no barrier follows
  const uint32_t row = unit / segs, seg = unit - row * segs;
  const int64_t c0 = (int64_t)seg * RF_COLS;
  const bool ok = c0 + 8 * (int64_t)lane < a.N;  // N % 128 == 0: a scale word's 16 lanes agree

  GU<LAYOUT> in;
  uint32_t dw[4];
  const uint16_t* gate = static_cast<const uint16_t*>(a.src);
  if constexpr (LAYOUT == SPLIT) {
    const int64_t base = (int64_t)row * a.ld_in + c0;
    const uint32_t off = ok ? 16u * lane : kOob;
    bld16(in.a, rsrc(gate + base), off);
    bld16(in.b, rsrc(a.up + base), off);
    if constexpr (MODE == MODE_BWD) bld16(dw, rsrc(a.dh + (int64_t)row * a.ld_dh + c0), off);
  } else {
    const auto r = rsrc(gate + (int64_t)row * a.ld_in + 2 * c0);
    uint32_t w0[4], w1[4];
    bld16(w0, r, ok ? 32u * lane : kOob);
    bld16(w1, r, ok ? 32u * lane + 16u : kOob);
#pragma unroll
    for (int k = 0; k < 4; k++) {
      in.a[k] = w0[k];
      in.a[4 + k] = w1[k];
    }
  }

  float g[8], u[8];
  unpack_gu<LAYOUT>(in, g, u);
  bool tail = false;
  if constexpr (tail_from_gate_bits<ACT>()) {
    uint32_t m = in.a[0];
#pragma unroll
    for (int k = 1; k < (LAYOUT == SPLIT ? 4 : 8); k++) m = pkmax(m, in.a[k]);
    tail = tail_possible<ACT>(LAYOUT == SPLIT ? umax(lo16(m), hi16(m)) : lo16(m));
  }
  const int64_t ldq = (MODE == MODE_BWD ? 2 : 1) * a.N;
  const auto rq = rsrc(a.q_row + (int64_t)row * ldq + c0);
  const auto rs = rsrc(a.s_row + (int64_t)row * (ldq / 32) + (int64_t)seg * (RF_COLS / 32));
  if constexpr (MODE == MODE_FWD) {
    float h[8];
#pragma unroll
    for (int c = 0; c < 8; c++) {
      h[c] = glu_fwd_fast<ACT>(g[c], u[c]);
      if constexpr (!tail_from_gate_bits<ACT>()) tail |= fwd_tail_needed<ACT>(g[c], u[c]);
    }
    if (tail) {  // rare: some element may need the FP64 tail path
#pragma unroll
      for (int c = 0; c < 8; c++)
        if (fwd_tail_needed<ACT>(g[c], u[c])) h[c] = glu_fwd_tail<ACT>(g[c], u[c]);
    }
    uint32_t H[4];
#pragma unroll
    for (int k = 0; k < 4; k++) H[k] = pack_bf16(h[2 * k], h[2 * k + 1]);
    row_quant_store(H, rq, rs, lane, ok, pol.nt);
  } else {
    float d[8], da[8], db[8];
#pragma unroll
    for (int c = 0; c < 8; c++) {
      d[c] = (c & 1) ? bf_hi(dw[c >> 1]) : bf_lo(dw[c >> 1]);
      glu_bwd_fast<ACT>(g[c], u[c], d[c], da[c], db[c]);
      if constexpr (!tail_from_gate_bits<ACT>()) tail |= bwd_tail_needed<ACT>(g[c], u[c], d[c]);
    }
    if (tail) {  // rare: some element may need the FP64 tail path
#pragma unroll
      for (int c = 0; c < 8; c++)
        if (bwd_tail_needed<ACT>(g[c], u[c], d[c])) glu_bwd_tail<ACT>(g[c], u[c], d[c], da[c], db[c]);
    }
    uint32_t A[4], B[4];
#pragma unroll
    for (int k = 0; k < 4; k++) {
      A[k] = pack_bf16(da[2 * k], da[2 * k + 1]);
      B[k] = pack_bf16(db[2 * k], db[2 * k + 1]);
    }
    row_quant_store(A, rq, rs, lane, ok, pol.nt);
    // db: N columns further along the row; its scales N / 32 bytes further
    row_quant_store(B, rsrc(a.q_row + (int64_t)row * ldq + a.N + c0),
                    rsrc(a.s_row + (int64_t)row * (ldq / 32) + a.N / 32 + (int64_t)seg * (RF_COLS / 32)), lane, ok,
                    pol.nt);
  }
}

// Launches the rowwise kernel above when it applies: row-major scales, N % 128 == 0 (whole
// scale words; at [1000, 4000], whose scales would leave byte by byte, the tiled kernel was
// faster: 11.7 vs 13.1 us forward), units numbered in 32 bits.  Returns false to leave the
// launch to k_mxfp8.
template <int ACT, int LAYOUT, int MODE>
bool launch_row(const MxArgs& a, hipStream_t s, hipError_t& err) {
  if (a.flags != ROWWISE || a.N % 128 != 0) return false;
  const int64_t segs = (a.N + RF_COLS - 1) / RF_COLS, units = a.M * segs;
  if (units >= (int64_t)1 << 31) return false;
  const int64_t wgs = (units + RF_WAVES - 1) / RF_WAVES, wg_per_xcd = (wgs + 7) / 8;
  const int64_t parts = MODE == MODE_BWD ? 2 : 1;
  err = launch_kernel(k_mxfp8_row<ACT, LAYOUT, MODE>, dim3((unsigned)(8 * wg_per_xcd)), dim3(64 * RF_WAVES), s,
                      a, (uint32_t)segs, (uint32_t)units, (uint32_t)wg_per_xcd,
                      launch_policy(a.flags, MODE, parts * a.M * a.N, true, (a.flags & SF_SWIZZLED) != 0));
  return true;
}

template <int ACT, int LAYOUT, int FLAGS, int MODE>
hipError_t launch(const MxArgs& a, hipStream_t s) {
  using T = TileOf<FLAGS, MODE>;
  int64_t tiles_m = (a.M + T::TM - 1) / T::TM, tiles_n = (a.N + T::TN - 1) / T::TN;
  if (a.flags & SF_SWIZZLED) {
    // tiles past the matrix (zero inputs, no codes written) cover the scale padding:
    // rowwise padding rows up to a multiple of 128 and padding scale columns up to a multiple
    // of 4 after the last part; colwise padding rows (columns of the quantized matrix) up to a
    // multiple of 128 after the last part
    const int64_t ldq = (MODE == MODE_BWD ? 2 : 1) * a.N, last = ldq - a.N;
    const int64_t rp = (a.M + 127) / 128 * 128, wp = (ldq + 127) / 128 * 128;
    if (FLAGS & ROWWISE) {
      tiles_m = (rp + T::TM - 1) / T::TM;
      const int64_t cpad = (ldq / 32 + 3) / 4 * 4 * 32;  // padded scale columns, in elements
      const int64_t need = (cpad - last + T::TN - 1) / T::TN;
      if (need > tiles_n) tiles_n = need;
    }
    if (FLAGS & COLWISE) {
      const int64_t need = (wp - last + T::TN - 1) / T::TN;
      if (need > tiles_n) tiles_n = need;
    }
  }
  const int64_t ntiles = tiles_m * tiles_n, per_xcd = (ntiles + 7) / 8;
  const int64_t code_bytes = (((FLAGS & ROWWISE) ? 1 : 0) + ((FLAGS & COLWISE) ? 1 : 0)) *
                             a.M * (MODE == MODE_BWD ? 2 : 1) * a.N;
  const LaunchPolicy pol = launch_policy(FLAGS, MODE, code_bytes, false, (a.flags & SF_SWIZZLED) != 0);
  // per-XCD runs need 8 * per_xcd workgroups (the last XCD's run may be short); round-robin
  // needs one per tile
  const int64_t grid = pol.xcd_runs != 0u ? 8 * per_xcd : ntiles;
  return launch_kernel(k_mxfp8<ACT, LAYOUT, FLAGS, MODE>, dim3((unsigned)grid), dim3(T::NTHREADS), s, a,
                       (uint32_t)tiles_m, (uint32_t)tiles_n, (uint32_t)ntiles, (uint32_t)per_xcd, pol);
}

template <int ACT, int LAYOUT, int MODE>
hipError_t by_flags(const MxArgs& a, hipStream_t s) {
  switch (a.flags & (ROWWISE | COLWISE)) {
    case ROWWISE: return launch<ACT, LAYOUT, ROWWISE, MODE>(a, s);
    case COLWISE: return launch<ACT, LAYOUT, COLWISE, MODE>(a, s);
    default: return launch<ACT, LAYOUT, ROWWISE | COLWISE, MODE>(a, s);
  }
}

}  // namespace

hipError_t launch_glu_fwd_mxfp8(const MxArgs& a, hipStream_t s) {
  return with_act(a.act, [&](auto A) {
    constexpr int ACT = decltype(A)::value;
    hipError_t err = hipSuccess;
    if (a.layout == SPLIT ? launch_row<ACT, SPLIT, MODE_FWD>(a, s, err) : launch_row<ACT, PAIRED, MODE_FWD>(a, s, err))
      return err;
    return a.layout == SPLIT ? by_flags<ACT, SPLIT, MODE_FWD>(a, s) : by_flags<ACT, PAIRED, MODE_FWD>(a, s);
  });
}

hipError_t launch_glu_bwd_mxfp8(const MxArgs& a, hipStream_t s) {
  return with_act(a.act, [&](auto A) {
    constexpr int ACT = decltype(A)::value;
    hipError_t err = hipSuccess;
    if (launch_row<ACT, SPLIT, MODE_BWD>(a, s, err)) return err;
    return by_flags<ACT, SPLIT, MODE_BWD>(a, s);
  });
}

hipError_t launch_quant_mxfp8_f32(const MxArgs& a, hipStream_t s) {
  return by_flags<SWIGLU, SPLIT, MODE_F32>(a, s);
}

}  // namespace glu
