// Merged gate/up block-scaled GEMM with the GLU as its epilogue (and optionally the MXFP8
// rowwise or the NVFP4 quantizer after it): "feat(phyai-kernel): add Thor NVFP4 GeGLU kernel for
// pi0.5" (Summary: the GeGLU fold follows the merged gate/up GEMM; Supported contract: packed
// E2M1 values and pairwise-interleaved gate/up weight rows), in the MXFP8 form of "Add swiglu +
// MXFP8 fused CuTe DSL kernel" (Performance: the fused-w13 MoE composite under an MXFP8 recipe;
// API: a fused w13 projection packs [gate | up]).  The pre-activation never reaches memory.
//
//   Y = X W^T, X [M, K] and W [2N, K] with E8M0 scales per 32-element block along K, codes E4M3
//   (one per byte) or E2M1 (two per byte, element 2j in the low nibble); W's rows are
//   [W_gate | W_up] or interleaved gate0, up0, gate1, ...; h = bf16(act(Y_gate) * Y_up).
//
// Matrix cores: v_mfma_scale_f32_16x16x128_f8f6f4 (E8M0 block scales; format code 0 for E4M3,
// 4 for E2M1).  Operand layouts, established on the device:
//   E4M3: lane l = 16 g + r (g = l / 16) holds row r of the 16-row operand and the 16-byte K
//     chunks g and g + 4 of the 128-byte K step; its scale byte covers K block g (chunks 2g,
//     2g + 1).
//   E2M1: lane l holds row r and K elements 32 g .. 32 g + 31 (16 bytes, the operand's first
//     four registers); its scale byte covers that block.
// The 16x16 result: lane l holds rows 4 g + i, i = 0..3, of column r.  The instruction does
// not add products as IEEE FP32 values.  E4M3: the products of each aligned 8-element K chunk
// are summed in a 14-bit fixed-point window anchored at the chunk's largest product (bits
// below it are dropped, whatever the sign).  E2M1: each aligned 16-element chunk is summed
// (exactly: its products share the block's scales and span at most 2^8).  The chunk sums are
// added to the FP32 accumulator one at a time with FP32 rounding.
//
// Work decomposition: a workgroup of 8 waves (two per SIMD, so one wave's LDS reads overlap
// the other's matrix instructions) owns 256 rows x 128 output columns, i.e. 128 gate and 128
// up rows of W.  Each wave holds a 64 x 64 block: the gate and the up accumulators of the
// same (row, column) positions (4 x 4 tiles of 16 x 16 each), so the GLU is applied in
// registers.
//
// Operand staging: a K step is one 128-byte line of every operand row (128 E4M3 codes, or 256
// E2M1 codes that feed two matrix instructions: the lane's chunk g, then its chunk g + 4).
// Each K step of the workgroup's 256 X rows and 256 W rows
// (64 KiB) is copied into LDS by direct-to-LDS buffer loads, which place lane l's 16 bytes at
// 16 l of a 1 KiB block.  Each group of 8 lanes fetches one row's whole 128-byte line, and
// lane l puts global chunk (l % 8) ^ ((row / 2) % 8) at chunk l % 8 of the row, so the
// fragment reads (row r, chunks g and g + 4 per lane) hit distinct LDS banks.  Two stages
// alternate: the loads of step t + 1 are issued right after the barrier of step t and have
// step t's matrix work to arrive.  The E8M0 scales come in groups of 16 blocks (4 E4M3 or 2
// E2M1 K steps; 16 bytes a row, 4 lanes a row) into a ring of two groups.  Interleaved W rows
// are gathered into the same LDS places as split ones (gate slices, then up slices), so the
// two layouts give identical results.  Rows past M read zeros.  The loop body runs
// two steps with the stage as a compile-time constant, so every fragment read is a lane base
// register plus an immediate offset and each load's K offset rides in the scalar offset: the
// loop carries almost no VALU work (a wave64 VALU instruction occupies its SIMD 4 cycles).
//
// Epilogue: the products are formed as W X^T, so each 16 x 16 result is a transposed tile of
// Y and a lane holds 4 consecutive columns of one row.  Per 16-row slice: the GLU in FP32 for
// all elements, one wave-wide branch for the rare tail elements, BF16 pairs by the hardware
// converter; then the block amax in the lane and over the row's 4 lanes (two exchanges), the
// block scale, the hardware converters, and one store per lane and tile.
//
// Tile order: workgroups are spread over the 8 XCDs in turn, so workgroup b is given tile
// (b mod 8) * (tiles / 8) + b / 8, which keeps each XCD on a contiguous run of tiles, and
// tiles run down groups of 8 row tiles before moving to the next column tile, so the
// workgroups resident on one XCD share X and W in its L2.
#include "glu_device.h"
#include "glu_launch.h"

namespace glu {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t v2u __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void* lds_ptr;

constexpr int GM_THREADS = 512;
constexpr int WM = 4, WN = 4;                         // 16x16 tiles per wave: rows, columns
constexpr int GM_BM = 4 * 16 * WM, GM_BN = 2 * 16 * WN, GM_BK = 128;  // workgroup tile, K step
static_assert(WN % 2 == 0, "an MXFP8 block is two 16-column tiles");
constexpr int GROUP_M = 8;                            // row tiles per group of the tile order

// LDS stage: 16 X slices, then 16 W slices (gate 0..7, up 8..15), 2 KiB each.
constexpr uint32_t X_SLICES = GM_BM / 16, W_SLICES = 2 * GM_BN / 16;
constexpr uint32_t W_OFF = X_SLICES * 2048u;
constexpr uint32_t STAGE = W_OFF + W_SLICES * 2048u;
constexpr int STAGES = 2;
// Scale ring: 2 groups of 4 K steps; a group holds 16 bytes (4 steps x 4 blocks) per row,
// X rows 0..255 then W rows 256..511.
constexpr uint32_t SC_ROWS = GM_BM + 2 * GM_BN, SC_GROUP = 16u * SC_ROWS, SC_OFF = STAGES * STAGE;
static_assert(SC_OFF + 2 * SC_GROUP <= 160u * 1024u, "LDS");
constexpr int SC_LOADS = SC_ROWS / 16 / 8;            // per wave and group: 16 rows each

enum {
  GEMM_H = 0, GEMM_MXFP8 = 1, GEMM_F32 = 2,
  GEMM_NV_ROWMAJOR = 3, GEMM_NV_128x4 = 4,         // NVFP4, global scale 1
  GEMM_NV_GS_ROWMAJOR = 5, GEMM_NV_GS_128x4 = 6    // NVFP4, two-level (global scale from *amax)
};
constexpr bool is_nv(int out) { return out >= GEMM_NV_ROWMAJOR; }

// Direct-to-LDS loads: lane l's bytes go to lds + size * l.  voffset is the lane's part,
// soffset the wave-uniform part (an out-of-range voffset stays out of range with it added).
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, uint8_t* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr)lds, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, uint8_t* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr)lds, 4, voff, soff, 0, 0);
}

// s_waitcnt on the vector-memory counter alone (gfx9 encoding: vmcnt in bits 3:0 and 15:14).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Barrier that also orders the workgroup's LDS accesses (no wait on global memory).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ v8i frag(const uint8_t* blk, uint32_t oa, uint32_t ob) {
  const u32x4 a = *(const u32x4*)(blk + oa);
  const u32x4 b = *(const u32x4*)(blk + ob);
  return (v8i){(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
}

template <int ACT, int OUT, int FMT>
__global__ __launch_bounds__(GM_THREADS) void k_glu_gemm(GemmArgs a, uint32_t tiles_m, uint32_t tiles_n) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[SC_OFF + 2 * SC_GROUP];
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t g = lane >> 4, r = lane & 15u;

  // tile of this workgroup: XCD-contiguous runs, grouped row-tile order
  const uint32_t tiles = tiles_m * tiles_n, per_xcd = tiles / 8u, b = blockIdx.x;
  const uint32_t t = b < 8u * per_xcd ? (b % 8u) * per_xcd + b / 8u : b;
  const uint32_t in_group = GROUP_M * tiles_n, first_m = (t / in_group) * GROUP_M;
  const uint32_t gm = min(tiles_m - first_m, (uint32_t)GROUP_M);
  const uint32_t tm = first_m + (t % in_group) % gm, tn = (t % in_group) / gm;

  const uint32_t row0 = tm * GM_BM + (wave >> 1) * (16 * WM);  // the wave's first row
  const uint32_t col0 = tn * GM_BN + (wave & 1) * (16 * WN);   // its first output column
  const uint32_t K = (uint32_t)a.K, KB = K / 32u, N = (uint32_t)a.N, M = (uint32_t)a.M;
  // A K step is one 128-byte line of every operand row: 128 E4M3 codes, or 256 E2M1 codes
  // (two matrix instructions of 128).  A scale group (16 bytes a row) covers SPG steps.
  constexpr uint32_t KPS = FMT == FMT_E2M1 ? 2u * GM_BK : GM_BK, SPG = 16u / (KPS / 32u);
  const uint32_t RB = FMT == FMT_E2M1 ? K / 2u : K;             // bytes per operand row
  const uint32_t T = K / KPS;                                   // K steps
  // W rows of output column n: gate n and up N + n, or gate 2n and up 2n + 1 (interleaved)
  const bool paired = a.w_layout == PAIRED;
  const uint32_t up_row0 = paired ? 1u : N, col_rows = paired ? 2u : 1u;

  // Load assignment (per wave, the same count every step): X slices 2w, 2w + 1 and W slices
  // 2w, 2w + 1, two loads of 8 rows each.  Lane l of load h of a slice: slice row
  // 8 h + l / 8, LDS chunk l % 8 <- global chunk (l % 8) ^ ((slice row / 2) % 8).
  const auto rx = rsrc(a.xq), rxs = rsrc(a.xs), rw = rsrc(a.wq), rws = rsrc(a.ws);
  uint32_t xoff[2], woff[2];
  const uint32_t lrow = lane >> 3;                                   // + 8 h
  uint32_t lchunk[2];
#pragma unroll
  for (int h = 0; h < 2; h++) lchunk[h] = 16u * ((lane & 7u) ^ (((8u * h + lrow) >> 1) & 7u));
  bool xokh[2][2];
#pragma unroll
  for (int i = 0; i < 2; i++) {
    const uint32_t row = tm * GM_BM + 16u * (2u * wave + i) + lrow;
    xoff[i] = row * RB;
#pragma unroll
    for (int h = 0; h < 2; h++) xokh[i][h] = row + 8u * h < M;
  }
#pragma unroll
  for (int i = 0; i < 2; i++) {
    const uint32_t sl = 2u * wave + i;                           // 0..7 gate, 8..15 up
    const uint32_t n = tn * GM_BN + 16u * (sl & 7u) + lrow;       // output column
    woff[i] = ((sl < 8u ? 0u : up_row0) + col_rows * n) * RB;
  }
  // scale load i of a group: rows 16 q .. 16 q + 15, q = SC_LOADS w + i; lane l reads the
  // word of step 4 j + l % 4 of row 16 q + l / 4
  uint32_t soff[SC_LOADS];
  bool sok[SC_LOADS], sx[SC_LOADS];
#pragma unroll
  for (int i = 0; i < SC_LOADS; i++) {
    const uint32_t row = 16u * (SC_LOADS * wave + i) + (lane >> 2);
    if (row < (uint32_t)GM_BM) {
      const uint32_t grow = tm * GM_BM + row;
      sx[i] = true; sok[i] = grow < M; soff[i] = grow * KB + 4u * (lane & 3u);
    } else {
      const uint32_t wr = row - GM_BM, n = tn * GM_BN + (wr % (uint32_t)GM_BN);
      const uint32_t wrow = (wr < (uint32_t)GM_BN ? 0u : up_row0) + col_rows * n;
      sx[i] = false; sok[i] = true; soff[i] = wrow * KB + 4u * (lane & 3u);
    }
  }
  auto issue_scales = [&](uint32_t grp) {
    uint8_t* sc = smem + SC_OFF + (grp & 1u) * SC_GROUP;
    const bool live = SPG * grp + (lane & 3u) * SPG / 4u < T;   // the step this word serves
#pragma unroll
    for (int i = 0; i < SC_LOADS; i++)
      dma4(sx[i] ? rxs : rws, sok[i] && live ? soff[i] : kOob, 16u * grp, sc + 256u * (SC_LOADS * wave + i));
  };
  // the lanes' parts of the operand loads (rows past M out of range); the K offset is added
  // as the instruction's scalar offset
  uint32_t vx[2][2], vw[2][2];
#pragma unroll
  for (int i = 0; i < 2; i++)
#pragma unroll
    for (int h = 0; h < 2; h++) {
      vx[i][h] = xokh[i][h] ? xoff[i] + 8u * h * RB + lchunk[h] : kOob;
      vw[i][h] = woff[i] + 8u * h * col_rows * RB + lchunk[h];
    }
  auto issue = [&](uint32_t step, uint32_t stage) {
    uint8_t* st = smem + stage * STAGE;
    const uint32_t k0 = step * GM_BK;
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
      for (int h = 0; h < 2; h++)
        dma16(rx, vx[i][h], k0, st + (2u * (2u * wave + i) + h) * 1024u);
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
      for (int h = 0; h < 2; h++)
        dma16(rw, vw[i][h], k0, st + W_OFF + (2u * (2u * wave + i) + h) * 1024u);
  };

  v4f acc[2][WM][WN];
#pragma unroll
  for (int h = 0; h < 2; h++)
#pragma unroll
    for (int i = 0; i < WM; i++)
#pragma unroll
      for (int j = 0; j < WN; j++) acc[h][i][j] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};

  // The lane's fragment bases (row r, chunks g and g + 4 at their swizzled positions) in
  // the wave's first X slice and first gate slice; the slices, the stage and the up half are
  // compile-time offsets from these.
  const uint32_t fo_a = 128u * r + 16u * (g ^ ((r >> 1) & 7u));
  const uint32_t fo_b = 128u * r + 16u * ((g + 4u) ^ ((r >> 1) & 7u));
  const uint32_t xb_a = fo_a + 2048u * ((wave >> 1) * WM), xb_b = fo_b + 2048u * ((wave >> 1) * WM);
  const uint32_t wb_a = fo_a + W_OFF + 2048u * ((wave & 1) * WN), wb_b = fo_b + W_OFF + 2048u * ((wave & 1) * WN);
  const uint32_t sc_x = 16u * (16u * ((wave >> 1) * WM) + r) + g;             // scale bytes
  const uint32_t sc_w = 16u * (GM_BM + 16u * ((wave & 1) * WN) + r) + g;
  auto run_step = [&](uint32_t step, auto STG) {
    constexpr uint32_t stage = decltype(STG)::value;
    wait_vm<0>();
    lds_barrier();   // every wave's loads of this step have landed; step - 1's stage is free
    if (step % SPG == 0u && step + SPG < T) issue_scales(step / SPG + 1u);
    if (step + 1u < T) issue(step + 1u, 1u - stage);
    const uint8_t* st = smem + stage * STAGE;
    const uint32_t sq = SC_OFF + ((step / SPG) & 1u) * SC_GROUP + (16u / SPG) * (step % SPG);
    v8i xa[WM], wb[2][WN];
#pragma unroll
    for (int i = 0; i < WM; i++) xa[i] = frag(st, xb_a + 2048u * i, xb_b + 2048u * i);
#pragma unroll
    for (int h = 0; h < 2; h++)
#pragma unroll
      for (int j = 0; j < WN; j++) wb[h][j] = frag(st, wb_a + 2048u * (8u * h + j), wb_b + 2048u * (8u * h + j));
    // E4M3: one instruction over the lane's 32 bytes (chunks g and g + 4).  E2M1: the line
    // holds two 128-element steps; the lane's chunk g (the low half of its fragment) feeds
    // the first and chunk g + 4 the second, with the scale bytes of blocks g and 4 + g.
    constexpr int SUBS = FMT == FMT_E2M1 ? 2 : 1, CODE = FMT == FMT_E2M1 ? 4 : 0;
#pragma unroll
    for (int u = 0; u < SUBS; u++) {
      int xs[WM], ws[2][WN];
#pragma unroll
      for (int i = 0; i < WM; i++) xs[i] = smem[sq + 4u * u + sc_x + 256u * i];
#pragma unroll
      for (int h = 0; h < 2; h++)
#pragma unroll
        for (int j = 0; j < WN; j++) ws[h][j] = smem[sq + 4u * u + sc_w + 256u * (8u * h + j)];
#pragma unroll
      for (int h = 0; h < 2; h++)
#pragma unroll
        for (int i = 0; i < WM; i++)
#pragma unroll
          for (int j = 0; j < WN; j++) {
            const v8i wop = u == 0 ? wb[h][j] : __builtin_shufflevector(wb[h][j], wb[h][j], 4, 5, 6, 7, 4, 5, 6, 7);
            const v8i xop = u == 0 ? xa[i] : __builtin_shufflevector(xa[i], xa[i], 4, 5, 6, 7, 4, 5, 6, 7);
            acc[h][i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                wop, xop, acc[h][i][j], CODE, CODE, 0, ws[h][j], 0, xs[i]);
          }
    }
  };
  static_assert(STAGES == 2, "two steps per iteration, one per stage");
  issue_scales(0);
  issue(0, 0);
  for (uint32_t step = 0; step < T; step += 2) {
    run_step(step, std::integral_constant<uint32_t, 0>{});
    if (step + 1u < T) run_step(step + 1u, std::integral_constant<uint32_t, 1>{});
  }

  // Epilogue.  The products are formed as W X^T (W the first operand), so each 16 x 16 result
  // is a transposed tile of Y: acc[h][i][j][e] is Y at row row0 + 16 i + r and column
  // col0 + 16 j + 4 g + e of the gate (h = 0) or up (h = 1) half.  A lane thus holds 4
  // consecutive columns of one row per tile, and a row's 16 columns of a tile sit in the 4
  // lanes r, 16 + r, 32 + r, 48 + r.
  if constexpr (OUT == GEMM_F32) {
    // test hook: the pre-activation itself, [M, 2N] FP32
    // one lane offset per 16-row slice; the gate/up half and the tile column are constants
    // added to it, so no per-store address arithmetic is kept live across the stores
    const auto ry = rsrc(a.y);
    const uint32_t pitch = 8u * N;  // bytes per row of y
    const uint32_t base = (row0 + r) * pitch + 4u * (col0 + 4u * g);
#pragma unroll
    for (int i = 0; i < WM; i++) {
      const uint32_t oi = row0 + 16u * i + r < M ? base + 16u * i * pitch : kOob;
#pragma unroll
      for (int h = 0; h < 2; h++)
#pragma unroll
        for (int j = 0; j < WN; j++) {
          const v4f v = acc[h][i][j];
          const uint32_t off = oi == kOob ? kOob : oi + 4u * N * h + 64u * j;
          __builtin_amdgcn_raw_buffer_store_b128((u32x4){__float_as_uint(v[0]), __float_as_uint(v[1]),
                                                         __float_as_uint(v[2]), __float_as_uint(v[3])},
                                                 ry, off, 0, 0);
        }
    }
  } else {
    // h = bf16(act(gate) * up), one 16-row slice i at a time (so that the slice's
    // accumulators die as it is written): the fast form for every element, then the tail
    // form where the fast one leaves FP32 (one branch per slice for the whole wave, rarely
    // taken).  P[j][0] holds columns 4g, 4g + 1 of tile j as a BF16 pair, P[j][1] 4g + 2, 4g + 3.
    auto xor32 = [&](uint32_t v) {   // the value of lane l ^ 32
      return (uint32_t)__builtin_amdgcn_ds_bpermute((int)(4u * (lane ^ 32u)), (int)v);
    };
    // the packed maxima of the lane's row over its 4 lanes g
    auto row_max = [&](uint32_t m) {
      m = pkmax(m, swz_xor16(m));
      return pkmax(m, xor32(m));
    };
    const auto rh = rsrc(a.h), rq = rsrc(a.q_row), rs = rsrc(a.s_row);
    GlobalScale gs;
    if constexpr (OUT >= GEMM_NV_GS_ROWMAJOR) gs = global_scale(*a.amax);
    const uint32_t NB = N / 32u;
#pragma unroll
    for (int i = 0; i < WM; i++) {
      const uint32_t row = row0 + 16u * i + r;
      const bool ok = row < M;
      float hv[WN][4];
      bool tail = false;
#pragma unroll
      for (int j = 0; j < WN; j++)
#pragma unroll
        for (int e = 0; e < 4; e++) hv[j][e] = glu_fwd_elem<ACT>(acc[0][i][j][e], acc[1][i][j][e], tail);
      if (tail) {
#pragma unroll
        for (int j = 0; j < WN; j++)
#pragma unroll
          for (int e = 0; e < 4; e++)
            if (fwd_tail_needed<ACT>(acc[0][i][j][e], acc[1][i][j][e]))
              hv[j][e] = glu_fwd_tail<ACT>(acc[0][i][j][e], acc[1][i][j][e]);
      }
      uint32_t P[WN][2];
#pragma unroll
      for (int j = 0; j < WN; j++) {
        P[j][0] = pack_bf16(hv[j][0], hv[j][1]);
        P[j][1] = pack_bf16(hv[j][2], hv[j][3]);
      }
      const uint32_t cl = col0 + 4u * g;   // the lane's first column in tile 0
      if constexpr (OUT == GEMM_H) {
#pragma unroll
        for (int j = 0; j < WN; j++)
          __builtin_amdgcn_raw_buffer_store_b64((v2u){P[j][0], P[j][1]}, rh,
                                                ok ? 2u * (row * (uint32_t)a.ld_h + cl + 16u * j) : kOob, 0, 0);
      } else if constexpr (OUT == GEMM_MXFP8) {
        // MXFP8 rowwise: the wave's 64 columns of a row are two blocks of 32 (tiles 2b and
        // 2b + 1); block amax in the lane (packed), then over the row's 4 lanes, both blocks
        // at once (block 0 in the low half)
        static_assert(WN == 4, "two MXFP8 blocks per row and wave");
        uint32_t mb[2];
#pragma unroll
        for (int b = 0; b < 2; b++) {
          const uint32_t t = pkmax(pkmax(P[2 * b][0] & 0x7fff7fffu, P[2 * b][1] & 0x7fff7fffu),
                                   pkmax(P[2 * b + 1][0] & 0x7fff7fffu, P[2 * b + 1][1] & 0x7fff7fffu));
          mb[b] = umax(lo16(t), hi16(t));
        }
        const uint32_t mm = row_max(mb[0] | (mb[1] << 16));
        uint32_t sbs = 0;
#pragma unroll
        for (int b = 0; b < 2; b++) {
          const uint32_t m = b ? hi16(mm) : lo16(mm);
          const bool nonfinite = m >= 0x7f80u;
          const uint32_t sb = nonfinite ? 0xffu : mx_scale_byte(m << 16);
          sbs |= sb << (8 * b);
          const float sc = e8m0_value(sb);
#pragma unroll
          for (int t = 0; t < 2; t++) {
            const int j = 2 * b + t;
            uint32_t c = fp8x2_scaled<false>(0u, P[j][0], sc);
            c = fp8x2_scaled<true>(c, P[j][1], sc);
            __builtin_amdgcn_raw_buffer_store_b32(nonfinite ? 0x7f7f7f7fu : c, rq,
                                                  ok ? row * N + cl + 16u * j : kOob, 0, 0);
          }
        }
        __builtin_amdgcn_raw_buffer_store_b16((uint16_t)sbs, rs, ok && g == 0 ? row * NB + col0 / 32u : kOob, 0, 0);
      } else {
        // NVFP4: a 16-column block is one tile j; its amax in the lane, then over the row's 4
        // lanes, two blocks at a time (packed)
        uint32_t mt[WN];
#pragma unroll
        for (int j = 0; j < WN; j++) {
          const uint32_t t = pkmax(P[j][0] & 0x7fff7fffu, P[j][1] & 0x7fff7fffu);
          mt[j] = umax(lo16(t), hi16(t));
        }
        const uint32_t m01 = row_max(mt[0] | (mt[1] << 16)), m23 = row_max(mt[2] | (mt[3] << 16));
        uint32_t sbs = 0;
#pragma unroll
        for (int j = 0; j < WN; j++) {
          const uint32_t mj = j == 0 ? lo16(m01) : j == 1 ? hi16(m01) : j == 2 ? lo16(m23) : hi16(m23);
          const bool nonfinite = mj >= 0x7f80u;
          const float x[4] = {bf_lo(P[j][0]), bf_hi(P[j][0]), bf_lo(P[j][1]), bf_hi(P[j][1])};
          uint32_t sc, word;
          if constexpr (OUT >= GEMM_NV_GS_ROWMAJOR) {
            // two-level: E4M3(fl(bamax * k)), saturating at 448; codes E2M1(fl(x * fl(s / S)))
            const float d = __builtin_fminf(__uint_as_float(mj << 16) * gs.k, 448.0f);
            sc = nonfinite ? 0x7fu : (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(d, 0.0f, 0, false) & 0xffu;
            const float S = e4m3_value(nonfinite ? 0u : sc);
            const float rs_ = S > 0.0f ? gs.s / S : 0.0f;   // IEEE division
            // |x * rs_| beyond 8 saturates to 6 either way; the clamp keeps the input finite
            float y[4];
#pragma unroll
            for (int e = 0; e < 4; e++) y[e] = nonfinite ? 0.0f : __builtin_amdgcn_fmed3f(x[e] * rs_, -8.0f, 8.0f);
            word = fp4x2<0>(0u, y[0], y[1]);
            word = fp4x2<1>(word, y[2], y[3]);
          } else {
            sc = nonfinite ? 0x7fu : nv_scale_code_bf16(__uint_as_float(mj << 16));
            const float S = e4m3_value(nonfinite ? 0u : sc);
            const float R = S > 0.0f ? __builtin_amdgcn_rcpf(S) : 0.0f;
            word = fp4x2_of_quotients<0>(0u, x[0], x[1], R);
            word = fp4x2_of_quotients<1>(word, x[2], x[3], R);
            if (nonfinite) word = 0u;
          }
          sbs |= sc << (8 * j);
          // (a block holding NaN or Inf gets scale 0x7F and zero codes)
          __builtin_amdgcn_raw_buffer_store_b16((uint16_t)word, rq, ok ? (row * N + cl + 16u * j) / 2u : kOob, 0, 0);
        }
        // the row's four scale bytes of this wave, blocks col0 / 16 .. + 3, as one word
        if constexpr (OUT == GEMM_NV_ROWMAJOR || OUT == GEMM_NV_GS_ROWMAJOR) {
          __builtin_amdgcn_raw_buffer_store_b32(sbs, rs, ok && g == 0 ? row * (N / 16u) + col0 / 16u : kOob, 0, 0);
        } else {
          // 128x4: rows padded to 128 with zero scales (N / 16 is a multiple of 4)
          const uint32_t off = (row >> 7) * (N / 64u) * 512u + (row & 31u) * 16u + ((row & 127u) >> 5) * 4u +
                               (col0 / 64u) * 512u;
          const bool pad_ok = row < ((M + 127u) & ~127u);
          __builtin_amdgcn_raw_buffer_store_b32(ok ? sbs : 0u, rs, pad_ok && g == 0 ? off : kOob, 0, 0);
        }
      }
    }
  }
}

template <int OUT, int FMT>
hipError_t launch_fmt(const GemmArgs& a, hipStream_t s) {
  const uint32_t tiles_m = (uint32_t)((a.M + GM_BM - 1) / GM_BM), tiles_n = (uint32_t)(a.N / GM_BN);
  const dim3 grid(tiles_m * tiles_n), block(GM_THREADS);
  if constexpr (OUT == GEMM_F32) {
    return launch_kernel(k_glu_gemm<SWIGLU, GEMM_F32, FMT>, grid, block, s, a, tiles_m, tiles_n);
  } else {
    return with_act(a.act, [&](auto A) {
      constexpr int ACT = decltype(A)::value;
      return launch_kernel(k_glu_gemm<ACT, OUT, FMT>, grid, block, s, a, tiles_m, tiles_n);
    });
  }
}

template <int OUT>
hipError_t launch(const GemmArgs& a, hipStream_t s) {
  return a.fmt == FMT_E2M1 ? launch_fmt<OUT, FMT_E2M1>(a, s) : launch_fmt<OUT, FMT_E4M3>(a, s);
}

}  // namespace

hipError_t launch_glu_gemm(const GemmArgs& a, hipStream_t s) { return launch<GEMM_H>(a, s); }
hipError_t launch_glu_gemm_mxfp8(const GemmArgs& a, hipStream_t s) { return launch<GEMM_MXFP8>(a, s); }
hipError_t launch_mx_gemm_f32(const GemmArgs& a, hipStream_t s) { return launch<GEMM_F32>(a, s); }
hipError_t launch_glu_gemm_nvfp4(const GemmArgs& a, int sf_layout, bool two_level, hipStream_t s) {
  if (two_level)
    return sf_layout == SF_128x4 ? launch<GEMM_NV_GS_128x4>(a, s) : launch<GEMM_NV_GS_ROWMAJOR>(a, s);
  return sf_layout == SF_128x4 ? launch<GEMM_NV_128x4>(a, s) : launch<GEMM_NV_ROWMAJOR>(a, s);
}

}  // namespace glu
