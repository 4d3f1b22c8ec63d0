// C-ABI entry points: host-side validation, then one kernel launch on the caller's stream.
//
// Contract ("feat(phyai-kernel): add Thor NVFP4 GeGLU kernel for pi0.5", Supported
// contract and Known limits: caller-owned buffers, unsupported inputs fail before launch,
// no hidden fallback; "Add swiglu + MXFP8 fused CuTe DSL kernel", Numerics and tests:
// launcher guards for the 32-bit bound, pointer alignment and geometry; "[WS1] Add
// batch-invariant h_aggregate kernel", Supported profile and fail-closed behavior: no silent
// copies).  Every check runs before any HIP call, and the glu_check_* exports run exactly
// the same checks without a device.
#include "../../include/glu_mx.h"

#include <hip/hip_runtime.h>

#include <initializer_list>

#include "glu_launch.h"

namespace {

using glu::BF16Args;
using glu::MxArgs;
using glu::NvArgs;
using glu::GemmArgs;

// Upper bound on MXFP8 tiles per launch (counted with the smallest tile, 32 x 64), so the
// tile index and the workgroup count stay within 32 bits.
constexpr int64_t kMaxTiles = (int64_t)1 << 30;
// Largest row pitch, in bytes, of an MXFP8 kernel operand: the kernels address 32 rows from a
// per-piece base with 32-bit offsets that must stay below 2^31.
constexpr int64_t kMaxMxPitchBytes = (int64_t)1 << 25;
// Largest row pitch, in bytes, of an MXFP8 code output (rowwise: the quantized matrix's
// width; colwise: M): the kernels address 128 output rows from a per-tile base with 32-bit
// offsets that must stay below 2^31.
constexpr int64_t kMaxMxOutPitch = (int64_t)1 << 24;
// Largest operand width (columns) of an NVFP4 launch: the kernels address one row from a
// per-row base with 32-bit offsets (FP32 hook loads 4 bytes per column; 128x4 scales of the
// backward's [M, 2N] reach 16 bytes per column) that must stay below 2^31.
constexpr int64_t kMaxNvWidth = (int64_t)1 << 26;
// Bytes an operand or output of the GEMM kernels may span (32-bit offsets from its base).
constexpr int64_t kOffsetLimit = (int64_t)1 << 31;

// Output pitches of an MXFP8 launch whose quantized matrix is [M, width].
glu_status check_mx_pitch(int flags, int64_t M, int64_t width) {
  if ((flags & glu::ROWWISE) && width > kMaxMxOutPitch) return GLU_ERR_SHAPE;
  if ((flags & glu::COLWISE) && M > kMaxMxOutPitch) return GLU_ERR_SHAPE;
  return GLU_OK;
}

// Byte extent of a row-major matrix: ((rows - 1) * ld + cols) * esz, or -1 on overflow.
int64_t extent_bytes(int64_t rows, int64_t cols, int64_t ld, int64_t esz) {
  int64_t a, b, c;
  if (__builtin_mul_overflow(rows - 1, ld, &a)) return -1;
  if (__builtin_add_overflow(a, cols, &b)) return -1;
  if (__builtin_mul_overflow(b, esz, &c)) return -1;
  return c;
}

struct Operand {
  uintptr_t base;
  int64_t rows, cols, ld, esz;  // cols and ld in elements
  int64_t bytes;                // extent, -1 on overflow
};

Operand mat(const void* p, int64_t rows, int64_t cols, int64_t ld, int64_t esz) {
  return Operand{(uintptr_t)p, rows, cols, ld, esz, extent_bytes(rows, cols, ld, esz)};
}

// True when the two operands may share a byte.  Operands with the same byte row stride
// are tested row by row (so [gate | up] halves of one buffer, or [dGate | dUp] outputs, do
// not count as overlapping); otherwise the byte spans are compared, which can only err
// on the side of rejecting.
bool overlaps(const Operand& A, const Operand& B) {
  if (A.base == 0 || B.base == 0) return false;
  const uintptr_t ahi = A.base + (uintptr_t)A.bytes, bhi = B.base + (uintptr_t)B.bytes;
  if (!(A.base < bhi && B.base < ahi)) return false;
  const int64_t L = A.ld * A.esz;
  if (L != B.ld * B.esz || L <= 0) return true;
  const int64_t wa = A.cols * A.esz, wb = B.cols * B.esz;
  const int64_t d = (int64_t)(B.base - A.base);  // two's complement difference
  // rows r of A and r' of B meet iff d - k L lies in (-wb, wa) for k = r - r'
  auto floordiv = [](int64_t x, int64_t y) { return x / y - ((x % y != 0) && ((x < 0) != (y < 0))); };
  for (int64_t k = floordiv(d - wa, L); k <= floordiv(d + wb, L) + 1; k++) {
    if (k > A.rows - 1 || k < -(B.rows - 1)) continue;
    const int64_t off = d - k * L;
    if (off > -wb && off < wa) return true;
  }
  return false;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool valid_act(int act) { return act >= glu::SWIGLU && act <= glu::RELU2; }
bool valid_layout(int l) { return l == glu::SPLIT || l == glu::PAIRED; }
// MXFP8 flags: one or both directions, optionally the 128x4 scale layout.
bool valid_flags(int f) {
  const int dir = f & ~glu::SF_SWIZZLED;
  return dir == glu::ROWWISE || dir == glu::COLWISE || dir == (glu::ROWWISE | glu::COLWISE);
}

// Shared checks on the BF16 operands.
glu_status check_inputs(int act, int layout, int64_t N, const void* gate, const void* up,
                        int64_t ld_in) {
  if (!valid_act(act) || !valid_layout(layout)) return GLU_ERR_ARG;
  if (gate == nullptr) return GLU_ERR_NULL;
  if (layout == glu::SPLIT && up == nullptr) return GLU_ERR_NULL;
  if (layout == glu::PAIRED && up != nullptr) return GLU_ERR_ARG;
  if (ld_in < (layout == glu::PAIRED ? 2 * N : N)) return GLU_ERR_STRIDE;
  return GLU_OK;
}

// A [rows, nb] MXFP8 scale matrix: row-major, or the zero-padded 128x4 layout.
Operand mx_scales(const void* p, int64_t rows, int64_t nb, int flags) {
  const int64_t bytes = glu_mxfp8_sf_bytes(rows, 32 * nb, (flags & glu::SF_SWIZZLED) ? 1 : 0);
  if (bytes < 0) return Operand{(uintptr_t)p, 1, 0, 0, 1, -1};  // extent overflows
  return mat(p, 1, bytes, bytes, 1);
}

bool any_overflow(std::initializer_list<Operand> ops) {
  for (const Operand& o : ops)
    if (o.base != 0 && (o.bytes < 0 || o.base + (uintptr_t)o.bytes < o.base)) return true;
  return false;
}

glu_status check_no_overlap(std::initializer_list<Operand> outs, std::initializer_list<Operand> ins) {
  for (auto i = outs.begin(); i != outs.end(); ++i) {
    for (const Operand& in : ins)
      if (overlaps(*i, in)) return GLU_ERR_OVERLAP;
    for (auto j = i + 1; j != outs.end(); ++j)
      if (overlaps(*i, *j)) return GLU_ERR_OVERLAP;
  }
  return GLU_OK;
}

glu_status check_mx_outputs(int flags, uint8_t* q_row, uint8_t* s_row, uint8_t* q_col,
                            uint8_t* s_col) {
  if (!valid_flags(flags)) return GLU_ERR_ARG;
  if (flags & glu::ROWWISE) {
    if (!q_row || !s_row) return GLU_ERR_NULL;
  } else if (q_row || s_row) {
    return GLU_ERR_ARG;
  }
  if (flags & glu::COLWISE) {
    if (!q_col || !s_col) return GLU_ERR_NULL;
  } else if (q_col || s_col) {
    return GLU_ERR_ARG;
  }
  return GLU_OK;
}

glu_status status_of(hipError_t e) { return e == hipSuccess ? GLU_OK : GLU_ERR_HIP; }

}  // namespace

extern "C" {

int glu_version(void) { return 100; }

const char* glu_status_string(glu_status s) {
  switch (s) {
    case GLU_OK: return "ok";
    case GLU_ERR_NULL: return "a required pointer is NULL";
    case GLU_ERR_SHAPE: return "unsupported or overflowing shape";
    case GLU_ERR_ALIGN: return "a base pointer is not 16-byte aligned";
    case GLU_ERR_STRIDE: return "bad row stride";
    case GLU_ERR_ARG: return "bad enum, flag or disabled-output pointer";
    case GLU_ERR_OVERLAP: return "an output overlaps an input or another output";
    case GLU_ERR_UNSUPPORTED: return "combination not implemented";
    case GLU_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

int64_t glu_mxfp8_sf_bytes(int64_t rows, int64_t cols, int swizzled) {
  if (rows < 0 || cols < 0 || cols % 32 != 0 || (swizzled != 0 && swizzled != 1)) return -1;
  const int64_t nb = cols / 32;
  const int64_t rp = swizzled ? (rows + 127) / 128 * 128 : rows;
  const int64_t cp = swizzled ? (nb + 3) / 4 * 4 : nb;
  int64_t r;
  return __builtin_mul_overflow(rp, cp, &r) ? -1 : r;
}

int64_t glu_nvfp4_sf_bytes(int64_t M, int64_t H, int sf_layout) {
  if (M < 0 || H < 0 || H % 16 != 0) return -1;
  const int64_t nb = H / 16;
  if (sf_layout == glu::SF_ROWMAJOR) {
    int64_t r;
    return __builtin_mul_overflow(M, nb, &r) ? -1 : r;
  }
  if (sf_layout == glu::SF_128x4) {
    int64_t r;
    const int64_t rp = (M + 127) / 128 * 128, cp = (nb + 3) / 4 * 4;
    return __builtin_mul_overflow(rp, cp, &r) ? -1 : r;
  }
  return -1;
}

glu_status glu_check_fwd(int act, int layout, int64_t M, int64_t N, const uint16_t* gate,
                         const uint16_t* up, int64_t ld_in, uint16_t* h, int64_t ld_h) {
  if (!valid_act(act) || !valid_layout(layout)) return GLU_ERR_ARG;
  if (M < 0 || N < 0) return GLU_ERR_SHAPE;
  if (M == 0 || N == 0) return GLU_OK;
  glu_status st = check_inputs(act, layout, N, gate, up, ld_in);
  if (st != GLU_OK) return st;
  if (h == nullptr) return GLU_ERR_NULL;
  if (ld_h < N) return GLU_ERR_STRIDE;
  const int64_t in_cols = layout == glu::PAIRED ? 2 * N : N;
  const bool flat = ld_in == in_cols && ld_h == N;
  if (!flat && (ld_in % 8 != 0 || ld_h % 8 != 0)) return GLU_ERR_STRIDE;
  if (!aligned16(gate) || !aligned16(up) || !aligned16(h)) return GLU_ERR_ALIGN;
  const Operand G = mat(gate, M, in_cols, ld_in, 2), U = mat(up, M, N, ld_in, 2),
                Hh = mat(h, M, N, ld_h, 2);
  if (any_overflow({G, U, Hh})) return GLU_ERR_SHAPE;
  return check_no_overlap({Hh}, {G, U});
}

glu_status glu_check_bwd(int act, int layout, int64_t M, int64_t N, const uint16_t* gate,
                         const uint16_t* up, int64_t ld_in, const uint16_t* dh, int64_t ld_dh,
                         uint16_t* da, uint16_t* db, int64_t ld_out) {
  if (!valid_act(act) || !valid_layout(layout)) return GLU_ERR_ARG;
  if (M < 0 || N < 0) return GLU_ERR_SHAPE;
  if (M == 0 || N == 0) return GLU_OK;
  glu_status st = check_inputs(act, layout, N, gate, up, ld_in);
  if (st != GLU_OK) return st;
  if (dh == nullptr || da == nullptr) return GLU_ERR_NULL;
  if (layout == glu::SPLIT && db == nullptr) return GLU_ERR_NULL;
  if (layout == glu::PAIRED && db != nullptr) return GLU_ERR_ARG;
  const int64_t in_cols = layout == glu::PAIRED ? 2 * N : N;
  if (ld_dh < N || ld_out < in_cols) return GLU_ERR_STRIDE;
  const bool flat = ld_in == in_cols && ld_dh == N && ld_out == in_cols;
  if (!flat && (ld_in % 8 != 0 || ld_dh % 8 != 0 || ld_out % 8 != 0)) return GLU_ERR_STRIDE;
  if (!aligned16(gate) || !aligned16(up) || !aligned16(dh) || !aligned16(da) || !aligned16(db))
    return GLU_ERR_ALIGN;
  const Operand G = mat(gate, M, in_cols, ld_in, 2), U = mat(up, M, N, ld_in, 2),
                D = mat(dh, M, N, ld_dh, 2), A = mat(da, M, in_cols, ld_out, 2),
                B = mat(db, M, N, ld_out, 2);
  if (any_overflow({G, U, D, A, B})) return GLU_ERR_SHAPE;
  // In place: the gradients overwrite the operands they were computed from.
  const bool in_place = ld_out == ld_in && da == gate && (layout == glu::PAIRED || db == up);
  if (in_place) return check_no_overlap({A, B}, {D});
  return check_no_overlap({A, B}, {G, U, D});
}

glu_status glu_check_fwd_mxfp8(int act, int layout, int64_t M, int64_t N, const uint16_t* gate,
                               const uint16_t* up, int64_t ld_in, int flags, uint8_t* q_row,
                               uint8_t* s_row, uint8_t* q_col, uint8_t* s_col) {
  if (!valid_act(act) || !valid_layout(layout) || !valid_flags(flags)) return GLU_ERR_ARG;
  if (M < 0 || N < 0) return GLU_ERR_SHAPE;
  if (M == 0 || N == 0) return GLU_OK;
  glu_status st = check_inputs(act, layout, N, gate, up, ld_in);
  if (st != GLU_OK) return st;
  if ((st = check_mx_outputs(flags, q_row, s_row, q_col, s_col)) != GLU_OK) return st;
  if (N % 32 != 0 || ((flags & glu::COLWISE) && M % 32 != 0)) return GLU_ERR_SHAPE;
  if ((st = check_mx_pitch(flags, M, N)) != GLU_OK) return st;
  if (ld_in % 8 != 0 || ld_in > kMaxMxPitchBytes / 2) return GLU_ERR_STRIDE;
  if (!aligned16(gate) || !aligned16(up) || !aligned16(q_row) || !aligned16(s_row) ||
      !aligned16(q_col) || !aligned16(s_col))
    return GLU_ERR_ALIGN;
  const int64_t in_cols = layout == glu::PAIRED ? 2 * N : N;
  const Operand G = mat(gate, M, in_cols, ld_in, 2), U = mat(up, M, N, ld_in, 2),
                QR = mat(q_row, M, N, N, 1), SR = mx_scales(s_row, M, N / 32, flags),
                QC = mat(q_col, N, M, M, 1), SC = mx_scales(s_col, N, M / 32, flags);
  if (any_overflow({G, U, QR, SR, QC, SC})) return GLU_ERR_SHAPE;
  if (((M + 31) / 32) * ((N + 63) / 64) > kMaxTiles) return GLU_ERR_SHAPE;
  return check_no_overlap({QR, SR, QC, SC}, {G, U});
}

glu_status glu_check_bwd_mxfp8(int act, int layout, int64_t M, int64_t N, const uint16_t* gate,
                               const uint16_t* up, int64_t ld_in, const uint16_t* dh,
                               int64_t ld_dh, int flags, uint8_t* q_row, uint8_t* s_row,
                               uint8_t* q_col, uint8_t* s_col) {
  if (!valid_act(act) || !valid_layout(layout) || !valid_flags(flags)) return GLU_ERR_ARG;
  if (M < 0 || N < 0) return GLU_ERR_SHAPE;
  if (layout == glu::PAIRED) return GLU_ERR_UNSUPPORTED;
  if (M == 0 || N == 0) return GLU_OK;
  glu_status st = check_inputs(act, layout, N, gate, up, ld_in);
  if (st != GLU_OK) return st;
  if (dh == nullptr) return GLU_ERR_NULL;
  if ((st = check_mx_outputs(flags, q_row, s_row, q_col, s_col)) != GLU_OK) return st;
  if (N % 32 != 0 || ((flags & glu::COLWISE) && M % 32 != 0)) return GLU_ERR_SHAPE;
  if ((st = check_mx_pitch(flags, M, 2 * N)) != GLU_OK) return st;
  if (ld_dh < N) return GLU_ERR_STRIDE;
  if (ld_in % 8 != 0 || ld_dh % 8 != 0) return GLU_ERR_STRIDE;
  if (ld_in > kMaxMxPitchBytes / 2 || ld_dh > kMaxMxPitchBytes / 2) return GLU_ERR_STRIDE;
  if (!aligned16(gate) || !aligned16(up) || !aligned16(dh) || !aligned16(q_row) ||
      !aligned16(s_row) || !aligned16(q_col) || !aligned16(s_col))
    return GLU_ERR_ALIGN;
  int64_t N2;
  if (__builtin_mul_overflow(N, (int64_t)2, &N2)) return GLU_ERR_SHAPE;
  const Operand G = mat(gate, M, N, ld_in, 2), U = mat(up, M, N, ld_in, 2),
                D = mat(dh, M, N, ld_dh, 2), QR = mat(q_row, M, N2, N2, 1),
                SR = mx_scales(s_row, M, N2 / 32, flags), QC = mat(q_col, N2, M, M, 1),
                SC = mx_scales(s_col, N2, M / 32, flags);
  if (any_overflow({G, U, D, QR, SR, QC, SC})) return GLU_ERR_SHAPE;
  if (((M + 31) / 32) * ((N + 63) / 64) > kMaxTiles) return GLU_ERR_SHAPE;
  return check_no_overlap({QR, SR, QC, SC}, {G, U, D});
}

glu_status glu_check_fwd_nvfp4(int act, int layout, int64_t M, int64_t H, const uint16_t* gate,
                               const uint16_t* up, int64_t ld_in, uint8_t* q, uint8_t* sf,
                               int sf_layout) {
  if (!valid_act(act) || !valid_layout(layout)) return GLU_ERR_ARG;
  if (sf_layout != glu::SF_ROWMAJOR && sf_layout != glu::SF_128x4) return GLU_ERR_ARG;
  if (M < 0 || H < 0) return GLU_ERR_SHAPE;
  if (M == 0 || H == 0) return GLU_OK;
  glu_status st = check_inputs(act, layout, H, gate, up, ld_in);
  if (st != GLU_OK) return st;
  if (q == nullptr || sf == nullptr) return GLU_ERR_NULL;
  if (H % 16 != 0 || H > kMaxNvWidth) return GLU_ERR_SHAPE;
  if (ld_in % 8 != 0) return GLU_ERR_STRIDE;
  if (!aligned16(gate) || !aligned16(up) || !aligned16(q) || !aligned16(sf)) return GLU_ERR_ALIGN;
  const int64_t sfb = glu_nvfp4_sf_bytes(M, H, sf_layout);
  if (sfb < 0) return GLU_ERR_SHAPE;
  const int64_t in_cols = layout == glu::PAIRED ? 2 * H : H;
  const Operand G = mat(gate, M, in_cols, ld_in, 2), U = mat(up, M, H, ld_in, 2),
                Q = mat(q, M, H / 2, H / 2, 1), S = mat(sf, 1, sfb, sfb, 1);
  if (any_overflow({G, U, Q, S})) return GLU_ERR_SHAPE;
  return check_no_overlap({Q, S}, {G, U});
}

glu_status glu_check_amax(int act, int layout, int64_t M, int64_t N, const uint16_t* gate,
                          const uint16_t* up, int64_t ld_in, float* amax) {
  if (!valid_act(act) || !valid_layout(layout)) return GLU_ERR_ARG;
  if (M < 0 || N < 0) return GLU_ERR_SHAPE;
  if (amax == nullptr) return GLU_ERR_NULL;
  if (((uintptr_t)amax & 3u) != 0) return GLU_ERR_ALIGN;
  if (M == 0 || N == 0) return GLU_OK;
  glu_status st = check_inputs(act, layout, N, gate, up, ld_in);
  if (st != GLU_OK) return st;
  if (N % 16 != 0 || N > kMaxNvWidth) return GLU_ERR_SHAPE;
  if (ld_in % 8 != 0) return GLU_ERR_STRIDE;
  if (!aligned16(gate) || !aligned16(up)) return GLU_ERR_ALIGN;
  const int64_t in_cols = layout == glu::PAIRED ? 2 * N : N;
  const Operand G = mat(gate, M, in_cols, ld_in, 2), U = mat(up, M, N, ld_in, 2),
                A = mat(amax, 1, 1, 1, 4);
  if (any_overflow({G, U})) return GLU_ERR_SHAPE;
  return check_no_overlap({A}, {G, U});
}

glu_status glu_check_fwd_nvfp4_gs(int act, int layout, int64_t M, int64_t H,
                                  const uint16_t* gate, const uint16_t* up, int64_t ld_in,
                                  const float* amax, uint8_t* q, uint8_t* sf, int sf_layout) {
  glu_status st = glu_check_fwd_nvfp4(act, layout, M, H, gate, up, ld_in, q, sf, sf_layout);
  if (st != GLU_OK || M == 0 || H == 0) return st;
  if (amax == nullptr) return GLU_ERR_NULL;
  if (((uintptr_t)amax & 3u) != 0) return GLU_ERR_ALIGN;
  const int64_t sfb = glu_nvfp4_sf_bytes(M, H, sf_layout);
  const Operand A = mat(amax, 1, 1, 1, 4), Q = mat(q, M, H / 2, H / 2, 1),
                S = mat(sf, 1, sfb, sfb, 1);
  return check_no_overlap({Q, S}, {A});
}

// Operands of the merged gate/up block-scaled GEMM.  The kernels address each operand from
// its base with 32-bit byte offsets, so every operand and output extent stays below 2^31
// bytes.  A K step is one 128-byte line of an operand row: 128 E4M3 or 256 E2M1 codes.
struct GemmOperands {
  Operand X, XS, W, WS;
};
bool valid_gemm_format(int fmt, int w_layout) {
  return (fmt == glu::FMT_E4M3 || fmt == glu::FMT_E2M1) && (w_layout == glu::SPLIT || w_layout == glu::PAIRED);
}
glu_status check_gemm_inputs(int fmt, int64_t M, int64_t N, int64_t K, const uint8_t* xq,
                             const uint8_t* xs, const uint8_t* wq, const uint8_t* ws, GemmOperands* ops) {
  if (xq == nullptr || xs == nullptr || wq == nullptr || ws == nullptr) return GLU_ERR_NULL;
  const int64_t kstep = fmt == glu::FMT_E2M1 ? 256 : 128;
  if (K <= 0 || K % kstep != 0 || N % 128 != 0) return GLU_ERR_SHAPE;
  const int64_t rb = fmt == glu::FMT_E2M1 ? K / 2 : K;   // bytes per operand row
  int64_t xb, wb;
  if (__builtin_mul_overflow(M, rb, &xb) || __builtin_mul_overflow(2 * N, rb, &wb)) return GLU_ERR_SHAPE;
  if (xb >= kOffsetLimit || wb >= kOffsetLimit) return GLU_ERR_SHAPE;
  if (!aligned16(xq) || !aligned16(xs) || !aligned16(wq) || !aligned16(ws)) return GLU_ERR_ALIGN;
  *ops = {mat(xq, M, rb, rb, 1), mat(xs, M, K / 32, K / 32, 1), mat(wq, 2 * N, rb, rb, 1),
          mat(ws, 2 * N, K / 32, K / 32, 1)};
  return GLU_OK;
}

glu_status glu_check_gemm(int act, int fmt, int w_layout, int64_t M, int64_t N, int64_t K,
                          const uint8_t* xq, const uint8_t* xs, const uint8_t* wq,
                          const uint8_t* ws, uint16_t* h, int64_t ld_h) {
  if (!valid_act(act) || !valid_gemm_format(fmt, w_layout)) return GLU_ERR_ARG;
  if (M < 0 || N < 0 || K < 0) return GLU_ERR_SHAPE;
  if (M == 0 || N == 0) return GLU_OK;
  GemmOperands o;
  glu_status st = check_gemm_inputs(fmt, M, N, K, xq, xs, wq, ws, &o);
  if (st != GLU_OK) return st;
  if (h == nullptr) return GLU_ERR_NULL;
  if (ld_h < N) return GLU_ERR_STRIDE;
  if (!aligned16(h) || ld_h % 8 != 0) return GLU_ERR_ALIGN;
  const Operand Hh = mat(h, M, N, ld_h, 2);
  if (any_overflow({Hh}) || Hh.bytes >= kOffsetLimit) return GLU_ERR_SHAPE;
  return check_no_overlap({Hh}, {o.X, o.XS, o.W, o.WS});
}

glu_status glu_check_gemm_mxfp8(int act, int fmt, int w_layout, int64_t M, int64_t N, int64_t K,
                                const uint8_t* xq, const uint8_t* xs, const uint8_t* wq,
                                const uint8_t* ws, uint8_t* q_row, uint8_t* s_row) {
  if (!valid_act(act) || !valid_gemm_format(fmt, w_layout)) return GLU_ERR_ARG;
  if (M < 0 || N < 0 || K < 0) return GLU_ERR_SHAPE;
  if (M == 0 || N == 0) return GLU_OK;
  GemmOperands o;
  glu_status st = check_gemm_inputs(fmt, M, N, K, xq, xs, wq, ws, &o);
  if (st != GLU_OK) return st;
  if (q_row == nullptr || s_row == nullptr) return GLU_ERR_NULL;
  if (!aligned16(q_row) || !aligned16(s_row)) return GLU_ERR_ALIGN;
  const Operand Q = mat(q_row, M, N, N, 1), S = mat(s_row, M, N / 32, N / 32, 1);
  if (any_overflow({Q, S}) || Q.bytes >= kOffsetLimit) return GLU_ERR_SHAPE;
  return check_no_overlap({Q, S}, {o.X, o.XS, o.W, o.WS});
}

glu_status glu_check_gemm_nvfp4(int act, int fmt, int w_layout, int64_t M, int64_t N, int64_t K,
                                const uint8_t* xq, const uint8_t* xs, const uint8_t* wq,
                                const uint8_t* ws, uint8_t* q, uint8_t* sf, int sf_layout) {
  if (!valid_act(act) || !valid_gemm_format(fmt, w_layout)) return GLU_ERR_ARG;
  if (sf_layout != glu::SF_ROWMAJOR && sf_layout != glu::SF_128x4) return GLU_ERR_ARG;
  if (M < 0 || N < 0 || K < 0) return GLU_ERR_SHAPE;
  if (M == 0 || N == 0) return GLU_OK;
  GemmOperands o;
  glu_status st = check_gemm_inputs(fmt, M, N, K, xq, xs, wq, ws, &o);
  if (st != GLU_OK) return st;
  if (q == nullptr || sf == nullptr) return GLU_ERR_NULL;
  if (!aligned16(q) || !aligned16(sf)) return GLU_ERR_ALIGN;
  const int64_t sfb = glu_nvfp4_sf_bytes(M, N, sf_layout);
  if (sfb < 0) return GLU_ERR_SHAPE;
  const Operand Q = mat(q, M, N / 2, N / 2, 1), S = mat(sf, 1, sfb, sfb, 1);
  if (any_overflow({Q, S}) || Q.bytes >= kOffsetLimit || S.bytes >= kOffsetLimit) return GLU_ERR_SHAPE;
  return check_no_overlap({Q, S}, {o.X, o.XS, o.W, o.WS});
}

glu_status glu_check_mx_gemm_f32(int fmt, int w_layout, int64_t M, int64_t N, int64_t K,
                                 const uint8_t* xq, const uint8_t* xs, const uint8_t* wq,
                                 const uint8_t* ws, float* y) {
  if (!valid_gemm_format(fmt, w_layout)) return GLU_ERR_ARG;
  if (M < 0 || N < 0 || K < 0) return GLU_ERR_SHAPE;
  if (M == 0 || N == 0) return GLU_OK;
  GemmOperands o;
  glu_status st = check_gemm_inputs(fmt, M, N, K, xq, xs, wq, ws, &o);
  if (st != GLU_OK) return st;
  if (y == nullptr) return GLU_ERR_NULL;
  if (!aligned16(y)) return GLU_ERR_ALIGN;
  const Operand Y = mat(y, M, 2 * N, 2 * N, 4);
  if (any_overflow({Y}) || Y.bytes >= kOffsetLimit) return GLU_ERR_SHAPE;
  return check_no_overlap({Y}, {o.X, o.XS, o.W, o.WS});
}

glu_status glu_check_bwd_nvfp4(int act, int layout, int64_t M, int64_t N, const uint16_t* gate,
                               const uint16_t* up, int64_t ld_in, const uint16_t* dh,
                               int64_t ld_dh, uint8_t* q, uint8_t* sf, int sf_layout) {
  if (!valid_act(act) || !valid_layout(layout)) return GLU_ERR_ARG;
  if (sf_layout != glu::SF_ROWMAJOR && sf_layout != glu::SF_128x4) return GLU_ERR_ARG;
  if (M < 0 || N < 0) return GLU_ERR_SHAPE;
  if (layout == glu::PAIRED) return GLU_ERR_UNSUPPORTED;
  if (M == 0 || N == 0) return GLU_OK;
  glu_status st = check_inputs(act, layout, N, gate, up, ld_in);
  if (st != GLU_OK) return st;
  if (dh == nullptr || q == nullptr || sf == nullptr) return GLU_ERR_NULL;
  if (N % 16 != 0 || N > kMaxNvWidth) return GLU_ERR_SHAPE;
  if (ld_dh < N) return GLU_ERR_STRIDE;
  if (ld_in % 8 != 0 || ld_dh % 8 != 0) return GLU_ERR_STRIDE;
  if (!aligned16(gate) || !aligned16(up) || !aligned16(dh) || !aligned16(q) || !aligned16(sf))
    return GLU_ERR_ALIGN;
  int64_t N2;
  if (__builtin_mul_overflow(N, (int64_t)2, &N2)) return GLU_ERR_SHAPE;
  const int64_t sfb = glu_nvfp4_sf_bytes(M, N2, sf_layout);
  if (sfb < 0) return GLU_ERR_SHAPE;
  const Operand G = mat(gate, M, N, ld_in, 2), U = mat(up, M, N, ld_in, 2),
                D = mat(dh, M, N, ld_dh, 2), Q = mat(q, M, N, N, 1), S = mat(sf, 1, sfb, sfb, 1);
  if (any_overflow({G, U, D, Q, S})) return GLU_ERR_SHAPE;
  return check_no_overlap({Q, S}, {G, U, D});
}

glu_status glu_check_quant_mxfp8_f32(int64_t M, int64_t N, const float* x, int64_t ld_x,
                                     int flags, uint8_t* q_row, uint8_t* s_row,
                                     uint8_t* q_col, uint8_t* s_col) {
  if (!valid_flags(flags)) return GLU_ERR_ARG;
  if (M < 0 || N < 0) return GLU_ERR_SHAPE;
  if (M == 0 || N == 0) return GLU_OK;
  if (x == nullptr) return GLU_ERR_NULL;
  glu_status st = check_mx_outputs(flags, q_row, s_row, q_col, s_col);
  if (st != GLU_OK) return st;
  if (N % 32 != 0 || ((flags & glu::COLWISE) && M % 32 != 0)) return GLU_ERR_SHAPE;
  if ((st = check_mx_pitch(flags, M, N)) != GLU_OK) return st;
  if (ld_x < N || ld_x % 4 != 0 || ld_x > kMaxMxPitchBytes / 4) return GLU_ERR_STRIDE;
  if (!aligned16(x) || !aligned16(q_row) || !aligned16(s_row) || !aligned16(q_col) ||
      !aligned16(s_col))
    return GLU_ERR_ALIGN;
  const Operand X = mat(x, M, N, ld_x, 4), QR = mat(q_row, M, N, N, 1),
                SR = mx_scales(s_row, M, N / 32, flags), QC = mat(q_col, N, M, M, 1),
                SC = mx_scales(s_col, N, M / 32, flags);
  if (any_overflow({X, QR, SR, QC, SC})) return GLU_ERR_SHAPE;
  if (((M + 31) / 32) * ((N + 63) / 64) > kMaxTiles) return GLU_ERR_SHAPE;
  return check_no_overlap({QR, SR, QC, SC}, {X});
}

glu_status glu_check_quant_nvfp4_f32(int64_t M, int64_t H, const float* x, int64_t ld_x,
                                     uint8_t* q, uint8_t* sf, int sf_layout) {
  if (sf_layout != glu::SF_ROWMAJOR && sf_layout != glu::SF_128x4) return GLU_ERR_ARG;
  if (M < 0 || H < 0) return GLU_ERR_SHAPE;
  if (M == 0 || H == 0) return GLU_OK;
  if (x == nullptr || q == nullptr || sf == nullptr) return GLU_ERR_NULL;
  if (H % 16 != 0 || H > kMaxNvWidth) return GLU_ERR_SHAPE;
  if (ld_x < H || ld_x % 4 != 0) return GLU_ERR_STRIDE;
  if (!aligned16(x) || !aligned16(q) || !aligned16(sf)) return GLU_ERR_ALIGN;
  const int64_t sfb = glu_nvfp4_sf_bytes(M, H, sf_layout);
  if (sfb < 0) return GLU_ERR_SHAPE;
  const Operand X = mat(x, M, H, ld_x, 4), Q = mat(q, M, H / 2, H / 2, 1),
                S = mat(sf, 1, sfb, sfb, 1);
  if (any_overflow({X, Q, S})) return GLU_ERR_SHAPE;
  return check_no_overlap({Q, S}, {X});
}

glu_status glu_check_stream_probe(int n_src, const void* const* src, int n_dst, void* const* dst,
                                  int64_t n_vec, int dst_bytes) {
  if (n_src < 1 || n_src > 3 || n_dst < 1 || n_dst > 4 || (dst_bytes != 4 && dst_bytes != 8 && dst_bytes != 16))
    return GLU_ERR_ARG;
  if (n_vec < 0 || n_vec > ((int64_t)1 << 36)) return GLU_ERR_SHAPE;
  if (src == nullptr || dst == nullptr) return GLU_ERR_NULL;
  if (n_vec == 0) return GLU_OK;
  Operand S[3], D[4];
  for (int k = 0; k < n_src; k++) {
    if (src[k] == nullptr) return GLU_ERR_NULL;
    if (!aligned16(src[k])) return GLU_ERR_ALIGN;
    S[k] = mat(src[k], 1, n_vec * 16, n_vec * 16, 1);
  }
  for (int k = 0; k < n_dst; k++) {
    if (dst[k] == nullptr) return GLU_ERR_NULL;
    if (!aligned16(dst[k])) return GLU_ERR_ALIGN;
    D[k] = mat(dst[k], 1, n_vec * dst_bytes, n_vec * dst_bytes, 1);
  }
  for (int k = 0; k < n_dst; k++) {
    for (int j = 0; j < n_src; j++)
      if (overlaps(D[k], S[j])) return GLU_ERR_OVERLAP;
    for (int j = k + 1; j < n_dst; j++)
      if (overlaps(D[k], D[j])) return GLU_ERR_OVERLAP;
  }
  return GLU_OK;
}

// ---- entry points -----------------------------------------------------------------

glu_status glu_fwd(int act, int layout, int64_t M, int64_t N, const uint16_t* gate,
                   const uint16_t* up, int64_t ld_in, uint16_t* h, int64_t ld_h, void* stream) {
  glu_status st = glu_check_fwd(act, layout, M, N, gate, up, ld_in, h, ld_h);
  if (st != GLU_OK || M == 0 || N == 0) return st;
  BF16Args a{};
  a.act = act;
  a.layout = layout;
  a.M = M;
  a.N = N;
  a.gate = gate;
  a.up = up;
  a.ld_in = ld_in;
  a.out0 = h;
  a.ld_out = ld_h;
  a.flat = ld_in == (layout == glu::PAIRED ? 2 * N : N) && ld_h == N;
  return status_of(glu::launch_glu_fwd_bf16(a, (hipStream_t)stream));
}

glu_status glu_bwd(int act, int layout, int64_t M, int64_t N, const uint16_t* gate,
                   const uint16_t* up, int64_t ld_in, const uint16_t* dh, int64_t ld_dh,
                   uint16_t* da, uint16_t* db, int64_t ld_out, void* stream) {
  glu_status st = glu_check_bwd(act, layout, M, N, gate, up, ld_in, dh, ld_dh, da, db, ld_out);
  if (st != GLU_OK || M == 0 || N == 0) return st;
  const int64_t in_cols = layout == glu::PAIRED ? 2 * N : N;
  BF16Args a{};
  a.act = act;
  a.layout = layout;
  a.M = M;
  a.N = N;
  a.gate = gate;
  a.up = up;
  a.ld_in = ld_in;
  a.dh = dh;
  a.ld_dh = ld_dh;
  a.out0 = da;
  a.out1 = db;
  a.ld_out = ld_out;
  a.flat = ld_in == in_cols && ld_dh == N && ld_out == in_cols;
  return status_of(glu::launch_glu_bwd_bf16(a, (hipStream_t)stream));
}

glu_status glu_fwd_mxfp8(int act, int layout, int64_t M, int64_t N, const uint16_t* gate,
                         const uint16_t* up, int64_t ld_in, int flags, uint8_t* q_row,
                         uint8_t* s_row, uint8_t* q_col, uint8_t* s_col, void* stream) {
  glu_status st = glu_check_fwd_mxfp8(act, layout, M, N, gate, up, ld_in, flags, q_row, s_row,
                                      q_col, s_col);
  if (st != GLU_OK || M == 0 || N == 0) return st;
  MxArgs a{act, layout, flags, M, N, gate, up, ld_in, nullptr, 0, q_row, s_row, q_col, s_col};
  return status_of(glu::launch_glu_fwd_mxfp8(a, (hipStream_t)stream));
}

glu_status glu_bwd_mxfp8(int act, int layout, int64_t M, int64_t N, const uint16_t* gate,
                         const uint16_t* up, int64_t ld_in, const uint16_t* dh, int64_t ld_dh,
                         int flags, uint8_t* q_row, uint8_t* s_row, uint8_t* q_col,
                         uint8_t* s_col, void* stream) {
  glu_status st = glu_check_bwd_mxfp8(act, layout, M, N, gate, up, ld_in, dh, ld_dh, flags,
                                      q_row, s_row, q_col, s_col);
  if (st != GLU_OK || M == 0 || N == 0) return st;
  MxArgs a{act, layout, flags, M, N, gate, up, ld_in, dh, ld_dh, q_row, s_row, q_col, s_col};
  return status_of(glu::launch_glu_bwd_mxfp8(a, (hipStream_t)stream));
}

glu_status glu_fwd_nvfp4(int act, int layout, int64_t M, int64_t H, const uint16_t* gate,
                         const uint16_t* up, int64_t ld_in, uint8_t* q, uint8_t* sf,
                         int sf_layout, void* stream) {
  glu_status st = glu_check_fwd_nvfp4(act, layout, M, H, gate, up, ld_in, q, sf, sf_layout);
  if (st != GLU_OK || M == 0 || H == 0) return st;
  NvArgs a{act, layout, sf_layout, M, H, gate, up, ld_in, q, sf, nullptr, 0, nullptr, nullptr};
  return status_of(glu::launch_glu_fwd_nvfp4(a, (hipStream_t)stream));
}

glu_status glu_amax(int act, int layout, int64_t M, int64_t N, const uint16_t* gate,
                    const uint16_t* up, int64_t ld_in, float* amax, void* stream) {
  glu_status st = glu_check_amax(act, layout, M, N, gate, up, ld_in, amax);
  if (st != GLU_OK) return st;
  NvArgs a{act, layout, glu::SF_ROWMAJOR, M, N, gate, up, ld_in, nullptr, nullptr,
           nullptr, 0, nullptr, amax};
  return status_of(glu::launch_glu_amax(a, (hipStream_t)stream));
}

glu_status glu_fwd_nvfp4_gs(int act, int layout, int64_t M, int64_t H, const uint16_t* gate,
                            const uint16_t* up, int64_t ld_in, const float* amax, uint8_t* q,
                            uint8_t* sf, int sf_layout, void* stream) {
  glu_status st =
      glu_check_fwd_nvfp4_gs(act, layout, M, H, gate, up, ld_in, amax, q, sf, sf_layout);
  if (st != GLU_OK || M == 0 || H == 0) return st;
  NvArgs a{act, layout, sf_layout, M, H, gate, up, ld_in, q, sf, nullptr, 0, amax, nullptr};
  return status_of(glu::launch_glu_fwd_nvfp4_gs(a, (hipStream_t)stream));
}

glu_status glu_gemm(int act, int fmt, int w_layout, int64_t M, int64_t N, int64_t K,
                    const uint8_t* xq, const uint8_t* xs, const uint8_t* wq, const uint8_t* ws,
                    uint16_t* h, int64_t ld_h, void* stream) {
  glu_status st = glu_check_gemm(act, fmt, w_layout, M, N, K, xq, xs, wq, ws, h, ld_h);
  if (st != GLU_OK || M == 0 || N == 0) return st;
  GemmArgs a{act, fmt, w_layout, M, N, K, xq, xs, wq, ws, h, ld_h, nullptr, nullptr, nullptr};
  return status_of(glu::launch_glu_gemm(a, (hipStream_t)stream));
}

glu_status glu_gemm_mxfp8(int act, int fmt, int w_layout, int64_t M, int64_t N, int64_t K,
                          const uint8_t* xq, const uint8_t* xs, const uint8_t* wq,
                          const uint8_t* ws, uint8_t* q_row, uint8_t* s_row, void* stream) {
  glu_status st = glu_check_gemm_mxfp8(act, fmt, w_layout, M, N, K, xq, xs, wq, ws, q_row, s_row);
  if (st != GLU_OK || M == 0 || N == 0) return st;
  GemmArgs a{act, fmt, w_layout, M, N, K, xq, xs, wq, ws, nullptr, 0, q_row, s_row, nullptr};
  return status_of(glu::launch_glu_gemm_mxfp8(a, (hipStream_t)stream));
}

glu_status glu_gemm_nvfp4(int act, int fmt, int w_layout, int64_t M, int64_t N, int64_t K,
                          const uint8_t* xq, const uint8_t* xs, const uint8_t* wq,
                          const uint8_t* ws, uint8_t* q, uint8_t* sf, int sf_layout, void* stream) {
  glu_status st = glu_check_gemm_nvfp4(act, fmt, w_layout, M, N, K, xq, xs, wq, ws, q, sf, sf_layout);
  if (st != GLU_OK || M == 0 || N == 0) return st;
  GemmArgs a{act, fmt, w_layout, M, N, K, xq, xs, wq, ws, nullptr, 0, q, sf, nullptr};
  return status_of(glu::launch_glu_gemm_nvfp4(a, sf_layout, false, (hipStream_t)stream));
}

glu_status glu_check_gemm_nvfp4_gs(int act, int fmt, int w_layout, int64_t M, int64_t N,
                                   int64_t K, const uint8_t* xq, const uint8_t* xs,
                                   const uint8_t* wq, const uint8_t* ws, const float* amax,
                                   uint8_t* q, uint8_t* sf, int sf_layout) {
  glu_status st = glu_check_gemm_nvfp4(act, fmt, w_layout, M, N, K, xq, xs, wq, ws, q, sf, sf_layout);
  if (st != GLU_OK || M == 0 || N == 0) return st;
  if (amax == nullptr) return GLU_ERR_NULL;
  if ((uintptr_t)amax % 4 != 0) return GLU_ERR_ALIGN;
  const int64_t sfb = glu_nvfp4_sf_bytes(M, N, sf_layout);
  const Operand A = mat(amax, 1, 1, 1, 4), Q = mat(q, M, N / 2, N / 2, 1), S = mat(sf, 1, sfb, sfb, 1);
  return check_no_overlap({Q, S}, {A});
}

glu_status glu_gemm_nvfp4_gs(int act, int fmt, int w_layout, int64_t M, int64_t N, int64_t K,
                             const uint8_t* xq, const uint8_t* xs, const uint8_t* wq,
                             const uint8_t* ws, const float* amax, uint8_t* q, uint8_t* sf,
                             int sf_layout, void* stream) {
  glu_status st =
      glu_check_gemm_nvfp4_gs(act, fmt, w_layout, M, N, K, xq, xs, wq, ws, amax, q, sf, sf_layout);
  if (st != GLU_OK || M == 0 || N == 0) return st;
  GemmArgs a{act, fmt, w_layout, M, N, K, xq, xs, wq, ws, nullptr, 0, q, sf, nullptr, amax};
  return status_of(glu::launch_glu_gemm_nvfp4(a, sf_layout, true, (hipStream_t)stream));
}

glu_status glu_mx_gemm_f32(int fmt, int w_layout, int64_t M, int64_t N, int64_t K,
                           const uint8_t* xq, const uint8_t* xs, const uint8_t* wq,
                           const uint8_t* ws, float* y, void* stream) {
  glu_status st = glu_check_mx_gemm_f32(fmt, w_layout, M, N, K, xq, xs, wq, ws, y);
  if (st != GLU_OK || M == 0 || N == 0) return st;
  GemmArgs a{glu::SWIGLU, fmt, w_layout, M, N, K, xq, xs, wq, ws, nullptr, 0, nullptr, nullptr, y};
  return status_of(glu::launch_mx_gemm_f32(a, (hipStream_t)stream));
}

glu_status glu_bwd_nvfp4(int act, int layout, int64_t M, int64_t N, const uint16_t* gate,
                         const uint16_t* up, int64_t ld_in, const uint16_t* dh, int64_t ld_dh,
                         uint8_t* q, uint8_t* sf, int sf_layout, void* stream) {
  glu_status st =
      glu_check_bwd_nvfp4(act, layout, M, N, gate, up, ld_in, dh, ld_dh, q, sf, sf_layout);
  if (st != GLU_OK || M == 0 || N == 0) return st;
  NvArgs a{act, layout, sf_layout, M, N, gate, up, ld_in, q, sf, dh, ld_dh, nullptr, nullptr};
  return status_of(glu::launch_glu_bwd_nvfp4(a, (hipStream_t)stream));
}

glu_status glu_quant_mxfp8_f32(int64_t M, int64_t N, const float* x, int64_t ld_x, int flags,
                               uint8_t* q_row, uint8_t* s_row, uint8_t* q_col, uint8_t* s_col,
                               void* stream) {
  glu_status st = glu_check_quant_mxfp8_f32(M, N, x, ld_x, flags, q_row, s_row, q_col, s_col);
  if (st != GLU_OK || M == 0 || N == 0) return st;
  MxArgs a{glu::SWIGLU, glu::SPLIT, flags, M, N, x, nullptr, ld_x, nullptr, 0,
           q_row, s_row, q_col, s_col};
  return status_of(glu::launch_quant_mxfp8_f32(a, (hipStream_t)stream));
}

glu_status glu_quant_nvfp4_f32(int64_t M, int64_t H, const float* x, int64_t ld_x, uint8_t* q,
                               uint8_t* sf, int sf_layout, void* stream) {
  glu_status st = glu_check_quant_nvfp4_f32(M, H, x, ld_x, q, sf, sf_layout);
  if (st != GLU_OK || M == 0 || H == 0) return st;
  NvArgs a{glu::SWIGLU, glu::SPLIT, sf_layout, M, H, x, nullptr, ld_x, q, sf, nullptr, 0, nullptr, nullptr};
  return status_of(glu::launch_quant_nvfp4_f32(a, (hipStream_t)stream));
}

glu_status glu_stream_probe(int n_src, const void* const* src, int n_dst, void* const* dst,
                            int64_t n_vec, int dst_bytes, void* stream) {
  glu_status st = glu_check_stream_probe(n_src, src, n_dst, dst, n_vec, dst_bytes);
  if (st != GLU_OK || n_vec == 0) return st;
  glu::StreamArgs a{n_src, n_dst, dst_bytes, n_vec, {nullptr, nullptr, nullptr}, {nullptr, nullptr, nullptr, nullptr}};
  for (int k = 0; k < n_src; k++) a.src[k] = src[k];
  for (int k = 0; k < n_dst; k++) a.dst[k] = dst[k];
  return status_of(glu::launch_stream_probe(a, (hipStream_t)stream));
}

}  // extern "C"
