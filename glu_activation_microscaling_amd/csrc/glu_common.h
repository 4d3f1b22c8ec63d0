// Enumerations shared by the host layer and the kernels; the values are those of the
// public C ABI (glu_mx.h).
#pragma once

namespace glu {

enum { SWIGLU = 0, GEGLU_TANH = 1, GEGLU_ERF = 2, RELU2 = 3 };
enum { SPLIT = 0, PAIRED = 1 };
enum { ROWWISE = 1, COLWISE = 2, SF_SWIZZLED = 4 };  // MXFP8 flags
enum { SF_ROWMAJOR = 0, SF_128x4 = 1 };
enum { FMT_E4M3 = 0, FMT_E2M1 = 1 };                // GEMM operand codes

}  // namespace glu
