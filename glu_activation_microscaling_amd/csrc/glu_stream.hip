// Streaming probe: the practical HBM ceiling for a given mix of read and write streams, the
// yardstick the fused kernels are measured against beside the nominal 8 TB/s.
//
// Each thread moves one 16-byte vector per source (non-temporal loads) and one 4-, 8- or
// 16-byte piece per destination (non-temporal stores); workgroup b covers vectors [256 b, 256 b + 256),
// so consecutive workgroups (dealt round-robin to the XCDs) stream consecutive addresses.
// This is the shape that measured fastest for plain streams on gfx950 (one vector per thread,
// non-temporal both ways, no per-XCD runs).  The destinations receive data derived from every
// source (their XOR, plus the destination's index), so no load can be dropped.
#include "glu_device.h"
#include "glu_launch.h"

namespace glu {
namespace {

constexpr int SP_THREADS = 256;

template <int NSRC, int NDST, int DB>
__global__ __launch_bounds__(SP_THREADS) void k_stream(StreamArgs a) {
  const int64_t i = (int64_t)blockIdx.x * SP_THREADS + threadIdx.x;
  if (i >= a.n_vec) return;
  const u32x4* s0 = static_cast<const u32x4*>(a.src[0]);
  u32x4 x = __builtin_nontemporal_load(s0 + i);
  if constexpr (NSRC > 1) x ^= __builtin_nontemporal_load(static_cast<const u32x4*>(a.src[1]) + i);
  if constexpr (NSRC > 2) x ^= __builtin_nontemporal_load(static_cast<const u32x4*>(a.src[2]) + i);
#pragma unroll
  for (int k = 0; k < NDST; k++) {
    if constexpr (DB == 16) {
      const u32x4 y = x + (u32x4){(uint32_t)k, 0u, 0u, 0u};
      __builtin_nontemporal_store(y, static_cast<u32x4*>(a.dst[k]) + i);
    } else if constexpr (DB == 8) {
      const u32x2 y = {(x.x ^ x.z) + (uint32_t)k, x.y ^ x.w};
      __builtin_nontemporal_store(y, static_cast<u32x2*>(a.dst[k]) + i);
    } else {
      const uint32_t y = (x.x ^ x.y ^ x.z ^ x.w) + (uint32_t)k;
      __builtin_nontemporal_store(y, static_cast<uint32_t*>(a.dst[k]) + i);
    }
  }
}

template <int NSRC, int NDST>
hipError_t by_width(const StreamArgs& a, dim3 grid, hipStream_t s) {
  switch (a.dst_bytes) {
    case 16: return launch_kernel(k_stream<NSRC, NDST, 16>, grid, dim3(SP_THREADS), s, a);
    case 8: return launch_kernel(k_stream<NSRC, NDST, 8>, grid, dim3(SP_THREADS), s, a);
    default: return launch_kernel(k_stream<NSRC, NDST, 4>, grid, dim3(SP_THREADS), s, a);
  }
}

template <int NSRC>
hipError_t by_dst(const StreamArgs& a, dim3 grid, hipStream_t s) {
  switch (a.n_dst) {
    case 1: return by_width<NSRC, 1>(a, grid, s);
    case 2: return by_width<NSRC, 2>(a, grid, s);
    case 3: return by_width<NSRC, 3>(a, grid, s);
    default: return by_width<NSRC, 4>(a, grid, s);
  }
}

}  // namespace

hipError_t launch_stream_probe(const StreamArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)((a.n_vec + SP_THREADS - 1) / SP_THREADS));
  switch (a.n_src) {
    case 1: return by_dst<1>(a, grid, s);
    case 2: return by_dst<2>(a, grid, s);
    default: return by_dst<3>(a, grid, s);
  }
}

}  // namespace glu
