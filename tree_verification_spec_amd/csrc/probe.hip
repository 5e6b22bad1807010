// Achievable HBM read bandwidth on this device: a streaming-read kernel whose
// access pattern is that of the weight GEMMs (each wavefront reads whole
// 1 KB blocks, 16 bytes per lane, with a rolling window of `depth` blocks in
// flight).  It is the measured ceiling the verify step's GEMMs are compared
// with, beside the vendor's peak (the byte lower bound of the besthub.dev
// article, section "Phase 0: Bottleneck Analysis", prices bytes at 90% of
// peak bandwidth; this says how much of the peak a kernel can reach).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/spec.h"

namespace {

// Wave gw of tw reads n blocks of 1 KB.  pattern 0: its own contiguous
// range (blocks gw * n + k); pattern 1: all waves sweep the buffer together
// (block k * tw + gw), as the K-major weight layout does.  Loads past the
// end re-read the last block; the XOR of everything read goes to sink[gw].
template <int D>
__global__ __launch_bounds__(1024) void stream_read_kernel(const uint8_t* __restrict__ src,
                                                           uint32_t n, uint32_t tw,
                                                           int pattern,
                                                           uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const uint32_t gw = __builtin_amdgcn_readfirstlane(blockIdx.x * (blockDim.x >> 6) +
                                                     (threadIdx.x >> 6));
  auto load = [&](uint32_t k) -> uint4 {
    const uint32_t kk = k < n ? k : n - 1;
    const size_t blk = pattern ? (size_t)kk * tw + gw : (size_t)gw * n + kk;
    return *reinterpret_cast<const uint4*>(src + blk * 1024 + lane * 16);
  };
  uint4 w[D];
#pragma unroll
  for (int u = 0; u < D; ++u) w[u] = load(u);
  uint32_t acc = 0;
  for (uint32_t k0 = 0; k0 < n; k0 += D) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
      acc ^= w[u].x ^ w[u].y ^ w[u].z ^ w[u].w;
      w[u] = load(k0 + u + D);
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o, 64);
  if (lane == 0) sink[gw] = acc;
}

template <int D>
hipError_t launch_stream(const void* src, uint32_t n, int grid, int waves, int pattern,
                         uint32_t* sink, hipStream_t s) {
  stream_read_kernel<D><<<grid, waves * 64, 0, s>>>((const uint8_t*)src, n,
                                                    (uint32_t)(grid * waves), pattern, sink);
  return hipGetLastError();
}

}  // namespace

extern "C" int32_t spec_probe_read_bandwidth(const void* d_src, size_t bytes, int32_t grid,
                                             int32_t waves, int32_t depth, int32_t pattern,
                                             uint32_t* d_sink, void* hip_stream) {
  if (!d_src || !d_sink || grid < 1 || waves < 1 || waves > 16 || (pattern != 0 && pattern != 1))
    return SPEC_E_INVAL;
  const size_t tw = (size_t)grid * waves;
  if (bytes == 0 || bytes % (1024 * tw)) return SPEC_E_INVAL;
  const size_t n = bytes / 1024 / tw;
  if (n > 0xFFFFFFFFull) return SPEC_E_INVAL;
  hipStream_t s = (hipStream_t)hip_stream;
  hipError_t e;
  switch (depth) {
    case 4: e = launch_stream<4>(d_src, (uint32_t)n, grid, waves, pattern, d_sink, s); break;
    case 8: e = launch_stream<8>(d_src, (uint32_t)n, grid, waves, pattern, d_sink, s); break;
    case 12: e = launch_stream<12>(d_src, (uint32_t)n, grid, waves, pattern, d_sink, s); break;
    case 16: e = launch_stream<16>(d_src, (uint32_t)n, grid, waves, pattern, d_sink, s); break;
    default: return SPEC_E_INVAL;
  }
  return e == hipSuccess ? SPEC_OK : SPEC_E_HIP;
}
