// Achievable HBM read bandwidth on this device: a streaming-read kernel whose
// access pattern is that of the weight GEMMs (each wavefront reads whole
// 1 KB blocks, 16 bytes per lane, with a rolling window of `depth` blocks in
// flight).  It is the measured ceiling the verify step's GEMMs are compared
// with, beside the vendor's peak (the byte lower bound of the besthub.dev
// article, section "Phase 0: Bottleneck Analysis", prices bytes at 90% of
// peak bandwidth; this says how much of the peak a kernel can reach).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

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

hipError_t launch_depth(int depth, const void* src, uint32_t n, int grid, int waves,
                        int pattern, uint32_t* sink, hipStream_t s) {
  switch (depth) {
    case 4: return launch_stream<4>(src, n, grid, waves, pattern, sink, s);
    case 8: return launch_stream<8>(src, n, grid, waves, pattern, sink, s);
    case 12: return launch_stream<12>(src, n, grid, waves, pattern, sink, s);
    case 16: return launch_stream<16>(src, n, grid, waves, pattern, sink, s);
    default: return hipErrorInvalidValue;
  }
}

// out[0] = XOR of sink[0, n): one workgroup, a fixed order of XORs (the
// result does not depend on it)
__global__ __launch_bounds__(256) void xor_reduce_kernel(const uint32_t* __restrict__ sink,
                                                         int n, uint32_t* __restrict__ out) {
  __shared__ uint32_t part[4];
  uint32_t acc = 0;
  for (int i = threadIdx.x; i < n; i += 256) acc ^= sink[i];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o, 64);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) out[0] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

// The variant that allocates nothing keeps the per-wavefront checksums in
// this array: one copy per device, held until the process ends.  Host code
// never passes the symbol itself to a kernel (in host code it is a stand-in,
// not a device address); it passes the device address that
// hipGetSymbolAddress returns, looked up once per device.
constexpr int kScratchWaves = 65536;  // 256 KB: grids of at most 65536 wavefronts
static __device__ __align__(256) uint32_t scratch[kScratchWaves];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
uint32_t* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch`, or nullptr if it cannot be found.
uint32_t* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = static_cast<uint32_t*>(ptr);
  }
  return g_scratch_ptr[dev];
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
  if (depth != 4 && depth != 8 && depth != 12 && depth != 16) return SPEC_E_INVAL;
  const hipError_t e = launch_depth(depth, d_src, (uint32_t)n, grid, waves, pattern, d_sink, s);
  return e == hipSuccess ? SPEC_OK : SPEC_E_HIP;
}

extern "C" int32_t spec_probe_read_bandwidth_noalloc(const void* d_src, size_t bytes,
                                                     int32_t grid, int32_t waves,
                                                     int32_t depth, int32_t pattern,
                                                     uint32_t* d_checksum, void* hip_stream) {
  if (!d_src || !d_checksum || grid < 1 || waves < 1 || waves > 16 ||
      (pattern != 0 && pattern != 1) || (depth != 4 && depth != 8 && depth != 12 && depth != 16))
    return SPEC_E_INVAL;
  const size_t tw = (size_t)grid * waves;
  if (tw > (size_t)kScratchWaves) return SPEC_E_INVAL;  // beyond the static scratch
  if (bytes == 0 || bytes % (1024 * tw)) return SPEC_E_INVAL;
  const size_t n = bytes / 1024 / tw;
  if (n > 0xFFFFFFFFull) return SPEC_E_INVAL;
  uint32_t* sink = scratch_on_current_device();
  if (!sink) return SPEC_E_HIP;
  hipStream_t s = (hipStream_t)hip_stream;
  // every wavefront writes its own sink word before the reduction reads it,
  // so the array needs no clearing
  if (launch_depth(depth, d_src, (uint32_t)n, grid, waves, pattern, sink, s) != hipSuccess)
    return SPEC_E_HIP;
  xor_reduce_kernel<<<1, 256, 0, s>>>(sink, (int)tw, d_checksum);
  return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_E_HIP;
}
