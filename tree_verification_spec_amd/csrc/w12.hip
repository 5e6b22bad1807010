// W12 encoding of bf16 weight matrices into the tiled layout (format in
// w12.h).  Runs once, when the weights are loaded.
#include "common.h"
#include "kernels.h"
#include "w12.h"

namespace {

// eb[row] = max(0, largest finite exponent of the row - 15): one workgroup
// per row.  Non-finite weights (exponent code 255) are exceptions whatever
// the window, so they do not move it; a row with no finite weight gets 0.
__global__ __launch_bounds__(256) void w12_rowexp_kernel(const uint16_t* src, int K,
                                                         uint8_t* eb) {
  __shared__ uint32_t part[4];
  const uint16_t* r = src + (size_t)blockIdx.x * K;
  uint32_t m = 0;
  for (int c = threadIdx.x; c < K; c += 256) {
    const uint32_t e = (r[c] >> 7) & 0xFFu;
    m = (e != 255u && e > m) ? e : m;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint32_t t = __shfl_xor(m, o, 64);
    m = t > m ? t : m;
  }
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = part[0];
    for (int w = 1; w < 4; ++w) t = part[w] > t ? part[w] : t;
    eb[blockIdx.x] = (uint8_t)(t >= 15 ? t - 15 : 0);
  }
}

// One wave per tile of a slab of source rows (row-major [nrows, K], bf16).
// Source tile row nb becomes destination tile row dst_tile0 + nb *
// tile_stride; tile (row tr, K-step kb) sits at tile index tr * wsn + kb *
// wsk of the destination.  eb: the bases of the slab's rows; eb_dst gets
// them at the destination rows.  A crowded tile (more than 7 exceptions)
// spills the rest into its overflow block (ovf: the matrix's blocks,
// w12.h); *err is set when a tile has more exceptions than the slot and its
// block hold.  dst8 (optional): the 8-bit view's tiles at the same tile
// indices.
__global__ __launch_bounds__(64) void w12_encode_kernel(
    const uint16_t* src, int K, const uint8_t* eb, uint8_t* eb_dst, uint8_t* dst,
    uint32_t* ovf, uint8_t* dst8, int dst_tile0, int tile_stride, int wsn, int wsk,
    int* err) {
  __shared__ uint32_t slot[8];
  const int ksteps = K / 32;
  const int tile = blockIdx.x;
  const int nb = tile / ksteps, kb = tile % ksteps;
  const int lane = threadIdx.x;
  const int row = nb * 16 + (lane & 15);
  const int col = kb * 32 + (lane >> 4) * 8;
  if (lane < 8) slot[lane] = 0;
  const uint4 raw = *reinterpret_cast<const uint4*>(src + (size_t)row * K + col);
  const uint16_t* w = reinterpret_cast<const uint16_t*>(&raw);
  const uint32_t base = eb[row];
  if (kb == 0 && lane < 16)  // the destination rows' bases, once per tile row
    eb_dst[(size_t)(dst_tile0 + nb * tile_stride) * 16 + lane] = (uint8_t)base;
  // the three data dwords (layout in w12.h); exceptions leave zeros
  uint32_t da = 0, db = 0, dc = 0, excmask = 0, v8lo = 0, v8hi = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t bits = w[e];
    const int exp = (int)((bits >> 7) & 0xFFu);
    const int d = exp - (int)base;
    const bool exc = d < 0 || d > 15 || exp == 255;
    const uint32_t dd = exc ? 0u : (uint32_t)d;
    const uint32_t sign = exc ? 0u : bits >> 15;
    const uint32_t lo = exc ? 0u : ((dd & 1u) << 7) | (bits & 0x7Fu);
    const uint32_t dh = dd >> 1;
    if (e < 4) {
      da |= lo << (8 * e);
      dc |= (dh | sign << 7) << (8 * e);
    } else {
      const int k = e - 4;
      db |= lo << (8 * k);
      dc |= dh << (8 * k + 4);
      dc |= sign << (8 * ((k + 1) & 3) + 3);
    }
    excmask |= (exc ? 1u : 0u) << e;
    // the 8-bit view: sign, offset, top 3 mantissa bits (sign only when out
    // of the window)
    const uint32_t c8 = ((bits >> 15) << 7) | (exc ? 0u : (dd << 3) | ((bits >> 4) & 7u));
    if (e < 4) v8lo |= c8 << (8 * e);
    else v8hi |= c8 << (8 * (e - 4));
  }
  // exclusive prefix of the exception counts over the wave
  const uint32_t cnt = __builtin_popcount(excmask);
  uint32_t incl = cnt;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  const uint32_t total = __shfl(incl, 63, 64);
  const uint32_t first = incl - cnt;
  const size_t tidx = (size_t)(dst_tile0 + nb * tile_stride) * wsn + (size_t)kb * wsk;
  uint8_t* t = dst + tidx * kW12TileBytes;
  if (dst8)
    *reinterpret_cast<uint2*>(dst8 + tidx * kW8TileBytes + lane * 8) = make_uint2(v8lo, v8hi);
  __syncthreads();
  if (total > (uint32_t)kW12MaxExc || (total > (uint32_t)kW12SlotExc && tidx >= (1u << 24))) {
    if (lane == 0) atomicOr(err, 1);
    return;
  }
  // entries k < 7 go to the slot, the rest to the tile's overflow block
  uint32_t* ob = ovf + tidx * kW12OvfDwords;
  uint32_t k = first;
#pragma unroll
  for (int e = 0; e < 8; ++e)
    if ((excmask >> e) & 1u) {
      const uint32_t ent = ((uint32_t)lane << 19) | ((uint32_t)e << 16) | w[e];
      if (k < (uint32_t)kW12SlotExc) slot[1 + k] = ent;
      else ob[k - kW12SlotExc] = ent;
      ++k;
    }
  if (lane == 0)
    slot[0] = total <= (uint32_t)kW12SlotExc
                  ? total
                  : (1u << 31) | ((total - kW12SlotExc) << 24) | (uint32_t)tidx;
  __syncthreads();
  uint32_t* td = reinterpret_cast<uint32_t*>(t);
  td[lane * 3 + 0] = da;
  td[lane * 3 + 1] = db;
  td[lane * 3 + 2] = dc;
  if (lane < 8) td[kW12SlotDword + lane] = slot[lane];
}

}  // namespace

hipError_t launch_w12_rowexp(const void* src, int nrows, int K, uint8_t* eb,
                             hipStream_t s) {
  if (nrows <= 0) return hipSuccess;
  w12_rowexp_kernel<<<nrows, 256, 0, s>>>((const uint16_t*)src, K, eb);
  return hipGetLastError();
}

hipError_t launch_w12_encode(const void* src, int nrows, int K, const uint8_t* eb,
                             uint8_t* eb_dst, void* dst, size_t dst_tiles, void* dst8,
                             int dst_tile0, int tile_stride, int wsn, int wsk, int* err,
                             hipStream_t s) {
  if (nrows % 16 || K % 32) return hipErrorInvalidValue;
  const unsigned tiles = (unsigned)(nrows / 16) * (K / 32);
  if (tiles == 0) return hipSuccess;
  uint32_t* ovf = const_cast<uint32_t*>(w12_overflow(dst, dst_tiles));
  w12_encode_kernel<<<tiles, 64, 0, s>>>((const uint16_t*)src, K, eb, eb_dst,
                                         (uint8_t*)dst, ovf, (uint8_t*)dst8, dst_tile0,
                                         tile_stride, wsn, wsk, err);
  return hipGetLastError();
}
