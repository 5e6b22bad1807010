// W12: a lossless 12-bit storage format for bf16 weight tiles.
//
// Every bf16 weight keeps its sign and its 7 mantissa bits; its 8-bit
// exponent is stored as a 4-bit offset d from a base exponent eb of its
// output row (eb = max(0, largest exponent of the row - 15)), so weights
// whose exponent lies in [eb, eb + 15] take 12 bits.  The others (exact
// zeros above the window's floor, values far below the row's largest, and
// non-finite values) are exceptions, restored exactly from a small list
// kept with each tile.  This follows the format the besthub.dev article
// describes in section "(1) W12: Lossless 12-bit Weight Format" (sign,
// 4-bit exponent offset, 7-bit mantissa, a sparse list for out-of-range
// weights, decoded in registers by the GEMM).
//
// Tile (16 rows x 32 reduction indices, the MFMA tile of kernels.h), 800
// bytes:
//   bytes [0, 768): lane l's 8 weights (row l % 16, indices (l / 16) * 8 +
//     e) in 3 dwords: dword 0 = byte e of (sign << 7 | mantissa) for e =
//     0..3, dword 1 the same for e = 4..7, dword 2 = nibble e of d.
//   bytes [768, 800): the exception slot, 8 dwords.  Dword 0 = number of
//     exceptions n <= 7, dwords 1..n = lane << 19 | e << 16 | bf16 bits.
// A matrix with a tile of more than 7 exceptions is not stored as W12 (the
// load reports it; such weights use their native storage).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

constexpr int kW12TileBytes = 800;
constexpr int kW12SlotDword = 192;         // first dword of the exception slot
constexpr int kW12MaxExc = 7;

// The raw words of one lane's weights of one tile: the 3 data dwords and
// dword (lane % 8) of the exception slot.
struct W12Raw {
  uint32_t d0, d1, d2, slot;
};

// One pair of weights (e = 2j, 2j + 1) as two bf16 in one dword.
__device__ __forceinline__ uint32_t w12_pair(uint32_t lo8x4, uint32_t nib, int j,
                                             uint32_t eb2) {
  // the two (sign | mantissa) bytes into the low byte of each 16-bit half
  const uint32_t b = (j & 1) ? ((lo8x4 >> 16) & 0xFFu) | ((lo8x4 >> 8) & 0xFF0000u)
                             : (lo8x4 & 0xFFu) | ((lo8x4 << 8) & 0xFF0000u);
  // the two exponent offsets into the low bits of each half
  const uint32_t n = (nib >> (8 * j)) & 0xFFu;
  const uint32_t d = (n & 0xFu) | ((n & 0xF0u) << 12);
  // bf16 = sign << 15 | (eb + d) << 7 | mantissa, per half
  return ((b & 0x00800080u) << 8) | ((d + eb2) << 7) | (b & 0x007F007Fu);
}

// Decode one lane's 8 weights into MFMA operand order (e = 0..7 as 4
// dwords of bf16 pairs).  eb2 = eb | eb << 16 of the lane's row.
__device__ __forceinline__ uint4 w12_decode(const W12Raw& w, uint32_t eb2) {
  uint4 v;
  v.x = w12_pair(w.d0, w.d2, 0, eb2);
  v.y = w12_pair(w.d0, w.d2, 1, eb2);
  v.z = w12_pair(w.d1, w.d2, 2, eb2);
  v.w = w12_pair(w.d1, w.d2, 3, eb2);
  return v;
}

// Patch the exceptions of a tile (count from lane 0's slot word); the
// element is selected arithmetically so the fragment stays in registers.
__device__ __forceinline__ void w12_patch(uint4& v, const W12Raw& w, int lane) {
  const uint32_t head = __builtin_amdgcn_readfirstlane(w.slot);
  if (head == 0) return;
  for (uint32_t k = 1; k <= head; ++k) {
    const uint32_t ent = __builtin_amdgcn_readlane(w.slot, k);
    const bool mine = (int)(ent >> 19) == lane;
    const uint32_t e = (ent >> 16) & 7u, val = ent & 0xFFFFu;
    const uint32_t keep = (e & 1u) ? 0x0000FFFFu : 0xFFFF0000u;
    const uint32_t put = (e & 1u) ? (val << 16) : val;
    const uint32_t dw = e >> 1;
    v.x = (mine && dw == 0) ? ((v.x & keep) | put) : v.x;
    v.y = (mine && dw == 1) ? ((v.y & keep) | put) : v.y;
    v.z = (mine && dw == 2) ? ((v.z & keep) | put) : v.z;
    v.w = (mine && dw == 3) ? ((v.w & keep) | put) : v.w;
  }
}
