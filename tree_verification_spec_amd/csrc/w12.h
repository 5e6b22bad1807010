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
//     e) in 3 dwords A, B, C.  With d = d0 + 2 d' (d0 one bit, d' three):
//     byte e of A (e < 4) or byte e - 4 of B = d0 << 7 | mantissa;
//     byte k of C (k < 4) = d'_k | s_(4 + (k + 3) % 4) << 3 | d'_(k + 4) << 4
//     | s_k << 7 (s = sign).  C rotated right by 4 bits puts weight 4 + k's
//     d' and sign where C has weight k's, so a mask and one byte permute per
//     weight pair leave sign << 15 | d << 7 | mantissa per 16 bits, and
//     adding eb << 7 gives the bf16 (eb + d <= 254 never carries).
//   bytes [768, 800): the exception slot, 8 dwords.  Dword 0 is the header,
//     dwords 1..7 hold entries lane << 19 | e << 16 | bf16 bits.  A tile of
//     n <= 7 exceptions has header n and its entries in dwords 1..n.  A
//     crowded tile (8 <= n <= kW12MaxExc) keeps its first 7 entries in the
//     slot and the other n - 7 in its overflow block; its header is
//     1 << 31 | (n - 7) << 24 | t, t = the tile's index in the matrix.
// Overflow blocks: the matrix region is sized for bf16 tiles (1024 bytes a
// tile) and W12 tiles fill only its first ntiles * 800 bytes; the block of
// tile t (56 entries, 224 bytes) follows at ntiles * 800 + t * 224, so the
// region still holds every tile's worst case.  A tile of more than
// kW12MaxExc exceptions does not fit: the load reports it and such weights
// use their native storage.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

constexpr int kW12TileBytes = 800;
constexpr int kW12SlotDword = 192;         // first dword of the exception slot
constexpr int kW12SlotExc = 7;             // entries held in the slot
constexpr int kW12OvfDwords = 56;          // entries of a tile's overflow block
constexpr int kW12MaxExc = kW12SlotExc + kW12OvfDwords;

// The overflow blocks of a W12 matrix of ntiles tiles starting at base.
__host__ __device__ inline const uint32_t* w12_overflow(const void* base, size_t ntiles) {
  return reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint8_t*>(base) +
                                           ntiles * kW12TileBytes);
}

// The raw words of one lane's weights of one tile: the 3 data dwords and
// dword (lane % 8) of the exception slot.
struct W12Raw {
  uint32_t d0, d1, d2, slot;
};

// Decode one lane's 8 weights into MFMA operand order (e = 0..7 as 4
// dwords of bf16 pairs).  eb7 = (eb | eb << 16) << 7 of the lane's row.
__device__ __forceinline__ uint4 w12_decode(const W12Raw& w, uint32_t eb7) {
  // the sign and d' bits of weights 0..3 (C) and 4..7 (C rotated right by 4)
  constexpr uint32_t kMask = 0x87878787u;
  const uint32_t c0 = w.d2 & kMask;
  const uint32_t c4 = __builtin_amdgcn_alignbit(w.d2, w.d2, 4) & kMask;
  constexpr uint32_t kLo = 0x05010400u, kHi = 0x07030602u;  // bytes {0,4,1,5}, {2,6,3,7}
  uint4 v;
  v.x = __builtin_amdgcn_perm(c0, w.d0, kLo) + eb7;
  v.y = __builtin_amdgcn_perm(c0, w.d0, kHi) + eb7;
  v.z = __builtin_amdgcn_perm(c4, w.d1, kLo) + eb7;
  v.w = __builtin_amdgcn_perm(c4, w.d1, kHi) + eb7;
  return v;
}

// Write one exception entry into the lane's fragment when it is the lane's;
// the element is selected arithmetically so the fragment stays in registers.
__device__ __forceinline__ void w12_put(uint4& v, uint32_t ent, int lane) {
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

// Patch the exceptions of a tile: the header from lane 0's slot word, slot
// entries from lanes 1..7, and for a crowded tile the rest from its
// overflow block (ovf: the matrix's overflow blocks, w12_overflow), read
// through the constant address space so that they are scalar loads.
__device__ __forceinline__ void w12_patch(uint4& v, const W12Raw& w, int lane,
                                          const uint32_t* ovf) {
  const uint32_t head = __builtin_amdgcn_readfirstlane(w.slot);
  if (head == 0) return;
  const uint32_t n = (head >> 31) ? (uint32_t)kW12SlotExc : head;
  for (uint32_t k = 1; k <= n; ++k) w12_put(v, __builtin_amdgcn_readlane(w.slot, k), lane);
  if (head >> 31) {
    typedef __attribute__((address_space(4))) const uint32_t cu32;
    cu32* ob = (cu32*)(ovf + (size_t)(head & 0xFFFFFFu) * kW12OvfDwords);
    const uint32_t extra = (head >> 24) & 63u;
    for (uint32_t j = 0; j < extra; ++j) w12_put(v, ob[j], lane);
  }
}

// The same patch as one assembly block (all 64 lanes active), so the
// rarely taken loops add no control flow to the compiler's view of the
// GEMM loop (which otherwise costs registers at many row tiles).  Every scalar
// value a vector instruction uses as a lane select or mask, and every
// scalar written by a vector instruction, is followed by s_nop 4 before
// use (these wait states cost nothing in the common path, which is the
// first four instructions).  The overflow entries of a crowded tile are
// scalar loads waited for inside the block (the blocks are written at load
// time and constant while a GEMM runs, so the block is a pure function of
// its operands).
#define W12_PUT_ASM(L)                                                  \
  "s_lshr_b32 %[t], %[ent], 19\n\t"                                     \
  "s_bfe_u32 %[e], %[ent], 0x30010\n\t"                                 \
  "s_and_b32 %[val], %[ent], 0xffff\n\t"                                \
  "s_lshl_b32 %[put], %[val], 16\n\t"                                   \
  "s_mov_b32 %[keep], 0xffff0000\n\t"                                   \
  "s_bitcmp1_b32 %[e], 0\n\t"                                           \
  "s_cselect_b32 %[put], %[put], %[val]\n\t"                            \
  "s_cselect_b32 %[keep], 0xffff, %[keep]\n\t"                          \
  "s_lshr_b32 %[dw], %[e], 1\n\t"                                       \
  "s_nop 4\n\t"                                                         \
  "v_cmp_eq_u32_e64 %[m], %[t], %[lane]\n\t"                            \
  "s_nop 4\n\t"                                                         \
  "s_cmp_eq_u32 %[dw], 0\n\t"                                           \
  "s_cselect_b64 %[mi], %[m], 0\n\t"                                    \
  "s_nop 4\n\t"                                                         \
  "v_and_b32 %[tmp], %[keep], %[x]\n\t"                                 \
  "v_or_b32 %[tmp], %[put], %[tmp]\n\t"                                 \
  "v_cndmask_b32_e64 %[x], %[x], %[tmp], %[mi]\n\t"                     \
  "s_cmp_eq_u32 %[dw], 1\n\t"                                           \
  "s_cselect_b64 %[mi], %[m], 0\n\t"                                    \
  "s_nop 4\n\t"                                                         \
  "v_and_b32 %[tmp], %[keep], %[y]\n\t"                                 \
  "v_or_b32 %[tmp], %[put], %[tmp]\n\t"                                 \
  "v_cndmask_b32_e64 %[y], %[y], %[tmp], %[mi]\n\t"                     \
  "s_cmp_eq_u32 %[dw], 2\n\t"                                           \
  "s_cselect_b64 %[mi], %[m], 0\n\t"                                    \
  "s_nop 4\n\t"                                                         \
  "v_and_b32 %[tmp], %[keep], %[z]\n\t"                                 \
  "v_or_b32 %[tmp], %[put], %[tmp]\n\t"                                 \
  "v_cndmask_b32_e64 %[z], %[z], %[tmp], %[mi]\n\t"                     \
  "s_cmp_eq_u32 %[dw], 3\n\t"                                           \
  "s_cselect_b64 %[mi], %[m], 0\n\t"                                    \
  "s_nop 4\n\t"                                                         \
  "v_and_b32 %[tmp], %[keep], %[q]\n\t"                                 \
  "v_or_b32 %[tmp], %[put], %[tmp]\n\t"                                 \
  "v_cndmask_b32_e64 %[q], %[q], %[tmp], %[mi]\n\t"

__device__ __forceinline__ void w12_patch_opaque(uint4& v, const W12Raw& w, int lane,
                                                 const uint32_t* ovf) {
  uint32_t x = v.x, y = v.y, z = v.z, q = v.w, tmp;
  uint32_t head, n, k, ent, t, e, val, keep, put, dw, off;
  uint64_t m, mi;
  asm(
      "v_readfirstlane_b32 %[head], %[slot]\n\t"
      "s_nop 4\n\t"
      "s_cmp_eq_u32 %[head], 0\n\t"
      "s_cbranch_scc1 .Lw12done%=\n\t"
      "s_bitcmp1_b32 %[head], 31\n\t"
      "s_cselect_b32 %[n], 7, %[head]\n\t"
      "s_mov_b32 %[k], 1\n"
      ".Lw12loop%=:\n\t"
      "s_nop 4\n\t"
      "v_readlane_b32 %[ent], %[slot], %[k]\n\t"
      "s_nop 4\n\t"
      W12_PUT_ASM(0)
      "s_add_u32 %[k], %[k], 1\n\t"
      "s_cmp_le_u32 %[k], %[n]\n\t"
      "s_cbranch_scc1 .Lw12loop%=\n\t"
      "s_bitcmp1_b32 %[head], 31\n\t"
      "s_cbranch_scc0 .Lw12done%=\n\t"
      "s_bfe_u32 %[n], %[head], 0x60018\n\t"
      "s_and_b32 %[off], %[head], 0xffffff\n\t"
      "s_mul_i32 %[off], %[off], 224\n\t"
      "s_mov_b32 %[k], 0\n"
      ".Lw12ovf%=:\n\t"
      "s_load_dword %[ent], %[ob], %[off]\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      W12_PUT_ASM(1)
      "s_add_u32 %[off], %[off], 4\n\t"
      "s_add_u32 %[k], %[k], 1\n\t"
      "s_cmp_lt_u32 %[k], %[n]\n\t"
      "s_cbranch_scc1 .Lw12ovf%=\n"
      ".Lw12done%=:\n\t"
      "s_nop 4"
      : [x] "+v"(x), [y] "+v"(y), [z] "+v"(z), [q] "+v"(q), [tmp] "=&v"(tmp),
        [head] "=&s"(head), [n] "=&s"(n), [k] "=&s"(k), [ent] "=&s"(ent), [t] "=&s"(t),
        [e] "=&s"(e), [val] "=&s"(val), [keep] "=&s"(keep), [put] "=&s"(put),
        [dw] "=&s"(dw), [off] "=&s"(off), [m] "=&s"(m), [mi] "=&s"(mi)
      : [slot] "v"(w.slot), [lane] "v"(lane), [ob] "s"(ovf)
      : "scc");
  v = make_uint4(x, y, z, q);
}
#undef W12_PUT_ASM

// ---- The 8-bit view (the low-precision pass of two-level verification):
// per weight one byte s << 7 | d << 3 | (top 3 mantissa bits), with the
// W12 base exponents of the same rows.  A tile is 512 bytes, lane l's 8
// weights at bytes l * 8 + e.  A weight outside its row's window keeps only
// its sign (d = 0, mantissa 0).  Decoding gives the weight with its
// mantissa truncated to 3 bits.
constexpr int kW8TileBytes = 512;

__device__ __forceinline__ uint4 w8_decode(uint2 w, uint32_t eb7) {
  // bytes 2j, 2j + 1 of a dword into the low byte of each 16-bit half
  constexpr uint32_t kP0 = 0x0C010C00u, kP1 = 0x0C030C02u;  // 0x0C selects a zero byte
  auto pair = [eb7](uint32_t h) -> uint32_t {
    return (((h & 0x007F007Fu) << 4) + eb7) | ((h & 0x00800080u) << 8);
  };
  uint4 v;
  v.x = pair(__builtin_amdgcn_perm(0u, w.x, kP0));
  v.y = pair(__builtin_amdgcn_perm(0u, w.x, kP1));
  v.z = pair(__builtin_amdgcn_perm(0u, w.y, kP0));
  v.w = pair(__builtin_amdgcn_perm(0u, w.y, kP1));
  return v;
}

