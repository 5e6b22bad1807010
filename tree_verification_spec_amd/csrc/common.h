// Device-side helpers shared by the gfx950 kernels: bf16 storage, MFMA
// operand fragments and wave reductions.
//
// Fragment convention used by every matrix kernel: a "K-step" covers 32
// reduction indices.  For a 16-row operand tile, lane l (0..63) holds row
// (l % 16) and the 8 consecutive reduction indices (l / 16) * 8 + e,
// e = 0..7.  For bf16 this is exactly the operand of
// v_mfma_f32_16x16x32_bf16; for fp32 the same 8 values feed eight
// v_mfma_f32_16x16x4_f32 (instruction e consumes item e, so A and B see the
// same permutation of the reduction index).  The 16x16 fp32 result is held
// as lane l, item r -> row 4 * (l / 16) + r, column l % 16.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

// bf16 values are stored as raw uint16_t bit patterns.
__device__ __forceinline__ float bf2f(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}

// float -> bf16, round to nearest even (gfx950 converts in hardware).
__device__ __forceinline__ uint16_t f2bf(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

typedef unsigned int u32x3_t __attribute__((ext_vector_type(3)));

// A raw (untyped, unswizzled) buffer resource over 4 GB from p, for
// streaming weights with scalar base and offsets.  Word 3 = 0x00020000 is
// the raw-buffer configuration of the gfx9-family CDNA descriptors.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t weight_rsrc(const void* p) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)0xFFFFFFFFu,
                                           0x00020000);
}

template <typename T> struct Frag;

// 8 bf16 = 16 bytes
template <> struct Frag<uint16_t> {
  uint4 v;
  __device__ __forceinline__ void zero() { v = make_uint4(0, 0, 0, 0); }
  __device__ __forceinline__ void load(const uint16_t* p) {
    v = *reinterpret_cast<const uint4*>(p);
  }
};

// 8 fp32 = 32 bytes
template <> struct Frag<float> {
  float4 lo, hi;
  __device__ __forceinline__ void zero() {
    lo = make_float4(0.f, 0.f, 0.f, 0.f);
    hi = lo;
  }
  __device__ __forceinline__ void load(const float* p) {
    lo = *reinterpret_cast<const float4*>(p);
    hi = *reinterpret_cast<const float4*>(p + 4);
  }
};

// acc += A(16 x 32) * B(32 x 16) for one K-step.
__device__ __forceinline__ void mma32(floatx4_t& acc, const Frag<uint16_t>& a,
                                      const Frag<uint16_t>& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
      __builtin_bit_cast(bf16x8_t, a.v), __builtin_bit_cast(bf16x8_t, b.v),
      acc, 0, 0, 0);
}

__device__ __forceinline__ void mma32(floatx4_t& acc, const Frag<float>& a,
                                      const Frag<float>& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.x, b.lo.x, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.y, b.lo.y, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.z, b.lo.z, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.w, b.lo.w, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.x, b.hi.x, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.y, b.hi.y, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.z, b.hi.z, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.w, b.hi.w, acc, 0, 0, 0);
}

template <typename T> __device__ __forceinline__ float to_f(T v);
template <> __device__ __forceinline__ float to_f<uint16_t>(uint16_t v) { return bf2f(v); }
template <> __device__ __forceinline__ float to_f<float>(float v) { return v; }

template <typename T> __device__ __forceinline__ T from_f(float v);
template <> __device__ __forceinline__ uint16_t from_f<uint16_t>(float v) { return f2bf(v); }
template <> __device__ __forceinline__ float from_f<float>(float v) { return v; }

// Activations kept at fp32 precision but fed to bf16 MFMAs are stored as
// two bf16 planes, hi = bf16(v) and lo = bf16(v - hi): hi + lo carries ~16
// mantissa bits.  fp32 activations are stored once (lo is unused).
__device__ __forceinline__ void store_act(uint16_t* hi, uint16_t* lo, size_t i,
                                          float v) {
  const uint16_t h = f2bf(v);
  hi[i] = h;
  lo[i] = f2bf(v - bf2f(h));
}
__device__ __forceinline__ void store_act(float* hi, float* /*lo*/, size_t i,
                                          float v) {
  hi[i] = v;
}
// Four consecutive activations (i a multiple of 4; each plane 8-byte
// aligned for bf16, 16-byte for fp32): one vector store per plane.
__device__ __forceinline__ void store_act4(uint16_t* hi, uint16_t* lo, size_t i,
                                           float4 v) {
  const uint16_t h0 = f2bf(v.x), h1 = f2bf(v.y), h2 = f2bf(v.z), h3 = f2bf(v.w);
  const uint16_t l0 = f2bf(v.x - bf2f(h0)), l1 = f2bf(v.y - bf2f(h1));
  const uint16_t l2 = f2bf(v.z - bf2f(h2)), l3 = f2bf(v.w - bf2f(h3));
  *reinterpret_cast<uint2*>(hi + i) =
      make_uint2((uint32_t)h0 | ((uint32_t)h1 << 16), (uint32_t)h2 | ((uint32_t)h3 << 16));
  *reinterpret_cast<uint2*>(lo + i) =
      make_uint2((uint32_t)l0 | ((uint32_t)l1 << 16), (uint32_t)l2 | ((uint32_t)l3 << 16));
}
__device__ __forceinline__ void store_act4(float* hi, float* /*lo*/, size_t i, float4 v) {
  *reinterpret_cast<float4*>(hi + i) = v;
}

// Four consecutive elements as fp32 (p 8-byte aligned for bf16, 16-byte
// for fp32).
__device__ __forceinline__ float4 load4(const uint16_t* p) {
  const uint2 w = *reinterpret_cast<const uint2*>(p);
  return make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xFFFF0000u),
                     __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xFFFF0000u));
}
__device__ __forceinline__ float4 load4(const float* p) {
  return *reinterpret_cast<const float4*>(p);
}

// Reductions over the four lanes {l, l^16, l^32, l^48} (one MFMA output
// column's four row groups) with the gfx950 row-swap instructions: after a
// swap of a register with itself, the two results hold, in every lane, the
// lane's own value and its partner's (in the same order in both lanes of a
// pair, so the reduction is bitwise symmetric).
__device__ __forceinline__ float quad_max(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float quad_sum(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Deferred RMSNorm.  A GEMM is linear in each input row, so
// (s * (h * w)) W^T = s * ((h * w) W^T) for the row's norm scale
// s = 1 / sqrt(mean(h^2) + eps).  The kernel that writes a normalised
// GEMM input therefore stores the planes of h * w and, per row, the sums of
// squares of h over chunks of kNormChunk columns (one workgroup each, so a
// row spreads over several CUs); the kernel that consumes that GEMM's output
// multiplies it by the row's scale, summing the chunks in order.
// All chunk loads are issued together (nc <= 16: d <= 16384); the chunks are
// added in order.
// The scale in two parts, so a caller can issue other loads between them:
// every lane loads 16 values (indexes past the row's chunks repeat its last
// one), so the loads are unconditional and all in flight together.
__device__ __forceinline__ void row_ss_load(const RowNorm& n, int row, float (&v)[16]) {
  const float* p = n.ss + (size_t)row * n.nc;
  const int last = n.nc > 0 ? n.nc - 1 : 0;
#pragma unroll
  for (int c = 0; c < 16; ++c) v[c] = p[c < last ? c : last];
}
__device__ __forceinline__ float row_scale_of(const RowNorm& n, const float (&v)[16]) {
  float t = 0.f;
#pragma unroll
  for (int c = 0; c < 16; ++c)
    if (c < n.nc) t += v[c];
  return 1.0f / sqrtf(t / (float)n.d + n.eps);
}
__device__ __forceinline__ float row_scale(const RowNorm& n, int row) {
  float v[16];
  row_ss_load(n, row, v);
  return row_scale_of(n, v);
}
