// Skinny GEMM for the verify pass: Y[M, N] = X[M, K] * W[N, K]^T with M
// (rows of the pass) small and W streamed once from HBM.
//
// Design for gfx950:
//  - W is pre-tiled (see kernels.h) so that one wavefront reads one 16 x 32
//    tile as a single contiguous 1 KB (bf16) load, 16 bytes per lane, which
//    is exactly that lane's MFMA operand.  A workgroup owns NT adjacent
//    16-column tiles and streams them over the whole K range.
//  - The K range is split across the WAVES wavefronts of the workgroup;
//    each wave keeps a block of U K-steps of W loads in flight
//    (double-buffered) while it multiplies the previous block.
//  - X (a few hundred KB at most) is read through L2; rows beyond M read
//    zeros, so the per-element result does not depend on M.  bf16 weights
//    meet activations held as hi + lo bf16 planes: two MFMAs per product,
//    which keeps the activations at ~16 mantissa bits while W is streamed
//    once (the kernel is HBM-bound, so the extra MFMA work is hidden).
//  - Partial sums of the waves are reduced in LDS in a fixed order, so the
//    result of a row is bitwise independent of how many rows the pass has
//    and of the launch's row chunking.
//  - Epilogues: plain store, residual add, SwiGLU (gate and up tiles are
//    interleaved so one workgroup owns both halves of 16 outputs), and the
//    LM-head argmax partial (per-row max over the workgroup's columns,
//    lowest index on ties).
#include "common.h"
#include "kernels.h"

namespace {

constexpr int kWaves = 8;

template <typename T, int MT, int NT, int EPI>
__global__ __launch_bounds__(kWaves * 64) void gemm_kernel(GemmArgs a) {
  constexpr int U = (sizeof(T) == 2) ? 8 : 4;  // K-steps per load block
  constexpr int TROWS = MT * 16;
  constexpr int TCOLS = NT * 16;
  constexpr int LDT = TCOLS + 1;
  __shared__ float red[kWaves * TROWS * LDT];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const int nb = blockIdx.x;
  const int ksteps = a.K >> 5;
  const int s0 = (wave * ksteps) / kWaves;
  const int s1 = ((wave + 1) * ksteps) / kWaves;

  const Frag<T>* Wt = reinterpret_cast<const Frag<T>*>(a.W);
  const T* X = reinterpret_cast<const T*>(a.X);

  constexpr bool kSplit = sizeof(T) == 2;
  const T* Xlo = reinterpret_cast<const T*>(a.X_lo);
  size_t xoff[MT];
  bool xok[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int row = a.row0 + mt * 16 + r16;
    xok[mt] = row < a.M;
    xoff[mt] = (size_t)(xok[mt] ? row : 0) * a.K + g * 8;
  }

  floatx4_t acc[NT][MT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[nt][mt] = floatx4_t{0.f, 0.f, 0.f, 0.f};

  const Frag<T>* wbase[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
    wbase[nt] = Wt + ((size_t)(nb * NT + nt) * ksteps) * 64 + lane;

  auto load_block = [&](Frag<T> (&w)[U][NT], int sb) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kb = sb + u;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        if (kb < s1) w[u][nt] = wbase[nt][(size_t)kb * 64];
        else w[u][nt].zero();
      }
    }
  };
  auto mul_block = [&](const Frag<T> (&w)[U][NT], int sb) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kb = sb + u;
      if (kb < s1) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          Frag<T> x, xl;
          if (xok[mt]) {
            x.load(X + xoff[mt] + kb * 32);
            if (kSplit) xl.load(Xlo + xoff[mt] + kb * 32);
          } else {
            x.zero();
            xl.zero();
          }
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            mma32(acc[nt][mt], w[u][nt], x);
            if (kSplit) mma32(acc[nt][mt], w[u][nt], xl);
          }
        }
      }
    }
  };

  Frag<T> wa[U][NT], wb[U][NT];
  int sb = s0;
  if (sb < s1) load_block(wa, sb);
  while (sb < s1) {
    if (sb + U < s1) load_block(wb, sb + U);
    mul_block(wa, sb);
    sb += U;
    if (sb >= s1) break;
    if (sb + U < s1) load_block(wa, sb + U);
    mul_block(wb, sb);
    sb += U;
  }

  // wave partials -> LDS, lane/item -> (row, col) as in common.h
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        red[(wave * TROWS + mt * 16 + r16) * LDT + nt * 16 + 4 * g + r] =
            acc[nt][mt][r];
  __syncthreads();

  const int col0 = nb * TCOLS;
  if (EPI == EPI_SWIGLU) {
    // columns [0,16) gate, [16,32) up of the same 16 outputs
    for (int e = threadIdx.x; e < TROWS * 16; e += kWaves * 64) {
      const int row = e >> 4, col = e & 15;
      const int m = a.row0 + row;
      if (m >= a.M) continue;
      float gv = 0.f, uv = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        gv += red[(w * TROWS + row) * LDT + col];
        uv += red[(w * TROWS + row) * LDT + col + 16];
      }
      const float act = gv / (1.0f + expf(-gv)) * uv;
      store_act(reinterpret_cast<T*>(a.act), reinterpret_cast<T*>(a.act_lo),
                (size_t)m * a.ldact + nb * 16 + col, act);
    }
    return;
  }

  for (int e = threadIdx.x; e < TROWS * TCOLS; e += kWaves * 64) {
    const int row = e / TCOLS, col = e % TCOLS;
    const int m = a.row0 + row;
    if (m >= a.M) continue;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) v += red[(w * TROWS + row) * LDT + col];
    const int n = col0 + col;
    if (EPI == EPI_STORE) {
      a.Y[(size_t)m * a.ldy + n] = v;
    } else if (EPI == EPI_RESID) {
      a.Y[(size_t)m * a.ldy + n] += v;
    } else {  // EPI_ARGMAX
      if (n == a.bias_tok && a.rows[m].pos >= a.bias_after) v += a.bias;
      if (a.logits) a.logits[(size_t)m * a.ldlog + n] = v;
      red[row * LDT + col] = v;
    }
  }
  if (EPI == EPI_ARGMAX) {
    __syncthreads();
    for (int row = threadIdx.x; row < TROWS; row += kWaves * 64) {
      const int m = a.row0 + row;
      if (m >= a.M) continue;
      float best = -INFINITY;
      int bi = col0;
      for (int col = 0; col < TCOLS; ++col) {
        const float v = red[row * LDT + col];
        if (v > best) { best = v; bi = col0 + col; }  // NaN never wins
      }
      a.part[(size_t)m * a.nblocks + nb] = make_float2(best, __int_as_float(bi));
    }
  }
}

template <typename T, int EPI, int NT>
hipError_t launch_mt(int mt, const GemmArgs& a, int grid, hipStream_t s) {
  dim3 blk(kWaves * 64);
  switch (mt) {
    case 1: gemm_kernel<T, 1, NT, EPI><<<grid, blk, 0, s>>>(a); break;
    case 2: gemm_kernel<T, 2, NT, EPI><<<grid, blk, 0, s>>>(a); break;
    case 3: gemm_kernel<T, 3, NT, EPI><<<grid, blk, 0, s>>>(a); break;
    case 4: gemm_kernel<T, 4, NT, EPI><<<grid, blk, 0, s>>>(a); break;
    case 5: gemm_kernel<T, 5, NT, EPI><<<grid, blk, 0, s>>>(a); break;
    default: gemm_kernel<T, 8, NT, EPI><<<grid, blk, 0, s>>>(a); break;
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_typed(int epi, const GemmArgs& a0, hipStream_t s) {
  GemmArgs a = a0;
  const int NT = (epi == EPI_SWIGLU) ? 2 : 1;
  const int grid = a.ntiles / NT;
  // rows per launch: up to 8 tiles of 16; smaller passes use the smallest
  // tile count that covers them
  for (int r0 = 0; r0 < a.M; r0 += 128) {
    const int rows = (a.M - r0 < 128) ? a.M - r0 : 128;
    const int need = (rows + 15) / 16;
    const int mt = need <= 5 ? need : 8;
    a.row0 = r0;
    hipError_t e;
    switch (epi) {
      case EPI_STORE: e = launch_mt<T, EPI_STORE, 1>(mt, a, grid, s); break;
      case EPI_RESID: e = launch_mt<T, EPI_RESID, 1>(mt, a, grid, s); break;
      case EPI_SWIGLU: e = launch_mt<T, EPI_SWIGLU, 2>(mt, a, grid, s); break;
      default: e = launch_mt<T, EPI_ARGMAX, 1>(mt, a, grid, s); break;
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_gemm(bool bf16, int epi, const GemmArgs& a, int /*nt*/,
                       hipStream_t s) {
  if (a.M <= 0) return hipSuccess;
  return bf16 ? launch_typed<uint16_t>(epi, a, s) : launch_typed<float>(epi, a, s);
}
