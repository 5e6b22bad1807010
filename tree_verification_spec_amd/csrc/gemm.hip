// Skinny GEMM for the verify pass: Y[M, N] = X[M, K] * W[N, K]^T with M
// (rows of the pass) small and W streamed once from HBM.
//
// Design for gfx950:
//  - W is pre-tiled (see kernels.h): one wavefront reads one 16 x 32 tile as
//    a single contiguous 1 KB (bf16) load, 16 bytes per lane, which is
//    exactly that lane's MFMA operand.  Each wave owns NTW adjacent tiles
//    and streams them over the workgroup's K range, keeping the next block
//    of U K-steps in flight while it multiplies the current one.
//  - The activations of the workgroup's K range are staged once per chunk
//    in LDS, shared by all waves, so the vector-memory path carries weights
//    only.  Activations arrive as planes of the weight type written once by
//    their producer (for bf16 weights hi + lo bf16 planes: two MFMAs per
//    product, ~16 mantissa bits), so staging is a plain copy.  Rows beyond M
//    stage zeros.  A preceding RMSNorm is deferred: the planes hold h * w and
//    the row's norm scale multiplies the output (in the SWIGLU and ARGMAX
//    epilogues here, in the consumer of split partials otherwise).
//  - The K range can be split over S workgroups.  Split GEMMs (EPI_PART)
//    write fp32 partials with plain stores and the consumer kernel adds the S
//    partials in split order (so no workgroup of this kernel waits for or
//    fences against another: on gfx950 a device-scope fence writes back and
//    invalidates the whole L2 of the XCD).
//  - Epilogues: partial store, SwiGLU (gate and up tiles are interleaved so a
//    wave owns both halves of 16 outputs; S = 1), and the LM-head argmax
//    partial (per-row max over the workgroup's columns, lowest index on ties;
//    S = 1).
#include <hip/hip_ext.h>

#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "w12.h"

namespace {

constexpr int kD = 8;  // minimum K-steps of W loads in flight per wave (rolling window)

// Staged chunk width (K elements) per row-tile count: up to 3 row tiles,
// two LDS buffers of MT*16 rows x (KC + pad) x 4 bytes stay near 64 KB (two
// workgroups per CU); from 4 row tiles the registers allow one workgroup
// per CU anyway, and chunks of ~130 KB halve the barriers.
template <int MT> struct ChunkK {
  static constexpr int value = MT <= 1 ? 256 : MT <= 2 ? 256 : MT <= 3 ? 160
                             : MT <= 4 ? 256 : MT <= 5 ? 192 : 128;
};
// With stacked hi / lo rows (one staged plane) 256-wide chunks stay within
// ~84 KB at every row-tile count used (up to 5).
constexpr int kChunkStk = 256;

// STK (bf16 activations, at most 40 rows a launch): the lo plane's rows are
// stacked under the hi plane's (rows [0, mc) hi, [mc, 2 mc) lo) in one staged
// plane, so each row tile is one MFMA per K-step instead of a hi and a lo
// MFMA on half-empty tiles; the epilogue adds row m + mc to row m.
template <typename T, int MT, int NTW, int WAVES, int EPI, int D, int WF, bool STK>
__global__ __launch_bounds__(WAVES * 64) void gemm_kernel(GemmArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr bool kBf = sizeof(T) == 2;
  static_assert(!STK || kBf, "stacked rows need bf16 activation planes");
  constexpr int NPL = (kBf && !STK) ? 2 : 1;  // staged planes
  constexpr int TROWS = MT * 16;
  constexpr int COLS = WAVES * NTW * 16;  // most output columns of a workgroup
  constexpr int NTHR = WAVES * 64;
  constexpr int KC = STK ? kChunkStk : ChunkK<MT>::value;
  constexpr int LDS_ROW = KC + (kBf ? 8 : 4);       // elements per staged row
  constexpr int EPU = 16 / sizeof(T);               // K values per 16-byte unit
  constexpr int QUADS = KC / EPU;                    // units per staged row
  constexpr int XQ = (TROWS * QUADS + NTHR - 1) / NTHR;  // units per thread
  // Loop shape by row tiles (measured on the 8B shapes): up to 32 rows the
  // compiler's own schedule streams best; from 48 rows on, activation loads
  // are unpredicated, each step's weight refill is pinned after its MFMAs,
  // and the W12 exception patch is one opaque block (its loop would
  // otherwise cost registers, and with them occupancy).
  constexpr bool kOrdered = STK ? MT >= 4 : MT >= 3;
  const int lane = threadIdx.x & 63;
  // wave-uniform (kept in scalar registers, so weight addresses are a
  // scalar base plus a per-lane offset)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, r16 = lane & 15;
  // Column partition: the launch has a.ncb workgroups per K split; workgroup
  // nb owns a balanced share [t0, t1) of the matrix's tiles, in whole
  // granules of a.gt tiles (a wave's NTW tiles; gate/up pairs stay in one
  // workgroup), one wave per NTW tiles.  Waves beyond the share shadow the
  // last live wave's tiles (their loads hit L2) and store nothing.
  const int nb = blockIdx.x % a.ncb;
  const int sk = blockIdx.x / a.ncb;
  const int ug = a.ntiles / a.gt;
  const int t0 = a.gt * (int)(((int64_t)nb * ug) / a.ncb);
  const int t1 = a.gt * (int)(((int64_t)(nb + 1) * ug) / a.ncb);
  const int live_waves = (t1 - t0) / NTW;
  const bool live = wave < live_waves;
  const int tbase = t0 + (live ? wave : live_waves - 1) * NTW;  // the wave's first tile
  const int kbeg = sk * a.KR;
  const int kend = min(a.K, kbeg + a.KR);

  // two staging buffers; each holds a bf16 hi plane then a lo plane, one
  // plane of stacked rows, or fp32
  constexpr int BUF_ELEMS = TROWS * LDS_ROW * NPL;
  // rows of this launch (stacked: the hi rows; their lo rows follow)
  const int mc = min(a.M - a.row0, 128);
  T* xbuf = reinterpret_cast<T*>(smem);
  // The SWIGLU and ARGMAX epilogues scale each row by its deferred RMSNorm
  // scale, computed once per row in the epilogue (loading the chunk sums at
  // the start measured slower: it delays the first weight loads).
  constexpr bool kNorm = EPI != EPI_PART;
  __shared__ float rsc[kNorm ? 128 : 1];

  // weights: bf16 / fp32 tiles (a Frag per lane), or W12 tiles (12 bytes
  // per lane plus one exception-slot word, decoded to a Frag before use)
  // weight format: 0 = bf16 / fp32 tiles, 1 = W12, 2 = the 8-bit view
  constexpr bool W12 = WF == 1, W8 = WF == 2;
  static_assert(WF == 0 || sizeof(T) == 2, "W12 and its 8-bit view hold bf16 weights");
  using WReg = typename std::conditional<
      W12, W12Raw, typename std::conditional<W8, uint2, Frag<T>>::type>::type;
  constexpr uint32_t TB = W12  ? kW12TileBytes
                          : W8 ? kW8TileBytes
                               : 64 * sizeof(Frag<T>);  // tile bytes
  // one buffer resource per tile row (scalar registers); a K-step's tile is
  // at the scalar offset k * wk, a lane's words at a fixed per-lane offset
  __amdgpu_buffer_rsrc_t wrs[NTW];
  uint32_t eb7[NTW];  // W12: the row's base exponent, (eb | eb << 16) << 7
#pragma unroll
  for (int t = 0; t < NTW; ++t) {
    const size_t tr = (size_t)(tbase + t);  // tile row
    wrs[t] = weight_rsrc(reinterpret_cast<const uint8_t*>(a.W) + tr * a.wsn * TB);
    if constexpr (W12 || W8) {
      const uint32_t e = a.eb[tr * 16 + r16];
      eb7[t] = (e | (e << 16)) << 7;
    } else {
      eb7[t] = 0;
    }
  }
  const uint32_t wk = (uint32_t)a.wsk * TB;  // bytes between K-steps (host-checked)
  // W12: the overflow blocks of crowded tiles (w12.h)
  const uint32_t* ovf = W12 ? w12_overflow(a.W, (size_t)a.ntiles * (a.K / 32)) : nullptr;

  // bf16 planes staged side by side: the hi and lo products accumulate
  // apart and are added once at the end, as the stacked rows are (so a
  // row's outputs are the same bits whatever the pass's row count)
  constexpr bool kSepLo = NPL == 2;
  floatx4_t acc[NTW][MT], acl[kSepLo ? NTW : 1][kSepLo ? MT : 1];
#pragma unroll
  for (int t = 0; t < NTW; ++t)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[t][mt] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  if constexpr (kSepLo) {
#pragma unroll
    for (int t = 0; t < NTW; ++t)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acl[t][mt] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  }

  // ---- activation chunk prefetch (registers) and store (LDS)
  // one unit = 16 bytes of one row: 8 consecutive K values of a bf16 plane,
  // or 4 of fp32
  using Unit = typename std::conditional<kBf, uint4, float4>::type;
  const T* Xh = reinterpret_cast<const T*>(a.X);
  const T* Xl = Xh + a.xlo;
  Unit xr[XQ], xl[NPL == 2 ? XQ : 1];
  auto fetch = [&](int kc0, int kcl) {
    // columns kc0 .. kc0 + min(kcl, KC) of the real K range; the rest zero
    const int quads = kcl <= 0 ? 0 : (kcl >= KC ? QUADS : kcl / EPU);
#pragma unroll
    for (int q = 0; q < XQ; ++q) {
      const int e = threadIdx.x + q * NTHR;
      const int r = e / QUADS, c = (e % QUADS) * EPU;
      if constexpr (STK) {
        // staged row r: hi row r, or lo row r - mc
        const bool low = r >= mc;
        const int m = a.row0 + (low ? r - mc : r);
        const bool in = r < TROWS && r < 2 * mc && c / EPU < quads;
        const T* src = low ? Xl : Xh;
        if constexpr (kOrdered) {
          const size_t off = in ? (size_t)m * a.ldx + kc0 + c : 0;
          const uint32_t mk = in ? 0xFFFFFFFFu : 0u;
          const uint4 h = *reinterpret_cast<const uint4*>((in ? src : Xh) + off);
          xr[q] = make_uint4(h.x & mk, h.y & mk, h.z & mk, h.w & mk);
        } else {
          const size_t off = (size_t)m * a.ldx + kc0 + c;
          xr[q] = in ? *reinterpret_cast<const uint4*>(src + off) : make_uint4(0, 0, 0, 0);
        }
      } else {
        const int m = a.row0 + r;
        const bool in = r < TROWS && m < a.M && c / EPU < quads;
        if constexpr (kOrdered) {
          // every lane loads (from the plane's first element when out of
          // range) and masks afterwards: no predicated loads, which the
          // compiler would otherwise count conservatively across the loop
          const size_t off = in ? (size_t)m * a.ldx + kc0 + c : 0;
          const uint32_t mk = in ? 0xFFFFFFFFu : 0u;
          if constexpr (NPL == 2) {
            const uint4 h = *reinterpret_cast<const uint4*>(Xh + off);
            const uint4 l = *reinterpret_cast<const uint4*>(Xl + off);
            xr[q] = make_uint4(h.x & mk, h.y & mk, h.z & mk, h.w & mk);
            xl[q] = make_uint4(l.x & mk, l.y & mk, l.z & mk, l.w & mk);
          } else {
            const uint4 h = *reinterpret_cast<const uint4*>(Xh + off);
            xr[q] = make_float4(__uint_as_float(h.x & mk), __uint_as_float(h.y & mk),
                                __uint_as_float(h.z & mk), __uint_as_float(h.w & mk));
          }
        } else {
          const size_t off = (size_t)m * a.ldx + kc0 + c;
          if constexpr (NPL == 2) {
            xr[q] = in ? *reinterpret_cast<const uint4*>(Xh + off) : make_uint4(0, 0, 0, 0);
            xl[q] = in ? *reinterpret_cast<const uint4*>(Xl + off) : make_uint4(0, 0, 0, 0);
          } else {
            xr[q] = in ? *reinterpret_cast<const float4*>(Xh + off)
                       : make_float4(0.f, 0.f, 0.f, 0.f);
          }
        }
      }
    }
  };
  auto store = [&](int buf) {
    // all KC columns are written (fetch zeroed those past the real range)
    T* hi = xbuf + buf * BUF_ELEMS;
    T* lo = hi + TROWS * LDS_ROW;
#pragma unroll
    for (int q = 0; q < XQ; ++q) {
      const int e = threadIdx.x + q * NTHR;
      const int r = e / QUADS, c = (e % QUADS) * EPU;
      if (r >= TROWS) continue;
      *reinterpret_cast<Unit*>(&hi[r * LDS_ROW + c]) = xr[q];
      if constexpr (NPL == 2) *reinterpret_cast<Unit*>(&lo[r * LDS_ROW + c]) = xl[q];
    }
  };

  const int kb_beg = kbeg >> 5, kb_end = kend >> 5;
  constexpr int CSTEPS = KC / 32;              // K-steps per staged chunk
  constexpr int CPW = (D + CSTEPS - 1) / CSTEPS;  // chunks per window
  constexpr int WIN = CPW * CSTEPS;            // K-steps of W loads in flight
  // Rolling window: slot u holds the W tiles of K-step (window start + u);
  // right after a slot is consumed it is reloaded with the step WIN ahead.
  // Slot indices are compile-time constants (the window is a whole number of
  // chunks) and the loop body has no branches around loads: loads past the
  // end are clamped to the last tile (an L2 hit) and staged activations past
  // the end are zero, so padded steps add nothing.  This keeps the
  // compiler's in-order load counters exact (no drain at chunk boundaries).
  WReg w[WIN][NTW];
  auto load_step = [&](WReg (&dst)[NTW], int kb) {
    const int k = kb < kb_end ? kb : kb_end - 1;
    const int so = (int)((uint32_t)k * wk);
#pragma unroll
    for (int t = 0; t < NTW; ++t) {
      if constexpr (W12) {
        const u32x3_t d = __builtin_amdgcn_raw_buffer_load_b96(wrs[t], lane * 12, so, 0);
        dst[t] = W12Raw{d.x, d.y, d.z,
                        __builtin_amdgcn_raw_buffer_load_b32(
                            wrs[t], (kW12SlotDword + (lane & 7)) * 4, so, 0)};
      } else if constexpr (W8) {
        dst[t] = __builtin_bit_cast(
            uint2, __builtin_amdgcn_raw_buffer_load_b64(wrs[t], lane * 8, so, 0));
      } else if constexpr (kBf) {
        dst[t].v = __builtin_bit_cast(
            uint4, __builtin_amdgcn_raw_buffer_load_b128(wrs[t], lane * 16, so, 0));
      } else {
        dst[t].lo = __builtin_bit_cast(
            float4, __builtin_amdgcn_raw_buffer_load_b128(wrs[t], lane * 32, so, 0));
        dst[t].hi = __builtin_bit_cast(
            float4, __builtin_amdgcn_raw_buffer_load_b128(wrs[t], lane * 32 + 16, so, 0));
      }
    }
  };
  // the weight operand of one K-step (W12: decoded, exceptions restored;
  // no memory access here, so the window's load counters stay exact)
  auto wfrag = [&](const WReg& r, int t) -> Frag<T> {
    if constexpr (W12) {
      Frag<T> f;
      f.v = w12_decode(r, eb7[t]);
      if constexpr (kOrdered) w12_patch_opaque(f.v, r, lane, ovf);
      else w12_patch(f.v, r, lane, ovf);
      return f;
    } else if constexpr (W8) {
      Frag<T> f;
      f.v = w8_decode(r, eb7[t]);
      return f;
    } else {
      (void)t;
      return r;
    }
  };
  // one staged chunk: CSTEPS K-steps from LDS (xat: the address of a row's
  // 8 values at K offset kk), weights from window slots cc * CSTEPS + j
  auto compute_chunk = [&](int kw, int cc, auto xat) {
    // activation fragments of K-step j + 1 are read from LDS while the
    // MFMAs of step j run (software pipelining hides the LDS latency)
    constexpr int XF = NPL;  // hi (+ lo) planes
    Frag<T> xc[MT][XF], xn[MT][XF];
    auto load_x = [&](Frag<T> (&x)[MT][XF], int j) {
      const int kk = j * 32 + g * 8;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int r = mt * 16 + r16;
        x[mt][0].load(xat(r, kk, 0));
        if constexpr (NPL == 2) x[mt][1].load(xat(r, kk, 1));
      }
    };
    load_x(xc, 0);
#pragma unroll
    for (int j = 0; j < CSTEPS; ++j) {
      const int u = cc * CSTEPS + j;
      if (j + 1 < CSTEPS) load_x(xn, j + 1);
      Frag<T> wf[NTW];
#pragma unroll
      for (int t = 0; t < NTW; ++t) wf[t] = wfrag(w[u][t], t);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int t = 0; t < NTW; ++t)
#pragma unroll
          for (int p = 0; p < XF; ++p) {
            if (kSepLo && p == 1) mma32(acl[t][mt], wf[t], xc[mt][1]);
            else mma32(acc[t][mt], wf[t], xc[mt][p]);
          }
      load_step(w[u], kw + u + WIN);
      // ordered: each step's refill is issued right after its MFMAs (the
      // scheduler would otherwise sink all refills to the end of the
      // chunk, and the next chunk would wait a full memory latency)
      if constexpr (kOrdered) __builtin_amdgcn_sched_barrier(0);
      if (j + 1 < CSTEPS) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int p = 0; p < XF; ++p) xc[mt][p] = xn[mt][p];
      }
    }
  };

  if constexpr (STK) {
    // Stacked rows: each chunk goes from memory straight into LDS (buffer
    // loads that write LDS, no registers), two buffers in turn.  A 1 KB
    // load of a wavefront fills two unpadded 512-byte rows; 16-byte unit u
    // of row r sits at position u ^ (r % 16), so the 16 rows of a fragment
    // read fall in distinct banks.  Rows past the stacked rows and K past
    // the split are loaded from an offset past the buffer's range, which
    // writes zeros.
    static_assert(CPW == 1, "the window is one chunk");
    typedef __attribute__((address_space(3))) void lds_void;
    __shared__ __align__(1024) T sx0[STK ? TROWS * KC : 1];
    __shared__ __align__(1024) T sx1[STK ? TROWS * KC : 1];
    const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void*>(a.X), (short)0, 0x7FFFFFFF, 0x00020000);
    // every wave issues the same number of loads (a wave past the chunk's
    // last load repeats it: the same bytes to the same place)
    constexpr int NB = TROWS / 2;  // 1 KB loads of the chunk
    constexpr int NQ = (NB + WAVES - 1) / WAVES;
    auto dma = [&](T* dst, int kc0, int kcl) {
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        const int gi = min(q * WAVES + wave, NB - 1);  // wave-uniform
        const int row = gi * 2 + (lane >> 5);
        const int u = (lane & 31) ^ (row & 15);
        const bool low = row >= mc;
        const int m = a.row0 + (low ? row - mc : row);
        const bool in = row < 2 * mc && u * 8 < kcl;
        const uint32_t voff =
            in ? (uint32_t)(((low ? (size_t)a.xlo : 0) + (size_t)m * a.ldx + kc0 + u * 8) *
                            sizeof(T))
               : 0x80000000u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xrs, (lds_void*)(dst + gi * 512), 16, voff, 0,
                                                 0, 0);
      }
    };
    // before a chunk is read: this wave's loads into it are done (they were
    // issued just before one window of weight loads: LPS loads per tile per
    // K-step, all issued in order after them), then every wave's are
    constexpr int LPS = W12 ? 2 : 1;
    constexpr int NAFTER = WIN * NTW * LPS;  // (the chunk's own loads: NQ, before them)
    static_assert(NAFTER < 64, "vmcnt range");
    constexpr int kWait = (NAFTER & 15) | ((NAFTER >> 4) << 14) | (7 << 4) | (15 << 8);
    auto arrive = [&]() {
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(kWait);
      __syncthreads();
    };
    auto swz = [](const T* buf) {
      return [buf](int r, int kk, int) {
        return buf + r * KC + ((((kk >> 3) ^ (r & 15))) << 3);
      };
    };
    dma(sx0, kbeg, kend - kbeg);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < WIN; ++u) load_step(w[u], kb_beg + u);
    // the first chunk, then the rest in pairs (buffer 1, buffer 0): with the
    // loop starting on buffer 1 the compiler's own load counting stays exact
    // across the loop edge (it then waits only for the weights it uses)
    arrive();
    dma(sx1, (kb_beg + CSTEPS) * 32, kend - (kb_beg + CSTEPS) * 32);
    __builtin_amdgcn_sched_barrier(0);
    compute_chunk(kb_beg, 0, swz(sx0));
    for (int kw = kb_beg + CSTEPS; kw < kb_end; kw += 2 * CSTEPS) {
      arrive();
      dma(sx0, (kw + CSTEPS) * 32, kend - (kw + CSTEPS) * 32);
      __builtin_amdgcn_sched_barrier(0);
      compute_chunk(kw, 0, swz(sx1));
      if (kw + CSTEPS < kb_end) {  // workgroup-uniform
        arrive();
        dma(sx1, (kw + 2 * CSTEPS) * 32, kend - (kw + 2 * CSTEPS) * 32);
        __builtin_amdgcn_sched_barrier(0);
        compute_chunk(kw + CSTEPS, 0, swz(sx0));
      }
    }
    // the loads of the chunk after the last (all zeros) land before the
    // workgroup can end and its LDS be reused
    __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));  // vmcnt(0)
  } else {
    // the first chunk is fetched now (before the W window, as in the steady
    // state); each chunk is stored into LDS at its start and the next one is
    // fetched into registers right after
    fetch(kbeg, kend - kbeg);
#pragma unroll
    for (int u = 0; u < WIN; ++u) load_step(w[u], kb_beg + u);

    int buf = 0;
    for (int kw = kb_beg; kw < kb_end; kw += WIN) {
#pragma unroll
      for (int cc = 0; cc < CPW; ++cc) {
        const int k0 = (kw + cc * CSTEPS) * 32;  // first K index of this chunk
        store(buf);
        fetch(k0 + KC, kend - k0 - KC);
        __syncthreads();
        const T* hi = xbuf + buf * BUF_ELEMS;
        buf ^= 1;
        compute_chunk(kw, cc, [hi](int r, int kk, int pl) {
          return hi + pl * TROWS * LDS_ROW + r * LDS_ROW + kk;
        });
      }
    }
  }

  if constexpr (kSepLo) {
#pragma unroll
    for (int t = 0; t < NTW; ++t)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[t][mt][r] = acc[t][mt][r] + acl[t][mt][r];
  }

  // ---- results
  const int col0 = t0 * 16;             // first output column of the workgroup
  const int width = (t1 - t0) * 16;     // its output columns (<= COLS)
  const int N = a.ntiles * 16;
  if (EPI == EPI_PART && !STK) {
    float* P = a.P + (size_t)sk * a.P_ld * N;
#pragma unroll
    for (int t = 0; t < NTW; ++t)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int m = a.row0 + mt * 16 + r16;
        if (m < a.M && live) {
          float* pp = P + (size_t)m * N + (tbase + t) * 16 + 4 * g;
          *reinterpret_cast<float4*>(pp) =
              make_float4(acc[t][mt][0], acc[t][mt][1], acc[t][mt][2], acc[t][mt][3]);
        }
      }
    return;
  }
  // S == 1 (or stacked rows): tile [TROWS][COLS] in LDS (reusing the
  // staging area)
  constexpr int LDT = COLS + 1;
  float* tile = reinterpret_cast<float*>(smem);
  __syncthreads();
#pragma unroll
  for (int t = 0; t < NTW; ++t)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        tile[(mt * 16 + r16) * LDT + (wave * NTW + t) * 16 + 4 * g + r] = acc[t][mt][r];
  if (kNorm && (int)threadIdx.x < mc)
    rsc[threadIdx.x] = a.norm.ss ? row_scale(a.norm, a.row0 + threadIdx.x) : 1.0f;
  __syncthreads();
  // output rows of the tile, and an output value (stacked: hi row + lo row)
  const int orows = STK ? mc : TROWS;
  auto val = [&](int row, int col) -> float {
    float v = tile[row * LDT + col];
    if constexpr (STK) v += tile[(row + mc) * LDT + col];
    return v;
  };

  if (EPI == EPI_PART) {  // stacked rows only
    float* P = a.P + (size_t)sk * a.P_ld * N;
    for (int e = threadIdx.x; e < orows * width; e += NTHR) {
      const int row = e / width, col = e % width;
      P[(size_t)(a.row0 + row) * N + col0 + col] = val(row, col);
    }
    return;
  }

  if (EPI == EPI_SWIGLU) {
    // tile pair p: columns [p*32, p*32+16) gate, [p*32+16, p*32+32) up
    const int outs = width / 2;
    for (int e = threadIdx.x; e < orows * outs; e += NTHR) {
      const int row = e / outs, j = e % outs;
      const int m = a.row0 + row;
      if (m >= a.M) continue;
      const int p = j >> 4, c = j & 15;
      const float gv = val(row, p * 32 + c) * rsc[row];
      const float uv = val(row, p * 32 + 16 + c) * rsc[row];
      T* Yh = reinterpret_cast<T*>(a.Y);
      store_act(Yh, Yh + a.ylo, (size_t)m * a.ldy + col0 / 2 + j,
                gv / (1.0f + expf(-gv)) * uv);
    }
    return;
  }
  // EPI_ARGMAX
  for (int e = threadIdx.x; e < orows * width; e += NTHR) {
    const int row = e / width, col = e % width;
    const int m = a.row0 + row;
    if (m >= a.M) continue;
    const int n = col0 + col;
    float v = val(row, col) * rsc[row];
    if (n >= a.ncols) v = -INFINITY;
    if (n == a.bias_tok && a.rows[m].pos >= a.bias_after) v += a.bias;
    if (a.logits && n < a.ncols) a.logits[(size_t)m * a.ldlog + n] = v;
    tile[row * LDT + col] = v;
  }
  __syncthreads();
  for (int row = threadIdx.x; row < orows; row += NTHR) {
    const int m = a.row0 + row;
    if (m >= a.M) continue;
    float best = -INFINITY;
    int bi = col0;
    for (int col = 0; col < width; ++col) {
      const float v = tile[row * LDT + col];
      if (v > best) { best = v; bi = col0 + col; }  // NaN never wins
    }
    a.part[(size_t)m * a.nblocks + nb] = make_float2(best, __int_as_float(bi));
  }
}

template <typename T, int MT, int NTW, int WAVES, int EPI, int D = kD, int WF = 0,
          bool STK = false>
hipError_t launch_one(const GemmArgs& a, const LaunchCtx& s) {
  auto k = gemm_kernel<T, MT, NTW, WAVES, EPI, D, WF, STK>;
  constexpr int KC = STK ? kChunkStk : ChunkK<MT>::value;
  // two buffers of MT*16 rows x (KC + pad) of 4 bytes (bf16 hi + lo, or fp32)
  // or 2 bytes (one plane of stacked bf16 rows)
  const size_t stage_b =
      2 * (size_t)MT * 16 * (KC + (sizeof(T) == 2 ? 8 : 4)) * (STK ? 2 : 4);
  const size_t tile_b = (size_t)MT * 16 * (WAVES * NTW * 16 + 1) * 4;
  // stacked rows stage in static LDS; the dynamic area holds the result tile
  const size_t lds = STK ? tile_b : (stage_b > tile_b ? stage_b : tile_b);
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void*)k,
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)lds);
    if (e != hipSuccess) return e;
  }
  if (s.t0 || s.t1) {
    GemmArgs arg = a;
    void* args[] = {&arg};
    return hipExtLaunchKernel((const void*)k, dim3(a.ncb * a.S), dim3(WAVES * 64), args, lds,
                              s.s, s.t0, s.t1, 0);
  }
  k<<<a.ncb * a.S, WAVES * 64, lds, s.s>>>(a);
  return hipGetLastError();
}

// ---------------------------------------------------------------- tall GEMM
// More than 128 rows (bf16 activation planes; fused multi-request verify
// passes and prefill chunks): the skinny kernel above gives each wave one
// column tile and every row, so each staged activation fragment feeds one
// MFMA and the LDS reads grow with the rows.  Here a wave owns a block of
// RT row tiles x kTallCT column tiles: per K-step it reads RT x 2 activation
// fragments (hi, lo) from LDS and kTallCT weight fragments from memory and
// issues RT x kTallCT x 2 MFMAs, so each fragment feeds several MFMAs.
// A workgroup is kTallWM x kTallWN waves: kTallWM row groups (all of a
// launch's rows up to 288, so a weight tile is streamed once per 288 rows)
// by kTallWN column groups (128 columns).  Activations go from memory
// straight into LDS in chunks of two K-steps (both planes), the next chunk
// in flight while one is used; weights stream through a window of four
// K-steps in registers.  (Staging one K-step at a time through registers,
// with one step of weights ahead, left each step waiting for its loads:
// 38% matrix-core use on the 8B gate/up at 288 rows.)  Epilogues as in the skinny
// kernel, written from registers: split partials, SwiGLU (the gate and up
// tiles of a pair are a wave's column tiles 2q and 2q + 1), and the per-row
// argmax partial of the workgroup's 128 columns.
// (3 x 4 waves of 6 x 2 tiles measured 158 us for the 8B gate/up at 288
// rows against 169 us for 3 x 2 waves of 6 x 4 tiles, and 258 us for 64
// columns a workgroup: each workgroup stages all its rows, so wider
// column blocks stage less per MFMA)
constexpr int kTallWM = 3;   // row groups
constexpr int kTallWN = 4;   // column groups
constexpr int kTallCT = 2;   // column tiles per wave
constexpr int kTallWaves = kTallWM * kTallWN;
constexpr int kTallCols = kTallWN * kTallCT * 16;  // columns of a workgroup (128)

template <int RT, int EPI, int WF>
__global__ __launch_bounds__(kTallWaves * 64) void gemm_tall_kernel(GemmArgs a) {
  constexpr int CT = kTallCT;
  constexpr int RB = kTallWM * RT * 16;  // rows of a workgroup
  constexpr int NTHR = kTallWaves * 64;
  constexpr bool W12 = WF == 1, W8 = WF == 2;
  __shared__ float rsc[RB];
  using WReg = typename std::conditional<
      W12, W12Raw, typename std::conditional<W8, uint2, Frag<uint16_t>>::type>::type;
  constexpr uint32_t TB = W12 ? kW12TileBytes : W8 ? kW8TileBytes : 1024;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave % kTallWM, wn = wave / kTallWM;
  const int g = lane >> 4, r16 = lane & 15;
  const int cb = blockIdx.x % a.ncb, sk = blockIdx.x / a.ncb;
  const int rbase = blockIdx.y * RB;  // first row of the workgroup
  const int rows = min(RB, a.M - rbase);
  const int tile0 = cb * (kTallCols / 16) + wn * CT;  // the wave's first column tile
  const int kbeg = sk * a.KR, kend = min(a.K, kbeg + a.KR);
  const int kb_beg = kbeg >> 5, kb_end = kend >> 5;

  __amdgpu_buffer_rsrc_t wrs[CT];
  uint32_t eb7[CT];
#pragma unroll
  for (int t = 0; t < CT; ++t) {
    const size_t tr = (size_t)(tile0 + t);
    wrs[t] = weight_rsrc(reinterpret_cast<const uint8_t*>(a.W) + tr * a.wsn * TB);
    if constexpr (W12 || W8) {
      const uint32_t e = a.eb[tr * 16 + r16];
      eb7[t] = (e | (e << 16)) << 7;
    } else {
      eb7[t] = 0;
    }
  }
  const uint32_t wk = (uint32_t)a.wsk * TB;
  const uint32_t* ovf = W12 ? w12_overflow(a.W, (size_t)a.ntiles * (a.K / 32)) : nullptr;
  auto load_step = [&](WReg (&dst)[CT], int kb) {
    const int k = kb < kb_end ? kb : kb_end - 1;  // past the end: the last tile again
    const int so = (int)((uint32_t)k * wk);
#pragma unroll
    for (int t = 0; t < CT; ++t) {
      if constexpr (W12) {
        const u32x3_t d = __builtin_amdgcn_raw_buffer_load_b96(wrs[t], lane * 12, so, 0);
        dst[t] = W12Raw{d.x, d.y, d.z,
                        __builtin_amdgcn_raw_buffer_load_b32(
                            wrs[t], (kW12SlotDword + (lane & 7)) * 4, so, 0)};
      } else if constexpr (W8) {
        dst[t] = __builtin_bit_cast(
            uint2, __builtin_amdgcn_raw_buffer_load_b64(wrs[t], lane * 8, so, 0));
      } else {
        dst[t].v = __builtin_bit_cast(
            uint4, __builtin_amdgcn_raw_buffer_load_b128(wrs[t], lane * 16, so, 0));
      }
    }
  };
  auto wfrag = [&](const WReg& r, int t) -> Frag<uint16_t> {
    if constexpr (W12) {
      Frag<uint16_t> f;
      f.v = w12_decode(r, eb7[t]);
      w12_patch_opaque(f.v, r, lane, ovf);
      return f;
    } else if constexpr (W8) {
      Frag<uint16_t> f;
      f.v = w8_decode(r, eb7[t]);
      return f;
    } else {
      (void)t;
      return r;
    }
  };

  // ---- activation staging: buffer loads that write LDS (no registers), in
  // chunks of two K-steps (32 values of every row, both planes, per step),
  // two chunk buffers in turn.  A step's part of a chunk is 2 x RB/16 blocks
  // of 1 KB (plane, row tile); one wavefront load fills one block: lane L
  // writes bytes [16 L, 16 L + 16) of it, row r = L / 4, 16-byte slot L % 4,
  // which holds that row's unit (L % 4) ^ sz(r), sz(r) = ((r / 2) % 4) ^
  // ((r / 8) % 2): the rows of a fragment read then fall in distinct banks
  // whether the LDS serves 8 lanes of 16 bytes a cycle (rows 0-7 and 8-15
  // apart) or 16 (all 16 rows).  (sz(r) = (r / 4) % 4, right for 16 only,
  // stalled half the LDS cycles on bank conflicts.)  Rows past M and steps past the
  // split load from an offset beyond the buffer's range, which writes zeros.
  // A chunk's loads are issued when no other chunk's are in flight (the
  // compiler orders loads into LDS that it cannot tell apart).
  typedef __attribute__((address_space(3))) void lds_void;
  constexpr int CS = 2;                            // K-steps per chunk
  constexpr int NBLK = 2 * RB / 16;                // blocks per K-step
  static_assert(NBLK % kTallWaves == 0, "whole block loads per wave");
  constexpr int NQS = NBLK / kTallWaves;           // block loads per wave per K-step
  constexpr int STEP = RB * 64;                    // elements per staged K-step
  // one array per (buffer, step), so that the compiler can tell a chunk's
  // loads from the reads of the other buffer
  __shared__ __align__(1024) uint16_t xs00[STEP];
  __shared__ __align__(1024) uint16_t xs01[STEP];
  __shared__ __align__(1024) uint16_t xs10[STEP];
  __shared__ __align__(1024) uint16_t xs11[STEP];
  const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(a.X), (short)0, 0x7FFFFFFF, 0x00020000);
  auto dma_step = [&](uint16_t* dst, int kb) {
    const bool kin = kb < kb_end;
#pragma unroll
    for (int q = 0; q < NQS; ++q) {
      const int b = q * kTallWaves + wave;  // wave-uniform
      const int pl = b / (RB / 16), rt = b % (RB / 16);
      const int r = lane >> 2;
      const int u = (lane & 3) ^ ((r >> 1) & 3) ^ ((r >> 3) & 1);
      const int row = rt * 16 + r;
      const bool in = kin && row < rows;
      const uint32_t voff =
          in ? (uint32_t)(((pl ? (size_t)a.xlo : 0) + (size_t)(rbase + row) * a.ldx + kb * 32 +
                           u * 8) * 2)
             : 0x80000000u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xrs, (lds_void*)(dst + b * 512), 16, voff, 0, 0,
                                               0);
    }
  };
  auto dma = [&](uint16_t* d0, uint16_t* d1, int kb0) {
    dma_step(d0, kb0);
    dma_step(d1, kb0 + 1);
  };

  constexpr bool kNorm = EPI != EPI_PART;
  if (kNorm) {
    for (int r = threadIdx.x; r < RB; r += NTHR)
      rsc[r] = (r < rows && a.norm.ss) ? row_scale(a.norm, rbase + r) : 1.0f;
  }

  floatx4_t acc[RT][CT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int t = 0; t < CT; ++t) acc[rt][t] = floatx4_t{0.f, 0.f, 0.f, 0.f};

  // Pipeline: weights stream through a window of kWin K-steps in
  // registers (a slot is refilled with the step kWin ahead right after its
  // MFMAs); chunk c + 1 is loaded into the other buffer while chunk c is
  // used.  Before a chunk is read each wave waits for its own loads of it
  // (the loads it issued after them are the previous chunk's weight
  // refills, NAFTER; loads complete in order for the counter), then the
  // barrier covers every wave's, and every wave is done with the other
  // buffer.
  constexpr int kWin = 2 * CS;
  constexpr int LPS = W12 ? 2 : 1;  // loads per weight tile per K-step
  constexpr int NAFTER = CS * CT * LPS;
  static_assert(NAFTER < 64, "vmcnt range");
  constexpr int kWait = (NAFTER & 15) | ((NAFTER >> 4) << 14) | (7 << 4) | (15 << 8);
  // the first loads in the order the loop leaves them at its edge (weights
  // of two steps, the first chunk, weights of two more steps), so that the
  // compiler's load counting is exact across the edge
  WReg w[kWin][CT];
  load_step(w[0], kb_beg);
  load_step(w[1], kb_beg + 1);
  __builtin_amdgcn_sched_barrier(0);
  dma(xs00, xs01, kb_beg);
  __builtin_amdgcn_sched_barrier(0);
  load_step(w[2], kb_beg + 2);
  load_step(w[3], kb_beg + 3);

  const int xrow = wm * RT * 16 + r16;  // the lane's row in the workgroup's first row tile
  const int sw = (g ^ ((r16 >> 1) & 3) ^ ((r16 >> 3) & 1)) * 8;  // the lane's slot in a staged row
  auto kstep = [&](int kb, const uint16_t* cur, WReg (&wu)[CT]) {
    Frag<uint16_t> xh[RT], xl[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const uint16_t* p = cur + (wm * RT + rt) * 512 + r16 * 32 + sw;
      xh[rt].load(p);
      xl[rt].load(p + RB * 32);
    }
    Frag<uint16_t> wf[CT];
#pragma unroll
    for (int t = 0; t < CT; ++t) wf[t] = wfrag(wu[t], t);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int t = 0; t < CT; ++t) {
        mma32(acc[rt][t], wf[t], xh[rt]);
        mma32(acc[rt][t], wf[t], xl[rt]);
      }
    // the slot's refill goes after the MFMAs that read it (bf16 tiles are
    // used as loaded): issued earlier, it would need other registers and a
    // copy back at the loop edge, which waits for the load
    __builtin_amdgcn_sched_barrier(0);
    load_step(wu, kb + kWin);
    __builtin_amdgcn_sched_barrier(0);
  };
  auto arrive = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(kWait);
    __syncthreads();
  };
  // steps past the end: zero activations (and the last weight tile again)
  for (int kb = kb_beg; kb < kb_end; kb += 2 * CS) {
    arrive();
    dma(xs10, xs11, kb + CS);
    __builtin_amdgcn_sched_barrier(0);
    kstep(kb, xs00, w[0]);
    kstep(kb + 1, xs01, w[1]);
    arrive();
    dma(xs00, xs01, kb + 2 * CS);
    __builtin_amdgcn_sched_barrier(0);
    kstep(kb + 2, xs10, w[2]);
    kstep(kb + 3, xs11, w[3]);
  }
  // the last chunk's loads (zeros) land before the LDS is reused or freed
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));  // vmcnt(0)

  // ---- results (registers: lane (r16, g) holds row r16, columns 4g..4g+3
  // of each tile)
  const int N = a.ntiles * 16;
  if constexpr (EPI == EPI_PART) {
    float* P = a.P + (size_t)sk * a.P_ld * N;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int lr = xrow + rt * 16;
      if (lr >= rows) continue;
      const size_t m = (size_t)(rbase + lr);
#pragma unroll
      for (int t = 0; t < CT; ++t)
        *reinterpret_cast<float4*>(P + m * N + (tile0 + t) * 16 + 4 * g) =
            make_float4(acc[rt][t][0], acc[rt][t][1], acc[rt][t][2], acc[rt][t][3]);
    }
    return;
  }
  __syncthreads();  // rsc
  if constexpr (EPI == EPI_SWIGLU) {
    uint16_t* Yh = reinterpret_cast<uint16_t*>(a.Y);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int lr = xrow + rt * 16;
      if (lr >= rows) continue;
      const float sc = rsc[lr];
      const size_t m = (size_t)(rbase + lr);
#pragma unroll
      for (int q = 0; q < CT / 2; ++q) {
        float o[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float gv = acc[rt][2 * q][r] * sc;
          const float uv = acc[rt][2 * q + 1][r] * sc;
          o[r] = gv / (1.0f + expf(-gv)) * uv;
        }
        const int col = ((tile0 + 2 * q) >> 1) * 16 + 4 * g;
        store_act4(Yh, Yh + a.ylo, m * a.ldy + col, make_float4(o[0], o[1], o[2], o[3]));
      }
    }
    return;
  }
  // EPI_ARGMAX: per row, the largest value of the workgroup's columns and
  // its lowest index: over the lane's 16 values, the 4 lanes of the row, then
  // the column groups (through LDS)
  float2* red = reinterpret_cast<float2*>(xs00);  // [kTallWN][RB]
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int lr = xrow + rt * 16;
    const bool live = lr < rows;
    const int m = rbase + (live ? lr : 0);
    const float sc = rsc[lr];
    float best = -INFINITY;
    int bi = cb * kTallCols;
#pragma unroll
    for (int t = 0; t < CT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int n = (tile0 + t) * 16 + 4 * g + r;
        float v = acc[rt][t][r] * sc;
        if (n >= a.ncols) v = -INFINITY;
        if (live && n == a.bias_tok && a.rows[m].pos >= a.bias_after) v += a.bias;
        if (live && a.logits && n < a.ncols) a.logits[(size_t)m * a.ldlog + n] = v;
        if (v > best || (v == best && n < bi)) {  // NaN never wins
          best = v;
          bi = n;
        }
      }
#pragma unroll
    for (int o = 16; o < 64; o <<= 1) {
      const float ov = __shfl_xor(best, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      if (ov > best || (ov == best && oi < bi)) {
        best = ov;
        bi = oi;
      }
    }
    if (g == 0) red[wn * RB + lr] = make_float2(best, __int_as_float(bi));
  }
  __syncthreads();
  for (int lr = threadIdx.x; lr < rows; lr += NTHR) {
    float2 b = red[lr];
#pragma unroll
    for (int c = 1; c < kTallWN; ++c) {
      const float2 o = red[c * RB + lr];
      if (o.x > b.x || (o.x == b.x && __float_as_int(o.y) < __float_as_int(b.y))) b = o;
    }
    a.part[(size_t)(rbase + lr) * a.nblocks + cb] = b;
  }
}

template <int RT, int EPI, int WF>
hipError_t launch_tall_rt(const GemmArgs& a, int nrb, const LaunchCtx& s) {
  auto k = gemm_tall_kernel<RT, EPI, WF>;
  const dim3 grid(a.ncb * a.S, nrb);
  if (s.t0 || s.t1) {
    GemmArgs arg = a;
    void* args[] = {&arg};
    return hipExtLaunchKernel((const void*)k, grid, dim3(kTallWaves * 64), args, 0, s.s, s.t0,
                              s.t1, 0);
  }
  k<<<grid, kTallWaves * 64, 0, s.s>>>(a);
  return hipGetLastError();
}

// Row tiles per wave by the launch's rows: 96, 192 or 288 rows per workgroup
// (more rows: several row blocks of 288).
template <int EPI, int WF>
hipError_t launch_tall_fmt(const GemmArgs& a, const LaunchCtx& s) {
  const int rt = a.M <= 96 ? 2 : a.M <= 192 ? 4 : 6;
  const int rb = kTallWM * rt * 16;
  const int nrb = (a.M + rb - 1) / rb;
  if (rt == 2) return launch_tall_rt<2, EPI, WF>(a, nrb, s);
  if (rt == 4) return launch_tall_rt<4, EPI, WF>(a, nrb, s);
  return launch_tall_rt<6, EPI, WF>(a, nrb, s);
}

template <int WF>
hipError_t launch_tall_epi(int epi, const GemmArgs& a, const LaunchCtx& s) {
  if (epi == EPI_PART) return launch_tall_fmt<EPI_PART, WF>(a, s);
  if (epi == EPI_SWIGLU) return launch_tall_fmt<EPI_SWIGLU, WF>(a, s);
  if (epi == EPI_ARGMAX) return launch_tall_fmt<EPI_ARGMAX, WF>(a, s);
  return hipErrorInvalidValue;
}

// Workgroup shapes: (tiles per wave, waves, workgroups per K split).  Up to
// 40 rows (bf16: the stacked-row limit) one tile per wave: up to 2048 tiles
// 8-tile workgroups (one round on 256 CUs); 2049-2560 tiles (the 27B gate/up,
// 2176 tiles) 256 workgroups of 8-10 tiles on 10 waves (a balanced share
// of every CU: 64.8 us against 77.5 us for 136 workgroups of two tiles per
// wave on 8 waves, and 96 us for 272 workgroups of 8, which leave a second
// round); more tiles (the LM heads) rounds of 256 workgroups of at most 8
// tiles (27B LM head 252 us against 268 us for 1188 workgroups of 8).  From
// 41 to 128 rows: 256 columns with two tiles per wave for wide matrices
// (>= 128 blocks of 256 columns: the LM head; half the LDS reads per MFMA),
// two tiles per wave on 4 waves for narrow ones up to 95 rows, and one tile
// per wave on 8 waves from 96 rows (8 row tiles; two waves per SIMD instead
// of one) (the 8B gate/up at 65 rows: 66 us, against 99 us for the tall
// kernel's 96-row workgroups).  More than 128 rows with bf16 activations:
// the tall kernel, one workgroup per 128 columns (ntw 0).  fp32 models: one
// tile per wave on 8 waves.  Measured on the 8B and 27B shapes, weights
// streamed from HBM.
struct Variant {
  int ntw, waves, ncb;
};

Variant gemm_variant(bool bf16, int N, int M) {
  const int nt = N / 16;
  if (!bf16) return {1, 8, nt / 8};
  if (M <= 40) {
    if (nt <= 2048) return {1, 8, nt / 8};
    if (nt <= 2560) return {1, 10, 256};
    return {1, 8, 256 * ((nt + 2047) / 2048)};
  }
  if (M <= 128) {
    if (N / 256 >= 128) return {2, 8, nt / 16};
    return M >= 96 ? Variant{1, 8, nt / 8} : Variant{2, 4, nt / 8};
  }
  // more rows: the tall kernel (ntw 0), 128 columns a workgroup
  return {0, kTallWaves, N / kTallCols};
}

template <typename T, int EPI, int NTW, int WAVES, int D, int WF>
hipError_t launch_mt(int mt, const GemmArgs& a, const LaunchCtx& s) {
  switch (mt) {
    case 1: return launch_one<T, 1, NTW, WAVES, EPI, D, WF>(a, s);
    case 2: return launch_one<T, 2, NTW, WAVES, EPI, D, WF>(a, s);
    case 3: return launch_one<T, 3, NTW, WAVES, EPI, D, WF>(a, s);
    case 4: return launch_one<T, 4, NTW, WAVES, EPI, (NTW > 1 ? 4 : D), WF>(a, s);
    case 5: return launch_one<T, 5, NTW, WAVES, EPI, (NTW > 1 ? 4 : D), WF>(a, s);
    default: return launch_one<T, 8, NTW, WAVES, EPI, (NTW > 1 ? 4 : D), WF>(a, s);
  }
}

// stacked hi / lo rows (bf16, one tile per wave, 8 or 10 waves): mt = row
// tiles of the 2 * rows stacked rows (1..5)
template <typename T, int EPI, int WF, int WAVES>
hipError_t launch_stk(int mt, const GemmArgs& a, const LaunchCtx& s) {
  if constexpr (sizeof(T) == 2) {
    switch (mt) {
      case 1: return launch_one<T, 1, 1, WAVES, EPI, kD, WF, true>(a, s);
      case 2: return launch_one<T, 2, 1, WAVES, EPI, kD, WF, true>(a, s);
      case 3: return launch_one<T, 3, 1, WAVES, EPI, kD, WF, true>(a, s);
      case 4: return launch_one<T, 4, 1, WAVES, EPI, kD, WF, true>(a, s);
      case 5: return launch_one<T, 5, 1, WAVES, EPI, kD, WF, true>(a, s);
      default: break;
    }
  }
  return hipErrorInvalidValue;
}

template <typename T, int EPI, int WF>
hipError_t launch_var(Variant v, int mt, bool stk, const GemmArgs& a,
                      const LaunchCtx& s) {
  if (stk) return v.waves == 10 ? launch_stk<T, EPI, WF, 10>(mt, a, s)
                                : launch_stk<T, EPI, WF, 8>(mt, a, s);
  if constexpr (sizeof(T) == 2) {
    if (v.ntw == 2 && v.waves == 8) return launch_mt<T, EPI, 2, 8, kD, WF>(mt, a, s);
    if (v.ntw == 2 && v.waves == 4) return launch_mt<T, EPI, 2, 4, kD, WF>(mt, a, s);
  }
  if (v.ntw == 1 && v.waves == 8) return launch_mt<T, EPI, 1, 8, kD, WF>(mt, a, s);
  return hipErrorInvalidValue;
}

template <typename T, int WF>
hipError_t launch_fmt(int epi, Variant v, const GemmArgs& a, int mt, bool stk,
                      const LaunchCtx& s) {
  if (epi == EPI_PART) return launch_var<T, EPI_PART, WF>(v, mt, stk, a, s);
  if (epi == EPI_SWIGLU) return launch_var<T, EPI_SWIGLU, WF>(v, mt, stk, a, s);
  if (epi == EPI_ARGMAX) return launch_var<T, EPI_ARGMAX, WF>(v, mt, stk, a, s);
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t launch_typed(int epi, Variant v, const GemmArgs& a, int mt, bool stk,
                        const LaunchCtx& s) {
  if constexpr (sizeof(T) == 2) {
    if (a.w12 == 1) return launch_fmt<T, 1>(epi, v, a, mt, stk, s);
    if (a.w12 == 2) return launch_fmt<T, 2>(epi, v, a, mt, stk, s);
  }
  if (a.w12) return hipErrorInvalidValue;
  return launch_fmt<T, 0>(epi, v, a, mt, stk, s);
}

}  // namespace

int gemm_pad_cols() { return 256; }

int gemm_argmax_blocks(bool bf16, int N, int M) { return gemm_variant(bf16, N, M).ncb; }

// K per split: whole K-steps, the last split possibly shorter.
static int split_k(int K, int S) { return (K / 32 + S - 1) / S * 32; }

int gemm_splits(bool bf16, int K, int N, int M) {
  // at most one workgroup per CU: the largest split count (of those the
  // consumers of the partials are built for) whose grid fits the 256 CUs,
  // with at least 256 reduction indices per split.  Splits of equal length
  // first (5 splits: 200 workgroups for the 40 column blocks of a 5120-wide
  // matrix, where 4 leave 96 CUs idle); if those fill under three quarters
  // of the CUs, a shorter last split is allowed (the 27B down GEMM, 544
  // K-steps: 6 splits, 240 workgroups instead of 160; where equal splits
  // already fill three quarters, the extra partials cost more than the
  // extra workgroups gain: the 8B QKV at 5 splits instead of 4 measured 1%
  // slower per step)
  const int nblk = gemm_variant(bf16, N, M).ncb;
  int S = 1;
  for (int c : {2, 4, 5, 8, 16, 32})
    if (c * nblk <= 256 && K % (32 * c) == 0 && K / c >= 256) S = c;
  if (4 * S * nblk < 3 * 256 && K % 32 == 0) {
    for (int c : {2, 4, 5, 6, 8, 16, 32})
      if (c > S && c * nblk <= 256 && K / c >= 256 && (c - 1) * split_k(K, c) < K) S = c;
  }
  return S;
}

hipError_t launch_gemm(bool bf16, int epi, const GemmArgs& a0, hipStream_t s,
                       hipEvent_t t0, hipEvent_t t1) {
  if (a0.M <= 0) return hipSuccess;
  GemmArgs a = a0;
  if (a.S < 1 || (epi != EPI_PART && a.S != 1) || a.K % 32) return hipErrorInvalidValue;
  a.KR = split_k(a.K, a.S);  // every split non-empty; the last may be shorter
  if ((a.S - 1) * a.KR >= a.K) return hipErrorInvalidValue;
  if (a.wsn <= 0 || a.wsk <= 0) return hipErrorInvalidValue;
  // weights are addressed through 32-bit buffer offsets: at most 4 GB a matrix
  if (a.w12 < 0 || a.w12 > 2) return hipErrorInvalidValue;
  const size_t tile_bytes = a.w12 == 1 ? kW12TileBytes
                            : a.w12 == 2 ? kW8TileBytes
                                         : (bf16 ? 1024 : 2048);
  if ((size_t)a.ntiles * (a.K / 32) * tile_bytes > 0xFFFFFFFFull) return hipErrorInvalidValue;
  // one workgroup shape for all row chunks (the ARGMAX block layout and the
  // partial sums must not depend on the chunk)
  const Variant v = gemm_variant(bf16, a.ntiles * 16, a.M);
  a.ncb = v.ncb;
  if (v.ntw == 0) {  // tall: all rows in one launch
    if (a.ntiles % (kTallCols / 16) || a.ncb < 1) return hipErrorInvalidValue;
    // activations are addressed through 31-bit byte offsets (both planes)
    if (((size_t)a.xlo + (size_t)a.M * a.ldx) * 2 >= 0x7FFFFFFFull) return hipErrorInvalidValue;
    if (epi == EPI_ARGMAX) a.nblocks = a.ncb;
    a.row0 = 0;
    const LaunchCtx lc{s, t0, t1};
    if (a.w12 == 1) return launch_tall_epi<1>(epi, a, lc);
    if (a.w12 == 2) return launch_tall_epi<2>(epi, a, lc);
    return launch_tall_epi<0>(epi, a, lc);
  }
  a.gt = (epi == EPI_SWIGLU && v.ntw == 1) ? 2 : v.ntw;
  // every workgroup's share of whole granules must fit its waves
  if (a.ntiles % a.gt || a.ncb < 1 || a.ncb > a.ntiles / a.gt ||
      ((a.ntiles / a.gt + a.ncb - 1) / a.ncb) * a.gt > v.waves * v.ntw)
    return hipErrorInvalidValue;
  if (epi == EPI_ARGMAX) a.nblocks = a.ncb;
  for (int r0 = 0; r0 < a.M; r0 += 128) {
    const int rows = (a.M - r0 < 128) ? a.M - r0 : 128;
    // up to 40 rows (bf16, one tile per wave) the lo rows are stacked under
    // the hi rows
    const bool stk = bf16 && v.ntw == 1 && (v.waves == 8 || v.waves == 10) && 2 * rows <= 80;
    const int need = ((stk ? 2 * rows : rows) + 15) / 16;
    const int mt = stk ? need : (need <= 5 ? need : 8);
    a.row0 = r0;
    // timing: the first chunk's start and the last chunk's end
    const LaunchCtx lc{s, r0 == 0 ? t0 : nullptr, r0 + 128 >= a.M ? t1 : nullptr};
    hipError_t e = bf16 ? launch_typed<uint16_t>(epi, v, a, mt, stk, lc)
                        : launch_typed<float>(epi, v, a, mt, false, lc);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}
