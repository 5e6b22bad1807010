// Tree-masked attention over the paged KV cache for one layer.
//
// Every row of the pass is a tree node (or a prompt token in prefill).  A
// node of request r attends to the request's committed keys [0, n_r) and,
// among the pass's own keys (written at slots n_r + node), to itself and its
// ancestors.  GQA: the G = n_heads / n_kv_heads query heads that share a KV
// head are processed together, so each K/V split staged in LDS serves
// (rows * G) query rows.
//
// Workgroup = 8 wavefronts = one (request, KV head, key split, group of
// query tiles of 16 query rows; all of a verify pass's tiles of that KV
// head).  The split's keys (at most 128) are staged in LDS once, with every
// load in flight; then the waves take the group's query tiles in turn and
// keep the transposed flash-attention state
// in registers: S^T = K Q^T (so a lane holds one query row's scores), an
// online softmax in fp32, and O^T += V^T P^T.  With a bf16 cache, the fp32
// operands q and P enter the MFMAs as bf16 hi + lo pairs, so only the stored
// K and V are rounded.  V pages are stored transposed ([dim][16 tokens]) in
// the cache so that the V^T operand is read directly.  Each split writes
// un-normalised partials (O, running max of the scores scaled by log2 e,
// running sum), merged in split order by attn_combine.
//
// Streamed variant (verify passes): a workgroup owns one range of keys of
// one (request, KV head) and one group of at most 8 of its query tiles, and
// walks the range in stages of 64 keys (a range that spans every request's
// keys writes the normalised output itself, with no combine).  The next stage's K
// and V are loaded into registers while the current one (in LDS) is used,
// so a workgroup keeps loads in flight for its whole range instead of
// loading once and computing once.  All 8 waves compute: wave w takes
// query tile w % qt and every kp-th 32-key block (kp = 4, 2 or 1, the
// largest with qt * kp <= 8, from block w / qt), and the kp states of a tile
// are merged in LDS, pairwise in block-part order, before the range's
// partial is written.  With one_part every tile takes kp = 1 (one wave
// walks all its blocks in key order), so a row's result does not depend on
// how many query tiles share its workgroup.
#include <hip/hip_ext.h>

#include "common.h"
#include "index_math.h"
#include "kernels.h"

namespace {

constexpr int kMaxSplitKeys = 128;  // keys of one split staged in LDS at once

// LDS layout of one staged split of `split` keys: K rows [split][HD + KPAD],
// then V^T [HD][split + VPAD] (pads keep 16-byte alignment and spread banks).
template <typename T, int HD>
struct SplitLds {
  static constexpr int KPAD = 16 / sizeof(T);
  static constexpr int VPAD = 16 / sizeof(T);
  static constexpr int KS = HD + KPAD;
  __host__ __device__ static size_t bytes(int split) {
    return ((size_t)split * KS + (size_t)HD * (split + VPAD)) * sizeof(T);
  }
};

template <typename T>
__device__ __forceinline__ void load_vfrag(Frag<T>& f, const T* p0, const T* p1);

template <>
__device__ __forceinline__ void load_vfrag<uint16_t>(Frag<uint16_t>& f,
                                                     const uint16_t* p0,
                                                     const uint16_t* p1) {
  const uint2 a = *reinterpret_cast<const uint2*>(p0);
  const uint2 b = *reinterpret_cast<const uint2*>(p1);
  f.v = make_uint4(a.x, a.y, b.x, b.y);
}

template <>
__device__ __forceinline__ void load_vfrag<float>(Frag<float>& f,
                                                  const float* p0,
                                                  const float* p1) {
  f.lo = *reinterpret_cast<const float4*>(p0);
  f.hi = *reinterpret_cast<const float4*>(p1);
}

__device__ __forceinline__ void pack_p(Frag<uint16_t>& f, const float* p) {
  f.v.x = (uint32_t)f2bf(p[0]) | ((uint32_t)f2bf(p[1]) << 16);
  f.v.y = (uint32_t)f2bf(p[2]) | ((uint32_t)f2bf(p[3]) << 16);
  f.v.z = (uint32_t)f2bf(p[4]) | ((uint32_t)f2bf(p[5]) << 16);
  f.v.w = (uint32_t)f2bf(p[6]) | ((uint32_t)f2bf(p[7]) << 16);
}

__device__ __forceinline__ void pack_p(Frag<float>& f, const float* p) {
  f.lo = make_float4(p[0], p[1], p[2], p[3]);
  f.hi = make_float4(p[4], p[5], p[6], p[7]);
}

// value actually multiplied by V (after rounding to the operand type)
__device__ __forceinline__ float op_round(float x, uint16_t) { return bf2f(f2bf(x)); }
__device__ __forceinline__ float op_round(float x, float) { return x; }

// One 32-key block [kb, kb + 32) of a staged split or stage against one
// query tile: scores S^T = K Q^T for the block's two 16-key tiles, the
// row's visibility mask, the online softmax update of (m_run, l_run, o) and
// O^T += V^T P^T.  sk: K rows [.][KS] with the block's first key at row
// kl; sv: V^T [HD][vs] with it at column kl.  Lane (g, r16) holds query row
// r16 of the tile (node `node` of the request; rows past the pass are
// !qvalid and see no key).
template <typename T, int HD, int KS>
__device__ __forceinline__ void attn_block(const T* sk, const T* sv, int vs, int kl, int kb,
                                           int kend, const ReqMeta& rm, int node, bool qvalid,
                                           uint64_t anc_lo, uint64_t anc_hi,
                                           const Frag<T> (&qf)[HD / 32],
                                           const Frag<T> (&qfl)[HD / 32], float scale2, int g,
                                           int r16, float& m_run, float& l_run,
                                           floatx4_t (&o)[HD / 16]) {
  constexpr bool kSplit = sizeof(T) == 2;
  // all K fragments of the block are read from LDS first, then the two
  // independent score chains are interleaved (hi and lo halves of q
  // accumulate separately: four chains of HD / 32 dependent MFMAs)
  floatx4_t s[2], sl[2];
  Frag<T> kf[2][HD / 32];
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int ks = 0; ks < HD / 32; ++ks)
      kf[kt][ks].load(&sk[(size_t)(kl + kt * 16 + r16) * KS + ks * 32 + g * 8]);
  s[0] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  s[1] = s[0];
  sl[0] = s[0];
  sl[1] = s[0];
#pragma unroll
  for (int ks = 0; ks < HD / 32; ++ks) {
    mma32(s[0], kf[0][ks], qf[ks]);
    mma32(s[1], kf[1][ks], qf[ks]);
    if (kSplit) {
      mma32(sl[0], kf[0][ks], qfl[ks]);
      mma32(sl[1], kf[1][ks], qfl[ks]);
    }
  }
  if (kSplit) {
    s[0] += sl[0];
    s[1] += sl[1];
  }
  // visibility of the block's 32 keys for this lane's row, as a bit mask
  // (bit i: key kb + i): keys past the range end are out; committed keys
  // are in; a pass key (tree node tn = key - nctx) is in along a chain up to
  // the row's own node, in a tree when tn is an ancestor or itself.  A block
  // of committed keys only (the common case) needs no mask arithmetic.
  uint32_t vis = 0;
  if (kb + 32 <= rm.nctx && kb + 32 <= kend) {  // uniform
    vis = qvalid ? 0xffffffffu : 0u;
  } else if (qvalid) {
    auto low_bits = [](int n) -> uint32_t {
      return n >= 32 ? 0xffffffffu : n <= 0 ? 0u : ((1u << n) - 1u);
    };
    const int c = rm.nctx - kb;  // committed keys in the block: [0, c)
    uint32_t pass;
    if (rm.chain) {
      pass = low_bits(c + node + 1);
    } else {
      // block bit i <-> tree node i - c: the ancestor mask shifted by c
      const int sh = -c;  // node of block bit 0 (may be negative)
      uint64_t w;
      if (sh >= 0) {
        w = sh >= 128 ? 0 : sh >= 64 ? (anc_hi >> (sh - 64))
                      : sh == 0 ? anc_lo : ((anc_lo >> sh) | (anc_hi << (64 - sh)));
      } else {
        w = -sh >= 64 ? 0 : (anc_lo << (-sh));
      }
      pass = (uint32_t)w;
    }
    vis = (low_bits(c) | pass) & low_bits(kend - kb);
  }
  // lane holds row r16, keys kb + kt*16 + 4g + r; scores in the base-2
  // domain (scaled by log2 e) so that every weight is one v_exp_f32
  float p[8];
  float mx = -INFINITY;
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const bool ok = (vis >> (kt * 16 + 4 * g + r)) & 1u;
      const float v = ok ? s[kt][r] * scale2 : -INFINITY;
      p[kt * 4 + r] = v;
      mx = fmaxf(mx, v);
    }
  mx = quad_max(mx);
  // No lane may skip the MFMAs below (they read operands of all lanes), so
  // a row with nothing visible yet uses a finite stand-in maximum: every
  // weight is then 2^-inf = 0 and the state stays (-inf, 0, O = 0).
  const float m_new = fmaxf(m_run, mx);
  const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
  const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);  // 2^-inf = 0
  float lsum = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    p[e] = __builtin_amdgcn_exp2f(p[e] - m_use);  // hidden keys: 2^-inf = 0
    lsum += p[e];
  }
  lsum = quad_sum(lsum);
  l_run = l_run * alpha + lsum;
  m_run = m_new;
  // rescale only when some row's maximum moved (alpha is exactly 1
  // otherwise, so skipping changes no bit)
  if (__any(alpha != 1.0f)) {
#pragma unroll
    for (int dt = 0; dt < HD / 16; ++dt) o[dt] *= alpha;
  }

  // P as an operand of the KV type; for bf16 it is carried as a hi + lo
  // pair (two MFMAs), which keeps ~16 mantissa bits of the weights
  Frag<T> pf, pf_lo;
  if (kSplit) {
    float lo[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) lo[e] = p[e] - op_round(p[e], T(0));
    pack_p(pf_lo, lo);
  }
  pack_p(pf, p);
  // V fragments in groups of four dim tiles, read before their MFMAs
#pragma unroll
  for (int d0 = 0; d0 < HD / 16; d0 += 4) {
    Frag<T> vf[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const T* vrow = sv + (size_t)((d0 + u) * 16 + r16) * vs + kl;
      load_vfrag<T>(vf[u], vrow + 4 * g, vrow + 16 + 4 * g);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) mma32(o[d0 + u], vf[u], pf);
    if (kSplit) {
#pragma unroll
      for (int u = 0; u < 4; ++u) mma32(o[d0 + u], vf[u], pf_lo);
    }
  }
}

constexpr int kAttnWaves = 8;
constexpr int kAttnThreads = kAttnWaves * 64;
static_assert(kAttnStreamTiles <= kAttnWaves, "a streamed tile per wave");

// Staging of one split (at most kMaxSplitKeys keys from kbeg) in chunks of
// 16 bytes: thread t takes chunk t + j * kAttnThreads (j < NC) of K and of
// V.  The loads are unconditional (chunk indexes past the split's repeat its
// last chunk, keys past kend read the last key's page slots; spg holds the
// split's pages, one per 16 keys) and the data is only stored to LDS
// afterwards, so all of a thread's loads are in flight together.  (Loads
// under per-lane conditions made the compiler wait for each one before
// issuing the next.)
template <typename T, int NC>
struct SplitChunks {
  uint4 k[NC], v[NC];
};

template <typename T, int HD, int NC>
__device__ __forceinline__ SplitChunks<T, NC> split_issue(const T* kc, const T* vc,
                                                          const int* spg, int nkv, int kvh,
                                                          int kbeg, int nkeys, int kch) {
  constexpr int EPC = 16 / sizeof(T);
  constexpr int KCH_ROW = HD / EPC;
  constexpr int VCH_ROW = 16 / EPC;
  static_assert(KCH_ROW * 16 == HD * VCH_ROW, "as many V chunks as K chunks");
  const int nslots = (nkeys + 15) >> 4;
  SplitChunks<T, NC> r;
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    const int c = min((int)threadIdx.x + j * kAttnThreads, kch - 1);
    {
      const int i = min(c / KCH_ROW, nkeys - 1), part = c % KCH_ROW;
      r.k[j] = *reinterpret_cast<const uint4*>(
          kc + kv_k_index(spg[i >> 4], nkv, kvh, (kbeg + i) & 15, HD, part * EPC));
    }
    {
      // chunk c of V: page blk = c / (HD * VCH_ROW), then (dim, part) in the
      // page's [dim][16 keys] order, so a wave reads contiguous memory
      const int blk = c / (HD * VCH_ROW), rest = c % (HD * VCH_ROW);
      const int dim = rest / VCH_ROW, part = rest % VCH_ROW;
      r.v[j] = *reinterpret_cast<const uint4*>(
          vc + kv_v_index(spg[min(blk, nslots - 1)], nkv, kvh, part * EPC, HD, dim));
    }
  }
  return r;
}

// The chunks into LDS (K rows [key][KS], V^T [dim][vs]); V of keys past kend
// (not written this pass) is cleared there after its chunk is stored (K of
// those keys is masked out of the scores).
// Chunks past the split's (c >= kch) are stored to `spill`, a 16-byte LDS
// slot that nothing reads, so that every store is unconditional (a guarded
// store let the compiler move its load under the guard, behind the wait for
// the previous chunk).
template <typename T, int HD, int KS, int NC>
__device__ __forceinline__ void split_place(const SplitChunks<T, NC>& r, T* sk, T* sv, int vs,
                                            int kbeg, int kend, int kch, uint4* spill) {
  constexpr int EPC = 16 / sizeof(T);
  constexpr int KCH_ROW = HD / EPC;
  constexpr int VCH_ROW = 16 / EPC;
  // every store first (one basic block, so no load is moved down to a
  // guarded use), then the clearing of V past kend
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    const int c = threadIdx.x + j * kAttnThreads;
    const bool in = c < kch;
    {
      const int i = c / KCH_ROW, part = c % KCH_ROW;
      *(in ? reinterpret_cast<uint4*>(&sk[(size_t)i * KS + part * EPC]) : spill) = r.k[j];
    }
    const int blk = c / (HD * VCH_ROW), rest = c % (HD * VCH_ROW);
    const int dim = rest / VCH_ROW, part = rest % VCH_ROW;
    *(in ? reinterpret_cast<uint4*>(&sv[(size_t)dim * vs + blk * 16 + part * EPC]) : spill) =
        r.v[j];
  }
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    const int c = threadIdx.x + j * kAttnThreads;
    const int blk = c / (HD * VCH_ROW), rest = c % (HD * VCH_ROW);
    const int dim = rest / VCH_ROW, part = rest % VCH_ROW;
    const int t0 = kbeg + blk * 16 + part * EPC;
    if (c < kch && t0 + EPC > kend) {
      T* dst = &sv[(size_t)dim * vs + blk * 16 + part * EPC];
#pragma unroll
      for (int e = 0; e < EPC; ++e)
        if (t0 + e >= kend) dst[e] = T(0);
    }
  }
}

template <typename T, int HD>
__global__ __launch_bounds__(kAttnThreads, 4) void attn_kernel(AttnArgs a) {
  extern __shared__ __align__(16) unsigned char attn_smem[];
  using L = SplitLds<T, HD>;
  T* sk = reinterpret_cast<T*>(attn_smem);      // [split][KS]
  T* sv = sk + (size_t)a.split * L::KS;          // [HD][VS]
  const int VS = a.split + L::VPAD;

  const int split = blockIdx.x, qg = blockIdx.y;
  const int req = blockIdx.z / a.nkv, kvh = blockIdx.z % a.nkv;
  const ReqMeta rm = a.reqs[req];
  const int G = a.nq / a.nkv;
  const int qrows = rm.nrows * G;
  const int qtiles = (qrows + 15) / 16;
  const int t_beg = qg * a.qtiles_per_wg;
  const int t_end = min(qtiles, t_beg + a.qtiles_per_wg);
  const int total_keys = rm.nctx + rm.nrows;
  const int kbeg = split * a.split;
  if (kbeg >= total_keys || t_beg >= qtiles) return;  // uniform per block
  const int kend = min(total_keys, kbeg + a.split);

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4, r16 = lane & 15;

  const T* kc = reinterpret_cast<const T*>(a.kc);
  const T* vc = reinterpret_cast<const T*>(a.vc);
  const int32_t* bt = a.btab + (size_t)rm.table * a.max_pages;

  constexpr bool kSplit = sizeof(T) == 2;
  const T* q = reinterpret_cast<const T*>(a.q);
  const T* qlo = reinterpret_cast<const T*>(a.q_lo);
  // q fragments of one query tile: hi + lo bf16 planes (bf16 KV) or fp32
  auto load_q = [&](int qtile, Frag<T> (&qf)[HD / 32], Frag<T> (&qfl)[HD / 32]) {
    const int qr = qtile * 16 + r16;
    const bool qvalid = qtile < t_end && qr < qrows;
    const int node = qvalid ? qr / G : 0;
    const int qhead = kvh * G + (qvalid ? qr % G : 0);
    const int grow = rm.row0 + node;
#pragma unroll
    for (int ks = 0; ks < HD / 32; ++ks) {
      const size_t off = ((size_t)grow * a.nq + qhead) * HD + ks * 32 + g * 8;
      if (qvalid) {
        qf[ks].load(q + off);
        if (kSplit) qfl[ks].load(qlo + off);
      } else {
        qf[ks].zero();
        qfl[ks].zero();
      }
    }
  };
  // ancestor masks of a tile's row for this lane
  auto load_anc = [&](int qtile, uint64_t& lo, uint64_t& hi) {
    const int qr = qtile * 16 + r16;
    lo = 0;
    hi = 0;
    if (qtile < t_end && qr < qrows && !rm.chain) {
      const uint64_t* am = a.anc + rm.anc0 + (size_t)(qr / G) * rm.anc_words;
      lo = am[0];
      if (rm.anc_words > 1) hi = am[1];
    }
  };
  // the split's pages (one per 16 keys), looked up once into LDS before any
  // other load is in flight
  __shared__ int spg[kMaxSplitKeys / 16];
  __shared__ uint4 spill;  // the target of chunk stores past the split (never read)
  if ((int)threadIdx.x < (kend - kbeg + 15) >> 4)
    spg[threadIdx.x] = kv_page(rm.page0, bt, kbeg + 16 * threadIdx.x);
  __syncthreads();
  // the wave's first tile (q and ancestor masks) is fetched before the K/V
  // staging (its latency overlaps the staging's)
  Frag<T> qf[HD / 32], qfl[HD / 32];
  load_q(t_beg + wave, qf, qfl);
  uint64_t anc_lo, anc_hi;
  load_anc(t_beg + wave, anc_lo, anc_hi);
  asm volatile("" ::: "memory");  // keep these loads ahead of the staging

  constexpr int EPC = 16 / sizeof(T);           // elements per 16-byte chunk
  constexpr int KCH_ROW = HD / EPC;              // chunks per K row
  // ---- stage the whole split (K rows and V^T, padded with zeros to a
  // multiple of 32 keys) with every load in flight, NC chunks of each per
  // thread, NC as small as the split allows
  {
    const int nkeys = kend - kbeg;  // <= a.split <= kMaxSplitKeys
    const int kch = ((nkeys + 31) & ~31) * KCH_ROW;  // chunks of K, and of V
    constexpr int MAXCH = kMaxSplitKeys * KCH_ROW / kAttnThreads;
    static_assert(MAXCH >= 1 && MAXCH * kAttnThreads == kMaxSplitKeys * KCH_ROW,
                  "chunks per thread");
    const int nc = (kch + kAttnThreads - 1) / kAttnThreads;  // uniform
    if (nc <= 1) {
      const auto r = split_issue<T, HD, 1>(kc, vc, spg, a.nkv, kvh, kbeg, nkeys, kch);
      split_place<T, HD, L::KS, 1>(r, sk, sv, VS, kbeg, kend, kch, &spill);
    } else if (nc == 2 || MAXCH <= 2) {
      const auto r = split_issue<T, HD, (MAXCH < 2 ? MAXCH : 2)>(kc, vc, spg, a.nkv, kvh, kbeg,
                                                                  nkeys, kch);
      split_place<T, HD, L::KS, (MAXCH < 2 ? MAXCH : 2)>(r, sk, sv, VS, kbeg, kend, kch,
                                                          &spill);
    } else if (nc == 3) {
      const auto r = split_issue<T, HD, (MAXCH < 3 ? MAXCH : 3)>(kc, vc, spg, a.nkv, kvh, kbeg,
                                                                  nkeys, kch);
      split_place<T, HD, L::KS, (MAXCH < 3 ? MAXCH : 3)>(r, sk, sv, VS, kbeg, kend, kch,
                                                          &spill);
    } else {
      const auto r = split_issue<T, HD, MAXCH>(kc, vc, spg, a.nkv, kvh, kbeg, nkeys, kch);
      split_place<T, HD, L::KS, MAXCH>(r, sk, sv, VS, kbeg, kend, kch, &spill);
    }
    __syncthreads();
  }

  // each wave takes the group's query tiles in turn (no barriers below)
  for (int qtile = t_beg + wave; qtile < t_end; qtile += kAttnWaves) {
    const int qr = qtile * 16 + r16;
    const bool qvalid = qr < qrows;
    const int node = qvalid ? qr / G : 0;
    const int qhead = kvh * G + (qvalid ? qr % G : 0);
    const int grow = rm.row0 + node;
    if (qtile != t_beg + wave) {  // the first was prefetched
      load_q(qtile, qf, qfl);
      load_anc(qtile, anc_lo, anc_hi);
    }

    const float scale2 = a.scale * 1.44269504088896340736f;  // log2(e)
    float m_run = -INFINITY, l_run = 0.f;
    floatx4_t o[HD / 16];
#pragma unroll
    for (int dt = 0; dt < HD / 16; ++dt) o[dt] = floatx4_t{0.f, 0.f, 0.f, 0.f};

    for (int kb = kbeg; kb < kend; kb += 32)
      attn_block<T, HD, L::KS>(sk, sv, VS, kb - kbeg, kb, kend, rm, node, qvalid, anc_lo, anc_hi,
                               qf, qfl, scale2, g, r16, m_run, l_run, o);

    if (qvalid) {
      const size_t slot = attn_part_slot(split, a.rows_total, a.nq, grow, qhead);
      float* po = a.part_o + slot * HD;
#pragma unroll
      for (int dt = 0; dt < HD / 16; ++dt)
        *reinterpret_cast<float4*>(po + dt * 16 + 4 * g) =
            make_float4(o[dt][0], o[dt][1], o[dt][2], o[dt][3]);
      if (g == 0) a.part_ml[slot] = make_float2(m_run, l_run);
    }
  }
}

constexpr int kStage = 64;  // keys per stage of the streamed kernel
constexpr int kStreamMaxPages = 512;  // 16-key pages of one workgroup's key range

// LDS of the streamed kernel: one stage (K rows, then V^T), reused at the
// end for the merge slots (per slot and lane: HD / 4 output values, then
// the running max and sum).
template <typename T, int HD>
struct StreamLds {
  using L = SplitLds<T, HD>;
  static constexpr int VS = kStage + L::VPAD;
  static constexpr size_t kv_bytes = ((size_t)kStage * L::KS + (size_t)HD * VS) * sizeof(T);
  static constexpr int SLOT = 64 * (HD / 4 + 2);  // floats per merge slot
  static constexpr size_t merge_bytes = (size_t)4 * SLOT * sizeof(float);
  static constexpr size_t bytes = kv_bytes > merge_bytes ? kv_bytes : merge_bytes;
};

// one workgroup per CU (two waves per SIMD): the next stage's loads in
// registers beside a tile's state need more than 128 registers
template <typename T, int HD>
__global__ __launch_bounds__(kAttnThreads, 2) void attn_stream_kernel(AttnArgs a) {
  extern __shared__ __align__(16) unsigned char attn_smem[];
  using L = SplitLds<T, HD>;
  using SL = StreamLds<T, HD>;
  constexpr int VS = SL::VS;
  T* sk = reinterpret_cast<T*>(attn_smem);      // [kStage][KS]
  T* sv = sk + (size_t)kStage * L::KS;           // [HD][VS]

  const int range = blockIdx.x;
  const int req = blockIdx.z / a.nkv, kvh = blockIdx.z % a.nkv;
  const ReqMeta rm = a.reqs[req];
  const int G = a.nq / a.nkv;
  const int qrows = rm.nrows * G;
  // this workgroup's query group: tiles [t_beg, t_beg + qt) of the request
  const int t_beg = blockIdx.y * a.qtiles_per_wg;  // qtiles_per_wg <= kAttnStreamTiles
  const int qt = min((qrows + 15) / 16 - t_beg, a.qtiles_per_wg);
  const int total_keys = rm.nctx + rm.nrows;
  const int kbeg = range * a.split;
  if (qt <= 0 || kbeg >= total_keys) return;  // uniform per block
  const int kend = min(total_keys, kbeg + a.split);
  // waves per query tile (each takes every kp-th key block of a stage; their
  // states merge at the end, so the rounding depends on kp)
  const int kp = a.one_part ? 1 : 4 * qt <= kAttnWaves ? 4 : 2 * qt <= kAttnWaves ? 2 : 1;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4, r16 = lane & 15;
  const int tile = t_beg + wave % qt, part = wave / qt;
  const bool active = part < kp;

  const T* kc = reinterpret_cast<const T*>(a.kc);
  const T* vc = reinterpret_cast<const T*>(a.vc);
  const int32_t* bt = a.btab + (size_t)rm.table * a.max_pages;

  constexpr bool kSplit = sizeof(T) == 2;
  const T* q = reinterpret_cast<const T*>(a.q);
  const T* qlo = reinterpret_cast<const T*>(a.q_lo);
  // the wave's query rows: q fragments (hi + lo bf16 planes, or fp32) and
  // the ancestor mask, loaded ahead of the first stage
  const int qr = tile * 16 + r16;
  const bool qvalid = active && qr < qrows;
  const int node = qvalid ? qr / G : 0;
  const int qhead = kvh * G + (qvalid ? qr % G : 0);
  const int grow = rm.row0 + node;
  Frag<T> qf[HD / 32], qfl[HD / 32];
#pragma unroll
  for (int ks = 0; ks < HD / 32; ++ks) {
    const size_t off = ((size_t)grow * a.nq + qhead) * HD + ks * 32 + g * 8;
    if (qvalid) {
      qf[ks].load(q + off);
      if (kSplit) qfl[ks].load(qlo + off);
    } else {
      qf[ks].zero();
      qfl[ks].zero();
    }
  }
  uint64_t anc_lo = 0, anc_hi = 0;
  if (qvalid && !rm.chain) {
    const uint64_t* am = a.anc + rm.anc0 + (size_t)node * rm.anc_words;
    anc_lo = am[0];
    if (rm.anc_words > 1) anc_hi = am[1];
  }
  asm volatile("" ::: "memory");  // keep these loads ahead of the staging

  // ---- staging of one stage: K rows and V^T of keys [s0, s0 + kStage)
  // (keys past kend are zeros)
  constexpr int EPC = 16 / sizeof(T);
  constexpr int KCH_ROW = HD / EPC;
  constexpr int VCH_ROW = 16 / EPC;
  constexpr int NCH = kStage * KCH_ROW / kAttnThreads;  // 16-byte chunks per thread, each of K, V
  static_assert(NCH * kAttnThreads == kStage * KCH_ROW, "stage chunks");
  // The range's pages (one per 16 keys) are looked up once into LDS; then
  // every load of a stage is unconditional, from page slots clamped to the
  // last one that holds keys, and the loaded data is only stored to LDS
  // (keys past kend are cleared there afterwards).  (Loads under per-lane
  // conditions, or arithmetic on the loaded data, made the compiler wait for
  // each load before going on.)
  __shared__ int spg[kStreamMaxPages];
  const int nslots = (kend - kbeg + 15) >> 4;  // <= kStreamMaxPages (checked by the launcher)
  for (int k = threadIdx.x; k < nslots; k += kAttnThreads)
    spg[k] = kv_page(rm.page0, bt, kbeg + 16 * k);
  __syncthreads();
  struct StageRegs {
    uint4 k[NCH], v[NCH];
  };
  auto issue = [&](int s0) __attribute__((always_inline)) {
    StageRegs r;
    const int slot0 = (s0 - kbeg) >> 4;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int c = threadIdx.x + j * kAttnThreads;
      {
        const int i = c / KCH_ROW, pt = c % KCH_ROW;  // key s0 + i (i < kStage)
        const int page = spg[min(slot0 + (i >> 4), nslots - 1)];
        r.k[j] = *reinterpret_cast<const uint4*>(
            kc + kv_k_index(page, a.nkv, kvh, i & 15, HD, pt * EPC));
      }
      {
        const int blk = c / (HD * VCH_ROW), rest = c % (HD * VCH_ROW);
        const int dim = rest / VCH_ROW, pt = rest % VCH_ROW;
        const int page = spg[min(slot0 + blk, nslots - 1)];
        r.v[j] = *reinterpret_cast<const uint4*>(
            vc + kv_v_index(page, a.nkv, kvh, pt * EPC, HD, dim));
      }
    }
    return r;
  };
  auto place = [&](const StageRegs& r, int s0) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int c = threadIdx.x + j * kAttnThreads;
      {
        const int i = c / KCH_ROW, pt = c % KCH_ROW;
        *reinterpret_cast<uint4*>(&sk[(size_t)i * L::KS + pt * EPC]) = r.k[j];
      }
      {
        const int blk = c / (HD * VCH_ROW), rest = c % (HD * VCH_ROW);
        const int dim = rest / VCH_ROW, pt = rest % VCH_ROW;
        *reinterpret_cast<uint4*>(&sv[(size_t)dim * VS + blk * 16 + pt * EPC]) = r.v[j];
      }
    }
    // the last stage: V of keys past kend (not written this pass) becomes
    // zeros in LDS, over the chunk just stored by the same thread (K needs
    // none: those keys' scores are masked out)
    if (s0 + kStage > kend) {  // uniform
#pragma unroll
      for (int j = 0; j < NCH; ++j) {
        const int c = threadIdx.x + j * kAttnThreads;
        const int blk = c / (HD * VCH_ROW), rest = c % (HD * VCH_ROW);
        const int dim = rest / VCH_ROW, pt = rest % VCH_ROW;
        const int t0 = s0 + blk * 16 + pt * EPC;
#pragma unroll
        for (int e = 0; e < EPC; ++e)
          if (t0 + e >= kend) sv[(size_t)dim * VS + blk * 16 + pt * EPC + e] = T(0);
      }
    }
  };

  const float scale2 = a.scale * 1.44269504088896340736f;  // log2(e)
  float m_run = -INFINITY, l_run = 0.f;
  floatx4_t o[HD / 16];
#pragma unroll
  for (int dt = 0; dt < HD / 16; ++dt) o[dt] = floatx4_t{0.f, 0.f, 0.f, 0.f};

  StageRegs nx = issue(kbeg);
  place(nx, kbeg);
  __syncthreads();
  for (int s0 = kbeg; s0 < kend; s0 += kStage) {
    const bool more = s0 + kStage < kend;  // uniform
    if (more) nx = issue(s0 + kStage);     // in flight while this stage is used
    if (active) {
#pragma unroll
      for (int b = 0; b < kStage / 32; ++b) {
        const int kb = s0 + 32 * b;
        if (kb < kend && ((kb - kbeg) / 32) % kp == part)
          attn_block<T, HD, L::KS>(sk, sv, VS, 32 * b, kb, kend, rm, node, qvalid, anc_lo,
                                   anc_hi, qf, qfl, scale2, g, r16, m_run, l_run, o);
      }
    }
    __syncthreads();  // every wave is done with this stage
    if (more) {
      place(nx, s0 + kStage);
      __syncthreads();
    }
  }

  // ---- merge the kp states of each tile, pairwise: parts [r, 2r) into
  // parts [0, r), in part order (the stage area is free after the last
  // barrier above)
  float* slots = reinterpret_cast<float*>(attn_smem);
  for (int r = kp / 2; r >= 1; r /= 2) {
    if (active && part >= r && part < 2 * r) {
      float* sp = slots + (size_t)((tile - t_beg) * r + (part - r)) * SL::SLOT;
#pragma unroll
      for (int dt = 0; dt < HD / 16; ++dt)
        *reinterpret_cast<floatx4_t*>(sp + (dt * 64 + lane) * 4) = o[dt];
      sp[HD / 4 * 64 + lane] = m_run;
      sp[HD / 4 * 64 + 64 + lane] = l_run;
    }
    __syncthreads();
    if (active && part < r) {
      const float* sp = slots + (size_t)((tile - t_beg) * r + part) * SL::SLOT;
      const float mb = sp[HD / 4 * 64 + lane], lb = sp[HD / 4 * 64 + 64 + lane];
      const float m_new = fmaxf(m_run, mb);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float wa = __builtin_amdgcn_exp2f(m_run - m_use);  // 2^-inf = 0
      const float wb = __builtin_amdgcn_exp2f(mb - m_use);
      l_run = l_run * wa + lb * wb;
      m_run = m_new;
#pragma unroll
      for (int dt = 0; dt < HD / 16; ++dt) {
        const floatx4_t ob = *reinterpret_cast<const floatx4_t*>(sp + (dt * 64 + lane) * 4);
        o[dt] = o[dt] * wa + ob * wb;
      }
    }
    __syncthreads();
  }

  if (qvalid && part == 0) {
    if (a.max_splits == 1) {  // uniform: the whole key range, so the output itself
      // (what the combine computes from one partial: o * (1 / l))
      const float inv = 1.0f / l_run;
      T* out = reinterpret_cast<T*>(a.out);
#pragma unroll
      for (int dt = 0; dt < HD / 16; ++dt)
        store_act4(out, out + a.out_lo, ((size_t)grow * a.nq + qhead) * HD + dt * 16 + 4 * g,
                   make_float4(o[dt][0] * inv, o[dt][1] * inv, o[dt][2] * inv, o[dt][3] * inv));
    } else {
      const size_t slot = attn_part_slot(range, a.rows_total, a.nq, grow, qhead);
      float* po = a.part_o + slot * HD;
#pragma unroll
      for (int dt = 0; dt < HD / 16; ++dt)
        *reinterpret_cast<float4*>(po + dt * 16 + 4 * g) =
            make_float4(o[dt][0], o[dt][1], o[dt][2], o[dt][3]);
      if (g == 0) a.part_ml[slot] = make_float2(m_run, l_run);
    }
  }
}

// One wave per (row, query head), four to a workgroup: merge the splits of
// the row's request.  Lane l reads the (max, sum) of splits l and l + 64 and
// every lane forms the same weights; each lane then adds the splits in order
// for its HD / 64 dims (16 splits' loads in flight together, the first 16
// issued with the (max, sum) loads).
template <typename T, int HD>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a, T* out, size_t olo) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wid = blockIdx.x * 4 + wave;  // row * nq + head
  if (wid >= a.rows_total * a.nq) return;  // uniform per wave (no barriers below)
  const int grow = wid / a.nq, qhead = wid % a.nq;
  const int nsplit = (a.rows[grow].keys + a.split - 1) / a.split;  // <= 128
  const size_t sstride = (size_t)a.rows_total * a.nq;
  float2 ml0 = make_float2(-INFINITY, 0.f), ml1 = ml0;
  if (lane < nsplit) ml0 = a.part_ml[attn_part_slot(lane, a.rows_total, a.nq, grow, qhead)];
  if (lane + 64 < nsplit)
    ml1 = a.part_ml[attn_part_slot(lane + 64, a.rows_total, a.nq, grow, qhead)];
  constexpr int PER = HD / 64;
  constexpr int U = 16;  // splits loaded together
  const float* po = a.part_o + (size_t)wid * HD + lane * PER;
  auto load_group = [&](int s0, float (&v)[U][PER]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int sp = min(s0 + u, nsplit - 1);
#pragma unroll
      for (int j = 0; j < PER; ++j) v[u][j] = po[(size_t)sp * sstride * HD + j];
    }
  };
  // the first group of partial outputs is loaded together with the (max,
  // sum) pairs, ahead of the reductions that form the weights
  float v[U][PER];
  load_group(0, v);
  const float M = wave_max(fmaxf(ml0.x, ml1.x));
  // the running maxima are in the base-2 domain of the split kernel
  const float w0 = (ml0.x == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(ml0.x - M);
  const float w1 = (ml1.x == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(ml1.x - M);
  const float L = wave_sum(ml0.y * w0 + ml1.y * w1);
  float acc[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) acc[j] = 0.f;
  for (int s0 = 0; s0 < nsplit; s0 += U) {
    if (s0 != 0) load_group(s0, v);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int sp = s0 + u;
      const float wu = __shfl(sp < 64 ? w0 : w1, sp & 63, 64);
      if (sp < nsplit) {
#pragma unroll
        for (int j = 0; j < PER; ++j) acc[j] += v[u][j] * wu;
      }
    }
  }
  const float inv = 1.0f / L;
#pragma unroll
  for (int j = 0; j < PER; ++j)
    store_act(out, out + olo, ((size_t)grow * a.nq + qhead) * HD + lane * PER + j, acc[j] * inv);
}

template <typename T, int HD>
hipError_t attn_launch(const AttnArgs& a, const LaunchCtx& s) {
  auto k = attn_kernel<T, HD>;
  const size_t lds = SplitLds<T, HD>::bytes(a.split);
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void*)k,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  dim3 grid(a.max_splits, a.max_qgroups, a.n_req * a.nkv);
  if (s.t0 || s.t1) {
    AttnArgs arg = a;
    void* args[] = {&arg};
    return hipExtLaunchKernel((const void*)k, grid, dim3(kAttnThreads), args, lds, s.s, s.t0,
                              s.t1, 0);
  }
  k<<<grid, kAttnThreads, lds, s.s>>>(a);
  return hipGetLastError();
}

template <typename T, int HD>
hipError_t attn_stream_launch(const AttnArgs& a, const LaunchCtx& s) {
  auto k = attn_stream_kernel<T, HD>;
  constexpr size_t lds = StreamLds<T, HD>::bytes;
  static_assert(StreamLds<T, HD>::merge_bytes <= 160 * 1024 && lds <= 160 * 1024, "LDS");
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void*)k,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  dim3 grid(a.max_splits, a.max_qgroups, a.n_req * a.nkv);
  if (s.t0 || s.t1) {
    AttnArgs arg = a;
    void* args[] = {&arg};
    return hipExtLaunchKernel((const void*)k, grid, dim3(kAttnThreads), args, lds, s.s, s.t0,
                              s.t1, 0);
  }
  k<<<grid, kAttnThreads, lds, s.s>>>(a);
  return hipGetLastError();
}

template <typename T>
hipError_t attn_typed(const AttnArgs& a, const LaunchCtx& s) {
  if (a.stream) {
    // a query group's tiles fit the waves of one workgroup
    if (a.split < kStage || a.split % kStage || a.split > 16 * kStreamMaxPages ||
        a.qtiles_per_wg < 1 || a.qtiles_per_wg > kAttnStreamTiles || a.max_qgroups < 1 ||
        (a.max_splits == 1 && !a.out))
      return hipErrorInvalidValue;
    if (a.hd == 128) return attn_stream_launch<T, 128>(a, s);
    if (a.hd == 64) return attn_stream_launch<T, 64>(a, s);
    return hipErrorInvalidValue;
  }
  if (a.split > kMaxSplitKeys || a.split < 32 || a.split % 32 || a.qtiles_per_wg < 1)
    return hipErrorInvalidValue;
  if (a.hd == 128) return attn_launch<T, 128>(a, s);
  if (a.hd == 64) return attn_launch<T, 64>(a, s);
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t combine_t(const AttnArgs& a, T* o, size_t olo, hipStream_t s) {
  if (a.max_splits > 128) return hipErrorInvalidValue;
  dim3 grid((a.rows_total * a.nq + 3) / 4);  // a wave per (row, head)
  if (a.hd == 128) attn_combine_kernel<T, 128><<<grid, 256, 0, s>>>(a, o, olo);
  else if (a.hd == 64) attn_combine_kernel<T, 64><<<grid, 256, 0, s>>>(a, o, olo);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention(bool bf16, const AttnArgs& a, hipStream_t s, hipEvent_t t0,
                            hipEvent_t t1) {
  const LaunchCtx lc{s, t0, t1};
  return bf16 ? attn_typed<uint16_t>(a, lc) : attn_typed<float>(a, lc);
}

hipError_t launch_attn_combine(bool bf16, const AttnArgs& a, void* o, size_t o_lo,
                               hipStream_t s) {
  return bf16 ? combine_t<uint16_t>(a, (uint16_t*)o, o_lo, s)
              : combine_t<float>(a, (float*)o, o_lo, s);
}
