// Tree-masked attention over the paged KV cache for one layer.
//
// Every row of the pass is a tree node (or a prompt token in prefill).  A
// node of request r attends to the request's committed keys [0, n_r) and,
// among the pass's own keys (written at slots n_r + node), to itself and its
// ancestors.  GQA: the G = n_heads / n_kv_heads query heads that share a KV
// head are processed together, so each K/V tile staged in LDS serves
// (rows * G) query rows.
//
// Workgroup = 4 wavefronts = one (request, KV head, query group of 64 query
// rows, key split).  Each wave owns one 16-row query tile and keeps the
// transposed flash-attention state in registers: S^T = K Q^T (so a lane holds
// one query row's scores), an online softmax in fp32, and O^T += V^T P^T.
// With a bf16 cache, the fp32 operands q and P enter the MFMAs as bf16
// hi + lo pairs, so only the stored K and V are rounded.  Keys are consumed in blocks of 32
// (two 16-token pages) staged in LDS; V pages are stored transposed
// ([dim][16 tokens]) in the cache so that the V^T operand is read directly.
// Each split writes un-normalised partials (O, running max, running sum),
// merged in split order by attn_combine.
#include "common.h"
#include "kernels.h"

namespace {

template <typename T, int HD>
struct alignas(16) AttnSmem {
  static constexpr int KPAD = 16 / sizeof(T) * 1;  // one 16-byte pad per row
  static constexpr int VPAD = 8 / sizeof(T) * 2;
  T k[32][HD + KPAD];
  T v[HD][32 + VPAD];
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

template <typename T, int HD>
__global__ __launch_bounds__(256) void attn_kernel(AttnArgs a) {
  __shared__ AttnSmem<T, HD> sm;
  const int split = blockIdx.x, qg = blockIdx.y;
  const int req = blockIdx.z / a.nkv, kvh = blockIdx.z % a.nkv;
  const ReqMeta rm = a.reqs[req];
  const int G = a.nq / a.nkv;
  const int qrows = rm.nrows * G;
  const int total_keys = rm.nctx + rm.nrows;
  const int kbeg = split * a.split;
  if (kbeg >= total_keys || qg * 64 >= qrows) return;  // uniform per block
  const int kend = min(total_keys, kbeg + a.split);

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4, r16 = lane & 15;
  const int qtile = qg * 4 + wave;
  const bool wave_active = qtile * 16 < qrows;
  const int qr = qtile * 16 + r16;
  const bool qvalid = wave_active && qr < qrows;
  const int node = qvalid ? qr / G : 0;
  const int qhead = kvh * G + (qvalid ? qr % G : 0);
  const int grow = rm.row0 + node;

  // q enters the score MFMA as hi + lo bf16 planes (bf16 KV) or as fp32
  constexpr bool kSplit = sizeof(T) == 2;
  const T* q = reinterpret_cast<const T*>(a.q);
  const T* qlo = reinterpret_cast<const T*>(a.q_lo);
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

  const T* kc = reinterpret_cast<const T*>(a.kc);
  const T* vc = reinterpret_cast<const T*>(a.vc);
  const int32_t* bt = a.btab + (size_t)rm.table * a.max_pages;

  float m_run = -INFINITY, l_run = 0.f;
  floatx4_t o[HD / 16];
#pragma unroll
  for (int dt = 0; dt < HD / 16; ++dt) o[dt] = floatx4_t{0.f, 0.f, 0.f, 0.f};

  constexpr int EPC = 16 / sizeof(T);        // elements per 16-byte chunk
  constexpr int KCH = 32 * HD / EPC;         // chunks in a K block
  constexpr int VCH_ROW = 16 / EPC;          // chunks per (dim, half page)
  constexpr int VCH = HD * 2 * VCH_ROW;      // chunks in a V block

  for (int kb = kbeg; kb < kend; kb += 32) {
    __syncthreads();
    // ---- stage K rows [kb, kb + 32) and V^T into LDS
    for (int c = threadIdx.x; c < KCH; c += 256) {
      const int i = c / (HD / EPC), part = c % (HD / EPC);
      const int t = kb + i;
      uint4 val = make_uint4(0, 0, 0, 0);
      if (t < kend) {
        const int page = bt[t >> 4];
        val = *reinterpret_cast<const uint4*>(
            kc + (((size_t)page * a.nkv + kvh) * 16 + (t & 15)) * HD + part * EPC);
      }
      *reinterpret_cast<uint4*>(&sm.k[i][part * EPC]) = val;
    }
    for (int c = threadIdx.x; c < VCH; c += 256) {
      const int dim = c / (2 * VCH_ROW);
      const int half = (c / VCH_ROW) & 1;
      const int part = c % VCH_ROW;
      const int t0 = kb + half * 16 + part * EPC;  // first key of the chunk
      uint4 val = make_uint4(0, 0, 0, 0);
      if (t0 < kend) {
        const int page = bt[t0 >> 4];
        val = *reinterpret_cast<const uint4*>(
            vc + (((size_t)page * a.nkv + kvh) * HD + dim) * 16 + (t0 & 15));
        // zero keys past the end (their memory is not written this pass)
        T* ve = reinterpret_cast<T*>(&val);
#pragma unroll
        for (int e = 0; e < EPC; ++e)
          if (t0 + e >= kend) ve[e] = T(0);
      }
      *reinterpret_cast<uint4*>(&sm.v[dim][half * 16 + part * EPC]) = val;
    }
    __syncthreads();
    if (!wave_active) continue;

    // ---- scores: S^T tiles for keys [kb, kb+16) and [kb+16, kb+32)
    floatx4_t s[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      s[kt] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < HD / 32; ++ks) {
        Frag<T> kf;
        kf.load(&sm.k[kt * 16 + r16][ks * 32 + g * 8]);
        mma32(s[kt], kf, qf[ks]);
        if (kSplit) mma32(s[kt], kf, qfl[ks]);
      }
    }
    // lane holds row r16, keys kb + kt*16 + 4g + r
    float p[8];
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = kb + kt * 16 + 4 * g + r;
        bool ok = qvalid && t < kend;
        if (ok && t >= rm.nctx) {
          const int tn = t - rm.nctx;  // tree node of this key
          if (rm.chain) ok = tn <= node;
          else ok = (tn < 64 ? (anc_lo >> tn) : (anc_hi >> (tn - 64))) & 1ull;
        }
        const float v = ok ? s[kt][r] * a.scale : -INFINITY;
        p[kt * 4 + r] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    // No lane may skip the MFMAs below (they read operands of all lanes), so
    // a row with nothing visible yet uses a finite stand-in maximum: every
    // weight is then 0 and the state stays (max = -inf, sum = 0, O = 0).
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = expf(m_run - m_use);  // exp(-inf) = 0 on first block
    float lsum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      p[e] = (p[e] == -INFINITY) ? 0.f : expf(p[e] - m_use);
      lsum += p[e];
    }
    lsum += __shfl_xor(lsum, 16, 64);
    lsum += __shfl_xor(lsum, 32, 64);
    l_run = l_run * alpha + lsum;
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < HD / 16; ++dt) o[dt] *= alpha;

    // P as an operand of the KV type; for bf16 it is carried as a hi + lo
    // pair (two MFMAs), which keeps ~16 mantissa bits of the weights
    Frag<T> pf, pf_lo;
    constexpr bool kSplitP = kSplit;
    if (kSplitP) {
      float lo[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) lo[e] = p[e] - op_round(p[e], T(0));
      pack_p(pf_lo, lo);
    }
    pack_p(pf, p);
#pragma unroll
    for (int dt = 0; dt < HD / 16; ++dt) {
      Frag<T> vf;
      load_vfrag<T>(vf, &sm.v[dt * 16 + r16][4 * g], &sm.v[dt * 16 + r16][16 + 4 * g]);
      mma32(o[dt], vf, pf);
      if (kSplitP) mma32(o[dt], vf, pf_lo);
    }
  }

  if (qvalid) {
    const size_t slot = (size_t)split * a.rows_total * a.nq + (size_t)grow * a.nq + qhead;
    float* po = a.part_o + slot * HD;
#pragma unroll
    for (int dt = 0; dt < HD / 16; ++dt)
      *reinterpret_cast<float4*>(po + dt * 16 + 4 * g) =
          make_float4(o[dt][0], o[dt][1], o[dt][2], o[dt][3]);
    if (g == 0) a.part_ml[slot] = make_float2(m_run, l_run);
  }
}

// One wave per (row, query head): merge the splits of the row's request.
template <typename T, int HD>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a, T* out,
                                                           T* out_lo) {
  const int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (wid >= a.rows_total * a.nq) return;
  const int grow = wid / a.nq, qhead = wid % a.nq;
  const ReqMeta rm = a.reqs[a.rows[grow].req];
  const int nsplit = (rm.nctx + rm.nrows + a.split - 1) / a.split;
  float M = -INFINITY;
  for (int s = 0; s < nsplit; ++s)
    M = fmaxf(M, a.part_ml[(size_t)s * a.rows_total * a.nq + wid].x);
  float L = 0.f;
  float acc[HD / 64 > 0 ? HD / 64 : 1] = {};
  constexpr int PER = HD / 64 > 0 ? HD / 64 : 1;
  for (int s = 0; s < nsplit; ++s) {
    const size_t slot = (size_t)s * a.rows_total * a.nq + wid;
    const float2 ml = a.part_ml[slot];
    if (ml.x == -INFINITY) continue;
    const float w = expf(ml.x - M);
    L += ml.y * w;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int dim = lane + 64 * j;
      if (dim < HD) acc[j] += a.part_o[slot * HD + dim] * w;
    }
  }
  const float inv = 1.0f / L;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int dim = lane + 64 * j;
    if (dim < HD) store_act(out, out_lo, ((size_t)grow * a.nq + qhead) * HD + dim, acc[j] * inv);
  }
}

template <typename T>
hipError_t attn_typed(const AttnArgs& a, hipStream_t s) {
  dim3 grid(a.max_splits, a.max_qgroups, a.n_req * a.nkv);
  if (a.hd == 128) attn_kernel<T, 128><<<grid, 256, 0, s>>>(a);
  else if (a.hd == 64) attn_kernel<T, 64><<<grid, 256, 0, s>>>(a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

template <typename T>
hipError_t combine_typed(const AttnArgs& a, void* o, void* o_lo, hipStream_t s) {
  const int waves = a.rows_total * a.nq;
  dim3 grid((waves + 3) / 4);
  if (a.hd == 128) attn_combine_kernel<T, 128><<<grid, 256, 0, s>>>(a, (T*)o, (T*)o_lo);
  else if (a.hd == 64) attn_combine_kernel<T, 64><<<grid, 256, 0, s>>>(a, (T*)o, (T*)o_lo);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention(bool bf16, const AttnArgs& a, hipStream_t s) {
  return bf16 ? attn_typed<uint16_t>(a, s) : attn_typed<float>(a, s);
}

hipError_t launch_attn_combine(bool bf16, const AttnArgs& a, void* o,
                               void* o_lo, hipStream_t s) {
  return bf16 ? combine_typed<uint16_t>(a, o, o_lo, s)
              : combine_typed<float>(a, o, o_lo, s);
}
