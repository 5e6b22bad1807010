// Small kernels of the verify pass: embedding gather, RoPE + KV store, argmax reduction, accepted-path walk, the per-branch recurrence of
// the hybrid layers, the commit kernels and the one-time weight re-layout.
#include "common.h"
#include "index_math.h"
#include "kernels.h"

// Products and sums are rounded separately, as written (RoPE and the
// recurrence follow the oracle's operation order; a fused multiply-add would
// round differently).
#pragma clang fp contract(off)

namespace {

// ------------------------------------------------------- block reduction
// Block-wide sum over blockDim.x threads (a multiple of 64, <= 1024).
__device__ __forceinline__ float block_sum(float v, float* part) {
  v = wave_sum(v);
  const int nw = blockDim.x >> 6;
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = v;
  __syncthreads();
  float t = 0.f;
  for (int w = 0; w < nw; ++w) t += part[w];  // same order in every thread
  return t;
}

// ---------------------------------------------------------------- embedding
// One workgroup per (row, chunk of kNormChunk columns): h = float(E[token]),
// u = h * nw as activation planes for the first layer's input GEMM, and the
// chunk's sum of squares of h (the deferred RMSNorm of u).  The workgroups of
// chunk 0 also copy the row's RoPE factors at its position into cs[row]
// (cos then sin, hd / 2 each), so that RoPE needs no position lookup.
template <typename T>
__global__ __launch_bounds__(256) void embed_kernel(const T* __restrict__ emb,
                                                    const RowMeta* __restrict__ rows, int d,
                                                    float* __restrict__ h,
                                                    const float* __restrict__ nw,
                                                    T* __restrict__ u, size_t ulo,
                                                    float* __restrict__ ss,
                                                    const float* __restrict__ cos_t,
                                                    const float* __restrict__ sin_t, int half,
                                                    float* __restrict__ cs) {
  __shared__ float part[4];
  const int row = blockIdx.x;
  if (blockIdx.y == 0) {
    const size_t pos = (size_t)rows[row].pos;
    for (int t = threadIdx.x; t < half; t += blockDim.x) {
      cs[(size_t)row * 2 * half + t] = cos_t[pos * half + t];
      cs[(size_t)row * 2 * half + half + t] = sin_t[pos * half + t];
    }
  }
  const int c = blockIdx.y * kNormChunk + threadIdx.x * 4;
  float acc = 0.f;
  if (c < d) {
    const T* e = emb + (size_t)rows[row].token * d;
    const float4 w = *reinterpret_cast<const float4*>(nw + c);
    const float4 v = load4(e + c);
    *reinterpret_cast<float4*>(h + (size_t)row * d + c) = v;
    acc = v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
    store_act4(u, u + ulo, (size_t)row * d + c,
               make_float4(v.x * w.x, v.y * w.y, v.z * w.z, v.w * w.w));
  }
  const float t = block_sum(acc, part);
  if (threadIdx.x == 0) ss[(size_t)row * gridDim.y + blockIdx.y] = t;
}

// ------------------------------------------------------------ RoPE + KV store
// Block = one row, one head (query, key or value head); threads cover the
// head_dim / 2 rotation pairs (i, i + hd/2).
template <typename T, int S>
__global__ __launch_bounds__(64) void rope_kv_kernel(const float* qkv, size_t sstride,
                               const RowMeta* rows, int nq, int nkv, int hd,
                               const float* cs, T* q_out, T* q_lo, T* kc, T* vc, int ld,
                               RowNorm norm) {
  const int row = blockIdx.x;
  const int head = blockIdx.y;  // [0, nq) q, [nq, nq+nkv) k, then v
  const int half = hd >> 1;
  const RowMeta rm = rows[row];
  const float sc = row_scale(norm, row);
  const float* x = qkv + (size_t)row * ld + (size_t)head * hd;
  const int page = rm.slot >> 4, off = rm.slot & 15;
  for (int i = threadIdx.x; i < half; i += blockDim.x) {
    float p1[S], p2[S];  // GEMM split partials, loaded together
#pragma unroll
    for (int k = 0; k < S; ++k) {
      p1[k] = x[k * sstride + i];
      p2[k] = x[k * sstride + i + half];
    }
    float x1 = 0.f, x2 = 0.f;  // added in split order, then scaled by the norm
#pragma unroll
    for (int k = 0; k < S; ++k) {
      x1 += p1[k];
      x2 += p2[k];
    }
    x1 *= sc;
    x2 *= sc;
    if (head < nq + nkv) {
      const float c = cs[(size_t)row * hd + i];
      const float s = cs[(size_t)row * hd + half + i];
      const float y1 = ((x1 * c) - (x2 * s));
      const float y2 = ((x2 * c) + (x1 * s));
      if (head < nq) {
        const size_t base = ((size_t)row * nq + head) * hd;
        store_act(q_out, q_lo, base + i, y1);
        store_act(q_out, q_lo, base + i + half, y2);
      } else {
        const int kvh = head - nq;
        T* dst = kc + kv_k_index(page, nkv, kvh, off, hd, 0);
        dst[i] = from_f<T>(y1);
        dst[i + half] = from_f<T>(y2);
      }
    } else {
      const int kvh = head - nq - nkv;
      T* dst = vc + kv_v_index(page, nkv, kvh, off, hd, 0);
      dst[(size_t)i * 16] = from_f<T>(x1);
      dst[(size_t)(i + half) * 16] = from_f<T>(x2);
    }
  }
}

// ------------------------------------------------------- residual reduce
// h[r] += (sum of the S split partials of the GEMM output, in split order),
// u = h[r] * nw as activation planes for the next GEMM and the chunk's sum of
// squares of h (the deferred RMSNorm of u).  One workgroup of 256 threads
// per (row, chunk of kNormChunk columns), a float4 per thread, so a row's
// loads spread over several CUs; all S partial loads of a thread are in
// flight together.
template <int S, typename T>
__global__ __launch_bounds__(256) void resid_reduce_kernel(const float* P, size_t sstride,
                                                           int ldp, int d, float* h,
                                                           const float* nw, T* u,
                                                           size_t ulo, float* ss) {
  __shared__ float part[4];
  const int row = blockIdx.x;
  const int c = blockIdx.y * kNormChunk + threadIdx.x * 4;
  float acc = 0.f;
  if (c < d) {
    const float4 w = *reinterpret_cast<const float4*>(nw + c);
    float4 pv[S];
#pragma unroll
    for (int k = 0; k < S; ++k)
      pv[k] = *reinterpret_cast<const float4*>(P + k * sstride + (size_t)row * ldp + c);
    float4 v = *reinterpret_cast<const float4*>(h + (size_t)row * d + c);
#pragma unroll
    for (int k = 0; k < S; ++k) {
      v.x += pv[k].x;
      v.y += pv[k].y;
      v.z += pv[k].z;
      v.w += pv[k].w;
    }
    *reinterpret_cast<float4*>(h + (size_t)row * d + c) = v;
    acc = v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
    store_act4(u, u + ulo, (size_t)row * d + c,
               make_float4(v.x * w.x, v.y * w.y, v.z * w.z, v.w * w.w));
  }
  const float t = block_sum(acc, part);
  if (threadIdx.x == 0) ss[(size_t)row * gridDim.y + blockIdx.y] = t;
}

// ----------------------------------------------------------- argmax reduce
__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

__global__ __launch_bounds__(256) void argmax_reduce_kernel(const float2* part,
                                                            int nblocks,
                                                            int32_t* amax) {
  __shared__ float sv[256];
  __shared__ int si[256];
  const int row = blockIdx.x;
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  for (int b = threadIdx.x; b < nblocks; b += 256) {
    const float2 p = part[(size_t)row * nblocks + b];
    const int i = __float_as_int(p.y);
    if (better(p.x, i, bv, bi)) { bv = p.x; bi = i; }
  }
  sv[threadIdx.x] = bv;
  si[threadIdx.x] = bi;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) {
      const float v = sv[threadIdx.x + o];
      const int i = si[threadIdx.x + o];
      if (better(v, i, sv[threadIdx.x], si[threadIdx.x])) {
        sv[threadIdx.x] = v;
        si[threadIdx.x] = i;
      }
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) amax[row] = (si[0] == 0x7fffffff) ? 0 : si[0];
}

// ------------------------------------------------------------- path walk
// ok(0) = 1; ok(i) = ok(parent) && token(i) == A(parent); best = deepest ok
// node (lowest index among equals); path = root..best; bonus = A(best).
// The request's parents, tokens and argmaxes are first loaded into LDS by
// all lanes together; one lane then walks the nodes in index order.
__global__ __launch_bounds__(64) void path_walk_kernel(const RowMeta* rows,
                                                       const ReqMeta* reqs,
                                                       const int32_t* amax, int max_path,
                                                       int32_t* res) {
  const int r = blockIdx.x;
  const ReqMeta rm = reqs[r];
  constexpr int MAXN = 512;
  __shared__ int16_t par[MAXN], dep[MAXN];
  __shared__ int32_t tok[MAXN], am[MAXN];
  __shared__ int8_t ok[MAXN];
  const int n = min(rm.nrows, MAXN);
  for (int i = threadIdx.x; i < n; i += 64) {
    par[i] = (int16_t)rows[rm.row0 + i].parent;
    tok[i] = rows[rm.row0 + i].token;
    am[i] = amax[rm.row0 + i];
  }
  __syncthreads();
  if (threadIdx.x != 0) return;
  walk_accepted_path(n, par, tok, am, ok, dep, res + (size_t)r * (2 + max_path));
}

// ------------------------------------------------------ recurrence (verify)
// A lane owns SPL states (s = SPL l + k, k < SPL) of one channel c; the
// S / SPL lanes of a channel are adjacent, and a workgroup of THR threads
// covers CPB = THR SPL / S channels.  For node i
//   H_i = sigmoid(a_i[c]) * H_parent + B_i[s] * x_i[c]   (no FMA contraction)
//   y_i[c] = sum_s H_i[s] * C_i[s];  o_i[c] = y_i * silu(z_i[c])
// where the root's parent state is the committed H_0.  The inputs of the
// staged rows (x, a, silu(z) of the workgroup's channels and every row's B
// and C, summed over the in_proj split partials in order and scaled by the
// row's norm scale) and sigmoid(a) are staged in LDS once per workgroup with
// all loads in flight; the walk then reads LDS only for inputs.  A chain
// keeps its running states in registers.  A tree is walked in depth-first
// order, in which the ancestors of the node being visited are exactly the
// last nodes visited at each smaller depth, so each lane keeps the states of
// the current root path in registers indexed by depth (16-entry vectors with
// a uniform index: indirect register moves, no copies).  Trees deeper than
// that recompute every node's state along its root path from H_0.  Either
// way a node's state comes from its own root path only, by the operations of
// a sequential walk along that path, in the same order.  y is summed over a
// lane's states in order, then over the channel's lanes in one fixed order,
// the same for every pass.
constexpr int kLrTreeRows = 72;  // rows of a tree pass staged at once (max_nodes <= 65)
constexpr int kLrSeg = 64;       // rows per staged segment of a chain pass
constexpr int kLrStack = kLrRegisterDepth + 2;  // H_0, then the root path's states by depth

typedef float lr_stack_t __attribute__((ext_vector_type(kLrStack)));

// Sum of v over each aligned segment of L lanes (L = 2, 4, 8 or 16); the sum
// is exact in the segment's last lane.  L = 16: DPP row shifts (a row is 16
// lanes); smaller segments: a butterfly of lane exchanges.
template <int L>
__device__ __forceinline__ float seg_sum(float v) {
  if constexpr (L == 16) {
#define LR_DPP_ADD(ctrl)                                                                 \
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), ctrl, 0xf, 0xf, true))
    LR_DPP_ADD(0x111);  // row_shr:1
    LR_DPP_ADD(0x112);  // row_shr:2
    LR_DPP_ADD(0x114);  // row_shr:4
    LR_DPP_ADD(0x118);  // row_shr:8: lane 15 of each row holds the row's sum
#undef LR_DPP_ADD
  } else {
#pragma unroll
    for (int o = L / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  }
  return v;
}

// N consecutive floats (N = 2, 4 or 8; p aligned to 4 N bytes, at most 16)
// to or from registers by vector accesses.
template <int N>
__device__ __forceinline__ void lr_vload(float (&v)[N], const float* p) {
  if constexpr (N == 2) {
    const float2 t = *reinterpret_cast<const float2*>(p);
    v[0] = t.x; v[1] = t.y;
  } else {
#pragma unroll
    for (int q = 0; q < N / 4; ++q) {
      const float4 t = *reinterpret_cast<const float4*>(p + 4 * q);
      v[4 * q] = t.x; v[4 * q + 1] = t.y; v[4 * q + 2] = t.z; v[4 * q + 3] = t.w;
    }
  }
}
template <int N>
__device__ __forceinline__ void lr_vstore(float* p, const float (&v)[N]) {
  if constexpr (N == 2) {
    *reinterpret_cast<float2*>(p) = make_float2(v[0], v[1]);
  } else {
#pragma unroll
    for (int q = 0; q < N / 4; ++q)
      *reinterpret_cast<float4*>(p + 4 * q) =
          make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
  }
}

// Units per thread in one staging batch: enough for `units` (one batch)
// but at most `cap` (and at least 1), which bounds the registers holding
// loads in flight.
constexpr int lr_batch(int units, int cap, int threads) {
  const int need = (units + threads - 1) / threads;
  const int c = cap > 0 ? cap : 1;
  return need < c ? need : c;
}

// Lanes per channel and threads per workgroup of the walk for state width S:
// 4 states a lane, 256 threads.
constexpr int lr_spl(int S) { return 4; }
constexpr int lr_threads(int S) { return 256; }

// MODE 0: chains; 1: trees of depth <= kLrRegisterDepth (register stack);
// 2: deeper trees
template <int S, int MODE, int NS, int SPL, int THR>
__global__ __launch_bounds__(THR) void lr_fork_kernel(
    const float* __restrict__ proj, size_t sstride, int ld, const RowMeta* __restrict__ rows,
    const ReqMeta* __restrict__ reqs, int d, float* __restrict__ H, void* o, size_t olo,
    bool obf, float* save, bool commit_last, RowNorm norm) {
  static_assert(S == 16 || S == 32 || S == 64, "state width");
  constexpr bool TREE = MODE > 0;
  static_assert(SPL == 2 || SPL == 4 || SPL == 8, "states per lane");
  constexpr int LPC = S / SPL;               // lanes per channel
  constexpr int CPB = THR / LPC;             // channels per workgroup
  static_assert(CPB % 4 == 0 && THR >= kLrTreeRows && THR >= kLrSeg, "workgroup shape");
  constexpr int ROWS = TREE ? kLrTreeRows : kLrSeg;
  constexpr int XU = CPB / 4;                // 4-channel units of x, a, z per row
  constexpr int BU = S / 2;                  // 4-value units of B and C per row
  // per (row, channel): sigmoid(a), x, silu(z), a (all scaled by the row's
  // norm scale); per row: B then C; per (row, channel): the output
  __shared__ __align__(16) float4 sgx[ROWS][CPB];
  __shared__ __align__(16) float sbc[ROWS][2 * S];
  __shared__ float so[ROWS][CPB];
  __shared__ float scs[ROWS];
  __shared__ int sord[ROWS], sdep[ROWS], spar[ROWS];
  const int r = blockIdx.y;
  const ReqMeta rm = reqs[r];
  const int l = threadIdx.x % LPC;           // the lane's place in its channel
  const int lc = threadIdx.x / LPC;          // the lane's channel within the workgroup
  const int c = blockIdx.x * CPB + lc;
  const bool live = c < d;
  const int cc = live ? c : 0;
  float* H0 = H + ((size_t)rm.table * d + cc) * S + SPL * l;
  float h0[SPL];
  lr_vload<SPL>(h0, H0);
  float hp[SPL];  // chains: the running states
#pragma unroll
  for (int k = 0; k < SPL; ++k) hp[k] = h0[k];
  if (rm.nrows <= 0) return;
  // a tree pass is one segment (its rows fit kLrTreeRows): straight-line
  // code, so no load waits at a loop header
  const int seg_end = TREE ? 1 : rm.nrows;
  for (int i0 = 0; i0 < seg_end; i0 += ROWS) {
    const int n = min(ROWS, rm.nrows - i0);
    // staging in batches: a batch's loads (the NS split partials of x, a, z
    // of the workgroup's channels, and of the rows' B and C) are all issued
    // before any is summed, from indexes clamped to the last unit so that
    // the loads are unconditional (no branch between them, so none waits for
    // another); only the stores are guarded.  The first batch's loads go out
    // with the rows' norm-scale loads, so the two round trips overlap.
    // (more than 8 partials: the first 8 are in flight together, the rest
    // are loaded and added in groups of 8 afterwards, in split order)
    constexpr int G = NS < 8 ? NS : 8;
    constexpr int UA = lr_batch(ROWS * XU, 6 / (3 * G), THR);  // x/a/z units per thread
    constexpr int UB = lr_batch(ROWS * BU, 12 / G, THR);       // B/C units per thread
    const float* pbase = proj + (size_t)(rm.row0 + i0) * ld;
    const int na = n * XU, nb = n * BU;  // units of this segment (n >= 1)
    // the first column of x/a/z unit q of a row (a partial workgroup's
    // surplus units repeat the last channels)
    auto a_col = [&](int q) { return min((int)blockIdx.x * CPB + q * 4, d - 4); };
    float4 ta[UA][3][G], tb[UB][G];
    auto issue = [&](int ea, int eb) {
#pragma unroll
      for (int u = 0; u < UA; ++u) {
        const int e = min(ea + (int)threadIdx.x + u * THR, na - 1);
        const float* p = pbase + (size_t)(e / XU) * ld + a_col(e % XU);
#pragma unroll
        for (int t = 0; t < 3; ++t)
#pragma unroll
          for (int s2 = 0; s2 < G; ++s2)
            ta[u][t][s2] = *reinterpret_cast<const float4*>(p + t * d + s2 * sstride);
      }
#pragma unroll
      for (int u = 0; u < UB; ++u) {
        const int e = min(eb + (int)threadIdx.x + u * THR, nb - 1);
        const float* p = pbase + (size_t)(e / BU) * ld + 3 * d + 4 * (e % BU);
#pragma unroll
        for (int s2 = 0; s2 < G; ++s2)
          tb[u][s2] = *reinterpret_cast<const float4*>(p + s2 * sstride);
      }
    };
    // the rows' norm-scale chunks and metadata (thread t: row min(t, n - 1))
    // first, then the first batch, all in flight together
    const int tr = min((int)threadIdx.x, n - 1);
    float ssv[16];
    row_ss_load(norm, rm.row0 + i0 + tr, ssv);
    RowMeta m{};
    if (TREE) m = rows[rm.row0 + tr];
    __syncthreads();  // the previous segment's values are no longer read
    issue(0, 0);
    if ((int)threadIdx.x < n) {
      scs[threadIdx.x] = row_scale_of(norm, ssv);
      if (TREE) {
        sord[threadIdx.x] = m.order;
        sdep[threadIdx.x] = m.pos - rm.nctx;
        spar[threadIdx.x] = m.parent;
      }
    }
    __syncthreads();  // scs
    // split-ordered sum of a unit's partials (the first G given), scaled
    auto sum = [&](const float4 (&t)[G], const float* p, float sc) {
      float4 v = t[0];
#pragma unroll
      for (int s2 = 1; s2 < G; ++s2) {
        v.x += t[s2].x;
        v.y += t[s2].y;
        v.z += t[s2].z;
        v.w += t[s2].w;
      }
      for (int q0 = G; q0 < NS; q0 += G) {
        float4 u[G];
#pragma unroll
        for (int s2 = 0; s2 < G; ++s2)
          if (q0 + s2 < NS) u[s2] = *reinterpret_cast<const float4*>(p + (q0 + s2) * sstride);
#pragma unroll
        for (int s2 = 0; s2 < G; ++s2)
          if (q0 + s2 < NS) {
            v.x += u[s2].x;
            v.y += u[s2].y;
            v.z += u[s2].z;
            v.w += u[s2].w;
          }
      }
      return make_float4(v.x * sc, v.y * sc, v.z * sc, v.w * sc);
    };
    for (int ea = 0, eb = 0; ea < na || eb < nb; ea += THR * UA, eb += THR * UB) {
      if (ea > 0 || eb > 0) issue(ea, eb);
#pragma unroll
      for (int u = 0; u < UA; ++u) {
        const int e = ea + threadIdx.x + u * THR;
        if (e < na) {
          const int j = e / XU, q = e % XU;
          const float sc = scs[j];
          const float* p = pbase + (size_t)j * ld + a_col(q);
          const float4 x = sum(ta[u][0], p, sc), a = sum(ta[u][1], p + d, sc),
                       z = sum(ta[u][2], p + 2 * d, sc);
          sgx[j][4 * q] = make_float4(1.0f / (1.0f + expf(-a.x)), x.x,
                                      z.x / (1.0f + expf(-z.x)), a.x);
          sgx[j][4 * q + 1] = make_float4(1.0f / (1.0f + expf(-a.y)), x.y,
                                          z.y / (1.0f + expf(-z.y)), a.y);
          sgx[j][4 * q + 2] = make_float4(1.0f / (1.0f + expf(-a.z)), x.z,
                                          z.z / (1.0f + expf(-z.z)), a.z);
          sgx[j][4 * q + 3] = make_float4(1.0f / (1.0f + expf(-a.w)), x.w,
                                          z.w / (1.0f + expf(-z.w)), a.w);
        }
      }
#pragma unroll
      for (int u = 0; u < UB; ++u) {
        const int e = eb + threadIdx.x + u * THR;
        if (e < nb) {
          const int j = e / BU, k = e % BU;
          *reinterpret_cast<float4*>(&sbc[j][4 * k]) =
              sum(tb[u], pbase + (size_t)j * ld + 3 * d + 4 * k, scs[j]);
        }
      }
    }
    __syncthreads();
    // The walk.  Each wave keeps the walk order (node, depth) in two lanes'
    // registers (position k in lane k % 64 of word k / 64) so a node index is
    // a register read, not an LDS round trip.  Two nodes' inputs are in
    // flight ahead of the one being computed (alternating register sets, no
    // copies), and each node's output goes to LDS, written out coalesced
    // after the walk.
    // trees: H_0, then the states of the current root path's nodes by depth + 1
    lr_stack_t st[SPL];
#pragma unroll
    for (int k = 0; k < SPL; ++k) {
      st[k] = lr_stack_t{};
      st[k][0] = h0[k];
    }
    int ordw0 = 0, ordw1 = 0;  // node | depth << 8 of positions lane, 64 + lane
    {
      const int lane = threadIdx.x & 63;
      auto at = [&](int q) {
        if (q >= n) return 0;
        return TREE ? (sord[q] | (sdep[sord[q]] << 8)) : q;
      };
      ordw0 = at(lane);
      ordw1 = at(64 + lane);
    }
    auto pos = [&](int k) {  // (node, depth) at walk position k (uniform)
      return __builtin_amdgcn_readlane(k < 64 ? ordw0 : ordw1, k & 63);
    };
    struct In {
      float4 gx;  // sigmoid(a), x, silu(z), a
      float b[SPL], c[SPL];
    };
    auto fetch = [&](int j) {
      In v;
      v.gx = sgx[j][lc];
      lr_vload<SPL>(v.b, &sbc[j][SPL * l]);
      lr_vload<SPL>(v.c, &sbc[j][S + SPL * l]);
      return v;
    };
    // one node's update from its parent's states
    auto step = [&](const In& v, float (&a)[SPL]) {
#pragma unroll
      for (int k = 0; k < SPL; ++k) a[k] = ((v.gx.x * a[k]) + (v.b[k] * v.gx.y));
    };
    auto node = [&](const In& cur, int wk) {
      const int j = wk & 0xFF, dj = wk >> 8;
      float a[SPL];
      if constexpr (MODE == 1) {
        // the parent's state is entry dj (H_0 for the root); every node's
        // state goes to entry dj + 1 unconditionally (no node of this class
        // is deeper than the last entry): a guarded insert into a register
        // vector compiles to a copy and a select of the whole vector
#pragma unroll
        for (int k = 0; k < SPL; ++k) a[k] = st[k][dj];
        step(cur, a);
#pragma unroll
        for (int k = 0; k < SPL; ++k) st[k][dj + 1] = a[k];
      } else if constexpr (MODE == 2) {
        // recompute along the root path of j, root first
#pragma unroll
        for (int k = 0; k < SPL; ++k) a[k] = h0[k];
        for (int t = 0; t <= dj; ++t) {
          int v = j;  // the ancestor of j at depth t
          for (int u = dj; u > t; --u) v = spar[v];
          step(fetch(__builtin_amdgcn_readfirstlane(v)), a);
        }
      } else {
#pragma unroll
        for (int k = 0; k < SPL; ++k) a[k] = hp[k];
        step(cur, a);
#pragma unroll
        for (int k = 0; k < SPL; ++k) hp[k] = a[k];
      }
      float y = (a[0] * cur.c[0]);
#pragma unroll
      for (int k = 1; k < SPL; ++k) y = (y + (a[k] * cur.c[k]));
      y = seg_sum<LPC>(y);
      if (l == LPC - 1) so[j][lc] = y * cur.gx.z;
    };
    if (n > 0) {
      auto at = [&](int k) { return pos(k < n ? k : n - 1); };
      int w0 = at(0), w1 = at(1);
      In A = fetch(w0 & 0xFF), B = fetch(w1 & 0xFF);
      for (int k = 0; k < n; k += 2) {
        node(A, w0);
        if (k + 2 < n) {
          w0 = at(k + 2);
          A = fetch(w0 & 0xFF);
        }
        if (k + 1 < n) node(B, w1);
        if (k + 3 < n) {
          w1 = at(k + 3);
          B = fetch(w1 & 0xFF);
        }
      }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < n * CPB; e += THR) {
      const int j = e / CPB, q = e % CPB;
      const int ch = blockIdx.x * CPB + q;
      if (ch >= d) continue;
      const size_t oi = (size_t)(rm.row0 + i0 + j) * d + ch;
      if (obf) store_act((uint16_t*)o, (uint16_t*)o + olo, oi, so[j][q]);
      else store_act((float*)o, (float*)o + olo, oi, so[j][q]);
    }
    if (save) {  // [x | a | B] of every row, for the commit
      for (int e = threadIdx.x; e < n * CPB; e += THR) {
        const int j = e / CPB, q = e % CPB;
        const int ch = blockIdx.x * CPB + q;
        if (ch >= d) continue;
        const size_t row = (size_t)(rm.row0 + i0 + j);
        const float4 v = sgx[j][q];
        save[row * (2 * d + S) + ch] = v.y;
        save[row * (2 * d + S) + d + ch] = v.w;
      }
      if (blockIdx.x == 0)
        for (int e = threadIdx.x; e < n * S; e += THR) {
          const int j = e / S, q = e % S;
          save[(size_t)(rm.row0 + i0 + j) * (2 * d + S) + 2 * d + q] = sbc[j][q];
        }
    }
  }
  if (commit_last && live) lr_vstore<SPL>(H0, hp);
}

// ----------------------------------------------------------- KV compaction
// Per (request, attention layer, KV head): read every accepted node's K and V
// first, then write them at their final positions (a node's destination may
// be another accepted node's source).
template <typename T>
__global__ __launch_bounds__(256) void kv_compact_kernel(
    const CommitReq* cr, const int32_t* btab, int max_pages, T* kbase,
    T* vbase, size_t layer_stride, int nkv, int hd) {
  __shared__ T buf[2][64 * 128];
  const int r = blockIdx.x, layer = blockIdx.y, kvh = blockIdx.z;
  const CommitReq& q = cr[r];  // read in place (nodes[] is indexed dynamically)
  const int32_t* bt = btab + (size_t)q.table * max_pages;
  T* kc = kbase + layer * layer_stride;
  T* vc = vbase + layer * layer_stride;
  const int n = q.plen * hd;
  for (int e = threadIdx.x; e < n; e += blockDim.x) {
    const int j = e / hd, dim = e % hd;
    const int t = q.nctx + q.slots[j];
    const int page = kv_page(-1, bt, t), off = t & 15;
    buf[0][e] = kc[kv_k_index(page, nkv, kvh, off, hd, dim)];
    buf[1][e] = vc[kv_v_index(page, nkv, kvh, off, hd, dim)];
  }
  __syncthreads();
  for (int e = threadIdx.x; e < n; e += blockDim.x) {
    const int j = e / hd, dim = e % hd;
    if (q.slots[j] == j + 1) continue;  // already in place
    const int t = q.nctx + j + 1;
    const int page = kv_page(-1, bt, t), off = t & 15;
    kc[kv_k_index(page, nkv, kvh, off, hd, dim)] = buf[0][e];
    vc[kv_v_index(page, nkv, kvh, off, hd, dim)] = buf[1][e];
  }
}

// ------------------------------------------------------ recurrence commit
// H <- state after the root and the accepted nodes, same op order as the
// verify pass, so the committed state equals the verified node's state.
__global__ __launch_bounds__(256) void lr_commit_kernel(
    const CommitReq* cr, const float* proj_all, size_t proj_layer_stride,
    int ld, int d, int S, float* H, size_t H_layer_stride) {
  const int r = blockIdx.z, layer = blockIdx.y;
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= d * S) return;
  const int c = e / S, s = e % S;
  const CommitReq& q = cr[r];  // read in place (nodes[] is indexed dynamically)
  float* hp = H + layer * H_layer_stride + (size_t)q.table * d * S + e;
  const float* proj = proj_all + layer * proj_layer_stride;
  float h = *hp;
  // the path's inputs are loaded 8 nodes at a time, ahead of the sequential
  // recurrence over them
  constexpr int B = 8;
  for (int k0 = 0; k0 <= q.plen; k0 += B) {
    float av[B], bv[B], xv[B];
#pragma unroll
    for (int u = 0; u < B; ++u) {
      const int k = k0 + u;
      if (k <= q.plen) {
        const int node = (k == 0) ? 0 : q.nodes[k - 1];
        const float* pr = proj + (size_t)(q.row0 + node) * ld;  // [x | a | B]
        av[u] = pr[d + c];
        bv[u] = pr[2 * d + s];
        xv[u] = pr[c];
      }
    }
#pragma unroll
    for (int u = 0; u < B; ++u) {
      if (k0 + u <= q.plen) {
        const float sig = 1.0f / (1.0f + expf(-av[u]));
        h = ((sig * h) + (bv[u] * xv[u]));
      }
    }
  }
  *hp = h;
}

// ---------------------------------------------------------- weight layout
template <typename T>
__global__ void relayout_kernel(const T* src, int nrows, int K, T* dst,
                                int dst_tile0, int tile_stride, int wsn, int wsk) {
  const int ksteps = K / 32;
  const size_t tid = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t total = (size_t)(nrows / 16) * ksteps * 64;
  if (tid >= total) return;
  const int lane = tid & 63;
  const size_t tile = tid >> 6;
  const int nb = (int)(tile / ksteps), kb = (int)(tile % ksteps);
  const int row = nb * 16 + (lane & 15);
  const int col = kb * 32 + (lane >> 4) * 8;
  const T* s = src + (size_t)row * K + col;
  const size_t dtr = (size_t)dst_tile0 + (size_t)nb * tile_stride;
  T* d = dst + ((dtr * wsn + (size_t)kb * wsk) * 64 + lane) * 8;
#pragma unroll
  for (int e = 0; e < 8; ++e) d[e] = s[e];
}

template <typename T>
__global__ void to_f32_kernel(const T* src, int n, float* dst) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = to_f<T>(src[i]);
}

}  // namespace

hipError_t launch_embed(bool bf16, const void* emb, const RowMeta* rows, int R,
                        int d, float* h, const float* nw, void* u, size_t u_lo, float* ss,
                        const float* cos_t, const float* sin_t, int hd, float* cs,
                        hipStream_t s) {
  if (d % 4 || d > 16384 || hd % 2) return hipErrorInvalidValue;
  const dim3 grid(R, (d + kNormChunk - 1) / kNormChunk);
  if (bf16)
    embed_kernel<uint16_t><<<grid, 256, 0, s>>>((const uint16_t*)emb, rows, d, h, nw,
                                                (uint16_t*)u, u_lo, ss, cos_t, sin_t,
                                                hd / 2, cs);
  else
    embed_kernel<float><<<grid, 256, 0, s>>>((const float*)emb, rows, d, h, nw, (float*)u,
                                             u_lo, ss, cos_t, sin_t, hd / 2, cs);
  return hipGetLastError();
}

template <typename T>
static hipError_t rope_t(const float* qkv, int S, size_t sstride, const RowMeta* rows,
                         int R, int nq, int nkv, int hd, const float* cs, T* q_out,
                         T* q_lo, T* kc, T* vc, int ld, RowNorm norm, hipStream_t s) {
  dim3 grid(R, nq + 2 * nkv);
  const int thr = 64;  // loops over hd / 2 rotation pairs
  switch (S) {
#define RO_CASE(SV)                                                                    \
  case SV:                                                                             \
    rope_kv_kernel<T, SV><<<grid, thr, 0, s>>>(qkv, sstride, rows, nq, nkv, hd, cs,    \
                                               q_out, q_lo, kc, vc, ld, norm);         \
    break;
    RO_CASE(1) RO_CASE(2) RO_CASE(4) RO_CASE(5) RO_CASE(6) RO_CASE(8) RO_CASE(16) RO_CASE(32)
#undef RO_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_rope_kv(bool bf16, const float* qkv, int S, size_t split_stride,
                          const RowMeta* rows, int R, int nq, int nkv, int hd,
                          const float* cs, void* q_out, void* q_lo, void* kc, void* vc,
                          int ld_qkv, RowNorm norm, hipStream_t s) {
  if (bf16)
    return rope_t<uint16_t>(qkv, S, split_stride, rows, R, nq, nkv, hd, cs,
                            (uint16_t*)q_out, (uint16_t*)q_lo, (uint16_t*)kc,
                            (uint16_t*)vc, ld_qkv, norm, s);
  return rope_t<float>(qkv, S, split_stride, rows, R, nq, nkv, hd, cs, (float*)q_out,
                       (float*)q_lo, (float*)kc, (float*)vc, ld_qkv, norm, s);
}

template <typename T>
static hipError_t resid_t(const float* P, int S, size_t split_stride, int ld_p, int R,
                          int d, float* h, const float* nw, T* u, size_t u_lo, float* ss,
                          hipStream_t s) {
  const dim3 grid(R, (d + kNormChunk - 1) / kNormChunk);
  switch (S) {
#define RR_CASE(SV)                                                                 \
  case SV:                                                                          \
    resid_reduce_kernel<SV, T><<<grid, 256, 0, s>>>(P, split_stride, ld_p, d, h, nw, \
                                                    u, u_lo, ss);                   \
    break;
    RR_CASE(1) RR_CASE(2) RR_CASE(4) RR_CASE(5) RR_CASE(6) RR_CASE(8) RR_CASE(16) RR_CASE(32)
#undef RR_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_resid_reduce(bool bf16, const float* P, int S, size_t split_stride,
                               int ld_p, int R, int d, float* h, const float* nw,
                               void* u, size_t u_lo, float* ss, hipStream_t s) {
  if (d % 4 || d > 16384) return hipErrorInvalidValue;
  if (bf16)
    return resid_t<uint16_t>(P, S, split_stride, ld_p, R, d, h, nw, (uint16_t*)u, u_lo, ss,
                             s);
  return resid_t<float>(P, S, split_stride, ld_p, R, d, h, nw, (float*)u, u_lo, ss, s);
}

hipError_t launch_argmax_reduce(const float2* part, int R, int nblocks,
                                int32_t* amax, hipStream_t s) {
  argmax_reduce_kernel<<<R, 256, 0, s>>>(part, nblocks, amax);
  return hipGetLastError();
}

hipError_t launch_path_walk(const RowMeta* rows, const ReqMeta* reqs,
                            int n_req, const int32_t* amax, int max_path,
                            int32_t* res, hipStream_t s) {
  path_walk_kernel<<<n_req, 64, 0, s>>>(rows, reqs, amax, max_path, res);
  return hipGetLastError();
}

template <int S, int NS>
static hipError_t lr_fork_s(const float* proj, size_t sstride, int ld,
                            const RowMeta* rows, const ReqMeta* reqs, int n_req, int d,
                            float* H, void* o, size_t olo, bool obf, float* save, int tree_depth,
                            bool commit_last, int max_rows_per_req, RowNorm norm,
                            hipStream_t s) {
  constexpr int SPL = lr_spl(S), THR = lr_threads(S);
  constexpr int CPB = THR / (S / SPL);
  if (tree_depth > 0 && max_rows_per_req > kLrTreeRows) return hipErrorInvalidValue;
  dim3 grid((d + CPB - 1) / CPB, n_req);
  if (tree_depth > kLrRegisterDepth)
    lr_fork_kernel<S, 2, NS, SPL, THR><<<grid, THR, 0, s>>>(proj, sstride, ld, rows, reqs, d, H,
                                                            o, olo, obf, save, commit_last, norm);
  else if (tree_depth > 0)
    lr_fork_kernel<S, 1, NS, SPL, THR><<<grid, THR, 0, s>>>(proj, sstride, ld, rows, reqs, d, H,
                                                            o, olo, obf, save, commit_last, norm);
  else
    lr_fork_kernel<S, 0, NS, SPL, THR><<<grid, THR, 0, s>>>(proj, sstride, ld, rows, reqs, d, H,
                                                            o, olo, obf, save, commit_last, norm);
  return hipGetLastError();
}

template <int S>
static hipError_t lr_fork_ns(int NS, const float* proj, size_t sstride, int ld,
                             const RowMeta* rows, const ReqMeta* reqs, int n_req, int d,
                             float* H, void* o, size_t olo, bool obf, float* save, int tree,
                             bool commit_last, int max_rows_per_req, RowNorm norm,
                             hipStream_t s) {
  switch (NS) {
#define NS_CASE(NV)                                                                    \
  case NV:                                                                             \
    return lr_fork_s<S, NV>(proj, sstride, ld, rows, reqs, n_req, d, H, o, olo, obf,    \
                            save, tree, commit_last, max_rows_per_req, norm, s);
    NS_CASE(1) NS_CASE(2) NS_CASE(4) NS_CASE(5) NS_CASE(6) NS_CASE(8) NS_CASE(16) NS_CASE(32)
#undef NS_CASE
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_lr_fork(bool bf16, const float* proj, int NS, size_t split_stride,
                          int ld, const RowMeta* rows, const ReqMeta* reqs, int n_req,
                          int d, int S, float* H, void* o, size_t o_lo, float* save,
                          int tree_depth, bool commit_last, int max_rows_per_req,
                          RowNorm norm, hipStream_t s) {
  switch (S) {
#define LR_CASE(SV)                                                                    \
  case SV:                                                                             \
    return lr_fork_ns<SV>(NS, proj, split_stride, ld, rows, reqs, n_req, d, H, o, o_lo, \
                          bf16, save, tree_depth, commit_last, max_rows_per_req, norm, s);
    LR_CASE(16)
    LR_CASE(32)
    LR_CASE(64)
#undef LR_CASE
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_kv_compact(bool bf16, const CommitReq* cr, int n_req,
                             const int32_t* btab, int max_pages, void* kbase,
                             void* vbase, size_t layer_stride_elems,
                             int n_attn_layers, int nkv, int hd,
                             hipStream_t s) {
  dim3 grid(n_req, n_attn_layers, nkv);
  if (bf16)
    kv_compact_kernel<uint16_t><<<grid, 256, 0, s>>>(cr, btab, max_pages, (uint16_t*)kbase,
                                                     (uint16_t*)vbase, layer_stride_elems,
                                                     nkv, hd);
  else
    kv_compact_kernel<float><<<grid, 256, 0, s>>>(cr, btab, max_pages, (float*)kbase,
                                                  (float*)vbase, layer_stride_elems, nkv,
                                                  hd);
  return hipGetLastError();
}

hipError_t launch_lr_commit(const CommitReq* cr, int n_req,
                            const float* proj_all, size_t proj_layer_stride,
                            int proj_ld, int n_lr, int d, int S, float* H,
                            size_t H_layer_stride, hipStream_t s) {
  dim3 grid((d * S + 255) / 256, n_lr, n_req);
  lr_commit_kernel<<<grid, 256, 0, s>>>(cr, proj_all, proj_layer_stride, proj_ld,
                                        d, S, H, H_layer_stride);
  return hipGetLastError();
}

hipError_t launch_relayout(bool bf16, const void* src, int nrows, int K,
                           void* dst, int dst_tile0, int tile_stride, int wsn, int wsk,
                           hipStream_t s) {
  const size_t total = (size_t)(nrows / 16) * (K / 32) * 64;
  const unsigned grid = (unsigned)((total + 255) / 256);
  if (bf16)
    relayout_kernel<uint16_t><<<grid, 256, 0, s>>>((const uint16_t*)src, nrows, K,
                                                   (uint16_t*)dst, dst_tile0, tile_stride,
                                                   wsn, wsk);
  else
    relayout_kernel<float><<<grid, 256, 0, s>>>((const float*)src, nrows, K,
                                                (float*)dst, dst_tile0, tile_stride,
                                                wsn, wsk);
  return hipGetLastError();
}

hipError_t launch_to_f32(bool bf16, const void* src, int n, float* dst,
                         hipStream_t s) {
  const int grid = (n + 255) / 256;
  if (bf16) to_f32_kernel<uint16_t><<<grid, 256, 0, s>>>((const uint16_t*)src, n, dst);
  else to_f32_kernel<float><<<grid, 256, 0, s>>>((const float*)src, n, dst);
  return hipGetLastError();
}
