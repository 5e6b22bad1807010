// Host runtime of the verification library: the C ABI declared in spec.h.
//
// One context = one model on one device and stream.  The caller's workspace
// is carved into: weights (matrices in the tiled MFMA layout, embedding
// row-major, norm vectors in fp32), the KV page pool (K pages
// [page][kv_head][16][head_dim], V pages transposed [page][kv_head]
// [head_dim][16], one pool per attention layer), recurrent states, RoPE
// tables, scratch activations and the per-pass metadata.
//
// A verify pass is: metadata upload (one async copy), embedding, per layer
// [RMSNorm, QKV GEMM, RoPE + KV store, tree attention + combine, O GEMM +
// residual] or [RMSNorm, in_proj GEMM, recurrence fork, out_proj GEMM +
// residual], then [RMSNorm, gate/up GEMM + SwiGLU, down GEMM + residual],
// then the final RMSNorm, LM-head GEMM with argmax partials, argmax
// reduction, path walk and the single device-to-host copy of the results.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/spec.h"
#include "kernels.h"
#include "w12.h"

namespace {

constexpr size_t kAlign = 256;
constexpr int kMaxSplits = 128;  // attention key splits per request (verify passes)
constexpr int kMaxSplitsPrefill = 64;  // prefill chunks: splits of 128 keys up to 8192
constexpr int kAttnSlots = 512;  // attention workgroups resident at once (2 per CU)
constexpr int kAttnStreamSlots = 256;  // streamed attention workgroups resident at once (1 per CU)
constexpr int kInvariantRows = 128;    // rows whose GEMM outputs do not depend on the row count
                                       // (the skinny kernel's shapes: one split count and K
                                       // order per matrix, hi and lo products summed apart)
constexpr int kMaxPath = 64;     // accepted-path slots per request in the walk result
constexpr size_t kMaxGraphs = 8; // captured verify-pass graphs kept per context
// tile order of the input projections (QKV, in_proj) and of the matrices
// whose output is added to the residual (O, out_proj, down); gate/up and the
// LM head are always K-major
constexpr bool kKmajorQkv = true;
constexpr bool kKmajorOut = false;
constexpr int kStagingBytes = 64 << 20;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Req {
  bool active = false;
  int n = 0;
  int root = 0;
  std::vector<int> pages;
  int page0 = -1;  // pages[i] == page0 + i for all i, else -1
};

// One weight matrix [N, K] in the tiled layout (kernels.h), as bf16 / fp32
// tiles or as W12 tiles (w12.h).  The region is sized for the uncompressed
// tiles (W12 uses ~78% of it).
struct WMat {
  void* p = nullptr;
  size_t bytes = 0;      // region size
  int n = 0, k = 0;      // padded output rows, reduction length
  bool kmajor = false;   // tile order
  uint8_t* eb = nullptr; // W12: per-row base exponents [n]
  int* err = nullptr;    // W12: set when a tile does not fit the format
  void* p8 = nullptr;    // the 8-bit view's tiles (W12_LOWP)
};

struct Layer {
  int kind = SPEC_LAYER_ATTN;
  int idx = 0;  // index among layers of its kind
  float* n1 = nullptr;
  float* n2 = nullptr;
  WMat wqkv;  // attention: [Wq; Wk; Wv]
  WMat wo;
  WMat win;   // recurrent: W_in
  WMat wout;
  WMat wgu;   // gate/up tiles interleaved
  WMat wd;
};

// tensor id -> where it goes
struct TensorSlot {
  int kind;  // 0 embed, 1 norm, 2 matrix (or part of a fused matrix)
  int layer;
  int rows, cols;
  void* dst;
  int tile0, tile_stride;
  int wsn = 0, wsk = 0;        // matrices: tile strides of the destination layout
  const WMat* mat = nullptr;   // matrices: the destination
};

// Tile order of a weight matrix [N, K] (N padded to whole workgroup column
// blocks).  K-major (the tiles of one K-step of every tile row adjacent):
// all workgroups of an unsplit GEMM sweep one contiguous region together,
// which streams best; used for the matrices whose GEMM runs with few or no
// K splits.  N-major (a tile row's K-steps adjacent) for the rest.
struct TileOrder {
  int wsn, wsk;
};
TileOrder tile_order(int N, int K, bool kmajor) {
  const int cb = gemm_pad_cols();
  const int nt = (N + cb - 1) / cb * cb / 16;
  return kmajor ? TileOrder{1, nt} : TileOrder{K / 32, 1};
}

struct GraphEntry {
  std::vector<int64_t> key;
  hipGraphExec_t exec;
  uint64_t used;
};

struct Plan {
  size_t total = 0;
  size_t cursor = 0;
  size_t take(size_t bytes) {
    const size_t off = cursor;
    cursor = align_up(cursor + bytes);
    total = cursor;
    return off;
  }
};

struct LastVerify {
  bool valid = false;
  std::vector<int> req, row0, nrows, nctx;
  std::vector<std::vector<int>> parent;  // node-local parents
  std::vector<std::vector<int>> rank;    // node -> depth-first rank (its KV slot past n)
};

}  // namespace

struct spec_ctx {
  spec_config cfg{};
  bool bf16 = true;
  size_t esz = 2;
  hipStream_t stream = nullptr;
  char* ws = nullptr;
  int device = 0;

  int d = 0, nq = 0, nkv = 0, hd = 0, F = 0, V = 0, S = 0;
  int n_attn = 0, n_lr = 0, qkv_n = 0, in_n = 0;
  std::vector<Layer> layers;
  std::vector<TensorSlot> slots;
  std::vector<char> loaded;

  void* embed = nullptr;
  WMat lm_head;
  bool w12 = false;          // weights stored as W12 tiles
  bool w8 = false;           // ... and as their 8-bit view
  bool cur_lowp = false;     // the pass being enqueued reads the 8-bit view
  uint8_t* eb_tmp = nullptr; // W12 encoding: base exponents of one slab's rows
  size_t w12_side0 = 0, w12_side_bytes = 0;  // W12 side data (zeroed at create)
  float* final_norm = nullptr;

  // KV pool
  char* kpool = nullptr;
  char* vpool = nullptr;
  size_t kv_layer_elems = 0;
  int n_pages = 0, max_pages = 0;
  int32_t* d_btab = nullptr;
  std::vector<int> free_pages;

  float* H = nullptr;  // [n_lr][max_requests][d][S]
  size_t H_layer = 0;
  float* cos_t = nullptr;
  float* sin_t = nullptr;
  int max_pos = 0;

  // scratch
  int Rmax = 0;
  float* h = nullptr;
  // activation planes [Rmax, width] feeding the GEMMs (bf16: hi plane then
  // lo plane, lo at + Rmax * width elements; fp32: one plane)
  void* u = nullptr;         // h * norm weight (QKV / in_proj / gate-up / LM head input)
  float* ss = nullptr;       // deferred RMSNorm of u: [Rmax][norm_nc] chunk sums of squares
  float* rope_cs = nullptr;  // the pass rows' RoPE factors [Rmax][hd] (cos, then sin)
  int norm_nc = 0;
  void* act = nullptr;       // SwiGLU output (down input)
  void* attn_o = nullptr;    // attention output (O input)
  void* q = nullptr;
  void* q_lo = nullptr;
  float* P = nullptr;        // GEMM split partials [S][Rmax][N]
  size_t split_rows = 0;     // capacity of the attention split table (splits x rows)
  // captured verify passes (see run_pass)
  bool use_graphs = true;
  std::vector<GraphEntry> graphs;
  uint64_t graph_tick = 0;
  float* lrsave = nullptr;   // per recurrent layer [max_rows][x | a | B]
  size_t lrsave_layer = 0;
  size_t weights_end = 0;
  void* lr_o = nullptr;      // recurrent mixer output (out_proj input)
  float* part_o = nullptr;
  float2* part_ml = nullptr;
  float2* am_part = nullptr;
  int32_t* amax = nullptr;
  int32_t* res = nullptr;
  void* staging = nullptr;  // aliases the scratch activations

  // metadata: device and pinned host mirrors
  RowMeta* d_rows = nullptr;
  ReqMeta* d_reqs = nullptr;
  uint64_t* d_anc = nullptr;
  CommitReq* d_commit = nullptr;
  char* h_meta = nullptr;  // pinned: rows | reqs | anc (same layout as device)
  char* d_meta = nullptr;
  size_t meta_bytes = 0, off_reqs = 0, off_anc = 0;
  CommitReq* h_commit = nullptr;
  int32_t* h_res = nullptr;
  int32_t* h_btab = nullptr;  // pinned mirror of the block tables [max_requests][max_pages]

  std::vector<Req> reqs;
  LastVerify last;
  std::string err;
  bool poisoned = false;
  int fault_tok = -1;
  bool table_only = false;   // debug: always look pages up in the block table
  int attn_mode = 0;         // debug: 0 = planner's choice, 1 = stream whenever the
                             // query tiles allow it, 2 = never stream
  float fault_bias = 0.f;
  int fault_after = 0;

  int timing_cls = 0;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> events;
  size_t events_used = 0;
  double timing_ms = 0.0;
  int64_t timing_n = 0;
};

namespace {

int fail(spec_ctx* c, int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  if (c) c->err = buf;
  return code;
}

#define HIP_TRY(expr)                                                        \
  do {                                                                       \
    hipError_t e_ = (expr);                                                  \
    if (e_ != hipSuccess) {                                                  \
      c->poisoned = true;                                                    \
      return fail(c, SPEC_E_HIP, "%s failed: %s", #expr, hipGetErrorString(e_)); \
    }                                                                        \
  } while (0)

bool valid_config(const spec_config* cfg, std::string* why) {
  auto bad = [&](const char* m) { if (why) *why = m; return false; };
  if (!cfg) return bad("null config");
  if (cfg->n_layers <= 0 || cfg->n_layers > SPEC_MAX_LAYERS) return bad("n_layers");
  if (cfg->dtype != SPEC_DTYPE_FP32 && cfg->dtype != SPEC_DTYPE_BF16) return bad("dtype");
  if (cfg->head_dim != 64 && cfg->head_dim != 128) return bad("head_dim must be 64 or 128");
  if (cfg->n_kv_heads <= 0 || cfg->n_heads % cfg->n_kv_heads) return bad("heads");
  if (cfg->d_model % 32 || cfg->d_model <= 0 || cfg->d_model > 16384)
    return bad("d_model must be a multiple of 32 in [32, 16384]");
  if (cfg->ffn_dim % 64) return bad("ffn_dim must be a multiple of 64");
  if (cfg->vocab % 16 || cfg->vocab <= 0) return bad("vocab must be a multiple of 16");
  if ((cfg->n_heads * cfg->head_dim) % 32) return bad("n_heads*head_dim");
  if (cfg->page_size != 16) return bad("page_size must be 16");
  if (cfg->weight_format != SPEC_WEIGHTS_NATIVE && cfg->weight_format != SPEC_WEIGHTS_W12 &&
      cfg->weight_format != SPEC_WEIGHTS_W12_LOWP)
    return bad("weight_format");
  if (cfg->weight_format != SPEC_WEIGHTS_NATIVE && cfg->dtype != SPEC_DTYPE_BF16)
    return bad("W12 weights need a bf16 model");
  if (cfg->max_requests <= 0 || cfg->max_ctx <= 0) return bad("capacity");
  if (cfg->max_nodes < 1 || cfg->max_nodes > 65) return bad("max_nodes must be in [1, 65]");
  if (cfg->max_rows < cfg->max_nodes) return bad("max_rows < max_nodes");
  if (cfg->prefill_chunk < 1 || cfg->prefill_chunk > 1024) return bad("prefill_chunk");
  if (cfg->max_ctx < cfg->max_nodes + 1) return bad("max_ctx");
  if (cfg->max_ctx > kMaxSplitsPrefill * 128) return bad("max_ctx must be <= 8192");
  if (cfg->kv_pages < 0 || cfg->kv_pages > (1 << 24)) return bad("kv_pages");
  bool any_lr = false;
  for (int i = 0; i < cfg->n_layers; ++i) {
    if (cfg->layer_kind[i] == SPEC_LAYER_LR) any_lr = true;
    else if (cfg->layer_kind[i] != SPEC_LAYER_ATTN) return bad("layer_kind");
  }
  if (any_lr && cfg->lr_state != 16 && cfg->lr_state != 32 && cfg->lr_state != 64)
    return bad("lr_state must be 16, 32 or 64");
  return true;
}

// Lay out the workspace; with base == nullptr only the size is computed.
size_t plan_workspace(spec_ctx* c, const spec_config& cfg, char* base) {
  Plan p;
  const size_t esz = cfg.dtype == SPEC_DTYPE_BF16 ? 2 : 4;
  const int d = cfg.d_model, hd = cfg.head_dim, nq = cfg.n_heads, nkv = cfg.n_kv_heads;
  const int F = cfg.ffn_dim, V = cfg.vocab, S = cfg.lr_state;
  int n_attn = 0, n_lr = 0;
  for (int i = 0; i < cfg.n_layers; ++i)
    (cfg.layer_kind[i] == SPEC_LAYER_LR ? n_lr : n_attn)++;
  const int qkv_n = (nq + 2 * nkv) * hd;
  const int in_n = 3 * d + 2 * S;
  auto at = [&](size_t off) -> char* { return base ? base + off : nullptr; };
  // GEMM output rows are padded to whole workgroup column blocks
  const int cb = gemm_pad_cols();
  auto npad = [&](int n) { return (n + cb - 1) / cb * cb; };

  // weights; every matrix region holds its uncompressed tiles, and with
  // W12 also a base exponent per output row and two counters
  const bool w12 = cfg.weight_format != SPEC_WEIGHTS_NATIVE;
  const bool w8 = cfg.weight_format == SPEC_WEIGHTS_W12_LOWP;
  struct MatPlan {
    size_t off = 0, bytes = 0, off_eb = 0, off_cnt = 0, off8 = 0;
    int n = 0, k = 0;
    bool kmajor = false;
  };
  auto mat = [&](int N, int K, bool kmajor) {
    MatPlan m;
    m.n = npad(N);
    m.k = K;
    m.kmajor = kmajor;
    m.bytes = (size_t)m.n * K * esz;
    m.off = p.take(m.bytes);
    return m;
  };
  std::vector<size_t> off_l1, off_l2;
  std::vector<MatPlan> m_qkv, m_o, m_in, m_out, m_gu, m_d;
  const size_t o_embed = p.take((size_t)V * d * esz);
  for (int i = 0; i < cfg.n_layers; ++i) {
    off_l1.push_back(p.take((size_t)d * 4));
    if (cfg.layer_kind[i] == SPEC_LAYER_ATTN) {
      m_qkv.push_back(mat(qkv_n, d, kKmajorQkv));
      m_o.push_back(mat(d, nq * hd, kKmajorOut));
      m_in.push_back(MatPlan{});
      m_out.push_back(MatPlan{});
    } else {
      m_qkv.push_back(MatPlan{});
      m_o.push_back(MatPlan{});
      m_in.push_back(mat(in_n, d, kKmajorQkv));
      m_out.push_back(mat(d, d, kKmajorOut));
    }
    off_l2.push_back(p.take((size_t)d * 4));
    m_gu.push_back(mat(2 * F, d, true));
    m_d.push_back(mat(d, F, kKmajorOut));
  }
  const size_t o_fnorm = p.take((size_t)d * 4);
  MatPlan m_lm = mat(V, d, true);
  const size_t weights_end = p.cursor;
  // W12 side data: base exponents and counters of every matrix, and the
  // base exponents of one slab during encoding
  auto side = [&](MatPlan& m) {
    if (!w12 || m.n == 0) return;
    m.off_eb = p.take((size_t)m.n);
    m.off_cnt = p.take(sizeof(int));
    if (w8) m.off8 = p.take((size_t)m.n * m.k);  // the 8-bit view: one byte a weight
  };
  for (int i = 0; i < cfg.n_layers; ++i) {
    side(m_qkv[i]);
    side(m_o[i]);
    side(m_in[i]);
    side(m_out[i]);
    side(m_gu[i]);
    side(m_d[i]);
  }
  side(m_lm);
  const size_t o_ebtmp = w12 ? p.take((size_t)std::max({npad(V), npad(2 * F), npad(in_n),
                                                        npad(qkv_n), npad(d)})) : 0;
  const size_t w12_end = p.cursor;

  // KV pool: kv_pages pages (default: every request at max_ctx), taken by
  // the requests as their contexts grow
  const int max_pages = (cfg.max_ctx + 15) / 16;  // per request
  const int n_pages = cfg.kv_pages > 0 ? cfg.kv_pages : max_pages * cfg.max_requests;
  const size_t kv_layer_elems = (size_t)n_pages * nkv * 16 * hd;
  const size_t o_k = p.take(kv_layer_elems * esz * std::max(n_attn, 1));
  const size_t o_v = p.take(kv_layer_elems * esz * std::max(n_attn, 1));
  const size_t o_btab = p.take((size_t)cfg.max_requests * max_pages * 4);
  const size_t H_layer = (size_t)cfg.max_requests * d * std::max(S, 1);
  const size_t o_H = p.take(H_layer * 4 * std::max(n_lr, 1));
  const int max_pos = cfg.max_ctx + 1;
  const size_t o_cos = p.take((size_t)max_pos * (hd / 2) * 4);
  const size_t o_sin = p.take((size_t)max_pos * (hd / 2) * 4);

  // scratch
  const int R = std::max(cfg.max_rows, cfg.prefill_chunk);
  const size_t scratch0 = p.cursor;
  const size_t o_h = p.take((size_t)R * d * 4);
  const size_t o_u = p.take((size_t)R * d * 4);
  const int norm_nc = (d + kNormChunk - 1) / kNormChunk;
  const size_t o_ss = p.take((size_t)R * norm_nc * 4);
  const size_t o_cs = p.take((size_t)R * hd * 4);
  const size_t o_act = p.take((size_t)R * F * 4);
  const size_t o_ao = p.take((size_t)R * nq * hd * 4);
  const size_t o_q = p.take((size_t)R * nq * hd * esz * 2);  // bf16: hi and lo planes
  const size_t o_lrs = p.take(n_lr ? (size_t)n_lr * cfg.max_rows * (2 * d + S) * 4 : 0);
  const size_t o_lro = p.take(n_lr ? (size_t)R * d * 4 : 0);
  // attention split partials: (splits x rows) of one pass
  const size_t split_rows = std::max((size_t)kMaxSplits * cfg.max_rows,
                                     (size_t)kMaxSplitsPrefill * R);
  const size_t o_po = p.take(split_rows * nq * hd * 4);
  const size_t o_pml = p.take(split_rows * nq * 8);
  int am_blocks = 1;  // LM-head argmax partials per row: the most column blocks of any row count
  for (int m = 1; m <= R; ++m)
    am_blocks = std::max(am_blocks, gemm_argmax_blocks(esz == 2, npad(V), m));
  const size_t o_amp = p.take((size_t)R * am_blocks * 8);
  const size_t o_amax = p.take((size_t)R * 4);
  const size_t o_res = p.take((size_t)cfg.max_requests * (2 + kMaxPath) * 4);
  // GEMM split partials: the largest S x N over the model's matrices, for
  // any row count up to R (the split count depends on the rows of a launch)
  size_t psz = 0;
  auto need_p = [&](int K, int N) {
    for (int m = 1; m <= R; ++m)
      psz = std::max(psz, (size_t)gemm_splits(esz == 2, K, npad(N), m) * npad(N));
  };
  need_p(d, qkv_n);
  need_p(nq * hd, d);
  need_p(d, 2 * F);
  need_p(F, d);
  if (n_lr) {
    need_p(d, in_n);
    need_p(d, d);
  }
  const size_t o_P = p.take(psz * R * 4);
  size_t scratch_bytes = p.cursor - scratch0;
  if (scratch_bytes < (size_t)kStagingBytes) p.take(kStagingBytes - scratch_bytes);

  // metadata
  const int anc_words = (cfg.max_nodes + 63) / 64;
  const size_t rows_b = align_up((size_t)R * sizeof(RowMeta));
  const size_t reqs_b = align_up((size_t)cfg.max_requests * sizeof(ReqMeta));
  const size_t anc_b = align_up((size_t)R * anc_words * 8);
  const size_t o_meta = p.take(rows_b + reqs_b + anc_b);
  const size_t o_commit = p.take((size_t)cfg.max_requests * sizeof(CommitReq));

  if (c && base) {
    auto wmat = [&](const MatPlan& m) {
      WMat w;
      if (m.n == 0) return w;
      w.p = at(m.off);
      w.bytes = m.bytes;
      w.n = m.n;
      w.k = m.k;
      w.kmajor = m.kmajor;
      if (w12) {
        w.eb = (uint8_t*)at(m.off_eb);
        w.err = (int*)at(m.off_cnt);
      }
      if (w8) w.p8 = at(m.off8);
      return w;
    };
    c->embed = at(o_embed);
    c->final_norm = (float*)at(o_fnorm);
    c->lm_head = wmat(m_lm);
    c->w12 = w12;
    c->w8 = w8;
    c->eb_tmp = w12 ? (uint8_t*)at(o_ebtmp) : nullptr;
    c->w12_side0 = weights_end;
    c->w12_side_bytes = w12_end - weights_end;
    int ia = 0, il = 0;
    c->layers.resize(cfg.n_layers);
    for (int i = 0; i < cfg.n_layers; ++i) {
      Layer& L = c->layers[i];
      L.kind = cfg.layer_kind[i];
      L.idx = L.kind == SPEC_LAYER_ATTN ? ia++ : il++;
      L.n1 = (float*)at(off_l1[i]);
      L.n2 = (float*)at(off_l2[i]);
      L.wqkv = wmat(m_qkv[i]);
      L.wo = wmat(m_o[i]);
      L.win = wmat(m_in[i]);
      L.wout = wmat(m_out[i]);
      L.wgu = wmat(m_gu[i]);
      L.wd = wmat(m_d[i]);
    }
    c->kpool = at(o_k);
    c->vpool = at(o_v);
    c->kv_layer_elems = kv_layer_elems;
    c->n_pages = n_pages;
    c->max_pages = max_pages;
    c->d_btab = (int32_t*)at(o_btab);
    c->H = (float*)at(o_H);
    c->H_layer = H_layer;
    c->cos_t = (float*)at(o_cos);
    c->sin_t = (float*)at(o_sin);
    c->max_pos = max_pos;
    c->Rmax = R;
    c->h = (float*)at(o_h);
    c->u = at(o_u);
    c->ss = (float*)at(o_ss);
    c->rope_cs = (float*)at(o_cs);
    c->norm_nc = norm_nc;
    c->act = at(o_act);
    c->attn_o = at(o_ao);
    c->q = at(o_q);
    c->q_lo = at(o_q + (size_t)R * nq * hd * esz);
    c->lrsave = (float*)at(o_lrs);
    c->lrsave_layer = (size_t)cfg.max_rows * (2 * d + S);
    c->lr_o = at(o_lro);
    c->P = (float*)at(o_P);
    c->weights_end = weights_end;
    c->part_o = (float*)at(o_po);
    c->part_ml = (float2*)at(o_pml);
    c->split_rows = split_rows;
    c->am_part = (float2*)at(o_amp);
    c->amax = (int32_t*)at(o_amax);
    c->res = (int32_t*)at(o_res);
    c->staging = at(scratch0);
    c->d_meta = at(o_meta);
    c->meta_bytes = rows_b + reqs_b + anc_b;
    c->off_reqs = rows_b;
    c->off_anc = rows_b + reqs_b;
    c->d_rows = (RowMeta*)c->d_meta;
    c->d_reqs = (ReqMeta*)(c->d_meta + rows_b);
    c->d_anc = (uint64_t*)(c->d_meta + rows_b + reqs_b);
    c->d_commit = (CommitReq*)at(o_commit);
  }
  return p.total;
}

void build_slots(spec_ctx* c) {
  const spec_config& cfg = c->cfg;
  const int d = c->d, hd = c->hd, F = c->F;
  c->slots.clear();
  auto mat = [&](int layer, int rows, int cols, const WMat& m, int tile0, int tstride) {
    const TileOrder o = tile_order(m.n, cols, m.kmajor);
    TensorSlot t{2, layer, rows, cols, m.p, tile0, tstride};
    t.wsn = o.wsn;
    t.wsk = o.wsk;
    t.mat = &m;
    c->slots.push_back(t);
  };
  c->slots.push_back({0, -1, c->V, d, c->embed, 0, 1});
  for (int i = 0; i < cfg.n_layers; ++i) {
    Layer& L = c->layers[i];
    c->slots.push_back({1, i, d, 1, L.n1, 0, 1});
    if (L.kind == SPEC_LAYER_ATTN) {
      mat(i, c->nq * hd, d, L.wqkv, 0, 1);
      mat(i, c->nkv * hd, d, L.wqkv, c->nq * hd / 16, 1);
      mat(i, c->nkv * hd, d, L.wqkv, (c->nq + c->nkv) * hd / 16, 1);
      mat(i, d, c->nq * hd, L.wo, 0, 1);
    } else {
      mat(i, c->in_n, d, L.win, 0, 1);
      mat(i, d, d, L.wout, 0, 1);
    }
    c->slots.push_back({1, i, d, 1, L.n2, 0, 1});
    mat(i, F, d, L.wgu, 0, 2);   // gate -> even tiles
    mat(i, F, d, L.wgu, 1, 2);   // up   -> odd tiles
    mat(i, d, F, L.wd, 0, 1);
  }
  c->slots.push_back({1, -1, d, 1, c->final_norm, 0, 1});
  mat(-1, c->V, d, c->lm_head, 0, 1);
  c->loaded.assign(c->slots.size(), 0);
}

int check(spec_ctx* c) {
  if (!c) return SPEC_E_INVAL;
  if (c->poisoned) return fail(c, SPEC_E_HIP, "context poisoned by an earlier HIP error");
  return SPEC_OK;
}

bool all_loaded(const spec_ctx* c) {
  for (char x : c->loaded)
    if (!x) return false;
  return true;
}

// Timing: the event pair for one launch of kernel class cls (both null when
// that class is not being timed).  The launch records the kernel's own start
// and end in them.
struct TimePair {
  hipEvent_t t0 = nullptr, t1 = nullptr;
};
TimePair time_pair(spec_ctx* c, int cls) {
  if (c->timing_cls != cls) return {};
  if (c->events_used == c->events.size()) {
    hipEvent_t a, b;
    if (hipEventCreate(&a) != hipSuccess) return {};
    if (hipEventCreate(&b) != hipSuccess) {
      (void)hipEventDestroy(a);
      return {};
    }
    c->events.push_back({a, b});
  }
  const auto& e = c->events[c->events_used++];
  return {e.first, e.second};
}

// The deferred RMSNorm of the rows of u from row0 on (the consumer of a
// GEMM over those rows applies it).
RowNorm row_norm(const spec_ctx* c, int row0 = 0) {
  return RowNorm{c->ss + (size_t)row0 * c->norm_nc, c->norm_nc, c->d, c->cfg.rms_eps};
}

// Element offset of the lo plane of an activation buffer of `width` columns.
size_t lo_off(const spec_ctx* c, int width) {
  return c->bf16 ? (size_t)c->Rmax * width : 0;
}

GemmArgs gemm_args(const spec_ctx* c, const WMat& W, const void* X, int ldx, int M,
                   int K, int N) {
  GemmArgs a{};
  a.W = W.p;
  const TileOrder o = tile_order(N, K, W.kmajor);
  a.wsn = o.wsn;
  a.wsk = o.wsk;
  a.w12 = c->w12 ? 1 : 0;
  a.eb = W.eb;
  if (c->cur_lowp) {
    a.W = W.p8;
    a.w12 = 2;
  }
  a.X = X;
  a.ldx = ldx;
  a.xlo = (int64_t)lo_off(c, ldx);
  a.M = M;
  a.K = K;
  const int cb = gemm_pad_cols();
  a.ntiles = (N + cb - 1) / cb * cb / 16;
  a.ncols = N;
  a.S = 1;
  a.P = c->P;
  a.P_ld = c->Rmax;
  a.bias_tok = -1;
  return a;
}

// Split GEMM into the partial buffer; returns the split count used.
int gemm_part(spec_ctx* c, GemmArgs& g, hipError_t* err, TimePair tp = {}) {
  g.S = gemm_splits(c->bf16, g.K, g.ntiles * 16, g.M);
  *err = launch_gemm(c->bf16, EPI_PART, g, c->stream, tp.t0, tp.t1);
  return g.S;
}

// Launch parameters of one forward pass: everything the kernel sequence
// depends on besides the device-side metadata (rows, requests, masks), so
// that two passes with equal parameters can replay one captured graph.
struct Pass {
  int R = 0, n_req = 0;
  int tree_depth = 0;  // 0: chains only; else the recurrent walk's depth class (16 or 64)
  bool prefill = false;
  int lm_row0 = 0, lm_rows = 0;
  float* d_logits = nullptr;
  int split = 0, max_splits = 0, tpw = 0, max_qgroups = 0, max_rows_req = 0;
  bool attn_stream = false;  // streamed attention (every request: <= 8 query tiles a KV head)
  bool one_part = false;     // streamed, one wave per query tile (row-count invariant)
  bool walk = false;  // append the accepted-path walk (verify passes)
  bool lowp = false;  // read the weights' 8-bit view
  std::vector<int64_t> key(const spec_ctx* c) const;
};

// Plan a forward pass over R rows already described in d_rows / d_reqs /
// d_anc.  lm_row0 / lm_rows: rows that go through the LM head (argmax into
// amax).  prefill: chain pass whose final recurrent states are committed.
int plan_pass(spec_ctx* c, Pass& P, int R, int n_req, const std::vector<int>& keys_per_req,
              const std::vector<int>& rows_per_req, int tree_depth, int lm_row0, int lm_rows,
              float* d_logits, bool prefill) {
  const spec_config& cfg = c->cfg;
  const int nq = c->nq, nkv = c->nkv;
  const int G = nq / nkv;
  P.R = R;
  P.n_req = n_req;
  P.tree_depth = tree_depth;
  P.prefill = prefill;
  P.lm_row0 = lm_row0;
  P.lm_rows = lm_rows;
  P.d_logits = d_logits;
  // attention launch shape.  Streamed (verify passes): a workgroup walks one
  // range of keys of one (request, KV head) in stages for a group of up to
  // kAttnStreamTiles query tiles of 16 query rows.  Otherwise (prefill
  // chunks) a workgroup stages one key split of one (request, KV head) and
  // serves a group of up to 32 query tiles of it.  The split is the smallest of
  // 32, 64, 96, 128 keys whose grid fits the resident workgroup slots (one
  // round, most parallelism), else 128 keys; the split table bounds it.  Key
  // counts are rounded up to 256 so that the launch shape (and a captured
  // graph) stays the same while a request grows; surplus splits exit early.
  auto keys_up = [&](int k) { return std::min((k + 255) / 256 * 256, cfg.max_ctx); };
  int keys_max = 0, qt_max = 0, max_rows_req = 0;
  for (int r = 0; r < n_req; ++r) {
    keys_max = std::max(keys_max, keys_up(keys_per_req[r]));
    qt_max = std::max(qt_max, (rows_per_req[r] * G + 15) / 16);
    max_rows_req = std::max(max_rows_req, rows_per_req[r]);
  }
  const int split_cap = R <= cfg.max_rows ? kMaxSplits : kMaxSplitsPrefill;
  const long pairs = (long)n_req * nkv;
  if (R <= cfg.max_rows && c->attn_mode != 2) {
    // streamed (verify passes): query groups of at most kAttnStreamTiles
    // tiles, and for each (request, KV head, query group) enough key ranges
    // (multiples of 64 keys) for about one workgroup per CU
    // (forced by the debug flag: two ranges, so each range has several stages)
    // One request, at most kInvariantRows rows: the GEMMs of such passes
    // give each output the same sums (split counts, K order), so with one wave per
    // query tile and a plan that does not depend on the pass's rows (query
    // groups sized for the largest tree, keys counted to the largest tree
    // by the caller) a row's logits are the same bits whatever the pass's
    // rows: a verify's rows and AR steps at their positions agree exactly
    // while the committed length stays in one 256-key bucket.
    const bool invariant = n_req == 1 && R <= kInvariantRows;
    if (invariant) qt_max = std::max(qt_max, (cfg.max_nodes * G + 15) / 16);
    const int qgroups = (std::max(qt_max, 1) + kAttnStreamTiles - 1) / kAttnStreamTiles;
    const long units = pairs * qgroups;
    const int ranges = c->attn_mode == 1
                           ? 2
                           : (int)std::max(1L, ((long)kAttnStreamSlots + units - 1) / units);
    int span = std::max(64, ((keys_max + ranges - 1) / ranges + 63) / 64 * 64);
    auto nsplit = [&](int sp) { return (keys_max + sp - 1) / sp; };
    while (nsplit(span) > split_cap || (size_t)nsplit(span) * R > c->split_rows) {
      if (span >= keys_max)
        return fail(c, SPEC_E_UNSUPPORTED, "context too long for the attention split table");
      span += 64;
    }
    P.attn_stream = true;
    P.one_part = invariant;
    P.split = span;
    P.max_splits = nsplit(span);
    P.tpw = (std::max(qt_max, 1) + qgroups - 1) / qgroups;  // tiles per group, balanced
    P.max_qgroups = qgroups;
    P.max_rows_req = max_rows_req;
    return SPEC_OK;
  }
  const int q_groups = (qt_max + 31) / 32;
  const int tpw = (qt_max + q_groups - 1) / q_groups;
  auto wgs_for = [&](int sp) {
    long w = 0;
    for (int r = 0; r < n_req; ++r)
      w += (long)(((rows_per_req[r] * G + 15) / 16 + tpw - 1) / tpw) * nkv *
           ((keys_up(keys_per_req[r]) + sp - 1) / sp);
    return w;
  };
  int split = 128;
  for (int sp : {32, 64, 96, 128}) {
    const int ns = (keys_max + sp - 1) / sp;
    if (ns > split_cap || (size_t)ns * R > c->split_rows) continue;
    if (wgs_for(sp) <= kAttnSlots) {
      split = sp;
      break;
    }
  }
  P.attn_stream = false;
  P.split = split;
  P.max_splits = (keys_max + split - 1) / split;
  P.tpw = tpw;
  P.max_qgroups = (qt_max + tpw - 1) / tpw;
  P.max_rows_req = max_rows_req;
  if (P.max_splits > split_cap || (size_t)P.max_splits * R > c->split_rows)
    return fail(c, SPEC_E_UNSUPPORTED, "context too long for the attention split table");
  return SPEC_OK;
}

std::vector<int64_t> Pass::key(const spec_ctx* c) const {
  return {R, n_req, tree_depth, prefill, lm_row0, lm_rows, (int64_t)(uintptr_t)d_logits,
          split, max_splits, tpw, max_qgroups, max_rows_req, attn_stream, one_part, walk, lowp,
          c->fault_tok,
          (int64_t)__builtin_bit_cast(uint32_t, c->fault_bias), c->fault_after};
}

// Enqueue the kernels of a planned pass on the context's stream.
int launch_pass_impl(spec_ctx* c, const Pass& P) {
  const spec_config& cfg = c->cfg;
  const bool bf = c->bf16;
  hipStream_t s = c->stream;
  const int d = c->d, hd = c->hd, nq = c->nq, nkv = c->nkv, F = c->F;
  const int R = P.R, n_req = P.n_req, max_rows_req = P.max_rows_req;
  const bool prefill = P.prefill;
  hipError_t e = hipSuccess;

  const size_t u_lo = lo_off(c, d);
  HIP_TRY(launch_embed(bf, c->embed, c->d_rows, R, d, c->h, c->layers[0].n1, c->u, u_lo,
                       c->ss, c->cos_t, c->sin_t, hd, c->rope_cs, s));
  const RowNorm norm = row_norm(c);

  AttnArgs aa{};
  aa.q = c->q;
  aa.q_lo = c->q_lo;
  aa.btab = c->d_btab;
  aa.max_pages = c->max_pages;
  aa.rows = c->d_rows;
  aa.reqs = c->d_reqs;
  aa.anc = c->d_anc;
  aa.part_o = c->part_o;
  aa.part_ml = c->part_ml;
  aa.nq = nq;
  aa.nkv = nkv;
  aa.hd = hd;
  aa.split = P.split;
  aa.max_splits = P.max_splits;
  aa.qtiles_per_wg = P.tpw;
  aa.one_part = P.one_part ? 1 : 0;
  aa.stream = P.attn_stream ? 1 : 0;
  aa.out = c->attn_o;
  aa.out_lo = lo_off(c, nq * hd);
  aa.max_qgroups = P.max_qgroups;
  aa.n_req = n_req;
  aa.rows_total = R;
  aa.scale = 1.0f / std::sqrt((float)hd);

  for (int li = 0; li < cfg.n_layers; ++li) {
    const Layer& L = c->layers[li];
    // the norm applied after this layer's down GEMM: the next layer's input
    // norm, or the final norm in front of the LM head
    const float* next_norm = li + 1 < cfg.n_layers ? c->layers[li + 1].n1 : c->final_norm;
    if (L.kind == SPEC_LAYER_ATTN) {
      GemmArgs g = gemm_args(c, L.wqkv, c->u, d, R, d, c->qkv_n);
      const int S = gemm_part(c, g, &e);
      HIP_TRY(e);
      char* kc = c->kpool + (size_t)L.idx * c->kv_layer_elems * c->esz;
      char* vc = c->vpool + (size_t)L.idx * c->kv_layer_elems * c->esz;
      const int ld = g.ntiles * 16;
      HIP_TRY(launch_rope_kv(bf, c->P, S, (size_t)c->Rmax * ld, c->d_rows, R, nq, nkv, hd,
                             c->rope_cs, c->q, c->q_lo, kc, vc, ld, norm, s));
      aa.kc = kc;
      aa.vc = vc;
      const TimePair ta = time_pair(c, 4);
      HIP_TRY(launch_attention(bf, aa, s, ta.t0, ta.t1));
      if (!(P.attn_stream && P.max_splits == 1))  // else written by the attention itself
        HIP_TRY(launch_attn_combine(bf, aa, c->attn_o, lo_off(c, nq * hd), s));
      GemmArgs o = gemm_args(c, L.wo, c->attn_o, nq * hd, R, nq * hd, d);
      const int So = gemm_part(c, o, &e);
      HIP_TRY(e);
      const int ldo = o.ntiles * 16;
      HIP_TRY(launch_resid_reduce(bf, c->P, So, (size_t)c->Rmax * ldo, ldo, R, d, c->h,
                                  L.n2, c->u, u_lo, c->ss, s));
    } else {
      GemmArgs g = gemm_args(c, L.win, c->u, d, R, d, c->in_n);
      const int S = gemm_part(c, g, &e);
      HIP_TRY(e);
      const int ld = g.ntiles * 16;
      float* H = c->H + (size_t)L.idx * c->H_layer;
      float* save = prefill ? nullptr : c->lrsave + (size_t)L.idx * c->lrsave_layer;
      HIP_TRY(launch_lr_fork(bf, c->P, S, (size_t)c->Rmax * ld, ld, c->d_rows, c->d_reqs,
                             n_req, d, c->S, H, c->lr_o, lo_off(c, d), save, P.tree_depth,
                             prefill, max_rows_req, norm, s));
      GemmArgs o = gemm_args(c, L.wout, c->lr_o, d, R, d, d);
      const int So = gemm_part(c, o, &e);
      HIP_TRY(e);
      const int ldo = o.ntiles * 16;
      HIP_TRY(launch_resid_reduce(bf, c->P, So, (size_t)c->Rmax * ldo, ldo, R, d, c->h,
                                  L.n2, c->u, u_lo, c->ss, s));
    }
    GemmArgs gu = gemm_args(c, L.wgu, c->u, d, R, d, 2 * F);
    gu.Y = c->act;
    gu.ldy = F;
    gu.ylo = (int64_t)lo_off(c, F);
    gu.norm = norm;
    const TimePair tg = time_pair(c, 1);
    HIP_TRY(launch_gemm(bf, EPI_SWIGLU, gu, s, tg.t0, tg.t1));
    GemmArgs dn = gemm_args(c, L.wd, c->act, F, R, F, d);
    const int Sd = gemm_part(c, dn, &e, time_pair(c, 2));
    HIP_TRY(e);
    const int ldd = dn.ntiles * 16;
    HIP_TRY(launch_resid_reduce(bf, c->P, Sd, (size_t)c->Rmax * ldd, ldd, R, d, c->h,
                                next_norm, c->u, u_lo, c->ss, s));
  }

  // final norm + LM head + argmax over rows [lm_row0, lm_row0 + lm_rows)
  if (P.lm_rows > 0) {
    GemmArgs lm = gemm_args(c, c->lm_head,
                            (const char*)c->u + (size_t)P.lm_row0 * d * c->esz, d, P.lm_rows,
                            d, c->V);
    lm.part = c->am_part;
    lm.nblocks = gemm_argmax_blocks(c->bf16, lm.ntiles * 16, P.lm_rows);
    lm.logits = P.d_logits;
    lm.ldlog = c->V;
    lm.rows = c->d_rows + P.lm_row0;
    lm.bias_tok = c->fault_tok;
    lm.bias = c->fault_bias;
    lm.bias_after = c->fault_after;
    lm.norm = row_norm(c, P.lm_row0);
    const TimePair tl = time_pair(c, 3);
    HIP_TRY(launch_gemm(bf, EPI_ARGMAX, lm, s, tl.t0, tl.t1));
    HIP_TRY(launch_argmax_reduce(c->am_part, P.lm_rows, lm.nblocks, c->amax, s));
  }
  if (P.walk)
    HIP_TRY(launch_path_walk(c->d_rows, c->d_reqs, n_req, c->amax, kMaxPath, c->res, s));
  return SPEC_OK;
}

int launch_pass(spec_ctx* c, const Pass& P) {
  c->cur_lowp = P.lowp;  // read by gemm_args while the pass is enqueued
  const int rc = launch_pass_impl(c, P);
  c->cur_lowp = false;
  return rc;
}

// Run a planned pass: replay a captured graph of its kernels when one with
// the same launch parameters exists (capturing it on first use), else
// launch eagerly.  Graphs are off while kernel timing is enabled.
int run_pass(spec_ctx* c, const Pass& P) {
  if (!c->use_graphs || c->timing_cls != 0) return launch_pass(c, P);
  const std::vector<int64_t> key = P.key(c);
  GraphEntry* hit = nullptr;
  for (auto& g : c->graphs)
    if (g.key == key) hit = &g;
  if (!hit) {
    hipGraph_t graph = nullptr;
    HIP_TRY(hipStreamBeginCapture(c->stream, hipStreamCaptureModeRelaxed));
    const int rc = launch_pass(c, P);
    const hipError_t ee = hipStreamEndCapture(c->stream, &graph);
    if (rc) {
      if (graph) (void)hipGraphDestroy(graph);
      return rc;
    }
    HIP_TRY(ee);
    hipGraphExec_t exec = nullptr;
    const hipError_t ie = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
    (void)hipGraphDestroy(graph);
    HIP_TRY(ie);
    if (c->graphs.size() >= kMaxGraphs) {  // drop the least recently used
      auto lru = std::min_element(c->graphs.begin(), c->graphs.end(),
                                  [](const GraphEntry& a, const GraphEntry& b) {
                                    return a.used < b.used;
                                  });
      (void)hipGraphExecDestroy(lru->exec);
      c->graphs.erase(lru);
    }
    c->graphs.push_back(GraphEntry{key, exec, 0});
    hit = &c->graphs.back();
  }
  hit->used = ++c->graph_tick;
  HIP_TRY(hipGraphLaunch(hit->exec, c->stream));
  return SPEC_OK;
}

int forward(spec_ctx* c, int R, int n_req, const std::vector<int>& keys_per_req,
            const std::vector<int>& rows_per_req, int tree_depth, int lm_row0, int lm_rows,
            float* d_logits, bool prefill, bool walk, bool lowp = false) {
  Pass P;
  const int rc = plan_pass(c, P, R, n_req, keys_per_req, rows_per_req, tree_depth, lm_row0,
                           lm_rows, d_logits, prefill);
  if (rc) return rc;
  P.walk = walk;
  P.lowp = lowp;
  // prefill chunks run eagerly (their shapes vary); verify passes replay graphs
  return prefill ? launch_pass(c, P) : run_pass(c, P);
}

RowMeta* h_rows(spec_ctx* c) { return (RowMeta*)c->h_meta; }
ReqMeta* h_reqs(spec_ctx* c) { return (ReqMeta*)(c->h_meta + c->off_reqs); }
uint64_t* h_anc(spec_ctx* c) { return (uint64_t*)(c->h_meta + c->off_anc); }

int slot_of(const spec_ctx* c, const Req& rq, int t) {
  return rq.pages[t >> 4] * 16 + (t & 15);
}

// Pages a request still needs to hold tokens [0, tokens).
int pages_needed(const Req& rq, int tokens) {
  return std::max(0, (tokens + 15) / 16 - (int)rq.pages.size());
}

// Give request `req` `count` more pages from the pool (the caller checked
// that it has them): the free list's last entries, so a request that grows
// alone takes ascending pages; page0 stays valid while its pages are
// consecutive.  The new block-table entries go to the device through the
// pinned mirror (an entry is written once per grant, before any pass reads
// it).
int take_pages(spec_ctx* c, int req, int count) {
  if (count <= 0) return SPEC_OK;
  Req& rq = c->reqs[req];
  const int first = (int)rq.pages.size();
  int32_t* row = c->h_btab + (size_t)req * c->max_pages;
  for (int i = 0; i < count; ++i) {
    const int p = c->free_pages.back();
    c->free_pages.pop_back();
    if (rq.pages.empty()) rq.page0 = p;
    else if (rq.page0 >= 0 && p != rq.page0 + (int)rq.pages.size()) rq.page0 = -1;
    rq.pages.push_back(p);
    row[first + i] = p;
  }
  if (hipMemcpyAsync(c->d_btab + (size_t)req * c->max_pages + first, row + first,
                     (size_t)count * 4, hipMemcpyHostToDevice, c->stream) != hipSuccess)
    return fail(c, SPEC_E_HIP, "block table upload failed");
  return SPEC_OK;
}

// A request's pages back to the pool, last first, so that the next request
// to grow takes them in ascending order again.
void give_back_pages(spec_ctx* c, Req& rq) {
  for (auto it = rq.pages.rbegin(); it != rq.pages.rend(); ++it) c->free_pages.push_back(*it);
  rq.pages.clear();
  rq.page0 = -1;
}

}  // namespace

// ====================================================================== ABI

extern "C" size_t spec_workspace_bytes(const spec_config* cfg) {
  if (!valid_config(cfg, nullptr)) return 0;
  return plan_workspace(nullptr, *cfg, nullptr);
}

extern "C" int32_t spec_create(const spec_config* cfg, void* d_workspace,
                               size_t bytes, void* hip_stream, spec_ctx** out) {
  if (!out) return SPEC_E_INVAL;
  *out = nullptr;
  std::string why;
  if (!valid_config(cfg, &why)) return SPEC_E_INVAL;
  const size_t need = plan_workspace(nullptr, *cfg, nullptr);
  if (!d_workspace || bytes < need || ((uintptr_t)d_workspace % kAlign))
    return SPEC_E_INVAL;
  spec_ctx* c = new spec_ctx();
  c->cfg = *cfg;
  c->bf16 = cfg->dtype == SPEC_DTYPE_BF16;
  c->esz = c->bf16 ? 2 : 4;
  c->stream = (hipStream_t)hip_stream;
  c->use_graphs = hip_stream != nullptr;  // the null stream cannot be captured
  c->ws = (char*)d_workspace;
  c->d = cfg->d_model;
  c->nq = cfg->n_heads;
  c->nkv = cfg->n_kv_heads;
  c->hd = cfg->head_dim;
  c->F = cfg->ffn_dim;
  c->V = cfg->vocab;
  c->S = cfg->lr_state;
  for (int i = 0; i < cfg->n_layers; ++i)
    (cfg->layer_kind[i] == SPEC_LAYER_LR ? c->n_lr : c->n_attn)++;
  c->qkv_n = (c->nq + 2 * c->nkv) * c->hd;
  c->in_n = 3 * c->d + 2 * c->S;
  (void)hipGetDevice(&c->device);
  plan_workspace(c, *cfg, c->ws);
  build_slots(c);
  c->reqs.resize(cfg->max_requests);
  for (int p = c->n_pages - 1; p >= 0; --p) c->free_pages.push_back(p);

  auto cleanup = [&](int code) {
    spec_destroy(c);
    return code;
  };
  if (hipHostMalloc((void**)&c->h_meta, c->meta_bytes, hipHostMallocDefault) != hipSuccess ||
      hipHostMalloc((void**)&c->h_commit, sizeof(CommitReq) * cfg->max_requests,
                    hipHostMallocDefault) != hipSuccess ||
      hipHostMalloc((void**)&c->h_res, sizeof(int32_t) * cfg->max_requests * (2 + kMaxPath),
                    hipHostMallocDefault) != hipSuccess ||
      hipHostMalloc((void**)&c->h_btab, sizeof(int32_t) * cfg->max_requests * c->max_pages,
                    hipHostMallocDefault) != hipSuccess)
    return cleanup(SPEC_E_HIP);
  memset(c->h_meta, 0, c->meta_bytes);

  // RoPE tables: angle = p * theta^(-2i/hd) in double, rounded once to float
  const int half = c->hd / 2;
  std::vector<float> ct((size_t)c->max_pos * half), st((size_t)c->max_pos * half);
  for (int i = 0; i < half; ++i) {
    const double inv = std::pow((double)cfg->rope_theta, -2.0 * i / c->hd);
    for (int p = 0; p < c->max_pos; ++p) {
      ct[(size_t)p * half + i] = (float)std::cos((double)p * inv);
      st[(size_t)p * half + i] = (float)std::sin((double)p * inv);
    }
  }
  if (hipMemcpy(c->cos_t, ct.data(), ct.size() * 4, hipMemcpyHostToDevice) != hipSuccess ||
      hipMemcpy(c->sin_t, st.data(), st.size() * 4, hipMemcpyHostToDevice) != hipSuccess ||
      hipMemsetAsync(c->d_btab, 0, (size_t)cfg->max_requests * c->max_pages * 4,
                     c->stream) != hipSuccess ||
      hipMemsetAsync(c->ws, 0, c->weights_end, c->stream) != hipSuccess ||
      (c->w12_side_bytes &&
       hipMemsetAsync(c->ws + c->w12_side0, 0, c->w12_side_bytes, c->stream) != hipSuccess) ||
      (c->n_lr && hipMemsetAsync(c->H, 0, c->H_layer * 4 * c->n_lr, c->stream) != hipSuccess) ||
      hipStreamSynchronize(c->stream) != hipSuccess)
    return cleanup(SPEC_E_HIP);
  *out = c;
  return SPEC_OK;
}

extern "C" int32_t spec_load_weights(spec_ctx* c, int32_t tensor_id,
                                     const void* src, size_t bytes,
                                     int32_t src_on_device) {
  int rc = check(c);
  if (rc) return rc;
  if (tensor_id < 0 || tensor_id >= (int)c->slots.size() || !src)
    return fail(c, SPEC_E_INVAL, "bad tensor id %d", tensor_id);
  const TensorSlot& t = c->slots[tensor_id];
  const size_t want = (size_t)t.rows * t.cols * c->esz;
  if (bytes != want)
    return fail(c, SPEC_E_INVAL, "tensor %d: %zu bytes given, %zu expected", tensor_id,
                bytes, want);
  hipStream_t s = c->stream;
  const hipMemcpyKind kind = src_on_device ? hipMemcpyDeviceToDevice : hipMemcpyHostToDevice;
  if (t.kind == 0) {  // embedding, row-major as given
    HIP_TRY(hipMemcpyAsync(t.dst, src, bytes, kind, s));
  } else if (t.kind == 1) {  // norm vector -> fp32
    const void* from = src;
    if (!src_on_device) {
      HIP_TRY(hipMemcpyAsync(c->staging, src, bytes, kind, s));
      from = c->staging;
    }
    HIP_TRY(launch_to_f32(c->bf16, from, t.rows, (float*)t.dst, s));
  } else {  // matrix -> tiles (bf16 / fp32, or W12)
    if (t.rows % 16 || t.cols % 32)
      return fail(c, SPEC_E_UNSUPPORTED, "tensor %d shape %dx%d not tileable", tensor_id,
                  t.rows, t.cols);
    const size_t row_bytes = (size_t)t.cols * c->esz;
    int slab = src_on_device ? t.rows : (int)((size_t)kStagingBytes / row_bytes) / 16 * 16;
    if (slab <= 0)
      return fail(c, SPEC_E_UNSUPPORTED, "tensor %d rows too long for staging", tensor_id);
    const WMat& m = *t.mat;
    // the matrix's overflow flag reports this tensor's tiles only
    if (c->w12) HIP_TRY(hipMemsetAsync(m.err, 0, sizeof(int), s));
    for (int r0 = 0; r0 < t.rows; r0 += slab) {
      const int nr = std::min(slab, t.rows - r0);
      const char* from = (const char*)src + (size_t)r0 * row_bytes;
      if (!src_on_device) {
        HIP_TRY(hipMemcpyAsync(c->staging, from, (size_t)nr * row_bytes, kind, s));
        from = (const char*)c->staging;
      }
      const int tile0 = t.tile0 + (r0 / 16) * t.tile_stride;
      if (c->w12) {
        HIP_TRY(launch_w12_rowexp(from, nr, t.cols, c->eb_tmp, s));
        HIP_TRY(launch_w12_encode(from, nr, t.cols, c->eb_tmp, m.eb, t.dst,
                                  (size_t)(m.n / 16) * (m.k / 32), m.p8, tile0,
                                  t.tile_stride, t.wsn, t.wsk, m.err, s));
      } else {
        HIP_TRY(launch_relayout(c->bf16, from, nr, t.cols, t.dst, tile0, t.tile_stride,
                                t.wsn, t.wsk, s));
      }
      if (!src_on_device) HIP_TRY(hipStreamSynchronize(s));
    }
    if (c->w12) {
      int err = 0;
      HIP_TRY(hipMemcpyAsync(&err, m.err, sizeof(int), hipMemcpyDeviceToHost, s));
      HIP_TRY(hipStreamSynchronize(s));
      if (err)
        return fail(c, SPEC_E_UNSUPPORTED,
                    "tensor %d: a tile has more than %d weights outside the W12 exponent "
                    "windows; load these weights in native format", tensor_id, kW12MaxExc);
    }
  }
  HIP_TRY(hipStreamSynchronize(s));
  c->loaded[tensor_id] = 1;
  return SPEC_OK;
}

extern "C" int32_t spec_prefill(spec_ctx* c, int32_t req, const int32_t* prompt,
                                int32_t n, int32_t* first_token, float* d_logits_opt) {
  int rc = check(c);
  if (rc) return rc;
  const spec_config& cfg = c->cfg;
  if (!all_loaded(c)) return fail(c, SPEC_E_STATE, "weights not loaded");
  if (req < 0 || req >= cfg.max_requests) return fail(c, SPEC_E_INVAL, "bad request id");
  if (c->reqs[req].active) return fail(c, SPEC_E_STATE, "request %d is active", req);
  if (!prompt || n < 1 || !first_token) return fail(c, SPEC_E_INVAL, "bad prompt");
  if (n + cfg.max_nodes > cfg.max_ctx)
    return fail(c, SPEC_E_CAPACITY, "prompt of %d tokens exceeds max_ctx", n);
  for (int i = 0; i < n; ++i)
    if (prompt[i] < 0 || prompt[i] >= c->V) return fail(c, SPEC_E_INVAL, "token out of range");
  Req& rq = c->reqs[req];
  // the prompt's pages (later passes take more as the context grows)
  const int need = pages_needed(rq, n);
  if ((int)c->free_pages.size() < need) return fail(c, SPEC_E_CAPACITY, "KV pages exhausted");
  auto undo = [&](int code) {
    give_back_pages(c, rq);
    return code;
  };
  rc = take_pages(c, req, need);
  if (rc) return undo(rc);
  // zero recurrent states of this request
  for (int l = 0; l < c->n_lr; ++l)
    if (hipMemsetAsync(c->H + l * c->H_layer + (size_t)req * c->d * c->S, 0,
                       (size_t)c->d * c->S * 4, c->stream) != hipSuccess)
      return undo(fail(c, SPEC_E_HIP, "state reset failed"));

  int done = 0;
  while (done < n) {
    const int C = std::min(cfg.prefill_chunk, n - done);
    // the previous upload from the pinned metadata buffer must have run
    // before the buffer is rewritten
    if (hipStreamSynchronize(c->stream) != hipSuccess) {
      c->poisoned = true;
      return undo(fail(c, SPEC_E_HIP, "stream synchronize failed"));
    }
    RowMeta* rows = h_rows(c);
    for (int i = 0; i < C; ++i) {
      RowMeta& r = rows[i];
      r.token = prompt[done + i];
      r.pos = done + i;
      r.slot = slot_of(c, rq, done + i);
      r.req = 0;
      r.node = i;
      r.parent = i - 1;
      r.keys = done + C;
      r.order = i;
    }
    ReqMeta& m = h_reqs(c)[0];
    m = ReqMeta{0, C, done, req, 0, 1, 1, c->table_only ? -1 : rq.page0};
    if (hipMemcpyAsync(c->d_meta, c->h_meta, c->meta_bytes, hipMemcpyHostToDevice,
                       c->stream) != hipSuccess) {
      c->poisoned = true;
      return undo(fail(c, SPEC_E_HIP, "metadata upload failed"));
    }
    const bool last = done + C == n;
    rc = forward(c, C, 1, {done + C}, {C}, 0, C - 1, last ? 1 : 0,
                 last ? d_logits_opt : nullptr, true, false);
    if (rc) return undo(rc);
    done += C;
  }
  if (hipMemcpyAsync(c->h_res, c->amax, 4, hipMemcpyDeviceToHost, c->stream) != hipSuccess ||
      hipStreamSynchronize(c->stream) != hipSuccess) {
    c->poisoned = true;
    return undo(fail(c, SPEC_E_HIP, "prefill result copy failed"));
  }
  rq.active = true;
  rq.n = n;
  rq.root = c->h_res[0];
  *first_token = rq.root;
  c->last.valid = false;
  return SPEC_OK;
}

namespace {

int verify_impl(spec_ctx* c, int32_t n_req, const int32_t* req, const int32_t* n_nodes,
                const int32_t* draft_tokens, const int32_t* parent_idx, int32_t* path,
                int32_t* path_len, int32_t* bonus, float* d_logits_opt, bool lowp) {
  int rc = check(c);
  if (rc) return rc;
  if (lowp && !c->w8)
    return fail(c, SPEC_E_UNSUPPORTED, "no 8-bit weight view (load with W12_LOWP)");
  const spec_config& cfg = c->cfg;
  if (n_req < 1 || n_req > cfg.max_requests || !req || !n_nodes || !path || !path_len ||
      !bonus)
    return fail(c, SPEC_E_INVAL, "bad arguments");
  std::vector<char> seen(cfg.max_requests, 0);
  int R = 0, total_drafts = 0;
  for (int r = 0; r < n_req; ++r) {
    if (req[r] < 0 || req[r] >= cfg.max_requests) return fail(c, SPEC_E_INVAL, "bad request id");
    if (seen[req[r]]) return fail(c, SPEC_E_INVAL, "request %d repeated", req[r]);
    seen[req[r]] = 1;
    if (!c->reqs[req[r]].active) return fail(c, SPEC_E_STATE, "request %d not active", req[r]);
    if (n_nodes[r] < 0 || n_nodes[r] + 1 > cfg.max_nodes)
      return fail(c, SPEC_E_INVAL, "request %d: %d drafts exceed max_nodes", req[r], n_nodes[r]);
    if (c->reqs[req[r]].n + n_nodes[r] + 1 > cfg.max_ctx)
      return fail(c, SPEC_E_CAPACITY, "request %d: context full", req[r]);
    R += n_nodes[r] + 1;
    total_drafts += n_nodes[r];
  }
  if (R > cfg.max_rows) return fail(c, SPEC_E_INVAL, "%d rows exceed max_rows", R);
  if (total_drafts && (!draft_tokens || !parent_idx))
    return fail(c, SPEC_E_INVAL, "missing drafts");
  for (int i = 0, off = 0; i < n_req; off += n_nodes[i], ++i)
    for (int j = 0; j < n_nodes[i]; ++j) {
      const int p = parent_idx[off + j], t = draft_tokens[off + j];
      if (p < -1 || p >= j) return fail(c, SPEC_E_INVAL, "parent_idx out of range");
      if (t < 0 || t >= c->V) return fail(c, SPEC_E_INVAL, "draft token out of range");
    }

  // pages for every request's new positions (all or none are taken)
  int new_pages = 0;
  for (int r = 0; r < n_req; ++r)
    new_pages += pages_needed(c->reqs[req[r]], c->reqs[req[r]].n + n_nodes[r] + 1);
  if (new_pages > (int)c->free_pages.size())
    return fail(c, SPEC_E_CAPACITY, "KV pages exhausted (%d more needed)", new_pages);
  for (int r = 0; r < n_req; ++r) {
    rc = take_pages(c, req[r], pages_needed(c->reqs[req[r]], c->reqs[req[r]].n + n_nodes[r] + 1));
    if (rc) return rc;
  }

  const int words = (cfg.max_nodes + 63) / 64;
  RowMeta* rows = h_rows(c);
  ReqMeta* rm = h_reqs(c);
  uint64_t* anc = h_anc(c);
  LastVerify lv;
  lv.valid = true;
  std::vector<int> keys(n_req), nrows(n_req);
  bool any_tree = false;
  int max_depth = 0;  // deepest node of the pass (chains included)
  int row = 0, off = 0;
  for (int r = 0; r < n_req; ++r) {
    const Req& rq = c->reqs[req[r]];
    const int K = n_nodes[r];
    std::vector<int> par(K + 1), dep(K + 1), rank(K + 1);
    bool chain = true;
    for (int i = 0; i <= K; ++i) {
      const int p = i == 0 ? -1 : parent_idx[off + i - 1] + 1;
      par[i] = p;
      dep[i] = p < 0 ? 0 : dep[p] + 1;
      if (p != i - 1) chain = false;
    }
    // depth-first (pre-order) walk of the tree, children in index order:
    // the recurrent layers visit the nodes in this order, and a node's KV
    // slot is n + its rank in it, so the first-child chain from the root
    // (in a best-first tree, the most probable branch) has its keys at its
    // own positions, contiguous after the committed ones: its rows see the
    // keys an AR step sees, in the same places, and its commit moves no KV
    {
      std::vector<int> kids_start(K + 2, 0), kids;
      for (int i = 1; i <= K; ++i) ++kids_start[par[i] + 1];
      for (int i = 0; i <= K; ++i) kids_start[i + 1] += kids_start[i];
      kids.assign(K > 0 ? K : 1, 0);
      std::vector<int> fill(kids_start.begin(), kids_start.end() - 1);
      for (int i = 1; i <= K; ++i) kids[fill[par[i]]++] = i;
      std::vector<int> stack{0};
      int k = 0;
      while (!stack.empty()) {
        const int v = stack.back();
        stack.pop_back();
        rank[v] = k;
        rows[row + k++].order = v;
        for (int e = kids_start[v + 1] - 1; e >= kids_start[v]; --e) stack.push_back(kids[e]);
      }
    }
    for (int i = 0; i <= K; ++i) {
      const int p = par[i];
      RowMeta& m = rows[row + i];
      m.token = i == 0 ? rq.root : draft_tokens[off + i - 1];
      m.pos = rq.n + dep[i];
      m.slot = slot_of(c, rq, rq.n + rank[i]);
      m.req = r;
      m.node = i;
      m.parent = p;
      m.keys = rq.n + K + 1;
      // ancestors (and the node itself) by KV slot: bit rank(a)
      uint64_t* a = anc + (size_t)(row + i) * words;
      for (int w = 0; w < words; ++w) a[w] = p < 0 ? 0 : anc[(size_t)(row + p) * words + w];
      a[rank[i] >> 6] |= 1ull << (rank[i] & 63);
    }
    if (!chain) any_tree = true;
    for (int i = 0; i <= K; ++i) max_depth = std::max(max_depth, dep[i]);
    rm[r] = ReqMeta{row, K + 1, rq.n, req[r], row * words, words, chain ? 1 : 0,
                    c->table_only ? -1 : rq.page0};
    // the attention plan (key ranges) from the committed length and the
    // largest tree, so that a pass's key ranges do not depend on its K
    keys[r] = rq.n + cfg.max_nodes;
    nrows[r] = K + 1;
    lv.req.push_back(req[r]);
    lv.row0.push_back(row);
    lv.nrows.push_back(K + 1);
    lv.nctx.push_back(rq.n);
    lv.parent.push_back(par);
    lv.rank.push_back(rank);
    row += K + 1;
    off += K;
  }
  HIP_TRY(hipMemcpyAsync(c->d_meta, c->h_meta, c->meta_bytes, hipMemcpyHostToDevice,
                         c->stream));
  // the recurrent walk of a pass with a tree walks every request as a tree
  // (a chain is a tree); its depth class: a register stack (depths 0..14)
  // unless a node of the pass is deeper (one class per pass keeps the
  // captured graphs few)
  const int depth_class = !any_tree ? 0 : max_depth <= kLrRegisterDepth ? kLrRegisterDepth : 64;
  rc = forward(c, R, n_req, keys, nrows, depth_class, 0, R, d_logits_opt, false, true, lowp);
  if (rc) return rc;
  const int max_path = kMaxPath;
  HIP_TRY(hipMemcpyAsync(c->h_res, c->res, (size_t)n_req * (2 + max_path) * 4,
                         hipMemcpyDeviceToHost, c->stream));
  HIP_TRY(hipStreamSynchronize(c->stream));
  const int slots = cfg.max_nodes - 1;
  for (int r = 0; r < n_req; ++r) {
    const int32_t* o = c->h_res + (size_t)r * (2 + max_path);
    path_len[r] = o[0];
    bonus[r] = o[1];
    for (int k = 0; k < o[0] && k < slots; ++k) path[(size_t)r * slots + k] = o[2 + k] - 1;
  }
  // only an exact verification may be committed
  c->last = lowp ? LastVerify{} : lv;
  return SPEC_OK;
}

}  // namespace

extern "C" int32_t spec_verify(spec_ctx* c, int32_t n_req, const int32_t* req,
                               const int32_t* n_nodes, const int32_t* draft_tokens,
                               const int32_t* parent_idx, int32_t* path,
                               int32_t* path_len, int32_t* bonus, float* d_logits_opt) {
  return verify_impl(c, n_req, req, n_nodes, draft_tokens, parent_idx, path, path_len, bonus,
                     d_logits_opt, false);
}

extern "C" int32_t spec_verify_lowp(spec_ctx* c, int32_t n_req, const int32_t* req,
                                    const int32_t* n_nodes, const int32_t* draft_tokens,
                                    const int32_t* parent_idx, int32_t* path,
                                    int32_t* path_len, int32_t* bonus, float* d_logits_opt) {
  return verify_impl(c, n_req, req, n_nodes, draft_tokens, parent_idx, path, path_len, bonus,
                     d_logits_opt, true);
}

extern "C" int32_t spec_commit(spec_ctx* c, int32_t n_req, const int32_t* req,
                               const int32_t* path, const int32_t* path_len,
                               const int32_t* next_root) {
  int rc = check(c);
  if (rc) return rc;
  const spec_config& cfg = c->cfg;
  if (!c->last.valid) return fail(c, SPEC_E_STATE, "commit without a matching verify");
  if (n_req != (int)c->last.req.size() || !req || !path_len || !next_root ||
      (!path && n_req > 0))
    return fail(c, SPEC_E_STATE, "commit does not match the last verify");
  const int slots = cfg.max_nodes - 1;
  bool need_compact = false;
  for (int r = 0; r < n_req; ++r) {
    if (req[r] != c->last.req[r]) return fail(c, SPEC_E_STATE, "request order differs");
    const std::vector<int>& par = c->last.parent[r];
    const int K = (int)par.size() - 1;
    if (path_len[r] < 0 || path_len[r] > K) return fail(c, SPEC_E_STATE, "bad path length");
    if (next_root[r] < 0 || next_root[r] >= c->V) return fail(c, SPEC_E_INVAL, "bad next root");
    int prev = 0;
    for (int k = 0; k < path_len[r]; ++k) {
      const int node = path[(size_t)r * slots + k] + 1;
      if (node < 1 || node > K || par[node] != prev)
        return fail(c, SPEC_E_STATE, "request %d: path is not a root path", req[r]);
      if (c->last.rank[r][node] != k + 1) need_compact = true;
      prev = node;
    }
  }
  for (int r = 0; r < n_req; ++r) {
    CommitReq& q = c->h_commit[r];
    q.table = req[r];
    q.nctx = c->last.nctx[r];
    q.row0 = c->last.row0[r];
    q.plen = path_len[r];
    for (int k = 0; k < path_len[r]; ++k) {
      q.nodes[k] = path[(size_t)r * slots + k] + 1;
      q.slots[k] = c->last.rank[r][q.nodes[k]];
    }
  }
  if (need_compact || c->n_lr) {
    HIP_TRY(hipMemcpyAsync(c->d_commit, c->h_commit, sizeof(CommitReq) * n_req,
                           hipMemcpyHostToDevice, c->stream));
    if (need_compact && c->n_attn)
      HIP_TRY(launch_kv_compact(c->bf16, c->d_commit, n_req, c->d_btab, c->max_pages,
                                c->kpool, c->vpool, c->kv_layer_elems, c->n_attn,
                                c->nkv, c->hd, c->stream));
    if (c->n_lr)
      HIP_TRY(launch_lr_commit(c->d_commit, n_req, c->lrsave, c->lrsave_layer,
                               2 * c->d + c->S, c->n_lr, c->d, c->S, c->H, c->H_layer,
                               c->stream));
  }
  for (int r = 0; r < n_req; ++r) {
    Req& rq = c->reqs[req[r]];
    rq.n += path_len[r] + 1;
    rq.root = next_root[r];
  }
  c->last.valid = false;
  return SPEC_OK;
}

extern "C" int32_t spec_release(spec_ctx* c, int32_t req) {
  int rc = check(c);
  if (rc) return rc;
  if (req < 0 || req >= c->cfg.max_requests) return fail(c, SPEC_E_INVAL, "bad request id");
  Req& rq = c->reqs[req];
  if (!rq.active) return fail(c, SPEC_E_STATE, "request %d not active", req);
  give_back_pages(c, rq);
  rq = Req();
  c->last.valid = false;
  return SPEC_OK;
}

extern "C" int32_t spec_request_state(const spec_ctx* c, int32_t req, int32_t* n_ctx,
                                      int32_t* pending_root) {
  if (!c || req < 0 || req >= c->cfg.max_requests || !c->reqs[req].active)
    return SPEC_E_INVAL;
  if (n_ctx) *n_ctx = c->reqs[req].n;
  if (pending_root) *pending_root = c->reqs[req].root;
  return SPEC_OK;
}

extern "C" int32_t spec_force_root(spec_ctx* c, int32_t req, int32_t token) {
  int rc = check(c);
  if (rc) return rc;
  if (req < 0 || req >= c->cfg.max_requests || !c->reqs[req].active)
    return fail(c, SPEC_E_INVAL, "request %d not active", req);
  if (token < 0 || token >= c->V) return fail(c, SPEC_E_INVAL, "token out of range");
  c->reqs[req].root = token;
  c->last.valid = false;
  return SPEC_OK;
}

extern "C" int32_t spec_debug_flags(spec_ctx* c, int32_t flags) {
  int rc = check(c);
  if (rc) return rc;
  if ((flags & ~7) || (flags & 6) == 6)
    return fail(c, SPEC_E_INVAL, "unknown debug flags %d", flags);
  c->table_only = (flags & 1) != 0;
  c->attn_mode = (flags & 2) ? 1 : (flags & 4) ? 2 : 0;
  return SPEC_OK;
}

extern "C" int32_t spec_set_fault(spec_ctx* c, int32_t token, float bias,
                                  int32_t after_position) {
  int rc = check(c);
  if (rc) return rc;
  if (token >= c->V) return fail(c, SPEC_E_INVAL, "fault token out of range");
  c->fault_tok = token < 0 ? -1 : token;
  c->fault_bias = bias;
  c->fault_after = after_position;
  return SPEC_OK;
}

extern "C" int32_t spec_use_graphs(spec_ctx* c, int32_t enable) {
  int rc = check(c);
  if (rc) return rc;
  if (enable && !c->stream)
    return fail(c, SPEC_E_UNSUPPORTED, "graphs need a stream other than the null stream");
  c->use_graphs = enable != 0;
  return SPEC_OK;
}

extern "C" int32_t spec_timing_enable(spec_ctx* c, int32_t cls) {
  int rc = check(c);
  if (rc) return rc;
  if (cls < 0 || cls > 4) return fail(c, SPEC_E_INVAL, "bad timing class");
  c->timing_cls = cls;
  return SPEC_OK;
}

extern "C" int32_t spec_timing_read(spec_ctx* c, double* total_ms, int64_t* launches) {
  int rc = check(c);
  if (rc) return rc;
  HIP_TRY(hipStreamSynchronize(c->stream));
  double ms = 0.0;
  for (size_t i = 0; i < c->events_used; ++i) {
    float t = 0.f;
    HIP_TRY(hipEventElapsedTime(&t, c->events[i].first, c->events[i].second));
    ms += t;
  }
  if (total_ms) *total_ms = ms;
  if (launches) *launches = (int64_t)c->events_used;
  c->events_used = 0;
  return SPEC_OK;
}

extern "C" void spec_destroy(spec_ctx* c) {
  if (!c) return;
  if (c->stream) (void)hipStreamSynchronize(c->stream);
  for (auto& g : c->graphs) (void)hipGraphExecDestroy(g.exec);
  c->graphs.clear();
  for (auto& e : c->events) {
    (void)hipEventDestroy(e.first);
    (void)hipEventDestroy(e.second);
  }
  if (c->h_meta) (void)hipHostFree(c->h_meta);
  if (c->h_commit) (void)hipHostFree(c->h_commit);
  if (c->h_res) (void)hipHostFree(c->h_res);
  if (c->h_btab) (void)hipHostFree(c->h_btab);
  delete c;
}

extern "C" const char* spec_last_error(const spec_ctx* c) {
  if (!c) return "null context";
  return c->err.c_str();
}
