// Internal interface between the host runtime (spec_api.cpp) and the gfx950
// kernels.  Not part of the public C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

// One row of a forward pass (a tree node, or a prompt token in prefill).
struct RowMeta {
  int32_t token;
  int32_t pos;     // RoPE position: committed length + depth
  int32_t slot;    // physical KV slot (page * 16 + offset) written by this row
  int32_t req;     // index of its request in this pass's ReqMeta array
  int32_t node;    // node index inside the request (0 = root)
  int32_t parent;  // node-local parent index, -1 for the root
  int32_t keys;    // keys of its request in this pass (committed + pass rows)
  int32_t order;   // the node visited k-th in a depth-first (pre-order) walk of
                   // the request's tree, for the row at node index k
};

// One request of a forward pass.
struct ReqMeta {
  int32_t row0;       // first row of the request in the pass
  int32_t nrows;      // rows (root + drafts)
  int32_t nctx;       // committed tokens: keys [0, nctx) are always visible
  int32_t table;      // request id: row of the block table
  int32_t anc0;       // u64 offset of the request's ancestor masks
  int32_t anc_words;  // u64 words per row
  int32_t chain;      // rows form a chain (parent == node - 1)
  int32_t page0;      // the request's pages are page0, page0 + 1, ... (its
                      // block table needs no lookup), or -1
};

// Tiled weight layout: a matrix [N, K] is stored as 16 x 32 tiles, tile
// (nb, kb) at element offset (nb * wsn + kb * wsk) * 512 (wsn, wsk: the
// matrix's tile strides, N-major or K-major), lane l of the tile holding
// W[nb * 16 + l % 16][kb * 32 + (l / 16) * 8 + e] at l * 8 + e.

// Activations that feed a GEMM are stored once, by the kernel that produces
// them, as "activation planes" of the weight type: for bf16 weights two bf16
// planes hi = bf16(v) and lo = bf16(v - hi) (lo at a fixed element offset
// from hi), so a bf16 MFMA pair sees ~16 mantissa bits of the fp32 value;
// for fp32 weights one fp32 plane.

// RMSNorm is deferred (see row_scale in common.h): the producer of a
// normalised input writes the planes of h * w and the row's chunk sums of
// squares; the consumer of the GEMM output applies the row's scale.
constexpr int kNormChunk = 1024;  // columns per sum-of-squares chunk (one workgroup)
struct RowNorm {
  const float* ss;  // [rows][nc] sums of squares of h, chunk by chunk
  int32_t nc;       // chunks per row: ceil(d / kNormChunk)
  int32_t d;
  float eps;
};

// EPI_PART: fp32 partial sums of split s at P[s][row][col] (any S); the
// consumer adds the S partials in order.  EPI_SWIGLU / EPI_ARGMAX need S = 1.
enum GemmEpi { EPI_PART = 0, EPI_SWIGLU = 2, EPI_ARGMAX = 3 };

struct GemmArgs {
  const void* W;        // tiled weights (bf16 bits or fp32, or W12 tiles), ntiles x 16 rows
  int32_t wsn, wsk;     // tile strides of W between tile rows and between K-steps
  int32_t w12;          // W holds 0: bf16 / fp32 tiles, 1: W12 tiles, 2: tiles of
                        // the 8-bit view (w12.h) ...
  const uint8_t* eb;    // ... with these per-row base exponents [ntiles * 16]
  const void* X;        // activation planes [M, ldx] (hi; lo at X + xlo)
  int32_t ldx;
  int64_t xlo;
  int32_t M, K;         // rows, reduction length
  int32_t ntiles;       // 16-column tiles of W (a multiple of 8)
  int32_t ncols;        // real output columns (<= ntiles * 16)
  int32_t row0;         // first row handled by this launch (set by launch_gemm)
  int32_t ncb;          // workgroups per K split, each a balanced share of the tiles
  int32_t gt;           // tiles per share granule (set by launch_gemm)
  int32_t S;            // K splits (EPI_PART only; see gemm_splits)
  int32_t KR;           // K per split (set by launch_gemm; the last split may be shorter)
  float* P;             // EPI_PART: partials [S][P_ld][ntiles * 16]
  int32_t P_ld;
  void* Y;              // SWIGLU: activation planes [M, ldy] (lo at Y + ylo)
  int32_t ldy;
  int64_t ylo;
  float2* part;         // ARGMAX: per (row, column block) (max, index bits)
  int32_t nblocks;      // ARGMAX: column blocks per row
  float* logits;        // ARGMAX: optional fp32 logits [M, ldlog]
  int32_t ldlog;
  const RowMeta* rows;  // ARGMAX fault injection: row positions
  int32_t bias_tok, bias_after;
  float bias;
  RowNorm norm;         // SWIGLU / ARGMAX: the input rows' deferred RMSNorm
                        // (norm.ss == NULL: none), rows indexed like X
};

// Weight matrices have their output rows padded to a multiple of
// gemm_pad_cols().  gemm_splits: the K split count launch_gemm expects for a
// matrix shape at M rows (EPI_PART); gemm_argmax_blocks: the per-row column
// blocks of the ARGMAX partials at M rows.
int gemm_pad_cols();
int gemm_splits(bool bf16, int K, int N, int M);
int gemm_argmax_blocks(bool bf16, int N, int M);

// A launch's stream and optional timing events: with t0 / t1 set, the
// first kernel of the call records its start in t0 and the last kernel its
// end in t1 (HIP's extended launch timestamps the dispatch itself, as a
// kernel trace does, so event setup and dispatch latency are left out).
struct LaunchCtx {
  hipStream_t s;
  hipEvent_t t0, t1;
};

// Launch the skinny GEMM for rows [0, M): picks the workgroup shape and the
// row-tile count, and splits rows into chunks of 128.  t0 / t1: optional
// timing events (LaunchCtx).
hipError_t launch_gemm(bool bf16, int epi, const GemmArgs& a, hipStream_t s,
                       hipEvent_t t0 = nullptr, hipEvent_t t1 = nullptr);

struct AttnArgs {
  const void* q;            // [rows, nq, hd] (bf16 bits or fp32), after RoPE
  const void* q_lo;         // bf16: low plane of q
  const void* kc;           // K pages of this layer: [page][nkv][16][hd]
  const void* vc;           // V pages of this layer: [page][nkv][hd][16]
  const int32_t* btab;      // block tables [max_requests][max_pages]
  int32_t max_pages;
  const RowMeta* rows;
  const ReqMeta* reqs;
  const uint64_t* anc;      // ancestor masks (self included)
  float* part_o;            // [split][rows * nq][hd]
  float2* part_ml;          // [split][rows * nq] (running max, sum)
  int32_t nq, nkv, hd;
  int32_t split;            // keys per split: a multiple of 32, <= 128; streamed:
                            // keys per workgroup range, a multiple of 64
  int32_t qtiles_per_wg;    // 16-row query tiles per workgroup (a query group)
  int32_t stream;           // 1: each workgroup streams a key range in stages
                            // for a group of at most 8 query tiles
  int32_t one_part;         // streamed: one wave per query tile walks each stage
                            // (else 2 or 4 waves split a tile's keys when the
                            // group has at most 4 tiles)
  void* out;                // streamed with one range per request (max_splits == 1):
  size_t out_lo;            // the normalised output, written as activation planes
                            // o[rows, nq*hd] (lo plane at out + out_lo elements)
                            // instead of partials (no combine)
  int32_t max_splits, max_qgroups, n_req;
  int32_t rows_total;
  float scale;
};

// Most 16-row query tiles per (request, KV head) of a streamed attention
// launch (one per wavefront of its workgroups).
constexpr int kAttnStreamTiles = 8;

hipError_t launch_attention(bool bf16, const AttnArgs& a, hipStream_t s,
                            hipEvent_t t0 = nullptr, hipEvent_t t1 = nullptr);

// Merge the per-split partials into the attention output, written as
// activation planes o[rows, nq*hd] (lo plane at o + o_lo elements).
hipError_t launch_attn_combine(bool bf16, const AttnArgs& a, void* o, size_t o_lo,
                               hipStream_t s);

// h[r] = E[token_r] in fp32, u[r] = h[r] * nw as activation planes (lo
// plane at u + u_lo elements) and ss[r][c] = the sum of h[r]^2 over chunk c
// of kNormChunk columns (the deferred RMSNorm of u); cs[r] = the RoPE
// factors at row r's position ([hd]: cos_t then sin_t rows, hd / 2 each).
hipError_t launch_embed(bool bf16, const void* emb, const RowMeta* rows,
                        int R, int d, float* h, const float* nw, void* u,
                        size_t u_lo, float* ss, const float* cos_t, const float* sin_t,
                        int hd, float* cs, hipStream_t s);

// q -> RoPE -> q_out; k -> RoPE -> K cache; v -> V cache, at each row's slot.
// qkv = the row's norm scale (norm) times the sum of the S GEMM partials
// qkv[s * split_stride + row * ld_qkv + c]; cs: the rows' RoPE factors as
// written by launch_embed.
hipError_t launch_rope_kv(bool bf16, const float* qkv, int S, size_t split_stride,
                          const RowMeta* rows, int R, int nq, int nkv, int hd,
                          const float* cs, void* q_out, void* q_lo, void* kc, void* vc,
                          int ld_qkv, RowNorm norm, hipStream_t s);

// h[r] += sum_s P[s * split_stride + r * ld_p + c] (c < d), then
// u[r] = h[r] * nw as activation planes and ss[r][c] = the sum of h[r]^2
// over chunk c: the residual add of a split GEMM and the input of the next
// GEMM (whose consumer applies the norm scale).  One workgroup per row and
// chunk of kNormChunk columns.
hipError_t launch_resid_reduce(bool bf16, const float* P, int S, size_t split_stride,
                               int ld_p, int R, int d, float* h, const float* nw,
                               void* u, size_t u_lo, float* ss, hipStream_t s);

// Per-row argmax over the column-block partials (lowest index on ties).
hipError_t launch_argmax_reduce(const float2* part, int R, int nblocks,
                                int32_t* amax, hipStream_t s);

// Accepted-path walk per request; writes res[req][2 + max_path]:
// {path_len, bonus, path...}.
hipError_t launch_path_walk(const RowMeta* rows, const ReqMeta* reqs,
                            int n_req, const int32_t* amax, int max_path,
                            int32_t* res, hipStream_t s);

// Gated diagonal recurrence over the pass's nodes for one recurrent layer.
// proj: in_proj output as NS split partials (stride split_stride floats),
// each [R, ld] = [x | a | z | B | C | pad], scaled by the row's norm scale
// (norm) after the partials are summed; H: committed states
// [max_requests][d][S]; o: [R, d] activation planes (lo at o + o_lo).
// save (or NULL): per row [x | a | B] ([R, 2d + S]) for the commit.  With
// commit_last (chain passes only) the state of each request's last row is
// written back to H.  tree_depth: 0 for a pass of chains, else at least the
// deepest node's depth (<= 64) of the pass's trees, which are walked in the
// rows' depth-first order (RowMeta.order) with depth = pos - the request's
// nctx.
// Deepest node depth that the recurrent walk keeps on its register stack
// (16 entries: H_0, then one per depth 0..14; deeper trees recompute each
// node's state along its root path).
constexpr int kLrRegisterDepth = 14;
hipError_t launch_lr_fork(bool bf16, const float* proj, int NS, size_t split_stride,
                          int ld, const RowMeta* rows, const ReqMeta* reqs, int n_req,
                          int d, int S, float* H, void* o, size_t o_lo, float* save,
                          int tree_depth, bool commit_last, int max_rows_per_req,
                          RowNorm norm, hipStream_t s);

struct CommitReq {
  int32_t table;     // request id
  int32_t nctx;      // committed length before the commit
  int32_t row0;      // first row of the request in the verified pass
  int32_t plen;      // accepted drafts
  int32_t nodes[64]; // accepted node indices (root excluded), root-to-leaf
  int32_t slots[64]; // their KV slots past nctx (the nodes' depth-first ranks)
};

// Move the accepted branch's K/V from slot (n + rank) to position
// (n + depth) for every attention layer.
hipError_t launch_kv_compact(bool bf16, const CommitReq* cr, int n_req,
                             const int32_t* btab, int max_pages, void* kbase,
                             void* vbase, size_t layer_stride_elems,
                             int n_attn_layers, int nkv, int hd,
                             hipStream_t s);

// Advance the committed recurrent state along root + accepted nodes (proj_all
// holds the summed in_proj outputs that the verify pass saved per layer).
hipError_t launch_lr_commit(const CommitReq* cr, int n_req,
                            const float* proj_all, size_t proj_layer_stride,
                            int proj_ld, int n_lr, int d, int S, float* H,
                            size_t H_layer_stride, hipStream_t s);

// Copy a row-major [nrows, K] slab into the tiled layout.  Source rows
// [0, nrows) become destination tile rows dst_tile0 + t * tile_stride; tile
// (row tr, K-step kb) of the destination starts at tile index
// tr * wsn + kb * wsk.
hipError_t launch_relayout(bool bf16, const void* src, int nrows, int K,
                           void* dst, int dst_tile0, int tile_stride, int wsn, int wsk,
                           hipStream_t s);

// W12 encoding (w12.h): eb[r] for the rows of a row-major bf16 slab
// [nrows, K]; then the slab's tiles, placed like launch_relayout places
// them (tile index tr * wsn + kb * wsk, 800 bytes each, in a matrix of
// dst_tiles tiles whose overflow blocks follow its tiles), and the rows'
// bases at their destination rows of eb_dst; with dst8, also the 8-bit
// view's tiles (512 bytes) at the same tile indices.  *err becomes nonzero
// if a tile has more exceptions than W12 holds.
hipError_t launch_w12_rowexp(const void* src, int nrows, int K, uint8_t* eb,
                             hipStream_t s);
hipError_t launch_w12_encode(const void* src, int nrows, int K, const uint8_t* eb,
                             uint8_t* eb_dst, void* dst, size_t dst_tiles, void* dst8,
                             int dst_tile0, int tile_stride, int wsn, int wsk, int* err,
                             hipStream_t s);

// Widen a norm vector (bf16 bits or fp32) to fp32.
hipError_t launch_to_f32(bool bf16, const void* src, int n, float* dst,
                         hipStream_t s);
