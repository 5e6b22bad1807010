/*
 * spec.h - C ABI of the MI355X speculative-decoding verification library.
 *
 * The library runs the target model's verification step of lossless greedy
 * speculative decoding on one gfx950 GPU: one forward pass scores a pending
 * root token plus a chain or tree of draft tokens against a paged KV cache,
 * takes the greedy argmax at every node and accepts the longest root path
 * whose tokens equal the target's own choices.  The emitted text is then
 * identical to plain autoregressive greedy decoding ("token forcing";
 * zicq.com article "SpecPilot Uses Agentic Discovery to Push Speculative
 * Decoding to 10.87x", section "Core Idea: Let Agents Discover the
 * Bottlenecks").  Tree verification, including hybrid targets whose recurrent
 * layers recompute their state along each root path, follows the besthub.dev
 * article "SpecPilot: AI Agent Framework Boosts Speculative Decoding 10.87x
 * for Qwen3.8-27B", section "(2) Best-first Tree Verification for Hybrid
 * Architectures".  Only the exact verification may accept tokens or update
 * the target's state (same article, "(3) Two-Level Verification"): this is
 * why verification (spec_verify) and the state update (spec_commit) are
 * separate calls.
 *
 * Conventions for every call:
 *  - All int32_t-returning calls return SPEC_OK (0) or a negative SPEC_E_*
 *    code; spec_last_error() then describes the failure.  On any error the
 *    committed state (KV cache contents below each request's length,
 *    recurrent states, lengths, pending roots) is unchanged.  After
 *    SPEC_E_HIP the context is poisoned: every later call except
 *    spec_last_error/spec_destroy returns SPEC_E_HIP.
 *  - "host" pointers are ordinary CPU memory, read or written before the
 *    call returns.  "device" pointers are GPU memory on the context's device.
 *  - The caller owns the device workspace and the HIP stream.  The library
 *    allocates no device memory of its own; it enqueues all GPU work on the
 *    given stream.  A context is single-stream and not thread-safe.
 */
#ifndef SPEC_H
#define SPEC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  SPEC_OK = 0,
  SPEC_E_INVAL = -1,       /* bad ids, shapes or tree (parent out of range) */
  SPEC_E_STATE = -2,       /* call-order violation or non-root path         */
  SPEC_E_CAPACITY = -3,    /* KV pages or max_ctx exhausted                 */
  SPEC_E_HIP = -4,         /* a HIP runtime error; the context is poisoned  */
  SPEC_E_UNSUPPORTED = -5  /* shape or option the library does not handle  */
};

enum { SPEC_DTYPE_FP32 = 0, SPEC_DTYPE_BF16 = 1 };
/* Weight storage: the weights' own type, or W12 for bf16 models: each
 * weight in 12 bits (sign, 4-bit exponent offset from its output row's
 * base exponent, 7-bit mantissa) plus per-tile lists of the exceptions,
 * restored exactly in registers by the GEMMs, so every result is bitwise
 * the same as with bf16 storage while the weights move in ~0.78x the bytes
 * (besthub.dev article, section "(1) W12: Lossless 12-bit Weight Format"). */
/* SPEC_WEIGHTS_W12_LOWP: W12 plus the 8-bit view of every weight (sign,
 * exponent offset, top 3 mantissa bits; one more byte per weight) that
 * spec_verify_lowp reads (besthub.dev article, section "(3) Two-Level
 * Verification"). */
enum { SPEC_WEIGHTS_NATIVE = 0, SPEC_WEIGHTS_W12 = 1, SPEC_WEIGHTS_W12_LOWP = 2 };
enum { SPEC_LAYER_ATTN = 0, SPEC_LAYER_LR = 1 };

#define SPEC_MAX_LAYERS 128

/*
 * Model shape and capacity.  Dense layers: RMSNorm, GQA attention with
 * rotate-half RoPE, SwiGLU FFN.  Recurrent layers (layer_kind SPEC_LAYER_LR)
 * replace attention with a gated diagonal linear recurrence of state width
 * lr_state per channel: [x|a|z|B|C] = norm(h) W_in^T,
 * H_t = sigmoid(a_t) * H_{t-1} + B_t (x) x_t, y_t = H_t C_t,
 * h += (y_t * silu(z_t)) W_out^T.
 */
typedef struct spec_config {
  /* d_model: a multiple of 32, at most 16384; head_dim: 64 or 128;
     ffn_dim: a multiple of 64; vocab: a multiple of 16 */
  int32_t n_layers, d_model, n_heads, n_kv_heads, head_dim, ffn_dim, vocab;
  int32_t dtype;                       /* SPEC_DTYPE_*: weights and KV cache  */
  int32_t lr_state;                    /* recurrent state width (0: none)     */
  int32_t layer_kind[SPEC_MAX_LAYERS]; /* SPEC_LAYER_* per layer              */
  float rms_eps, rope_theta;
  int32_t max_requests;   /* requests alive at once                          */
  int32_t max_ctx;        /* per request: committed tokens + one tree;
                             at most 8192                                    */
  int32_t max_nodes;      /* per request: rows of one verify (root + K)      */
  int32_t max_rows;       /* rows of one verify over all its requests        */
  int32_t prefill_chunk;  /* prompt rows per prefill pass                    */
  int32_t page_size;      /* tokens per KV page; must be 16                  */
  int32_t weight_format;  /* SPEC_WEIGHTS_*; W12 (_LOWP) need SPEC_DTYPE_BF16 */
  int32_t kv_pages;       /* KV pages in the pool, shared by all requests and
                             taken as their contexts grow (prefill: the
                             prompt's; verify: the pass's new positions);
                             0: max_requests * ceil(max_ctx / 16), enough
                             for every request at max_ctx                   */
} spec_config;

typedef struct spec_ctx spec_ctx;

/* Device bytes the caller must provide to spec_create for this config:
 * weights in the library's tiled layout, the KV page pool (kv_pages pages
 * of 16 tokens), recurrent states and scratch.  0 if cfg is invalid. */
size_t spec_workspace_bytes(const spec_config* cfg);

/* Create a context on the current HIP device.  d_workspace: device buffer of
 * at least spec_workspace_bytes(cfg) bytes, 256-byte aligned, owned by the
 * caller and used exclusively by the context until spec_destroy.
 * hip_stream: a hipStream_t (NULL = default stream).  *out receives the
 * context (NULL on failure). */
int32_t spec_create(const spec_config* cfg, void* d_workspace, size_t bytes,
                    void* hip_stream, spec_ctx** out);

/* Load one weight tensor.  tensor_id follows this order: embedding [V, d];
 * per layer, attention layers: attn_norm [d], Wq [nq*hd, d], Wk [nkv*hd, d],
 * Wv [nkv*hd, d], Wo [d, nq*hd], ffn_norm [d], Wg [F, d], Wu [F, d],
 * Wd [d, F]; recurrent layers: attn_norm [d], W_in [3d+2S, d], W_out [d, d],
 * ffn_norm [d], Wg, Wu, Wd; then final_norm [d], lm_head [V, d].
 * src: row-major [out, in] in the config's dtype (fp32, or bf16 bit
 * patterns), `bytes` long, on the host (src_on_device = 0) or the device
 * (src_on_device = 1).  src is only borrowed for the call; the library
 * re-lays the tensor out once into its own tiled layout.  The call is
 * synchronous.  Errors: SPEC_E_INVAL for a bad id or size;
 * SPEC_E_UNSUPPORTED with W12 storage when a 16 x 32 tile of the tensor
 * holds more than 63 weights outside its rows' exponent windows (the
 * tensor may be loaded again, e.g. after a change of weights; such a model
 * loads in native storage). */
int32_t spec_load_weights(spec_ctx* ctx, int32_t tensor_id, const void* src,
                          size_t bytes, int32_t src_on_device);

/* Start request `req` (0 <= req < max_requests, not active) with the host
 * prompt[n] (1 <= n, n + max_nodes <= max_ctx).  Writes the prompt's KV,
 * runs the recurrent layers over it from a zero state, and returns in
 * *first_token (host) the greedy argmax of the last prompt row, which becomes
 * the request's pending root.  d_logits_opt: NULL or device float[vocab]
 * receiving that row's logits.  Synchronous.  Errors: SPEC_E_STATE if any
 * weight is missing or req is active, SPEC_E_INVAL, SPEC_E_CAPACITY. */
int32_t spec_prefill(spec_ctx* ctx, int32_t req, const int32_t* prompt,
                     int32_t n, int32_t* first_token, float* d_logits_opt);

/* Verify one draft tree per request, all in one forward pass.
 * host arrays: req[n_req] (distinct active requests); n_nodes[n_req] draft
 * counts K_r >= 0 with K_r + 1 <= max_nodes and sum(K_r + 1) <= max_rows;
 * draft_tokens and parent_idx concatenated per request (sum K_r entries):
 * parent_idx[i] in [-1, i-1] within its request, -1 meaning the pending
 * root, so every parent precedes its children.  A draft node at depth j
 * (the root has depth 0) is placed at position n_r + j.
 * Outputs (host): path, concatenated per request with max_nodes - 1 slots
 * each, holding the accepted draft indices in root-to-leaf order;
 * path_len[n_req]; bonus[n_req], the target's greedy token after the
 * accepted path.  d_logits_opt: NULL or device float[sum(K_r+1), vocab],
 * each request's rows being its root then its drafts in order.
 * The committed state is not modified.  Returns after the single
 * device-to-host copy of the results.
 * Row-count invariance: with one request and at most 128 rows, the rows of
 * the root and of the first-child chain from it (children in index order:
 * a best-first tree's first branch) get logits (hence argmaxes)
 * bit-identical to those of a pass with K_r = 0 at that row's position and
 * prefix (an AR step), as long as the committed length plus max_nodes
 * stays within one 256-key bucket; other rows, and larger or multi-request
 * passes, agree with AR steps to rounding only. */
int32_t spec_verify(spec_ctx* ctx, int32_t n_req, const int32_t* req,
                    const int32_t* n_nodes, const int32_t* draft_tokens,
                    const int32_t* parent_idx, int32_t* path,
                    int32_t* path_len, int32_t* bonus, float* d_logits_opt);

/* The low-precision first round of two-level verification (besthub.dev,
 * "SpecPilot: AI Agent Framework Boosts Speculative Decoding 10.87x for
 * Qwen3.8-27B", section "(3) Two-Level Verification"): the same pass and
 * arguments as spec_verify, with every weight read through its 8-bit view
 * (weights with mantissas truncated to 3 bits), returning that model's
 * greedy path and bonus token as a candidate chain.  It accepts nothing:
 * the committed state is not modified and a following spec_commit is
 * refused (SPEC_E_STATE) until an exact spec_verify has run.  Needs weights
 * loaded with SPEC_WEIGHTS_W12_LOWP (else SPEC_E_UNSUPPORTED). */
int32_t spec_verify_lowp(spec_ctx* ctx, int32_t n_req, const int32_t* req,
                         const int32_t* n_nodes, const int32_t* draft_tokens,
                         const int32_t* parent_idx, int32_t* path, int32_t* path_len,
                         int32_t* bonus, float* d_logits_opt);

/* Commit after a spec_verify of the same requests (same order).  host
 * arrays: path concatenated with max_nodes - 1 slots per request as returned
 * by spec_verify; path_len[n_req]: any prefix of a root path of the verified
 * tree may be committed; next_root[n_req] in [0, vocab) becomes the pending
 * root (normally the bonus token; any token may be forced).  The root and
 * the path's drafts are appended to the context, the KV of the accepted
 * branch is moved to its final positions and the recurrent state advances
 * along the path.  Asynchronous (stream-ordered).  Errors: SPEC_E_STATE if
 * there is no matching verify or the path is not a root path. */
int32_t spec_commit(spec_ctx* ctx, int32_t n_req, const int32_t* req,
                    const int32_t* path, const int32_t* path_len,
                    const int32_t* next_root);

/* End request `req` and free its KV pages. */
int32_t spec_release(spec_ctx* ctx, int32_t req);

/* Committed length and pending root of an active request. */
int32_t spec_request_state(const spec_ctx* ctx, int32_t req, int32_t* n_ctx,
                           int32_t* pending_root);

/* Token forcing: replace the pending root of an active request (for
 * example with a reference token where the target's own choice was a
 * near-tie).  Invalidates a pending verify of that request.  Host-only. */
int32_t spec_force_root(spec_ctx* ctx, int32_t req, int32_t token);

/* Test hooks: flags bit 0 makes attention look every KV page up in the
 * block table even where a request's pages are consecutive (where it
 * otherwise computes the page from the first one).  Verify passes stream
 * attention (each workgroup walks a range of keys in stages for a group of
 * at most 8 query tiles of 16 query rows); bit 1 makes the ranges two per
 * request, KV head and query group, so that each spans several stages;
 * bit 2 never streams (every pass stages one key split per workgroup).
 * Bits 1 and 2 together, or other bits: SPEC_E_INVAL.  Results agree within
 * rounding either way (the key ranges, and so the order of the softmax
 * sums, differ). */
int32_t spec_debug_flags(spec_ctx* ctx, int32_t flags);

/* Fault injection for checking the token-forcing harness: adds `bias` to
 * the logit of `token` at every row whose position is >= after_position
 * (an analogue of the logit-bias fault of the besthub.dev article, "Phase 4:
 * Final Validation").  token < 0 disables it (the default). */
int32_t spec_set_fault(spec_ctx* ctx, int32_t token, float bias,
                       int32_t after_position);

/* Verify passes replay a captured HIP graph of their kernel sequence when a
 * pass with the same launch parameters (rows, requests, tree or chain,
 * attention split shape, logits buffer, fault setting) ran before; the
 * first such pass captures it (up to 8 are kept per context, least recently
 * used dropped).  Results are identical either way.  enable = 0 launches
 * every kernel individually.  The default is 1 unless the context was
 * created on the null stream (which cannot be captured; enabling graphs
 * there returns SPEC_E_UNSUPPORTED).  Kernel timing (below) also launches
 * individually while enabled.  Host-only. */
int32_t spec_use_graphs(spec_ctx* ctx, int32_t enable);

/* Per-launch timing of one kernel class, for roofline measurement: while
 * enabled, every launch of that class records the kernel's own start and
 * end in a pair of HIP events on the library's stream (HIP's extended
 * launch, which timestamps the dispatch as a kernel trace does; passes then
 * run without graph replay).  cls: 0 = off, 1 = FFN gate/up GEMM, 2 = FFN
 * down GEMM, 3 = LM head GEMM, 4 = attention.  spec_timing_read
 * synchronizes the stream, returns the summed milliseconds and launch
 * count since the last read, and resets them. */
int32_t spec_timing_enable(spec_ctx* ctx, int32_t cls);
int32_t spec_timing_read(spec_ctx* ctx, double* total_ms, int64_t* launches);

/* Diagnostics (no context): the device's achievable streaming-read
 * bandwidth, measured by a kernel with the weight GEMMs' access pattern.
 * Enqueues one read of `bytes` of device memory at d_src on hip_stream:
 * grid workgroups of `waves` (1..16) wavefronts; each wavefront reads whole
 * 1 KB blocks, 16 bytes per lane, keeping `depth` (4, 8, 12 or 16) block
 * loads in flight; pattern 0: each wavefront reads its own contiguous
 * range, pattern 1: all wavefronts sweep the buffer together (block
 * k * grid * waves + wavefront).  d_sink: device memory of grid * waves
 * uint32 that receives a checksum per wavefront.  bytes must be a multiple
 * of 1024 * grid * waves.  The caller times the enqueued kernel (events on
 * the same stream).  SPEC_E_INVAL on bad arguments, SPEC_E_HIP if the
 * launch fails. */
int32_t spec_probe_read_bandwidth(const void* d_src, size_t bytes, int32_t grid,
                                  int32_t waves, int32_t depth, int32_t pattern,
                                  uint32_t* d_sink, void* hip_stream);

/* The same read for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the per-wavefront checksums go to a scratch array held by the library
 * (256 KB per device, kept until the process ends), and d_checksum (device
 * memory, one uint32, the caller's) receives their XOR, which equals the
 * XOR of the d_sink words spec_probe_read_bandwidth writes for the same
 * arguments.  Allocates nothing.  grid * waves must be at most 65536
 * (SPEC_E_INVAL beyond, and for the same bad arguments as above).  Calls
 * that overlap on one GPU share its scratch array and race; serialize them
 * (one stream, or events).  SPEC_E_HIP if the launch fails. */
int32_t spec_probe_read_bandwidth_noalloc(const void* d_src, size_t bytes, int32_t grid,
                                          int32_t waves, int32_t depth, int32_t pattern,
                                          uint32_t* d_checksum, void* hip_stream);

/* Destroy the context (the workspace stays the caller's). */
void spec_destroy(spec_ctx* ctx);

/* Message describing the last error (never NULL). */
const char* spec_last_error(const spec_ctx* ctx);

/* ---- Batched draft planning (host only; no context, no GPU).
 * besthub.dev, "SpecPilot: AI Agent Framework Boosts Speculative Decoding
 * 10.87x for Qwen3.8-27B", section "(4) Three Batch Optimization
 * Mechanisms": dynamic draft length (each request picks one of a few draft
 * lengths from its recent acceptance) and a shared node budget (a batch's
 * draft nodes go to the candidates with the highest path probability).
 * These only choose how many draft positions each request offers; the
 * verification itself, and so every emitted token, is unchanged.
 *
 * spec_acceptance_update: after a step in which request r offered
 * offered[r] chain positions and accepted[r] of them (its accepted prefix),
 * decays the request's counts and adds the step:
 *   succ[r] = decay * succ[r] + accepted[r]
 *   fail[r] = decay * fail[r] + (accepted[r] < offered[r] ? 1 : 0).
 * Arrays of n_req (host memory, caller-owned; succ and fail start at 0).
 * SPEC_E_INVAL if accepted > offered, a count is negative or decay is
 * outside [0, 1] (nothing is changed then).
 *
 * spec_plan_drafts: the estimated per-position acceptance of request r is
 * p_r = (succ[r] + 1) / (succ[r] + fail[r] + 2), and its position j (1-based)
 * has path probability p_r^j.  Each request's maximum length L_r is the
 * largest of choices[0..n_choices) whose last position has p_r^L >= min_prob
 * (the smallest choice when none does).  Of all positions j <= L_r over the
 * batch, the `budget` most probable are kept (ties: lower request, then lower
 * position), which is a prefix of every request's chain; len[r] receives its
 * length (0..L_r; sum(len) <= budget).  choices in [1, 1024].  SPEC_E_INVAL
 * on bad arguments (len is then not written). */
int32_t spec_acceptance_update(int32_t n_req, const int32_t* offered, const int32_t* accepted,
                               float decay, float* succ, float* fail);
int32_t spec_plan_drafts(int32_t n_req, const float* succ, const float* fail,
                         const int32_t* choices, int32_t n_choices, float min_prob,
                         int32_t budget, int32_t* len);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_H */
