// Index arithmetic of the kernels that address the paged KV cache, the
// attention split partials and the accepted-path walk, written once for
// the device code and for a CPU build (tests/index_math_check.cpp) that
// checks every offset against the buffer sizes under the address and
// undefined-behaviour sanitizers.
#pragma once

#include <stddef.h>
#include <stdint.h>

#if defined(__HIPCC__)
#define SPEC_HD __host__ __device__
#else
#define SPEC_HD
#endif

// One layer's paged KV cache: K pages [page][nkv][16 tokens][hd], V pages
// [page][nkv][hd][16 tokens] (transposed, so attention reads V^T
// directly).  t16 = the token's place in its page.
SPEC_HD inline size_t kv_k_index(int page, int nkv, int kvh, int t16, int hd, int dim) {
  return (((size_t)page * nkv + kvh) * 16 + t16) * hd + dim;
}
SPEC_HD inline size_t kv_v_index(int page, int nkv, int kvh, int t16, int hd, int dim) {
  return (((size_t)page * nkv + kvh) * hd + dim) * 16 + t16;
}

// The page holding token t of a request: consecutive pages from page0, or
// (page0 < 0) its row of the block table.
SPEC_HD inline int kv_page(int page0, const int32_t* bt_row, int t) {
  return page0 >= 0 ? page0 + (t >> 4) : bt_row[t >> 4];
}

// Attention partials of (key split, pass row, query head): [split][rows *
// nq] (the output rows are hd floats each).
SPEC_HD inline size_t attn_part_slot(int split, int rows_total, int nq, int row, int head) {
  return (size_t)split * rows_total * nq + (size_t)row * nq + head;
}

// Greedy acceptance over one request's n nodes (node 0 the root, parents
// before children): node i is accepted when its parent is and its token is
// the parent's argmax; the deepest accepted node wins, the lowest index
// among equals.  Writes out[0] = path length, out[1] = the bonus token (the
// winner's argmax), out[2 + k] = the k-th node of the path below the root.
// ok and dep are scratch arrays of n entries.
SPEC_HD inline void walk_accepted_path(int n, const int16_t* par, const int32_t* tok,
                                       const int32_t* am, int8_t* ok, int16_t* dep,
                                       int32_t* out) {
  int best = 0;
  ok[0] = 1;
  dep[0] = 0;
  for (int i = 1; i < n; ++i) {
    const int p = par[i];
    ok[i] = ok[p] && tok[i] == am[p];
    dep[i] = (int16_t)(dep[p] + 1);
    if (ok[i] && dep[i] > dep[best]) best = i;
  }
  const int plen = dep[best];
  out[0] = plen;
  out[1] = am[best];
  int v = best;
  for (int k = plen - 1; k >= 0; --k) {
    out[2 + k] = v;
    v = par[v];
  }
}
