// CPU build of the kernels' index arithmetic (csrc/index_math.h), run under
// the address and undefined-behaviour sanitizers by test_index_math_cpu.py.
// Every buffer is a std::vector of exactly the size the library allocates,
// so an index one past the end is reported by the sanitizer; the checks
// also compare each map with a plain enumeration.
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "index_math.h"

static int failures = 0;
#define CHECK(c, ...)                         \
  do {                                        \
    if (!(c)) {                               \
      std::printf("FAIL %s:%d ", __FILE__, __LINE__); \
      std::printf(__VA_ARGS__);               \
      std::printf("\n");                      \
      if (++failures > 20) std::exit(1);      \
    }                                         \
  } while (0)

// K and V page layouts: every (page, head, token, dim) maps to a distinct
// element of a cache of n_pages * nkv * 16 * hd elements.
static void check_kv_layout(int n_pages, int nkv, int hd) {
  const size_t n = (size_t)n_pages * nkv * 16 * hd;
  std::vector<unsigned char> seen_k(n, 0), seen_v(n, 0);
  std::vector<float> cache(n);  // touched through the computed indices
  for (int page = 0; page < n_pages; ++page)
    for (int kvh = 0; kvh < nkv; ++kvh)
      for (int t = 0; t < 16; ++t)
        for (int dim = 0; dim < hd; ++dim) {
          const size_t ik = kv_k_index(page, nkv, kvh, t, hd, dim);
          const size_t iv = kv_v_index(page, nkv, kvh, t, hd, dim);
          CHECK(ik < n && iv < n, "kv index past the cache");
          cache.at(ik) += 1.f;
          cache.at(iv) += 1.f;
          seen_k[ik]++;
          seen_v[iv]++;
        }
  for (size_t i = 0; i < n; ++i) CHECK(seen_k[i] == 1 && seen_v[i] == 1, "kv map not one-to-one at %zu", i);
}

// Page lookups of a request's tokens, through consecutive pages or a block
// table row of max_pages entries.
static void check_pages(int n_pages, int max_pages, std::mt19937& rng) {
  std::vector<int32_t> bt(max_pages);
  for (int i = 0; i < max_pages; ++i) bt[i] = (int32_t)(rng() % n_pages);
  for (int t = 0; t < max_pages * 16; ++t) {
    const int p = kv_page(-1, bt.data(), t);
    CHECK(p >= 0 && p < n_pages, "table page out of range");
    const int page0 = n_pages - max_pages;
    const int q = kv_page(page0, bt.data(), t);
    CHECK(q >= 0 && q < n_pages, "consecutive page out of range");
  }
}

// Attention partials: the library sizes them for split_rows (split, row)
// pairs of nq heads; a pass of R rows may use max_splits splits when
// max_splits * R <= split_rows.
static void check_partials(int split_rows, int R, int nq, int hd) {
  const int max_splits = split_rows / R;
  std::vector<float> part_o((size_t)split_rows * nq * hd);
  std::vector<float> part_ml((size_t)split_rows * nq * 2);
  for (int sp = 0; sp < max_splits; ++sp)
    for (int row = 0; row < R; ++row)
      for (int h = 0; h < nq; ++h) {
        const size_t slot = attn_part_slot(sp, R, nq, row, h);
        part_o.at(slot * hd + hd - 1) = 1.f;
        part_ml.at(slot * 2 + 1) = 1.f;
      }
}

// Acceptance walk against a plain recomputation: a node is accepted when
// every node on its root path matches its parent's argmax.
static void check_walk(int n, std::mt19937& rng, int max_path, int match_pct) {
  std::vector<int16_t> par(n), dep(n);
  std::vector<int32_t> tok(n), am(n);
  std::vector<int8_t> ok(n);
  std::vector<int32_t> out(2 + max_path, -7);
  par[0] = -1;
  const bool chain = rng() % 3 == 0;
  for (int i = 1; i < n; ++i) par[i] = (int16_t)(chain ? i - 1 : rng() % i);
  for (int i = 0; i < n; ++i) am[i] = (int32_t)(rng() % 3);
  tok[0] = 0;
  for (int i = 1; i < n; ++i)  // a draft matches its parent's argmax with this chance
    tok[i] = (int)(rng() % 100) < match_pct ? am[par[i]] : (int32_t)(rng() % 3);
  walk_accepted_path(n, par.data(), tok.data(), am.data(), ok.data(), dep.data(), out.data());
  int best = 0, best_d = 0;
  for (int i = 1; i < n; ++i) {
    bool acc = true;
    int d = 0;
    for (int v = i; v != 0; v = par[v], ++d) acc = acc && tok[v] == am[par[v]];
    if (acc && d > best_d) {
      best = i;
      best_d = d;
    }
  }
  CHECK(out[0] == best_d, "path length %d, want %d", out[0], best_d);
  CHECK(out[1] == am[best], "bonus");
  for (int k = best_d - 1, v = best; k >= 0; --k, v = par[v]) CHECK(out[2 + k] == v, "path node");
  for (int k = best_d; k < max_path; ++k) CHECK(out[2 + k] == -7, "write past the path");
}

int main() {
  std::mt19937 rng(12345);
  check_kv_layout(3, 2, 64);
  check_kv_layout(2, 8, 128);
  for (int i = 0; i < 50; ++i) check_pages(64, 1 + (int)(rng() % 64), rng);
  // verify passes (kMaxSplits = 128 splits of max_rows rows) and prefill
  // chunks (64 splits of the chunk's rows), with the planner's rule
  check_partials(128 * 17, 17, 32, 128);
  check_partials(128 * 33, 33, 40, 128);
  check_partials(64 * 512, 512, 8, 64);
  check_partials(128 * 288, 288, 32, 128);
  // trees and chains up to the library's 65 nodes; the walk result holds
  // 64 path slots
  for (int it = 0; it < 4000; ++it) check_walk(1 + (int)(rng() % 65), rng, 64, (int)(rng() % 101));
  for (int it = 0; it < 200; ++it) check_walk(65, rng, 64, 100);  // every node accepted
  check_walk(1, rng, 64, 100);
  std::printf("index math: %d failures\n", failures);
  return failures ? 1 : 0;
}
