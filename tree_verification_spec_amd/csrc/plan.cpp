// Batched draft planning: dynamic draft length and a shared node budget
// (host code; see include/spec.h for the contract).
//
// Follows besthub.dev, "SpecPilot: AI Agent Framework Boosts Speculative
// Decoding 10.87x for Qwen3.8-27B", section "(4) Three Batch Optimization
// Mechanisms": each request picks one of a few draft lengths from its recent
// acceptance, and the requests of a batch share a fixed budget of draft
// nodes that goes to the candidates with the highest path probability.
// Without a drafter's own confidence, a request's position-j candidate has
// the estimated path probability rate^j, where rate is the request's
// estimated per-position acceptance probability.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <vector>

#include "spec.h"

namespace {

// Laplace-smoothed acceptance estimate from decayed success / failure counts.
float rate_of(float succ, float fail) { return (succ + 1.f) / (succ + fail + 2.f); }

}  // namespace

extern "C" int32_t spec_acceptance_update(int32_t n_req, const int32_t* offered,
                                          const int32_t* accepted, float decay, float* succ,
                                          float* fail) {
  if (n_req < 0 || (n_req > 0 && (!offered || !accepted || !succ || !fail)) ||
      !(decay >= 0.f && decay <= 1.f))
    return SPEC_E_INVAL;
  for (int r = 0; r < n_req; ++r)
    if (offered[r] < 0 || accepted[r] < 0 || accepted[r] > offered[r]) return SPEC_E_INVAL;
  for (int r = 0; r < n_req; ++r) {
    // a chain's accepted prefix is `accepted` matches, then one mismatch
    // unless every offered position matched
    succ[r] = decay * succ[r] + (float)accepted[r];
    fail[r] = decay * fail[r] + (accepted[r] < offered[r] ? 1.f : 0.f);
  }
  return SPEC_OK;
}

extern "C" int32_t spec_plan_drafts(int32_t n_req, const float* succ, const float* fail,
                                    const int32_t* choices, int32_t n_choices, float min_prob,
                                    int32_t budget, int32_t* len) {
  if (n_req < 0 || n_choices < 1 || budget < 0 || !choices || !(min_prob >= 0.f) ||
      (n_req > 0 && (!succ || !fail || !len)))
    return SPEC_E_INVAL;
  int cmin = choices[0];
  for (int i = 0; i < n_choices; ++i) {
    if (choices[i] < 1 || choices[i] > 1024) return SPEC_E_INVAL;
    cmin = std::min(cmin, choices[i]);
  }
  for (int r = 0; r < n_req; ++r)
    if (!(succ[r] >= 0.f) || !(fail[r] >= 0.f)) return SPEC_E_INVAL;

  // dynamic draft length: the longest choice whose last position is still
  // reached with probability >= min_prob (the shortest choice otherwise)
  struct Cand {
    double logp;
    int req, pos;
  };
  std::vector<Cand> cand;
  for (int r = 0; r < n_req; ++r) {
    const double p = rate_of(succ[r], fail[r]);
    int L = cmin;
    for (int i = 0; i < n_choices; ++i)
      if (choices[i] > L && std::pow(p, choices[i]) >= (double)min_prob) L = choices[i];
    for (int j = 1; j <= L; ++j) cand.push_back({j * std::log(p), r, j});
    len[r] = 0;
  }
  // shared budget: the most probable candidates over the batch; the order
  // (probability, then request, then position) keeps each request's kept
  // positions a prefix of its chain
  std::sort(cand.begin(), cand.end(), [](const Cand& a, const Cand& b) {
    if (a.logp != b.logp) return a.logp > b.logp;
    if (a.req != b.req) return a.req < b.req;
    return a.pos < b.pos;
  });
  const size_t keep = std::min(cand.size(), (size_t)budget);
  for (size_t i = 0; i < keep; ++i) len[cand[i].req] = std::max(len[cand[i].req], cand[i].pos);
  return SPEC_OK;
}
