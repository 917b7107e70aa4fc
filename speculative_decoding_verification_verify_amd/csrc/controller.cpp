// Host-side draft-length controller and acceptance statistics.
//
// devpost "phoenix", "How we built it", "The bandit": an epsilon-greedy
// bandit picks how many tokens to draft from a set of arms (there {0, 2, 4,
// 6, 8}; 0 = no drafting); every arm is tried twice first; then it explores
// with probability eps_t = max(0.05, 0.3 * 0.97^t) and otherwise takes the
// arm with the best running-average reward, mean_a += (r - mean_a) / n_a;
// the reward is output tokens per second (the caller measures it: the
// verify calls' num_accepted, or their counters, give the tokens).
// quickscale.ai, "Quand et pourquoi utiliser le speculative decoding",
// section 4: per-position acceptance a_i and the mean acceptance length.
//
// Choices the page leaves open: the warm-up visits the arms in list order,
// twice around; t counts every decision already made (warm-up included);
// exploring takes arm floor(u_arm * n_arms) over all arms; exploiting takes
// the highest mean, the lowest index on ties.  The two uniforms of a
// decision come from the caller, so a run replays exactly.  Not
// thread-safe.

#include <algorithm>
#include <cmath>
#include <new>
#include <vector>

#include "specverify.h"

struct sv_bandit {
  int n_arms = 0;
  long long warm = 0;
  long long t = 0;
  std::vector<long long> pulls;
  std::vector<double> mean;
};

namespace {
double explore_prob(long long t) { return std::max(0.05, 0.3 * std::pow(0.97, (double)t)); }
}  // namespace

extern "C" sv_bandit* spec_bandit_create(int n_arms, int warmup_rounds) {
  if (n_arms < 1 || warmup_rounds < 0) return nullptr;
  sv_bandit* b = new (std::nothrow) sv_bandit;
  if (!b) return nullptr;
  try {
    b->n_arms = n_arms;
    b->warm = (long long)warmup_rounds * n_arms;
    b->pulls.assign(n_arms, 0);
    b->mean.assign(n_arms, 0.0);
  } catch (...) {
    delete b;
    return nullptr;
  }
  return b;
}

extern "C" void spec_bandit_destroy(sv_bandit* b) { delete b; }

extern "C" int spec_bandit_select(const sv_bandit* b, double u_explore, double u_arm) {
  if (!b || !(u_explore >= 0.0 && u_explore < 1.0) || !(u_arm >= 0.0 && u_arm < 1.0))
    return SV_ERR_INVALID_ARG;
  const int k = b->n_arms;
  if (b->t < b->warm) return (int)(b->t % k);
  if (u_explore < explore_prob(b->t)) return std::min((int)(u_arm * k), k - 1);
  int best = 0;
  for (int a = 1; a < k; ++a)
    if (b->mean[a] > b->mean[best]) best = a;
  return best;
}

extern "C" int spec_bandit_update(sv_bandit* b, int arm, double reward) {
  if (!b || arm < 0 || arm >= b->n_arms || !std::isfinite(reward)) return SV_ERR_INVALID_ARG;
  b->pulls[arm] += 1;
  b->mean[arm] = b->mean[arm] + (reward - b->mean[arm]) / (double)b->pulls[arm];
  b->t += 1;
  return SV_OK;
}

extern "C" int spec_bandit_stats(const sv_bandit* b, long long* pulls, double* means, long long* t) {
  if (!b) return SV_ERR_INVALID_ARG;
  for (int a = 0; a < b->n_arms; ++a) {
    if (pulls) pulls[a] = b->pulls[a];
    if (means) means[a] = b->mean[a];
  }
  if (t) *t = b->t;
  return SV_OK;
}

extern "C" int spec_accept_stats(const int32_t* num_accepted, int B, int K, double* a,
                                 double* mean_len) {
  if (!num_accepted || B < 1 || K < 0 || (K > 0 && !a) || !mean_len) return SV_ERR_INVALID_ARG;
  std::vector<long long> ge(K + 2, 0);      // ge[i] = #sequences with n >= i
  long long sum = 0;
  for (int b = 0; b < B; ++b) {
    const int n = std::max(0, std::min(num_accepted[b], K));
    ge[n] += 1;
    sum += n + 1;
  }
  for (int i = K - 1; i >= 0; --i) ge[i] += ge[i + 1];
  for (int i = 1; i <= K; ++i) a[i - 1] = (double)ge[i] / B;
  *mean_len = (double)sum / B;
  return SV_OK;
}
