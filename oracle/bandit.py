"""Oracle: the adaptive draft-length controller and the acceptance statistics.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[PHX] "How we built it", "The bandit": an epsilon-greedy bandit picks how
many tokens to draft per request from the arms {0, 2, 4, 6, 8} (0 = no
drafting); every arm is tried twice first; afterwards it explores with
probability eps_t = max(0.05, 0.3 * 0.97^t) and otherwise takes the arm with
the best running-average reward, updated incrementally
(mean_a <- mean_a + (r - mean_a) / n_a); the reward is output tokens per
second.  [QS] section 4: per-position acceptance a_i and the mean acceptance
length.

Readings (the page leaves these open):
  * warm-up order: the arms in list order, twice around (a0..a4, a0..a4);
  * t counts every decision made before this one, warm-up included (the
    first decision has t = 0);
  * exploring picks arm floor(u_arm * n_arms) uniformly over all arms, the
    best one included; exploiting picks the highest mean, the lowest index
    on ties;
  * the two uniforms of a decision are inputs (u_explore, u_arm in [0, 1)),
    so a run can be replayed exactly.
Acceptance statistics (reading of [QS] section 4): a_i = P(n >= i) for
i = 1..K over the sequences of a batch (the fraction whose first i drafts
were all accepted), and L = mean(n + 1), the tokens emitted per verify.
"""

import numpy as np

__all__ = ["epsilon", "EpsGreedy", "acceptance_stats"]

EPS_FLOOR, EPS_START, EPS_DECAY = 0.05, 0.3, 0.97


def epsilon(t):
    """Exploration probability of decision t."""
    return max(EPS_FLOOR, EPS_START * EPS_DECAY ** t)


class EpsGreedy:
    def __init__(self, arms, warmup_rounds=2):
        self.arms = list(arms)
        self.n = [0] * len(self.arms)
        self.mean = [0.0] * len(self.arms)
        self.t = 0
        self.warm = warmup_rounds * len(self.arms)

    def select(self, u_explore, u_arm):
        """Index of the arm for decision t (t advances on update)."""
        k = len(self.arms)
        if self.t < self.warm:
            return self.t % k
        if u_explore < epsilon(self.t):
            return min(int(u_arm * k), k - 1)
        best = 0
        for a in range(1, k):
            if self.mean[a] > self.mean[best]:
                best = a
        return best

    def update(self, arm, reward):
        self.n[arm] += 1
        self.mean[arm] = self.mean[arm] + (reward - self.mean[arm]) / self.n[arm]
        self.t += 1


def acceptance_stats(num_accepted, K):
    """(a [K], L): a[i-1] = fraction of sequences with n >= i; L = mean(n + 1)."""
    n = np.asarray(num_accepted, dtype=np.int64)
    a = np.array([np.mean(n >= i) for i in range(1, K + 1)], dtype=np.float64)
    return a, float(np.mean(n + 1))
