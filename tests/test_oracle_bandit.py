"""Pins of oracle.bandit: the exploration schedule, the warm-up, the
incremental mean, explore/exploit choices, convergence on stationary rewards,
and the acceptance statistics against hand counts and E[n] = sum P(n >= i)."""

import math

import numpy as np
import pytest

from oracle import bandit as ob

ARMS = [0, 2, 4, 6, 8]


def test_epsilon_schedule():
    assert ob.epsilon(0) == 0.3
    vals = [ob.epsilon(t) for t in range(200)]
    assert all(a >= b for a, b in zip(vals, vals[1:]))          # non-increasing
    # 0.3 * 0.97^t reaches the 0.05 floor at t = ln 6 / ln(1 / 0.97) = 58.8.
    t_star = math.log(6) / math.log(1 / 0.97)
    assert 58 < t_star < 59
    assert ob.epsilon(58) > 0.05 and ob.epsilon(59) == 0.05 and ob.epsilon(10 ** 6) == 0.05


def test_warmup_tries_every_arm_twice_in_order():
    b = ob.EpsGreedy(ARMS)
    rng = np.random.default_rng(0)
    seq = []
    for _ in range(10):
        a = b.select(*rng.random(2))
        seq.append(a)
        b.update(a, 1.0)
    assert seq == [0, 1, 2, 3, 4] * 2
    assert b.n == [2] * 5 and b.t == 10


def test_incremental_mean_is_the_mean():
    b = ob.EpsGreedy(ARMS)
    rng = np.random.default_rng(1)
    hist = {a: [] for a in range(5)}
    for _ in range(500):
        a = b.select(*rng.random(2))
        r = float(rng.normal(10 * a, 3))
        hist[a].append(r)
        b.update(a, r)
    for a in range(5):
        assert b.n[a] == len(hist[a])
        assert abs(b.mean[a] - np.mean(hist[a])) < 1e-9 * max(1, abs(np.mean(hist[a])))


def test_explore_and_exploit_choices():
    b = ob.EpsGreedy(ARMS)
    for a, r in zip([0, 1, 2, 3, 4] * 2, [5, 9, 9, 1, 2] * 2):
        b.update(a, r)
    eps = ob.epsilon(10)
    assert b.select(eps, 0.0) == 1            # u >= eps: exploit, tie 1 vs 2 -> lowest index
    assert b.select(0.999, 0.99) == 1
    for u_arm, arm in [(0.0, 0), (0.199, 0), (0.2, 1), (0.61, 3), (0.9999, 4)]:
        assert b.select(eps / 2, u_arm) == arm   # explore: floor(5 u)


@pytest.mark.parametrize("best", [0, 3])
def test_converges_on_stationary_rewards(best):
    rng = np.random.default_rng(7 + best)
    means = np.array([20.0, 15.0, 16.0, 14.0, 12.0])
    means[best], means[0] = means[0], means[best]
    b = ob.EpsGreedy(ARMS)
    picks = []
    for _ in range(400):
        a = b.select(*rng.random(2))
        picks.append(a)
        b.update(a, float(rng.normal(means[a], 1.0)))
    late = np.array(picks[-100:])
    assert np.argmax(b.n) == best
    assert (late == best).mean() > 0.85        # exploration is 5% of late decisions


def test_acceptance_stats_by_hand():
    a, L = ob.acceptance_stats([0, 1, 3, 3], 3)
    assert a.tolist() == [0.75, 0.5, 0.5] and L == 2.75
    rng = np.random.default_rng(3)
    n = rng.integers(0, 8, size=1000)
    a, L = ob.acceptance_stats(n, 7)
    assert abs(1 + a.sum() - L) < 1e-12          # E[n] = sum_i P(n >= i)
    assert all(x >= y for x, y in zip(a, a[1:]))
