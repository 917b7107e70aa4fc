"""The native draft-length controller and acceptance statistics, on the CPU,
replayed against oracle.bandit with the same uniforms and rewards: identical
arm choices and bit-identical running means."""

import numpy as np
import pytest

import speculative_decoding_verification_verify_amd as sv
from oracle import bandit as ob


@pytest.fixture(scope="module")
def lib():
    return sv.load()


@pytest.mark.parametrize("seed,arms,warm", [(0, (0, 2, 4, 6, 8), 2), (1, (2, 4, 8), 1),
                                            (2, (7,), 2), (3, tuple(range(1, 17)), 0)])
def test_replays_the_oracle(lib, seed, arms, warm):
    rng = np.random.default_rng(seed)
    c, o = sv.DraftLengthBandit(arms, warm), ob.EpsGreedy(arms, warm)
    true = rng.normal(100, 20, size=len(arms))
    for step in range(2000):
        u = rng.random(2)
        a_c, a_o = c.select(*u), o.select(*u)
        assert a_c == a_o, step
        r = float(rng.normal(true[a_c], 5))
        c.update(a_c, r)
        o.update(a_o, r)
    pulls, means, t = c.stats()
    assert pulls == o.n and t == o.t == 2000
    assert means == o.mean                       # same operations in the same order
    c.close()


def test_learns_to_skip_drafting_when_it_does_not_pay(lib):
    # The page's finding: with drafts as costly as target passes, no drafting
    # (arm 0) gives the most tokens/s and the bandit settles on it.
    rng = np.random.default_rng(5)
    tps = {0: 21.6, 2: 17.0, 4: 15.0, 6: 13.5, 8: 12.0}
    c = sv.DraftLengthBandit()
    picks = []
    for _ in range(200):
        a = c.select(*rng.random(2))
        picks.append(c.arms[a])
        c.update(a, tps[c.arms[a]] * rng.uniform(0.9, 1.1))
    assert np.mean(np.array(picks[-50:]) == 0) > 0.85
    c.close()


def test_bad_arguments(lib):
    assert not lib.spec_bandit_create(0, 2)
    assert not lib.spec_bandit_create(3, -1)
    c = sv.DraftLengthBandit((2, 4))
    for u in [(1.0, 0.5), (-0.1, 0.5), (0.5, 1.0), (float("nan"), 0.5)]:
        with pytest.raises(sv.SpecVerifyError):
            c.select(*u)
    with pytest.raises(sv.SpecVerifyError):
        c.update(2, 1.0)
    with pytest.raises(sv.SpecVerifyError):
        c.update(0, float("inf"))
    assert c.stats()[2] == 0                     # nothing was counted
    c.close()


@pytest.mark.parametrize("K", [1, 4, 7, 16])
def test_accept_stats_match_the_oracle(lib, K):
    rng = np.random.default_rng(K)
    n = rng.integers(0, K + 1, size=777).astype(np.int32)
    a, L = sv.accept_stats(n, K)
    a_o, L_o = ob.acceptance_stats(n, K)
    assert np.array_equal(a, a_o) and L == L_o
