"""Pins of oracle.filter: top-k and top-p sets against hand-computed cases,
the off settings, and losslessness of the filtered verifier against the
filtered target law (the drafts drawn from the filtered draft law)."""

import numpy as np
import pytest

from oracle import filter as of
from oracle import reject as orj
from synth import gen


def test_top_k_by_hand():
    x = np.array([1.0, 5.0, 3.0, 5.0, 2.0, 4.0])
    assert of.filter_mask(x, 1.0, top_k=1)[0].tolist() == [0, 1, 0, 1, 0, 0]   # tie kept
    assert of.filter_mask(x, 1.0, top_k=3)[0].tolist() == [0, 1, 0, 1, 0, 1]
    assert of.filter_mask(x, 1.0, top_k=4)[0].tolist() == [0, 1, 1, 1, 0, 1]
    for k in (0, -1, 6, 100):
        assert of.filter_mask(x, 1.0, top_k=k)[0].all()


def test_top_p_by_hand():
    prob = np.array([0.05, 0.5, 0.15, 0.3])
    x = np.log(prob)
    cases = [(0.5, [0, 1, 0, 0]), (0.7, [0, 1, 0, 1]), (0.9, [0, 1, 1, 1]),
             (0.96, [1, 1, 1, 1])]
    for p, want in cases:
        keep, flag = of.filter_mask(x, 1.0, top_p=p)
        assert keep.tolist() == [bool(w) for w in want], p
    assert of.filter_mask(x, 1.0, top_p=0.8)[1]            # cum mass exactly 0.8: flagged
    assert not of.filter_mask(x, 1.0, top_p=0.79999)[1]    # 1e-5 away: outside the band
    assert not of.filter_mask(x, 1.0, top_p=0.7)[1]
    for p in (0.0, 1.0, 1.5):
        assert of.filter_mask(x, 1.0, top_p=p)[0].all()
    # Temperature reshapes the law first: at T = 0.5 the top two hold 0.5^2 + 0.3^2 over
    # the sum of squares = 0.34 / 0.365 = 0.93 > 0.9.
    assert of.filter_mask(x, 0.5, top_p=0.9)[0].tolist() == [False, True, False, True]


def test_top_k_then_top_p_renormalises():
    prob = np.array([0.05, 0.5, 0.15, 0.3])
    x = np.log(prob)
    # top-3 = {0.5, 0.3, 0.15} / 0.95: 0.5263, then 0.8421 >= 0.8.
    keep, _ = of.filter_mask(x, 1.0, top_k=3, top_p=0.8)
    assert keep.tolist() == [False, True, False, True]
    keep, _ = of.filter_mask(x, 1.0, top_k=3, top_p=0.85)      # 0.8421 < 0.85: add 0.15
    assert keep.tolist() == [False, True, True, True]


def test_filters_off_is_the_plain_verifier():
    inp = gen.make_reject_inputs(seed=3, B=50, K=4, V=200, dtype="f32", draft_sigma=1.0)
    a = orj.reject_sample(inp["target"], inp["draft"], inp["draft_tokens"], inp["uniforms"],
                          inp["temperature"])
    b = of.reject_sample_filtered(inp["target"], inp["draft"], inp["draft_tokens"],
                                  inp["uniforms"], inp["temperature"], 0, 1.0)
    assert np.array_equal(a["out_tokens"], b["out_tokens"]) and not b["flag_filter"].any()


@pytest.mark.parametrize("top_k,top_p", [(5, 1.0), (0, 0.8), (8, 0.9)])
def test_filtered_verifier_is_lossless_for_the_filtered_target(top_k, top_p):
    # One shared row pair, fresh drafts (from the filtered draft law) and
    # uniforms per trial: the first emitted token must follow the filtered q.
    V, trials = 16, 100_000
    rng = np.random.default_rng(11)
    tgt = rng.standard_normal((1, 2, V))
    drf = tgt[:, :1] + rng.standard_normal((1, 1, V))
    tf, _ = of.filtered_logits(tgt, 1.0, top_k, top_p)
    df, _ = of.filtered_logits(drf, 1.0, top_k, top_p)
    g = -np.log(-np.log(rng.random((trials, V))))
    d = np.argmax(df[0, 0][None, :] + g, axis=1)[:, None]
    u = gen.uniforms24(rng, (trials, 2))
    # The filtered verifier on a subset equals the plain verifier on the
    # filtered rows, which then runs all trials at once (shared rows).
    sub = slice(0, 500)
    a = of.reject_sample_filtered(np.broadcast_to(tgt, (500, 2, V)), np.broadcast_to(drf, (500, 1, V)),
                                  d[sub], u[sub], np.ones(500), top_k, top_p)
    res = orj.reject_sample(np.broadcast_to(tf, (trials, 2, V)), np.broadcast_to(df, (trials, 1, V)),
                            d, u, np.ones(trials))
    assert np.array_equal(a["out_tokens"], res["out_tokens"][sub])
    first = np.bincount(res["out_tokens"][:, 0], minlength=V) / trials
    q = np.exp(tf[0, 0] - tf[0, 0].max())
    q /= q.sum()
    assert (first[q == 0] == 0).all()                       # nothing outside the kept set
    assert 0.5 * np.abs(first - q).sum() < 0.01


def test_f3_band_edges():
    # Masses 0.5, 0.3, 0.2 in value order: cumulative 0.5, 0.8, 1.0.  F3 flags
    # a row when top_p is within 1e-6 of the mass of the kept set or of the
    # set one value smaller.
    x = np.log(np.array([0.3, 0.5, 0.2]))
    for p, flag in [(0.8 - 0.99e-6, True), (0.8 - 1.01e-6, False), (0.8 + 0.99e-6, True),
                    (0.8 + 1.01e-6, False), (0.5 + 0.99e-6, True), (0.5 + 1.01e-6, False),
                    (0.65, False)]:
        keep, f = of.filter_mask(x, 1.0, top_p=p)
        assert bool(f) == flag, p
    # The kept sets on both sides of the 0.8 edge.
    assert of.filter_mask(x, 1.0, top_p=0.8 - 1.01e-6)[0].tolist() == [True, True, False]
    assert of.filter_mask(x, 1.0, top_p=0.8 + 1.01e-6)[0].tolist() == [True, True, True]
