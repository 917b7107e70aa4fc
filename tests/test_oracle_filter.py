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


def test_filtered_trees_per_sequence_are_independent_calls():
    # One tree per sequence: each sequence's filtered walk is its own
    # one-sequence call (filters of its rows by its own shape).
    from synth.tree import mixed_parents
    B, N, V = 8, 6, 70
    par = mixed_parents(31, B, N)
    r = gen.make_tree_reject_inputs(31, B, par, V, dtype="bf16", draft_sigma=1.0,
                                    temperature=np.array([1.0, 0.0, 0.9, 1.2] * 2, np.float32))
    tk = np.array([0, 5, 20, 3, 0, 40, 7, 0], np.int64)
    tp = np.array([0.9, 1.0, 0.8, 0.95, 1.0, 0.7, 1.0, 0.6])
    batch = of.reject_sample_tree_filtered(r["target"], r["draft"], par, r["tokens"],
                                            r["uniforms"], r["temperature"], tk, tp)
    for b in range(B):
        one = of.reject_sample_tree_filtered(r["target"][b:b + 1], r["draft"][b:b + 1], par[b],
                                              r["tokens"][b:b + 1], r["uniforms"][b:b + 1],
                                              r["temperature"][b:b + 1], tk[b:b + 1], tp[b:b + 1])
        for k in ("out_tokens", "out_nodes", "num_accepted", "flag_accept", "flag_sample",
                  "flag_filter"):
            assert np.array_equal(batch[k][b], one[k][0]), (b, k)


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


# --------------------------------------------------------------------------
# Trees: the same filters on the tree verifier.
# --------------------------------------------------------------------------

def _chain_as_tree(r):
    """A chain call's inputs recast as a chain-shaped tree call (node i's
    children law = chain draft row i; u[i] <-> u_{i-1}, u[0] <-> u_K)."""
    B, K, V = r["draft"].shape
    n = K + 1
    draft = np.zeros((B, n, V), dtype=r["draft"].dtype)
    draft[:, :K] = r["draft"]
    tokens = np.zeros((B, n), np.int32)
    tokens[:, 1:] = r["draft_tokens"]
    u = np.zeros((B, n), np.float32)
    u[:, 1:] = r["uniforms"][:, :K]
    u[:, 0] = r["uniforms"][:, K]
    return draft, tokens, u


def test_tree_filters_off_is_the_plain_tree_verifier():
    from oracle import tree as otr
    from synth.tree import tree_parents
    par = tree_parents((2, 2))
    inp = gen.make_tree_reject_inputs(seed=5, B=60, parent=par, V=300, dtype="bf16",
                                      draft_sigma=1.2, temperature=1.0)
    a = otr.reject_sample_tree(inp["target"], inp["draft"], par, inp["tokens"], inp["uniforms"],
                               inp["temperature"])
    b = of.reject_sample_tree_filtered(inp["target"], inp["draft"], par, inp["tokens"],
                                       inp["uniforms"], inp["temperature"], 0, 1.0)
    for k in ("out_tokens", "out_nodes", "num_accepted", "flag_accept", "flag_sample"):
        assert np.array_equal(a[k], b[k]), k
    assert not b["flag_filter"].any()


@pytest.mark.parametrize("top_k,top_p", [(5, 1.0), (0, 0.8), (20, 0.9)])
def test_chain_shaped_filtered_tree_is_the_filtered_chain(top_k, top_p):
    from synth.tree import chain_parents
    r = gen.make_reject_inputs(seed=9, B=40, K=5, V=200, dtype="bf16", draft_sigma=1.0,
                               temperature=np.array([0.7, 1.0, 1.3, 0.0] * 10, np.float32))
    chain = of.reject_sample_filtered(r["target"], r["draft"], r["draft_tokens"], r["uniforms"],
                                      r["temperature"], top_k, top_p)
    draft, tokens, u = _chain_as_tree(r)
    tr = of.reject_sample_tree_filtered(r["target"], draft, chain_parents(6), tokens, u,
                                        r["temperature"], top_k, top_p)
    for k in ("out_tokens", "num_accepted", "flag_accept", "flag_sample", "flag_filter"):
        assert np.array_equal(tr[k], chain[k]), k


def test_top_k_one_tree_is_the_greedy_tree():
    """top_k = 1 leaves each row's argmax alone (no ties here): q'_v and p'_v
    are point masses, the filtered drafter can only propose p'_v's argmax,
    a child passes iff that token is q_v's argmax, and the residual after a
    rejection is the point mass at q_v's argmax.  So at any T > 0 the walk is
    the greedy walk (T = 0) on the same rows."""
    from oracle import tree as otr
    from synth.tree import tree_parents, children
    par = tree_parents((2, 2, 2))
    B, V = 80, 64
    inp = gen.make_tree_reject_inputs(seed=21, B=B, parent=par, V=V, dtype="f32",
                                      logit_std=1.0, draft_sigma=0.7, temperature=1.0)
    tgt, drf = inp["target"].astype(np.float64), inp["draft"].astype(np.float64)
    tokens = inp["tokens"].copy()
    kids = children(par)
    for v, cs in enumerate(kids):
        for c in cs:
            tokens[:, c] = np.argmax(drf[:, v], axis=1)
    got = of.reject_sample_tree_filtered(tgt, drf, par, tokens, inp["uniforms"],
                                         np.full(B, 0.9), 1, 1.0)
    greedy = otr.reject_sample_tree(tgt, None, par, tokens, inp["uniforms"], np.zeros(B))
    for k in ("out_tokens", "out_nodes", "num_accepted"):
        assert np.array_equal(got[k], greedy[k]), k
    assert (greedy["num_accepted"] > 0).any() and (greedy["num_accepted"] < 3).any()


def test_filtered_tree_is_lossless_for_the_filtered_root():
    # Shared rows, children drawn from the filtered draft laws, fresh
    # uniforms per trial: the first emitted token follows the filtered q_root.
    from synth.tree import tree_parents, children
    par = tree_parents((2, 2))
    V, trials, top_k, top_p = 16, 200_000, 8, 0.9
    rng = np.random.default_rng(13)
    tgt = rng.standard_normal((1, 7, V))
    drf = tgt + rng.standard_normal((1, 7, V))
    tf, _ = of.filtered_logits(tgt, 1.0, top_k, top_p)
    df, _ = of.filtered_logits(drf, 1.0, top_k, top_p)
    tokens = np.zeros((trials, 7), np.int32)
    for v, cs in enumerate(children(par)):
        for c in cs:
            g = -np.log(-np.log(rng.random((trials, V))))
            tokens[:, c] = np.argmax(df[0, v][None, :] + g, axis=1)
    u = gen.uniforms24(rng, (trials, 7))
    # The filtered verifier on a subset equals the plain tree verifier on the
    # filtered rows, which then runs all trials (shared rows).
    from oracle import tree as otr
    sub = slice(0, 300)
    a = of.reject_sample_tree_filtered(np.broadcast_to(tgt, (300, 7, V)),
                                       np.broadcast_to(drf, (300, 7, V)), par, tokens[sub], u[sub],
                                       np.ones(300), top_k, top_p)
    res = otr.reject_sample_tree(np.broadcast_to(tf, (trials, 7, V)),
                                 np.broadcast_to(df, (trials, 7, V)), par, tokens, u,
                                 np.ones(trials))
    assert np.array_equal(a["out_tokens"], res["out_tokens"][sub])
    first = np.bincount(res["out_tokens"][:, 0], minlength=V) / trials
    q = np.exp(tf[0, 0] - tf[0, 0].max())
    q /= q.sum()
    assert (first[q == 0] == 0).all()                       # nothing outside the kept set
    assert 0.5 * np.abs(first - q).sum() < 0.01


def test_tree_f3_counts_only_the_rows_the_walk_uses():
    """A draft row whose top-p boundary sits on the F3 band flags the
    sequence when it belongs to a node with children, not when it belongs to
    a leaf (leaf draft rows are never used)."""
    edge = np.log(np.array([0.3, 0.5, 0.2]))            # cumulative 0.5, 0.8, 1.0
    flat = np.zeros(3)                                   # one value: mass 1, never on the band
    par = np.array([-1, 0])                              # root with one leaf child
    tgt = np.stack([flat, flat])[None]
    tokens = np.array([[0, 1]], np.int32)
    u = np.array([[0.5, 0.5]], np.float32)
    leaf_edge = np.stack([flat, edge])[None]             # the leaf's row is on the band
    root_edge = np.stack([edge, flat])[None]             # the root's (its child's law) is
    a = of.reject_sample_tree_filtered(tgt, leaf_edge, par, tokens, u, np.ones(1), 0, 0.8)
    b = of.reject_sample_tree_filtered(tgt, root_edge, par, tokens, u, np.ones(1), 0, 0.8)
    assert not a["flag_filter"][0] and b["flag_filter"][0]
