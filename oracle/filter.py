"""Oracle: top-k / top-p filtering of the target and draft distributions
before the lossless verifier.

TEST INFRASTRUCTURE ONLY (see the package docstring).  float64 throughout.

[QS] "Influence du sampling": a higher temperature, or a wider top-p /
top-k, makes the drafted tokens more diverse and lowers the acceptance; a
more deterministic regime gives longer accepted prefixes.  The pages fix no
filtering rule; the readings here (also in the design notes):

  * order: logits / T, then top-k, then top-p over the top-k set, then
    renormalise; one (top_k, top_p) per sequence, applied to every target
    row and, with the same parameters, to every draft row (the drafter
    samples from its own filtered law);
  * top-k keeps the tokens whose logit is >= the k-th largest logit (ties
    at the boundary kept); k <= 0 or k >= V keeps all;
  * top-p keeps the tokens whose logit is >= v*, v* the largest logit value
    whose set {x >= v*} holds at least top_p of the (top-k) mass (ties kept);
    top_p <= 0 or >= 1 keeps all;
  * the verifier then runs unchanged on the filtered laws q', p' (accept
    with min(1, q'(d)/p'(d)), residual (q' - p')_+, bonus from q'), so its
    output law is the filtered target's, which is what "lossless" means
    under filtering.
Filtering a row is the same as setting its dropped logits to -inf, which is
how reject_sample_filtered calls the plain verifier.  F3 flags a sequence
when a row's top-p boundary is within eps_filter (1e-6) of top_p (the set's
mass or the mass without the boundary value).  The device takes that
decision on fp32 weights (one rounding in the exponent, ~1 ulp in exp2)
summed in 40-bit fixed point: its cumulative masses are within ~2e-7 of the
exact ones, so it can differ only inside that band.
"""

import numpy as np

from .reject import widen, reject_sample
from .tree import children_of, reject_sample_tree

__all__ = ["filter_mask", "filtered_logits", "reject_sample_filtered",
           "reject_sample_tree_filtered"]


def filter_mask(logits, temperature, top_k=0, top_p=1.0, eps_filter=1e-6):
    """Kept-token mask [V] of one row, and the F3 flag."""
    x = np.asarray(logits, dtype=np.float64)
    v = x.shape[0]
    keep = np.ones(v, dtype=bool)
    if 0 < top_k < v:
        kth = np.sort(x)[::-1][top_k - 1]
        keep &= x >= kth
    flag = False
    if 0.0 < top_p < 1.0 and temperature > 0:
        z = np.where(keep, x / temperature, -np.inf)
        e = np.exp(z - z.max())
        prob = e / e.sum()
        # Mass of {x >= u} for every distinct kept value u, descending: a
        # cumulative sum in value order, read at the last entry of each value.
        xs, ps = x[keep], prob[keep]
        order = np.argsort(-xs, kind="stable")
        xs, cs = xs[order], np.cumsum(ps[order])
        ends = np.nonzero(np.r_[xs[1:] != xs[:-1], True])[0]
        vals, mass_at = xs[ends], cs[ends]
        idx = int(np.argmax(mass_at >= top_p))               # first (largest) value reaching top_p
        keep &= x >= vals[idx]
        before = mass_at[idx - 1] if idx > 0 else 0.0
        flag = abs(mass_at[idx] - top_p) < eps_filter or abs(before - top_p) < eps_filter
    return keep, flag


def filtered_logits(logits, temperature, top_k, top_p, eps_filter=1e-6):
    """float64 copy of rows [..., V] with the dropped logits at -inf, and a flag per row."""
    x = widen(logits)
    out = x.copy()
    flags = np.zeros(x.shape[:-1], dtype=bool)
    for idx in np.ndindex(*x.shape[:-1]):
        keep, f = filter_mask(x[idx], temperature, top_k, top_p, eps_filter)
        out[idx] = np.where(keep, x[idx], -np.inf)
        flags[idx] = f
    return out, flags


def reject_sample_filtered(target_logits, draft_logits, draft_tokens, uniforms, temperature,
                           top_k, top_p, eps_accept=1e-5, eps_sample=1e-10, eps_filter=1e-6):
    """reject_sample on the filtered laws.  top_k [B] int, top_p [B] float.

    Returns reject_sample's dict plus flag_filter [B] (F3).  Greedy sequences
    are unaffected (the argmax is always kept).
    """
    tl = widen(target_logits)
    b_sz, k1, v = tl.shape
    t = np.asarray(temperature, dtype=np.float64).reshape(b_sz)
    tk = np.broadcast_to(np.asarray(top_k, dtype=np.int64), (b_sz,))
    tp = np.broadcast_to(np.asarray(top_p, dtype=np.float64), (b_sz,))
    dl = None if draft_logits is None else widen(draft_logits).reshape(b_sz, k1 - 1, v)
    tf = tl.copy()
    df = None if dl is None else dl.copy()
    f3 = np.zeros(b_sz, dtype=bool)
    for b in range(b_sz):
        if t[b] <= 0:
            continue
        tf[b], ft = filtered_logits(tl[b], t[b], tk[b], tp[b], eps_filter)
        f = ft.any()
        if df is not None:
            df[b], fd = filtered_logits(dl[b], t[b], tk[b], tp[b], eps_filter)
            f = f or fd.any()
        f3[b] = f
    res = reject_sample(tf, df, draft_tokens, uniforms, temperature, eps_accept, eps_sample)
    res["flag_filter"] = f3
    return res


def reject_sample_tree_filtered(target_logits, draft_logits, parent, tokens, uniforms, temperature,
                                top_k, top_p, eps_accept=1e-5, eps_sample=1e-10, eps_filter=1e-6):
    """reject_sample_tree on the filtered laws.  top_k [B] int, top_p [B] float.

    The same reading as the chain's: every target row q_v, and the draft row
    p_v of every node with children (the law its children were drawn from),
    is filtered with the sequence's (top_k, top_p); the tree walk then runs
    unchanged on q', p' ([QS] "Influence du sampling" with the verifier of
    [TC] "Grading every branch in one pass").  Draft rows of leaves are never
    used and stay as given.  Returns reject_sample_tree's dict plus
    flag_filter [B] (F3 on any of the rows filtered).  Greedy sequences are
    unaffected.
    """
    tl = widen(target_logits)
    b_sz, n, v = tl.shape
    par = np.asarray(parent, dtype=np.int64)
    if par.ndim == 1:
        par = np.broadcast_to(par, (b_sz, n))
    t = np.asarray(temperature, dtype=np.float64).reshape(b_sz)
    tk = np.broadcast_to(np.asarray(top_k, dtype=np.int64), (b_sz,))
    tp = np.broadcast_to(np.asarray(top_p, dtype=np.float64), (b_sz,))
    dl = None if draft_logits is None else widen(draft_logits).reshape(b_sz, n, v)
    tf = tl.copy()
    df = None if dl is None else dl.copy()
    f3 = np.zeros(b_sz, dtype=bool)
    for b in range(b_sz):
        if t[b] <= 0:
            continue
        tf[b], ft = filtered_logits(tl[b], t[b], tk[b], tp[b], eps_filter)
        f = ft.any()
        if df is not None:
            kids = children_of(par[b])
            inner = [u for u in range(n) if kids[u]]
            if inner:
                rows, fd = filtered_logits(dl[b, inner], t[b], tk[b], tp[b], eps_filter)
                df[b, inner] = rows
                f = f or fd.any()
        f3[b] = f
    res = reject_sample_tree(tf, df, parent, tokens, uniforms, temperature, eps_accept, eps_sample)
    res["flag_filter"] = f3
    return res
