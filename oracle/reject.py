"""Oracle: the lossless rejection-sampling verifier and the KV-length commit.

TEST INFRASTRUCTURE ONLY (see the package docstring).  float64 throughout.

What is computed, per sequence b of a batch (the method of [AIE] "Concept"
and "Build it" steps 1-4, with the letters of [AIE]: q is the target /
verifier distribution, p the draft distribution):

  rows      target row i (i = 0..K) is q_{i+1}, the verifier's distribution
            after the last accepted token x0 and drafts d_1..d_i; draft row
            i (i = 0..K-1) is p_{i+1}, the law d_{i+1} was drawn from.
  softmax   q_i = softmax(target_row / T), p_i = softmax(draft_row / T),
            with one temperature T per sequence.
  accept    draft d_i is accepted iff u_{i-1} < min(1, q_i(d_i) / p_i(d_i));
            a draft with p_i(d_i) <= 0 is always accepted ([AIE] step 1).
  scan      n = number of leading accepts; drafts after the first rejection
            are discarded ([QS] section 2, step 4).
  resample  if n < K the emitted token is drawn from the normalised
            residual (q_{n+1} - p_{n+1})_+; if that residual has zero mass
            the draw is from q_{n+1} itself ([AIE] step 2).  If n == K a bonus
            token is drawn from q_{K+1} ([AIE] "Concept", step 3).  The draw
            uses u_K by inverse CDF: the smallest v with C(v) > u_K * Z,
            C the inclusive prefix sum of the weights and Z their total.
  greedy    T <= 0: d_i is accepted iff it equals argmax(target row i-1)
            (lowest index on ties), and the emitted token is
            argmax(target row n): the target's own greedy output ([PHX]
            "What it does"; [QS] section 2).
  emit      out[0..n-1] = d_1..d_n, out[n] = the sampled token, rest -1.
  commit    kv_len <- kv_len + n + 1: x0 plus the n accepted drafts stay in
            the logical cache, the K - n rejected slots are rolled back
            ([AIE] "Rolling back the KV cache" and step 4, with
            prefix_length := L0 and j := n).

Readings where the pages are silent (each also listed in the design notes):
  * one uniform per accept test plus one for the final draw, u[0..K]; only
    one of the residual / bonus draws happens, so u[K] serves both;
  * strict "<" in the accept test, as [AIE] step 1 writes it;
  * inverse-CDF boundary: smallest v with C(v) > u*Z, which never picks a
    zero-weight token; if rounding leaves no such v (u*Z >= C(V-1)), the
    largest v with positive weight is taken;
  * temperature divides both target and draft logits.

Boundary flags (parity bands, reported, never used to decide):
  F1  some examined accept test (positions 1..min(n+1, K)) has
      |u_{i-1} - q_i(d_i)/p_i(d_i)| < eps_accept (1e-5);
  F2  the final draw's target u_K * Z lies within eps_sample (1e-10
      probability mass) of C(t-1) or C(t) for the chosen token t.  Adjacent
      CDF edges of a 128K-entry vocabulary are ~1e-5 apart, so this band has
      to be far narrower than F1's; it is sized for an implementation that
      computes the final draw's weights and sums in float64.
"""

import numpy as np

__all__ = ["widen", "softmax_rows", "reject_sample", "commit_kv_len",
           "acceptance_rate", "leading_true"]


def widen(x):
    """Exact float64 view of logits given as float32, float64 or bf16 bits.

    bf16 is carried as uint16 bit patterns; widening places those 16 bits in
    the high half of a float32, which is exact, then converts to float64.
    """
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def softmax_rows(logits, temperature):
    """softmax(logits / T) along the last axis, in float64.

    ``temperature`` broadcasts against the leading axes (shape [..., 1]
    after expansion by the caller).  Max-subtracted for range, which does not
    change the value.
    """
    z = logits / temperature
    z = z - z.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=-1, keepdims=True)


def leading_true(mask):
    """Number of leading True values along the last axis (the first-rejection scan)."""
    mask = np.asarray(mask, dtype=bool)
    k = mask.shape[-1]
    if k == 0:
        return np.zeros(mask.shape[:-1], dtype=np.int64)
    first_false = np.argmin(mask, axis=-1)          # first False (0 if none)
    return np.where(mask.all(axis=-1), k, first_false)


def acceptance_rate(target_row, draft_row, temperature):
    """Per-token acceptance probability alpha = sum_v min(p(v), q(v)).

    The probability that d ~ p passes the accept test, summed over d:
    sum_d p(d) * min(1, q(d)/p(d)) ([AIE] "What determines the speed-up",
    the alpha of the expected-accepted-tokens formula).
    """
    q = softmax_rows(widen(target_row), temperature)
    p = softmax_rows(widen(draft_row), temperature)
    return np.minimum(p, q).sum(axis=-1)


def _inverse_cdf(w, u, eps):
    """Draw one index per row of weights ``w`` [S, V] with uniforms ``u`` [S].

    Returns (token, flag): token = smallest v with C(v) > u * Z, falling back
    to the largest positive-weight v; flag marks draws within ``eps`` of a
    CDF edge.
    """
    c = np.cumsum(w, axis=-1)
    z = c[:, -1]
    tgt = u * z
    hit = c > tgt[:, None]
    any_hit = hit.any(axis=-1)
    first_hit = np.argmax(hit, axis=-1)
    v = w.shape[-1]
    last_pos = v - 1 - np.argmax((w > 0)[:, ::-1], axis=-1)
    tok = np.where(any_hit, first_hit, last_pos)
    rows = np.arange(w.shape[0])
    c_hi = c[rows, tok]
    c_lo = np.where(tok > 0, c[rows, np.maximum(tok - 1, 0)], 0.0)
    flag = (np.abs(tgt - c_lo) < eps) | (np.abs(tgt - c_hi) < eps)
    return tok.astype(np.int64), flag


def reject_sample(target_logits, draft_logits, draft_tokens, uniforms,
                  temperature, eps_accept=1e-5, eps_sample=1e-10):
    """One verify call for a batch of sequences.

    Args:
      target_logits: [B, K+1, V] float32 / float64 / bf16 bits (uint16).
      draft_logits:  [B, K, V] same kinds, or None when every T_b <= 0.
      draft_tokens:  [B, K] integer token ids in [0, V).
      uniforms:      [B, K+1] in [0, 1): u[:, :K] accept tests, u[:, K]
                     the residual or bonus draw.
      temperature:   [B]; T_b <= 0 selects greedy for sequence b.
      eps_accept:    half-width of the F1 band (on u - q/p).
      eps_sample:    half-width of the F2 band (probability mass).

    Returns a dict with
      out_tokens   [B, K+1] int32, -1 padded
      num_accepted [B] int32
      flag_accept  [B] bool  (F1)
      flag_sample  [B] bool  (F2)
      ratio        [B, K] float64, q_i(d_i)/p_i(d_i) (nan for greedy rows)
    """
    tl = widen(target_logits)
    b_sz, k1, v = tl.shape
    k = k1 - 1
    d = np.asarray(draft_tokens, dtype=np.int64).reshape(b_sz, k)
    u = np.asarray(uniforms, dtype=np.float64).reshape(b_sz, k1)
    t = np.asarray(temperature, dtype=np.float64).reshape(b_sz)

    out = np.full((b_sz, k1), -1, dtype=np.int32)
    n_acc = np.zeros(b_sz, dtype=np.int32)
    f1 = np.zeros(b_sz, dtype=bool)
    f2 = np.zeros(b_sz, dtype=bool)
    ratio = np.full((b_sz, k), np.nan)

    greedy = t <= 0
    gi = np.nonzero(greedy)[0]
    if gi.size:
        # np.argmax returns the first maximal index: lowest index on ties.
        am = np.argmax(tl[gi], axis=-1)                     # [G, K+1]
        n = leading_true(am[:, :k] == d[gi])                # row i-1 checks d_i
        tok = am[np.arange(gi.size), n]
        n_acc[gi] = n
        for j, b in enumerate(gi):
            out[b, :n[j]] = d[b, :n[j]]
            out[b, n[j]] = tok[j]

    si = np.nonzero(~greedy)[0]
    if si.size:
        if draft_logits is None:
            raise ValueError("draft_logits required when some T_b > 0")
        dl = widen(draft_logits).reshape(b_sz, k, v)
        ts = t[si][:, None, None]
        q = softmax_rows(tl[si], ts)                        # [S, K+1, V]
        p = softmax_rows(dl[si], ts)                        # [S, K, V]
        ds = d[si]
        qd = np.take_along_axis(q[:, :k, :], ds[..., None], axis=-1)[..., 0]
        pd = np.take_along_axis(p, ds[..., None], axis=-1)[..., 0]
        with np.errstate(divide="ignore", invalid="ignore"):
            r = np.where(pd > 0, qd / pd, np.inf)
        accept = (pd <= 0) | (u[si, :k] < np.minimum(1.0, r))
        n = leading_true(accept)                            # [S]
        rows = np.arange(si.size)

        # F1: accept tests actually examined are positions 1..min(n+1, K).
        examined = np.arange(k)[None, :] <= np.minimum(n, k - 1)[:, None]
        f1[si] = (examined & (np.abs(u[si, :k] - r) < eps_accept)).any(axis=-1)

        # Residual (n < K) or bonus (n == K) weights.
        q_row = q[rows, n]                                  # q_{n+1}
        p_row = p[rows, np.minimum(n, k - 1)] if k > 0 else np.zeros_like(q_row)
        resid = np.maximum(0.0, q_row - p_row)
        w = np.where((n < k)[:, None], resid, q_row)
        zero_mass = w.sum(axis=-1) == 0
        w = np.where(zero_mass[:, None], q_row, w)          # [AIE] step 2 fallback
        tok, flag = _inverse_cdf(w, u[si, k], eps_sample)
        f2[si] = flag
        n_acc[si] = n
        ratio[si] = r
        for j, b in enumerate(si):
            out[b, :n[j]] = d[b, :n[j]]
            out[b, n[j]] = tok[j]

    return {"out_tokens": out, "num_accepted": n_acc, "flag_accept": f1,
            "flag_sample": f2, "ratio": ratio}


def commit_kv_len(kv_len, num_accepted):
    """Logical KV length after the verify: L0 + n + 1 ([AIE] "Rolling back the KV cache")."""
    return (np.asarray(kv_len, dtype=np.int64)
            + np.asarray(num_accepted, dtype=np.int64) + 1).astype(np.int32)
