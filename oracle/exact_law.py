"""Oracle: the exact output law of one verify call, in closed form.

TEST INFRASTRUCTURE ONLY (see the package docstring).  float64.

For fixed rows q_1..q_{K+1} (target) and p_1..p_K (draft), with each draft
d_i drawn from p_i and the accept / residual / bonus rule of [AIE]
"Concept", the probability of emitting exactly m accepted drafts d_1..d_m
followed by token y is

    P(m, d_1..d_m, y) = prod_{i<=m} min(p_i(d_i), q_i(d_i))
                        * ( (q_{m+1}(y) - p_{m+1}(y))_+   if m < K
                            q_{K+1}(y)                    if m == K ).

Derivation: d_i ~ p_i is drawn and accepted with probability
p_i(d_i) * min(1, q_i(d_i)/p_i(d_i)) = min(p_i(d_i), q_i(d_i)); a rejection at
position m+1 has total probability sum_d (p - q)_+ = sum_y (q - p)_+ =: Z and
is followed by a draw from (q - p)_+ / Z, so the product is (q - p)_+(y).
Summing the m = 0 term and the accepted-first-draft terms over the first
token gives min(p_1, q_1) + (q_1 - p_1)_+ = q_1: the first emitted token has
exactly the target's law ([AIE] "Concept"; [QS] section 2, losslessness).
"""

import itertools

import numpy as np

__all__ = ["joint_law", "first_token_law", "expected_emitted"]


def joint_law(q_rows, p_rows):
    """Map (m, (d_1..d_m), y) -> probability, for small V and K.

    q_rows: [K+1, V] probabilities; p_rows: [K, V] probabilities.
    """
    q_rows = np.asarray(q_rows, dtype=np.float64)
    p_rows = np.asarray(p_rows, dtype=np.float64)
    k1, v = q_rows.shape
    k = k1 - 1
    law = {}
    for m in range(k + 1):
        for ds in itertools.product(range(v), repeat=m):
            pref = 1.0
            for i, di in enumerate(ds):
                pref *= min(p_rows[i, di], q_rows[i, di])
            if m < k:
                tail = np.maximum(0.0, q_rows[m] - p_rows[m])
            else:
                tail = q_rows[k]
            for y in range(v):
                pr = pref * tail[y]
                if pr > 0:
                    law[(m, tuple(ds), y)] = pr
    return law


def first_token_law(law, v):
    """Marginal law of the first emitted token (slot 0) under ``law``."""
    out = np.zeros(v)
    for (m, ds, y), pr in law.items():
        out[ds[0] if m > 0 else y] += pr
    return out


def expected_emitted(alpha, k):
    """E[n + 1] for a constant per-token acceptance alpha: (1 - a^{K+1}) / (1 - a).

    [AIE] "What determines the speed-up"; equal to the geometric sum
    sum_{i=0..K} alpha^i, which is used when alpha == 1.
    """
    if alpha == 1.0:
        return float(k + 1)
    return (1.0 - alpha ** (k + 1)) / (1.0 - alpha)
