"""Oracle: grouped-query attention of the K+1 verify positions over a paged KV cache.

TEST INFRASTRUCTURE ONLY (see the package docstring).  float64 throughout.

The verifier scores the last accepted token x0 and the drafts d_1..d_K in
one forward pass over prefix + drafts ([AIE] "Concept": the verifier runs
once over prefix + d_1 + ... + d_N and returns q_1..q_{N+1}; [PHX] "What it
does": all guesses are checked in one pass).  Inside that pass each
attention layer computes, for sequence b with committed length L0 = kv_len[b],
query position i in 0..K (absolute position t = L0 + i) and query head h:

    g   = h // (Hq / Hkv)                     (the KV head shared by h)
    s_j = scale * <q[b, i, h], k_j>            for keys j = 0..t
    o   = sum_j softmax(s)_j * v_j

Keys after t are masked: causal inside the draft window.  The window's own
K/V (positions L0..L0+K) are already in the cache when the call is made.

Paged cache layout (a reading: the pages fix no layout).  Token j of
sequence b lives in page ``block_table[b, j // 16]`` at slot ``j % 16``:
  k_cache [num_blocks, Hkv, D // x, 16, x]   x = 16 bytes / element size
  v_cache [num_blocks, Hkv, D, 16]
so key j is ``k_cache[blk, g, :, j % 16, :].reshape(D)`` and value j is
``v_cache[blk, g, :, j % 16]``.
"""

import numpy as np

from .reject import widen

__all__ = ["gather_kv", "verify_attention", "verify_attention_row"]


def gather_kv(k_cache, v_cache, block_table, b, length):
    """Contiguous float64 keys / values [length, Hkv, D] of sequence b, by page lookup.

    The pages are gathered first and widened afterwards, so only the
    sequence's own tokens are converted.
    """
    nb, hkv, dx, blk, x = k_cache.shape
    d = dx * x
    pos = np.arange(length)
    blocks = np.asarray(block_table)[b, pos // blk]
    slots = pos % blk
    # Advanced indices split by slices put the token axis first.
    keys = widen(k_cache[blocks, :, :, slots, :]).reshape(length, hkv, d)
    vals = widen(v_cache[blocks, :, :, slots]).reshape(length, hkv, d)
    return keys, vals


def verify_attention_row(q, keys, vals, t, h, hq, scale):
    """Attention output of one query row (head h, absolute position t)."""
    hkv = keys.shape[1]
    g = h // (hq // hkv)
    kk = keys[: t + 1, g, :]
    vv = vals[: t + 1, g, :]
    s = scale * (kk @ q)
    s = s - s.max()
    e = np.exp(s)
    return (e / e.sum()) @ vv


def verify_attention(q, k_cache, v_cache, block_table, kv_len, scale=None,
                     batch_indices=None):
    """Attention outputs [B, K+1, Hq, D] (float64) for the verify window.

    Args:
      q:           [B, K+1, Hq, D] float32 or bf16 bits (uint16).
      k_cache:     [num_blocks, Hkv, D//x, 16, x] same kind.
      v_cache:     [num_blocks, Hkv, D, 16] same kind.
      block_table: [B, max_blocks_per_seq] int.
      kv_len:      [B] committed length L0 before the window.
      scale:       softmax scale; None or <= 0 means 1/sqrt(D).
      batch_indices: optional subset of sequences to compute (others are nan).
    """
    qq = widen(q)
    b_sz, k1, hq, d = qq.shape
    if scale is None or scale <= 0:
        scale = 1.0 / np.sqrt(d)
    out = np.full(qq.shape, np.nan)
    idx = range(b_sz) if batch_indices is None else batch_indices
    for b in idx:
        l0 = int(kv_len[b])
        keys, vals = gather_kv(k_cache, v_cache, block_table, b, l0 + k1)
        for i in range(k1):
            for h in range(hq):
                out[b, i, h] = verify_attention_row(qq[b, i, h], keys, vals,
                                                    l0 + i, h, hq, scale)
    return out
