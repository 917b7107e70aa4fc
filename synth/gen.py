"""Seeded generators for the verify step's inputs.

Only randomness and encodings live here (no softmax, no accept test, no
attention): normal logits rounded to bf16, a noisy draft, draft tokens drawn
by the Gumbel-max trick (the drafter's job, upstream of the verifier),
24-bit uniforms, context lengths, shuffled page tables and random Q/K/V.

Every generator takes a ``numpy.random.Generator``; callers derive those from
``numpy.random.SeedSequence`` so that each stream is independent.
"""

import numpy as np

__all__ = ["bf16_bits", "bf16_to_f32", "uniforms24", "make_reject_inputs",
           "make_tree_reject_inputs", "make_attn_inputs", "make_window_kv", "kv_layout_x",
           "BLOCK"]

BLOCK = 16  # tokens per KV page


def bf16_bits(x):
    """Round float32 values to bf16 (round to nearest, ties to even) -> uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    rounding = ((u >> 16) & 1) + np.uint32(0x7FFF)
    out = ((u + rounding) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_to_f32(bits):
    """bf16 bits (uint16) -> the float32 values they encode (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def uniforms24(rng, shape):
    """Uniforms on the 24-bit grid k * 2^-24, k in [0, 2^24): exactly representable
    in float32 and never equal to 1."""
    k = rng.integers(0, 1 << 24, size=shape, dtype=np.uint32)
    return (k.astype(np.float32) * np.float32(2.0 ** -24)).astype(np.float32)


def _encode(x, dtype):
    if dtype == "bf16":
        return bf16_bits(x)
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    raise ValueError(dtype)


def _decode(x, dtype):
    return bf16_to_f32(x) if dtype == "bf16" else np.asarray(x, dtype=np.float32)


def _draft_tokens(rng, draft_vals, temperature):
    """Draft tokens: argmax(draft / T + Gumbel) when T > 0 (an exact draw from
    softmax(draft / T)), plain argmax of the draft logits when T <= 0.

    ``draft_vals`` [B, K, V] float32 values of the encoded draft logits.
    Processed one sequence at a time to bound memory at large V.
    """
    b_sz, k, v = draft_vals.shape
    out = np.empty((b_sz, k), dtype=np.int32)
    for b in range(b_sz):
        t = float(temperature[b])
        x = draft_vals[b].astype(np.float64)
        if t > 0:
            g = -np.log(-np.log(rng.random((k, v)) * (1 - 2e-16) + 1e-16))
            out[b] = np.argmax(x / t + g, axis=-1)
        else:
            out[b] = np.argmax(x, axis=-1)
    return out


def make_reject_inputs(seed, B, K, V, dtype="bf16", logit_std=2.0,
                       draft_sigma=0.51, temperature=1.0, shared_rows=False):
    """Inputs of one reject-sample call.

    target logits ~ N(0, logit_std), draft = target + N(0, draft_sigma)
    (standard deviations), both encoded as ``dtype``.  ``temperature`` is a
    scalar or a length-B array.  With ``shared_rows`` every sequence gets the
    same target / draft rows (batched trials of one verify) while the draft
    tokens and uniforms stay independent per sequence.

    Returns a dict of numpy arrays: target [B,K+1,V], draft [B,K,V] (uint16
    bf16 bits or float32), draft_tokens [B,K] int32, uniforms [B,K+1]
    float32, temperature [B] float32.
    """
    ss = np.random.SeedSequence(seed)
    r_t, r_n, r_g, r_u = [np.random.default_rng(s) for s in ss.spawn(4)]
    temps = np.broadcast_to(np.asarray(temperature, dtype=np.float32), (B,)).copy()
    rows_b = 1 if shared_rows else B
    tgt = (r_t.standard_normal((rows_b, K + 1, V), dtype=np.float32)
           * np.float32(logit_std))
    noise = (r_n.standard_normal((rows_b, K, V), dtype=np.float32)
             * np.float32(draft_sigma))
    drf = tgt[:, :K, :] + noise
    tgt_e = _encode(tgt, dtype)
    drf_e = _encode(drf, dtype)
    del tgt, noise, drf
    if shared_rows:
        tgt_e = np.broadcast_to(tgt_e, (B, K + 1, V))
        drf_e = np.broadcast_to(drf_e, (B, K, V))
    if shared_rows:
        # Per-trial Gumbel draws over the one shared row set.
        vals = _decode(drf_e[0], dtype).astype(np.float64)
        toks = np.empty((B, K), dtype=np.int32)
        pos_t = temps > 0
        if (~pos_t).any():
            toks[~pos_t] = np.argmax(vals, axis=-1)
        idx = np.nonzero(pos_t)[0]
        step = max(1, (1 << 22) // max(1, K * V))
        for s in range(0, idx.size, step):
            sel = idx[s:s + step]
            g = -np.log(-np.log(r_g.random((sel.size, K, V)) * (1 - 2e-16) + 1e-16))
            toks[sel] = np.argmax(vals[None] / temps[sel, None, None] + g, axis=-1)
    else:
        toks = _draft_tokens(r_g, _decode(drf_e, dtype), temps)
    u = uniforms24(r_u, (B, K + 1))
    return {"target": tgt_e, "draft": drf_e, "draft_tokens": toks,
            "uniforms": u, "temperature": temps}


def make_tree_reject_inputs(seed, B, parent, V, dtype="bf16", logit_std=2.0,
                            draft_sigma=0.51, temperature=1.0, shared_rows=False):
    """Inputs of one tree-verify call over the tree given by ``parent`` (N nodes):
    one tree [N] for the batch, or one per sequence [B, N].

    Rows as in make_reject_inputs, one target and one draft row per node
    (target [B,N,V], draft [B,N,V]).  Node i's token is a fresh draw from
    softmax(draft[parent[i]] / T) by the Gumbel-max trick, independently for
    every child (T > 0); a greedy drafter (T <= 0) gives the children of a
    node the top-ranked tokens of its draft row, in order.  Token 0 (the
    root's) is 0 and unused.  uniforms [B,N] float32.
    """
    par = np.asarray(parent, dtype=np.int64)
    n = par.shape[-1]
    par2 = np.broadcast_to(par, (B, n))
    ss = np.random.SeedSequence(seed)
    r_t, r_n, r_g, r_u = [np.random.default_rng(s) for s in ss.spawn(4)]
    temps = np.broadcast_to(np.asarray(temperature, dtype=np.float32), (B,)).copy()
    rows_b = 1 if shared_rows else B
    tgt = r_t.standard_normal((rows_b, n, V), dtype=np.float32) * np.float32(logit_std)
    drf = tgt + r_n.standard_normal((rows_b, n, V), dtype=np.float32) * np.float32(draft_sigma)
    tgt_e = _encode(tgt, dtype)
    drf_e = _encode(drf, dtype)
    del tgt, drf
    if shared_rows:
        tgt_e = np.broadcast_to(tgt_e, (B, n, V))
        drf_e = np.broadcast_to(drf_e, (B, n, V))
    toks = np.zeros((B, n), dtype=np.int32)
    rank = np.zeros((B, n), dtype=np.int64)     # position of node i among its siblings
    for b in range(B if par.ndim == 2 else 1):
        seen = {}
        for i in range(1, n):
            rank[b, i] = seen.get(int(par2[b, i]), 0)
            seen[int(par2[b, i])] = rank[b, i] + 1
    if par.ndim == 1:
        rank[1:] = rank[0]
    step = max(1, (1 << 22) // max(1, (n - 1) * V))
    for s0 in range(0, B, step):
        sel = np.arange(s0, min(B, s0 + step))
        vals = _decode(drf_e[sel], dtype).astype(np.float64)          # [S, N, V]
        pv = np.take_along_axis(vals, par2[sel, 1:, None], axis=1)    # [S, N-1, V]
        t = temps[sel].astype(np.float64)
        g = -np.log(-np.log(r_g.random(pv.shape) * (1 - 2e-16) + 1e-16))
        sampled = np.argmax(pv / np.where(t > 0, t, 1.0)[:, None, None] + g, axis=-1)
        order = np.argsort(-pv, axis=-1, kind="stable")               # greedy: top-k
        greedy_tok = np.take_along_axis(order, rank[sel, 1:, None], axis=-1)[..., 0]
        toks[sel, 1:] = np.where((t > 0)[:, None], sampled, greedy_tok)
    u = uniforms24(r_u, (B, n))
    return {"target": tgt_e, "draft": drf_e, "tokens": toks, "parent": par.astype(np.int32),
            "uniforms": u, "temperature": temps}


def make_window_kv(seed, B, N, Hkv, D, dtype="bf16"):
    """The window's K/V as the projection produces them: k_new, v_new
    [B, N, Hkv, D], N(0, 1), bf16 bits or float32."""
    r_k, r_v = [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(2)]
    kn = r_k.standard_normal((B, N, Hkv, D), dtype=np.float32)
    vn = r_v.standard_normal((B, N, Hkv, D), dtype=np.float32)
    return _encode(kn, dtype), _encode(vn, dtype)


def kv_layout_x(dtype):
    """Elements per 16-byte chunk in the key layout [NB, Hkv, D/x, 16, x]."""
    return 8 if dtype == "bf16" else 4


def make_attn_inputs(seed, B, K, Hq, Hkv, D, ctx, dtype="bf16",
                     q_scale=1.0, spare_blocks=7, max_blocks_per_seq=None):
    """Inputs of one verify-attention call with a shuffled paged KV cache.

    ``ctx`` is an int (every sequence's committed length L0) or a (lo, hi)
    pair: L0 ~ uniform integers in [lo, hi].  Every position 0..L0+K (the
    committed prefix plus the K+1 window) holds random K/V.  Pages are a
    random permutation of the physical blocks, plus ``spare_blocks``
    unused ones; unused block-table entries are 0.

    Returns numpy arrays: q [B,K+1,Hq,D], k_cache [NB,Hkv,D/x,16,x],
    v_cache [NB,Hkv,D,16] (bf16 bits or float32), block_table
    [B, max_blocks_per_seq] int32, kv_len [B] int32.
    """
    ss = np.random.SeedSequence(seed)
    r_l, r_p, r_q, r_k, r_v = [np.random.default_rng(s) for s in ss.spawn(5)]
    if np.isscalar(ctx):
        l0 = np.full(B, int(ctx), dtype=np.int64)
    else:
        l0 = r_l.integers(int(ctx[0]), int(ctx[1]) + 1, size=B)
    need = (l0 + K + 1 + BLOCK - 1) // BLOCK
    mbps = int(need.max()) if max_blocks_per_seq is None else int(max_blocks_per_seq)
    assert mbps >= need.max()
    nb = int(need.sum()) + spare_blocks
    perm = r_p.permutation(nb).astype(np.int32)
    bt = np.zeros((B, mbps), dtype=np.int32)
    off = 0
    for b in range(B):
        bt[b, :need[b]] = perm[off:off + need[b]]
        off += need[b]
    x = kv_layout_x(dtype)
    q = r_q.standard_normal((B, K + 1, Hq, D), dtype=np.float32) * np.float32(q_scale)
    kc = r_k.standard_normal((nb, Hkv, D // x, BLOCK, x), dtype=np.float32)
    vc = r_v.standard_normal((nb, Hkv, D, BLOCK), dtype=np.float32)
    return {"q": _encode(q, dtype), "k_cache": _encode(kc, dtype),
            "v_cache": _encode(vc, dtype), "block_table": bt,
            "kv_len": l0.astype(np.int32)}
