"""Oracle: verification of a draft *tree* (attention and the lossless verifier).

TEST INFRASTRUCTURE ONLY (see the package docstring).  float64 throughout.

The drafter proposes a tree of continuations instead of one chain; the tree
is flattened into one window, an attention mask lets every candidate see only
its ancestors, and the verifier grades every branch in one forward pass; the
surviving path is kept ([TC] "Grading every branch in one pass"; [AIE]
"Concept", EAGLE-2's draft tree and tree attention with a mask that follows
the tree's topology).

Tree encoding (a reading: the pages fix none).  A window of N nodes,
node 0 the root (the last accepted token x0), parent[i] < i for i >= 1
(topological order), so node i's ancestors all precede it.  Node i's K/V
sit at absolute position L0 + i of the cache.  anc[i] is a bit set: bit j is
set iff node j is node i or one of its ancestors (the device's input
encoding, built by the input generators; here the path is found from
parent[] directly).

Attention.  Query node i attends keys [0, L0) and the window keys
{L0 + j : j on the path root -> i}: exactly causal attention over that
path, for every node in one pass.  (Rotary positions follow the node's depth, not
its slot; they are applied to q and k before this step.)

Verifier (the reading of "the surviving path is kept" that keeps the
lossless guarantee of [AIE] "Concept").  Rows: target row v is q_v, the
verifier's distribution after the path to node v; draft row v is p_v, the
law node v's children were drawn from, independently of one another.
Starting at the root with q' = q_v:
  * the children c of v are tested in index order: accept c iff
    u[c] < min(1, q'(d_c) / p_v(d_c)) (p_v(d_c) <= 0 accepts);
  * after a rejected child, q' <- (q' - p_v)_+ normalised (recursive rejection
    sampling; a zero-mass residual leaves q' unchanged);
  * the first accepted child is emitted and becomes v (q' <- q_v);
  * when every child of v is rejected, or v is a leaf, the final token is
    drawn from q' with u[0] by inverse CDF and the call ends.
With children drawn independently from p_v, the token emitted at every node
has exactly the law q_v, the same property the chain verifier has.  A chain
(parent[i] = i - 1) is exactly the chain verifier with u[i] <-> u_{i-1} and
u[0] <-> u_K.

Greedy (T <= 0): at node v the first child whose token equals argmax(q_v)
(lowest index on ties) is accepted; otherwise argmax(q_v) is emitted and the
call ends: the target's own greedy continuation ([PHX] "What it does").

Commit: n accepted nodes; the caller compacts their K/V (slots L0 + node)
into positions L0 + 1 .. L0 + n, and kv_len becomes L0 + n + 1 ([AIE]
"Rolling back the KV cache").
"""

import numpy as np

from .reject import widen, softmax_rows, _inverse_cdf
from .attention import gather_kv

__all__ = ["children_of", "path_to_root", "tree_attention", "reject_sample_tree"]


def children_of(parent):
    """Children lists in increasing index order."""
    parent = np.asarray(parent, dtype=np.int64)
    kids = [[] for _ in range(parent.shape[0])]
    for i in range(1, parent.shape[0]):
        kids[parent[i]].append(i)
    return kids


def path_to_root(parent, i):
    """Nodes on the path root -> i (both included), in increasing index
    order, by walking parent links from i."""
    parent = np.asarray(parent, dtype=np.int64)
    path = [i]
    while parent[path[-1]] >= 0:
        p = int(parent[path[-1]])
        if p >= path[-1]:
            raise ValueError("parents must precede their children")
        path.append(p)
    if path[-1] != 0:
        raise ValueError("node %d does not reach the root" % i)
    return path[::-1]


def tree_attention(q, k_cache, v_cache, block_table, kv_len, parent, scale=None,
                   batch_indices=None):
    """Attention outputs [B, N, Hq, D] (float64) for a flattened draft tree.

    Args as oracle.attention.verify_attention, plus parent: [N] or [B, N]
    parent arrays (one tree shape per sequence allowed).  Node i sees keys
    [0, L0) and L0 + j for every node j on its path from the root (itself
    included), found by walking its parent links.
    """
    qq = widen(q)
    b_sz, n, hq, d = qq.shape
    if scale is None or scale <= 0:
        scale = 1.0 / np.sqrt(d)
    par = np.asarray(parent, dtype=np.int64)
    if par.ndim == 1:
        par = np.broadcast_to(par, (b_sz, n))
    out = np.full(qq.shape, np.nan)
    idx = range(b_sz) if batch_indices is None else batch_indices
    for b in idx:
        l0 = int(kv_len[b])
        keys, vals = gather_kv(k_cache, v_cache, block_table, b, l0 + n)
        hkv = keys.shape[1]
        for i in range(n):
            win = path_to_root(par[b], i)
            pos = np.concatenate([np.arange(l0), l0 + np.asarray(win, dtype=np.int64)])
            for h in range(hq):
                g = h // (hq // hkv)
                s = scale * (keys[pos, g, :] @ qq[b, i, h])
                s = s - s.max()
                e = np.exp(s)
                out[b, i, h] = (e / e.sum()) @ vals[pos, g, :]
    return out


def reject_sample_tree(target_logits, draft_logits, parent, tokens, uniforms,
                       temperature, eps_accept=1e-5, eps_sample=1e-10):
    """One tree-verify call for a batch of sequences.

    Args:
      target_logits: [B, N, V] (float or bf16 bits): row v is q_v.
      draft_logits:  [B, N, V] or None when every T_b <= 0: row v is p_v
                     (rows of leaves are not used).
      parent:        [N] or [B, N] parent indices (parent[0] = -1).
      tokens:        [B, N] token of node i (entry 0 unused).
      uniforms:      [B, N] in [0, 1): u[i] tests node i, u[0] the final draw.
      temperature:   [B]; T_b <= 0 selects greedy.

    Returns a dict with
      out_tokens   [B, N] int32: path tokens, then the final token, -1 padded
      out_nodes    [B, N] int32: accepted nodes along the path, -1 padded
      num_accepted [B] int32
      flag_accept  [B] bool (F1: an examined test with |u - ratio| < eps_accept)
      flag_sample  [B] bool (F2: final draw within eps_sample of a CDF edge)
    """
    tl = widen(target_logits)
    b_sz, n, v = tl.shape
    par = np.asarray(parent, dtype=np.int64)
    if par.ndim == 1:
        par = np.broadcast_to(par, (b_sz, n))
    tok = np.asarray(tokens, dtype=np.int64).reshape(b_sz, n)
    u = np.asarray(uniforms, dtype=np.float64).reshape(b_sz, n)
    t = np.asarray(temperature, dtype=np.float64).reshape(b_sz)
    dl = None if draft_logits is None else widen(draft_logits).reshape(b_sz, n, v)

    out_tok = np.full((b_sz, n), -1, dtype=np.int32)
    out_node = np.full((b_sz, n), -1, dtype=np.int32)
    n_acc = np.zeros(b_sz, dtype=np.int32)
    f1 = np.zeros(b_sz, dtype=bool)
    f2 = np.zeros(b_sz, dtype=bool)

    for b in range(b_sz):
        kids = children_of(par[b])
        path = []
        node = 0
        if t[b] <= 0:
            while True:
                am = int(np.argmax(tl[b, node]))     # lowest index on ties
                nxt = next((c for c in kids[node] if tok[b, c] == am), None)
                if nxt is None:
                    final = am
                    break
                path.append(nxt)
                node = nxt
        else:
            if dl is None:
                raise ValueError("draft_logits required when some T_b > 0")
            q = softmax_rows(tl[b], t[b])            # [N, V]
            p = softmax_rows(dl[b], t[b])
            while True:
                qv = q[node]
                accepted = None
                for c in kids[node]:
                    d = tok[b, c]
                    pd = p[node, d]
                    r = qv[d] / pd if pd > 0 else np.inf
                    if abs(u[b, c] - r) < eps_accept:
                        f1[b] = True
                    if pd <= 0 or u[b, c] < min(1.0, r):
                        accepted = c
                        break
                    resid = np.maximum(0.0, qv - p[node])
                    z = resid.sum()
                    if z > 0:
                        qv = resid / z
                if accepted is None:
                    tk, fl = _inverse_cdf(qv[None, :], np.array([u[b, 0]]), eps_sample)
                    final = int(tk[0])
                    f2[b] = bool(fl[0])
                    break
                path.append(accepted)
                node = accepted
        m = len(path)
        n_acc[b] = m
        out_node[b, :m] = path
        out_tok[b, :m] = tok[b, path]
        out_tok[b, m] = final
    return {"out_tokens": out_tok, "out_nodes": out_node, "num_accepted": n_acc,
            "flag_accept": f1, "flag_sample": f2}
