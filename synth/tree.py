"""Draft-tree shapes and their encoding as device inputs.

Topology only (no verify arithmetic): parent arrays of chains and of full
trees given by branching factors, children lists, and the ancestor-or-self
bit sets that spec_verify_attn_tree takes as its ``anc`` input (bit j of
node i's word is set iff node j is node i or one of its ancestors).
"""

import numpy as np

__all__ = ["chain_parents", "tree_parents", "random_parents", "mixed_parents", "children",
           "ancestor_bits"]


def chain_parents(n):
    """parent[] of a chain of n nodes: node i's parent is i - 1."""
    return np.arange(-1, n - 1, dtype=np.int32)


def tree_parents(shape):
    """parent[] of a full tree given by branching factors per level, breadth
    first: shape (2, 2, 2) is a root with 2 children, each with 2, each with 2
    (15 nodes)."""
    parents = [-1]
    level = [0]
    for k in shape:
        nxt = []
        for v in level:
            for _ in range(k):
                parents.append(v)
                nxt.append(len(parents) - 1)
        level = nxt
    return np.asarray(parents, dtype=np.int32)


def random_parents(rng, n):
    """parent[] of a random tree of n nodes in topological order: node i's
    parent uniform over 0 .. i - 1."""
    par = np.full(n, -1, dtype=np.int32)
    for i in range(1, n):
        par[i] = rng.integers(0, i)
    return par


def mixed_parents(seed, B, n):
    """[B, n] parent arrays, one tree per sequence, cycling through a chain,
    a star (the root's n - 1 children), a two-level tree (root with two
    children, the rest spread under them) and a random tree."""
    rng = np.random.default_rng(seed)
    two = np.full(n, -1, dtype=np.int32)
    for i in range(1, n):
        two[i] = 0 if i <= 2 else 1 + (i - 3) % 2
    out = np.empty((B, n), dtype=np.int32)
    for b in range(B):
        k = b % 4
        out[b] = (chain_parents(n) if k == 0 else np.r_[-1, np.zeros(n - 1, np.int32)]
                  if k == 1 else two if k == 2 else random_parents(rng, n))
    return out


def children(parent):
    """Children lists in increasing index order."""
    parent = np.asarray(parent, dtype=np.int64)
    kids = [[] for _ in range(parent.shape[0])]
    for i in range(1, parent.shape[0]):
        kids[parent[i]].append(i)
    return kids


def ancestor_bits(parent):
    """Ancestor-or-self bit sets [N] (uint64) of a parent[] array in
    topological order (parent[i] < i); raises ValueError otherwise."""
    parent = np.asarray(parent, dtype=np.int64)
    n = parent.shape[0]
    anc = np.zeros(n, dtype=np.uint64)
    for i in range(n):
        a = np.uint64(1) << np.uint64(i)
        if i > 0:
            if not 0 <= parent[i] < i:
                raise ValueError("parent[%d] = %d: parents must precede their children"
                                 % (i, parent[i]))
            a |= anc[parent[i]]
        anc[i] = a
    return anc
