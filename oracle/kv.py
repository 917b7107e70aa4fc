"""Oracle: the window's K/V in the paged cache, the commit, and the page pool.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Plain numpy copies and
a pure-Python page pool; no arithmetic on the values.

What the pages fix ([AIE] "Rolling back the KV cache"; [SGL] the provisional
KV layer): verification extends the verifier's KV cache by the window; a
rejection at position j makes everything after it wrong; two common ways to
handle it are to write the window into a scratch buffer and commit on
acceptance, or to keep the physical cache plus a logical length.  The
readings below fill in what the pages leave open.

Layouts (as the verify attention takes them): K cache [NB, Hkv, D/x, 16, x],
V cache [NB, Hkv, D, 16] (x = 8 for bf16, 4 for fp32); token p of sequence
b lives in page block_table[b][p // 16], slot p % 16.  The window's K/V as
the projection produces them: [B, N, Hkv, D], row i for position L0 + i
(chain) or for tree node i.

append_window  -- write the window rows into their cache slots L0 + i.
commit         -- after the verifier: the root and the accepted nodes'
                  K/V at L0 + 0 .. L0 + n, taken from a scratch buffer or
                  from the window slots in place (tree compaction; a chain
                  in place is a no-op).
PagePool       -- the host-side page list: reserve (provisional pages for
                  the window), commit (free every page wholly past the
                  committed length), release; the lowest-numbered free page
                  is always handed out first.
"""

import heapq

import numpy as np

__all__ = ["append_window", "commit", "accepted_sources", "PagePool"]

BLOCK = 16


def _slot(block_table, b, p):
    return int(np.asarray(block_table)[b, p // BLOCK]), p % BLOCK


def _put(k_cache, v_cache, blk, tok, g, krow, vrow):
    nb, hkv, dx, blk_sz, x = k_cache.shape
    k_cache[blk, g, :, tok, :] = np.asarray(krow).reshape(dx, x)
    v_cache[blk, g, :, tok] = vrow


def _get(k_cache, v_cache, blk, tok, g):
    return k_cache[blk, g, :, tok, :].reshape(-1).copy(), v_cache[blk, g, :, tok].copy()


def append_window(k_cache, v_cache, block_table, kv_len, k_new, v_new):
    """Copies of the caches with window row i of sequence b at position L0_b + i."""
    kc, vc = np.array(k_cache, copy=True), np.array(v_cache, copy=True)
    b_sz, n, hkv, d = k_new.shape
    for b in range(b_sz):
        l0 = int(kv_len[b])
        for i in range(n):
            blk, tok = _slot(block_table, b, l0 + i)
            for g in range(hkv):
                _put(kc, vc, blk, tok, g, k_new[b, i, g], v_new[b, i, g])
    return kc, vc


def accepted_sources(num_accepted, nodes, b):
    """Window rows that survive in sequence b, in order: the root, then the
    accepted nodes (a chain's accepted drafts are rows 1..n)."""
    n = int(num_accepted[b])
    if nodes is None:
        return list(range(n + 1))
    return [0] + [int(x) for x in np.asarray(nodes)[b, :n]]


def commit(k_cache, v_cache, block_table, kv_len_after, num_accepted, nodes=None,
           k_src=None, v_src=None):
    """Copies of the caches after the commit of one verify call.

    kv_len_after is the verifier's committed length L0 + n + 1, so
    L0 = kv_len_after - n - 1.  Surviving row j (accepted_sources) goes to
    position L0 + j, from k_src/v_src [B, N, Hkv, D] when given, else from
    its window slot L0 + row of the cache.  Every source is read before any
    slot is written.  The emitted token's K/V are not here: the next verify
    call writes them as its root.
    """
    kc, vc = np.array(k_cache, copy=True), np.array(v_cache, copy=True)
    hkv = kc.shape[1]
    for b in range(len(num_accepted)):
        n = int(num_accepted[b])
        l0 = int(kv_len_after[b]) - n - 1
        src_rows = accepted_sources(num_accepted, nodes, b)
        vals = []
        for row in src_rows:
            per_head = []
            for g in range(hkv):
                if k_src is not None:
                    per_head.append((np.array(k_src[b, row, g]), np.array(v_src[b, row, g])))
                else:
                    blk, tok = _slot(block_table, b, l0 + row)
                    per_head.append(_get(k_cache, v_cache, blk, tok, g))
            vals.append(per_head)
        for j, per_head in enumerate(vals):
            blk, tok = _slot(block_table, b, l0 + j)
            for g, (kr, vr) in enumerate(per_head):
                _put(kc, vc, blk, tok, g, kr, vr)
    return kc, vc


class PagePool:
    """Pure-Python model of the host page list.

    Every page is either free or owned by exactly one sequence.  A sequence
    owns pages for positions [0, reserved); reserve() grows that range (new
    pages are the lowest-numbered free ones, appended in order); commit(len)
    frees every page whose first position is >= len (the provisional pages
    a rejection left empty, or an explicit rollback) and keeps the rest;
    release() frees all of a sequence's pages.  Errors raise ValueError and
    leave the pool unchanged.
    """

    def __init__(self, num_blocks, max_seqs, max_blocks_per_seq):
        self.num_blocks = num_blocks
        self.max_seqs = max_seqs
        self.mbps = max_blocks_per_seq
        self.free = list(range(num_blocks))
        heapq.heapify(self.free)
        self.pages = [[] for _ in range(max_seqs)]

    def _check_seq(self, seq):
        if not 0 <= seq < self.max_seqs:
            raise ValueError("sequence out of range")

    def reserve(self, seq, total_len):
        self._check_seq(seq)
        need = -(-int(total_len) // BLOCK)
        if need > self.mbps:
            raise ValueError("more pages than a block table row holds")
        extra = need - len(self.pages[seq])
        if extra > len(self.free):
            raise ValueError("out of pages")
        for _ in range(max(0, extra)):
            self.pages[seq].append(heapq.heappop(self.free))

    def commit(self, seq, length):
        self._check_seq(seq)
        keep = -(-int(length) // BLOCK)
        if length < 0 or keep > len(self.pages[seq]):
            raise ValueError("commit past the reserved pages")
        for blk in self.pages[seq][keep:]:
            heapq.heappush(self.free, blk)
        del self.pages[seq][keep:]

    def release(self, seq):
        self.commit(seq, 0)

    def free_count(self):
        return len(self.free)

    def block_table(self):
        t = np.zeros((self.max_seqs, self.mbps), dtype=np.int32)
        for s, pg in enumerate(self.pages):
            t[s, :len(pg)] = pg
        return t

    def seq_blocks(self, seq):
        return len(self.pages[seq])
