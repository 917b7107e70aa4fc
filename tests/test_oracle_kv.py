"""Pins of oracle.kv: the window append and the commit against hand-computed
layouts and against oracle.attention.gather_kv (an independent page lookup,
itself pinned by the attention tests), and the page pool's invariants."""

import numpy as np
import pytest

from oracle import kv as okv
from oracle.attention import gather_kv


def _cache(rng, nb, hkv, d, x):
    kc = rng.standard_normal((nb, hkv, d // x, 16, x))
    vc = rng.standard_normal((nb, hkv, d, 16))
    return kc, vc


def test_append_layout_by_hand():
    # One sequence, L0 = 14, window of 4: positions 14, 15 in page 2 (slots
    # 14, 15) and 16, 17 in page 0 (slots 0, 1).  D = 16, x = 8.
    kc = np.zeros((3, 1, 2, 16, 8))
    vc = np.zeros((3, 1, 16, 16))
    bt = np.array([[2, 0]], np.int32)
    kn = np.arange(4 * 16, dtype=np.float64).reshape(1, 4, 1, 16) + 1
    vn = -kn
    k2, v2 = okv.append_window(kc, vc, bt, np.array([14]), kn, vn)
    assert k2[2, 0, 1, 15, 3] == kn[0, 1, 0, 11]      # row 1 -> pos 15, d = 8 + 3
    assert k2[2, 0, 0, 14, 0] == kn[0, 0, 0, 0]
    assert k2[0, 0, 0, 1, 7] == kn[0, 3, 0, 7]        # row 3 -> pos 17 -> page 0 slot 1
    assert v2[0, 0, 5, 0] == vn[0, 2, 0, 5]           # row 2 -> pos 16 -> page 0 slot 0
    assert v2[2, 0, 15, 15] == vn[0, 1, 0, 15]
    assert np.count_nonzero(k2) == 64 and np.count_nonzero(v2) == 64
    assert not k2[1].any() and not v2[1].any()        # page 1 untouched


@pytest.mark.parametrize("x", [8, 4])
def test_append_then_gather(x):
    rng = np.random.default_rng(5)
    B, N, hkv, d, nb = 3, 5, 2, 16, 20
    kc, vc = _cache(rng, nb, hkv, d, x)
    bt = rng.permutation(nb)[:B * 6].reshape(B, 6).astype(np.int32)
    kv_len = np.array([0, 17, 60], np.int32)
    kn = rng.standard_normal((B, N, hkv, d))
    vn = rng.standard_normal((B, N, hkv, d))
    k2, v2 = okv.append_window(kc, vc, bt, kv_len, kn, vn)
    for b in range(B):
        L = int(kv_len[b]) + N
        k_old, v_old = gather_kv(kc, vc, bt, b, 6 * 16)
        k_new, v_new = gather_kv(k2, v2, bt, b, 6 * 16)
        l0 = int(kv_len[b])
        assert np.array_equal(k_new[l0:L], kn[b]) and np.array_equal(v_new[l0:L], vn[b])
        assert np.array_equal(k_new[:l0], k_old[:l0]) and np.array_equal(k_new[L:], k_old[L:])
        assert np.array_equal(v_new[:l0], v_old[:l0]) and np.array_equal(v_new[L:], v_old[L:])


def test_commit_chain_in_place_is_identity():
    rng = np.random.default_rng(6)
    kc, vc = _cache(rng, 8, 2, 16, 8)
    bt = np.arange(8, dtype=np.int32).reshape(2, 4)
    n = np.array([0, 3], np.int32)
    kv_after = np.array([10, 40], np.int32) + n + 1
    k2, v2 = okv.commit(kc, vc, bt, kv_after, n)
    assert np.array_equal(k2, kc) and np.array_equal(v2, vc)


def test_commit_chain_from_scratch():
    rng = np.random.default_rng(7)
    kc, vc = _cache(rng, 8, 2, 16, 8)
    bt = np.arange(8, dtype=np.int32).reshape(2, 4)
    N = 6
    ks = rng.standard_normal((2, N, 2, 16))
    vs = rng.standard_normal((2, N, 2, 16))
    n = np.array([2, 5], np.int32)
    l0 = np.array([13, 30], np.int32)
    k2, v2 = okv.commit(kc, vc, bt, l0 + n + 1, n, k_src=ks, v_src=vs)
    for b in range(2):
        kk, vv = gather_kv(k2, v2, bt, b, 64)
        k0, v0 = gather_kv(kc, vc, bt, b, 64)
        m = int(n[b]) + 1
        assert np.array_equal(kk[l0[b]:l0[b] + m], ks[b, :m])
        assert np.array_equal(vv[l0[b]:l0[b] + m], vs[b, :m])
        keep = np.r_[0:l0[b], l0[b] + m:64]
        assert np.array_equal(kk[keep], k0[keep]) and np.array_equal(vv[keep], v0[keep])


def test_commit_tree_in_place_overlap_by_hand():
    # L0 = 3, accepted path nodes 2 then 5: position 3 keeps the root (slot 3),
    # position 4 gets old slot 5 (node 2), position 5 gets old slot 8 (node 5).
    # Slot 5 is both a source and a destination: it must be read first.
    kc = np.zeros((1, 1, 1, 16, 8))
    vc = np.zeros((1, 1, 8, 16))
    for p in range(16):
        kc[0, 0, 0, p, :] = 100 + p
        vc[0, 0, :, p] = 200 + p
    nodes = np.array([[2, 5, -1, -1, -1, -1, -1]], np.int32)
    k2, v2 = okv.commit(kc, vc, np.zeros((1, 1), np.int32), np.array([3 + 2 + 1]),
                        np.array([2]), nodes=nodes)
    got = [k2[0, 0, 0, p, 0] for p in range(16)]
    want = [100 + p for p in range(16)]
    want[4], want[5] = 105, 108
    assert got == want
    assert [v2[0, 0, 3, p] for p in (3, 4, 5, 6)] == [203, 205, 208, 206]


def test_page_pool_by_hand():
    pool = okv.PagePool(num_blocks=6, max_seqs=2, max_blocks_per_seq=4)
    pool.reserve(0, 20)            # pages 0, 1
    pool.reserve(1, 5)             # page 2
    pool.reserve(0, 40)            # + page 3
    assert pool.block_table()[0].tolist() == [0, 1, 3, 0]
    pool.commit(0, 17)             # positions 0..16 stay: pages 0, 1; page 3 freed
    assert pool.free_count() == 3 and pool.seq_blocks(0) == 2
    pool.reserve(1, 33)            # lowest free first: 3, then 4
    assert pool.block_table()[1].tolist() == [2, 3, 4, 0]
    pool.release(0)
    assert pool.free_count() == 3
    pool.reserve(0, 1)
    assert pool.block_table()[0, 0] == 0
    with pytest.raises(ValueError):
        pool.reserve(0, 16 * 5)    # more than a table row
    with pytest.raises(ValueError):
        pool.commit(1, 16 * 4)     # past what was reserved


def test_page_pool_random_ops_keep_every_page_once():
    rng = np.random.default_rng(11)
    nb, S, mbps = 40, 5, 10
    pool = okv.PagePool(nb, S, mbps)
    lens = [0] * S
    for step in range(3000):
        s = int(rng.integers(S))
        op = rng.integers(3)
        try:
            if op == 0:
                k = int(rng.integers(1, 9))
                pool.reserve(s, lens[s] + k)          # window of k provisional slots
                n = int(rng.integers(0, k))           # any rejection pattern
                lens[s] += n + 1
                pool.commit(s, lens[s])
            elif op == 1:
                pool.release(s)
                lens[s] = 0
            else:
                back = int(rng.integers(0, lens[s] + 1))
                lens[s] = back                          # roll back further
                pool.commit(s, back)
        except ValueError:
            pass                                        # out of pages: pool unchanged
        owned = [b for pg in pool.pages for b in pg]
        assert len(owned) + pool.free_count() == nb
        assert sorted(owned + pool.free) == list(range(nb))
        for t in range(S):
            assert pool.seq_blocks(t) == -(-lens[t] // 16)
