"""The host page pool (spec_pages_*), on the CPU: it matches the oracle's
model page for page (the lowest-numbered free page first), keeps every page
owned exactly once across every rejection pattern, and reports errors
without changing its state."""

import numpy as np
import pytest

import speculative_decoding_verification_verify_amd as sv
from oracle import kv as okv


@pytest.fixture(scope="module")
def lib():
    return sv.load()


def _both(nb, seqs, mbps):
    return sv.PagePool(nb, seqs, mbps), okv.PagePool(nb, seqs, mbps)


def _same(c, o):
    assert c.check() == 0
    assert c.free_count() == o.free_count()
    assert np.array_equal(c.block_table(), o.block_table())


def _apply(pool, op, *args):
    try:
        getattr(pool, op)(*args)
        return 0
    except sv.SpecVerifyError as e:
        return e.status
    except ValueError:
        return "err"


def test_matches_the_model_on_random_ops(lib):
    rng = np.random.default_rng(3)
    c, o = _both(48, 6, 12)
    lens = [0] * 6
    for step in range(4000):
        s = int(rng.integers(6))
        op = int(rng.integers(4))
        if op <= 1:
            k = int(rng.integers(1, 18))               # window of k = N slots
            rc, ro = _apply(c, "reserve", s, lens[s] + k), _apply(o, "reserve", s, lens[s] + k)
            assert (rc == 0) == (ro == 0), (step, rc, ro)
            if rc == 0:
                n = int(rng.integers(0, k))            # any rejection pattern
                lens[s] += n + 1
                c.commit(s, lens[s])
                o.commit(s, lens[s])
            else:
                assert rc in (-5, -1) and ro == "err"
        elif op == 2:
            c.release(s)
            o.release(s)
            lens[s] = 0
        else:
            back = int(rng.integers(0, lens[s] + 1))
            lens[s] = back
            c.commit(s, back)
            o.commit(s, back)
        _same(c, o)
        assert c.seq_blocks(s) == -(-lens[s] // 16)
    c.close()


@pytest.mark.parametrize("K", [1, 4, 7, 16])
def test_every_rejection_pattern_frees_the_tail(lib, K):
    # From every start offset in a page, with every number of accepted drafts:
    # reserve the window, commit, and the pool holds exactly ceil(len / 16)
    # pages for the sequence and every other page is free.
    for l0 in range(0, 33):
        for n in range(0, K + 1):
            c = sv.PagePool(8, 1, 8)
            c.reserve(0, l0)
            c.commit(0, l0)
            c.reserve(0, l0 + K + 1)
            assert c.seq_blocks(0) == -(-(l0 + K + 1) // 16)
            c.commit(0, l0 + n + 1)
            assert c.seq_blocks(0) == -(-(l0 + n + 1) // 16)
            assert c.free_count() == 8 - c.seq_blocks(0)
            assert c.check() == 0
            c.release(0)
            assert c.free_count() == 8 and c.check() == 0
            c.close()


def test_errors_leave_the_pool_unchanged(lib):
    c = sv.PagePool(4, 2, 3)
    c.reserve(0, 20)                                   # pages 0, 1
    before = (c.free_count(), c.block_table().copy())
    for op, args, status in [("reserve", (2, 5), -1),           # no such sequence
                             ("reserve", (0, 16 * 3 + 1), -1),  # more than a table row
                             ("reserve", (1, 16 * 3), -5),      # 3 pages, 2 free
                             ("commit", (0, 33), -1),           # past the reserved pages
                             ("commit", (0, -1), -1),
                             ("release", (-1,), -1)]:
        with pytest.raises(sv.SpecVerifyError) as e:
            getattr(c, op)(*args)
        assert e.value.status == status, (op, args)
        assert c.free_count() == before[0] and np.array_equal(c.block_table(), before[1])
        assert c.check() == 0
    c.reserve(1, 32)                                   # exactly the 2 free pages
    assert c.free_count() == 0 and c.block_table()[1, :2].tolist() == [2, 3]
    c.close()


def test_create_rejects_bad_sizes(lib):
    assert not lib.spec_pages_create(0, 1, 1)
    assert not lib.spec_pages_create(4, 0, 1)
    assert lib.spec_pages_free_count(None) == -1
    assert lib.spec_pages_check(None) == -1
