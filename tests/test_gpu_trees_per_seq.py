"""GPU parity of spec_reject_sample_trees (one draft tree per sequence)
against the CPU oracle, which takes [B, N] parent arrays.

Bars as for the shared-tree call: accepted paths, emitted tokens and the
committed kv_len bit-exact with oracle.tree.reject_sample_tree (float64) on
every sequence the oracle does not flag (F1 / F2, and F3 with filters),
flagged ones checked for validity; greedy sequences bit-exact always.  A
batch whose sequences all share one tree must give exactly the outputs of
spec_reject_sample_tree.
"""

import numpy as np
import pytest

from oracle import filter as ofl
from oracle import tree as otr
from synth import gen
from synth.device import to_device, from_device
from synth.tree import mixed_parents, random_parents, tree_parents

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def dev(gpu_lib):
    return "cuda:0"


def _run(sv, inp, par, kv0, dev, top_k=None, top_p=None, with_draft=True):
    kv = to_device(kv0, dev)
    ot, on, n = sv.reject_sample_trees(
        to_device(inp["target"], dev), to_device(inp["draft"], dev) if with_draft else None,
        to_device(np.ascontiguousarray(par, dtype=np.int32), dev), to_device(inp["tokens"], dev),
        to_device(inp["uniforms"], dev), to_device(inp["temperature"], dev), kv,
        top_k=None if top_k is None else to_device(top_k.astype(np.int32), dev),
        top_p=None if top_p is None else to_device(top_p.astype(np.float32), dev))
    return from_device(ot), from_device(on), from_device(n), from_device(kv)


def _valid_path(parent, tokens, nodes, toks, n, V):
    prev = 0
    for j in range(n):
        c = nodes[j]
        assert 0 < c < len(parent) and parent[c] == prev
        assert toks[j] == tokens[c]
        prev = c
    assert 0 <= toks[n] < V
    assert (toks[n + 1:] == -1).all() and (nodes[n:] == -1).all()


def _compare(ref, got, inp, par, kv0, label, max_flag=None):
    ot, on, n, kv = got
    V = inp["target"].shape[-1]
    flag = ref["flag_accept"] | ref["flag_sample"]
    if "flag_filter" in ref:
        flag = flag | ref["flag_filter"]
    ok = ~flag
    assert (n >= 0).all(), label + ": a walk did not finish"
    assert np.array_equal(n[ok], ref["num_accepted"][ok]), label
    assert np.array_equal(on[ok], ref["out_nodes"][ok]), label
    assert np.array_equal(ot[ok], ref["out_tokens"][ok]), label
    assert np.array_equal(kv, kv0 + n + 1), label
    for b in np.nonzero(flag)[0]:
        _valid_path(par[b], inp["tokens"][b], on[b], ot[b], n[b], V)
    _say("%s: %d sequences, mean accepted %.2f, flagged %d"
         % (label, len(n), n.mean(), int(flag.sum())))
    lim = 2 + len(n) // 1000 if max_flag is None else max_flag
    assert int(flag.sum()) <= lim, (label, int(flag.sum()))
    return int(flag.sum())


def _case(sv, dev, seed, B, par, V, dtype="bf16", sigma=0.51, temp=1.0, top_k=None, top_p=None,
          max_flag=None):
    par = np.asarray(par, dtype=np.int32)
    label = "trees seed=%d B=%d N=%d V=%d %s sigma=%s filters=%s" % (
        seed, B, par.shape[1], V, dtype, sigma, top_k is not None or top_p is not None)
    _say(label)
    inp = gen.make_tree_reject_inputs(seed=seed, B=B, parent=par, V=V, dtype=dtype,
                                      draft_sigma=sigma, temperature=temp)
    kv0 = np.random.default_rng(seed).integers(100, 5000, size=B).astype(np.int32)
    got = _run(sv, inp, par, kv0, dev, top_k, top_p)
    if top_k is None and top_p is None:
        ref = otr.reject_sample_tree(inp["target"], inp["draft"], par, inp["tokens"],
                                     inp["uniforms"], inp["temperature"])
    else:
        tk = np.zeros(B, np.int64) if top_k is None else top_k
        tp = np.ones(B) if top_p is None else top_p
        ref = ofl.reject_sample_tree_filtered(inp["target"], inp["draft"], par, inp["tokens"],
                                              inp["uniforms"], inp["temperature"], tk, tp)
    _compare(ref, got, inp, par, kv0, label, max_flag)
    return inp, ref, got


@pytest.mark.parametrize("sigma", [0.5, 2.0])
def test_mixed_shapes_vs_oracle(gpu_lib, dev, sigma):
    # Chains, stars, two-level and random trees in one batch; sigma 2.0
    # rejects most first children, so the stars' sibling rounds run long.
    _case(gpu_lib, dev, 101, 48, mixed_parents(101, 48, 8), 5000, sigma=sigma)


def test_mixed_temperatures_with_greedy(gpu_lib, dev):
    temps = np.array([0.0, 1.0, 0.7, 0.0, 1.4, 0.0], np.float32)
    _case(gpu_lib, dev, 102, 48, mixed_parents(102, 48, 8), 3000, sigma=1.0,
          temp=np.tile(temps, 8))


def test_fp32_and_unaligned_vocab(gpu_lib, dev):
    _case(gpu_lib, dev, 103, 32, mixed_parents(103, 32, 6), 777, dtype="f32", sigma=1.0)
    _case(gpu_lib, dev, 104, 32, mixed_parents(104, 32, 6), 777, dtype="bf16", sigma=1.0)


def test_max_nodes(gpu_lib, dev):
    # N = 17: a star needs 16 rounds, the most the call launches.
    _case(gpu_lib, dev, 105, 24, mixed_parents(105, 24, 17), 3000, sigma=2.5)


def test_root_only_and_two_nodes(gpu_lib, dev):
    _case(gpu_lib, dev, 106, 16, np.full((16, 1), -1, np.int32), 500)
    _case(gpu_lib, dev, 107, 16, mixed_parents(107, 16, 2), 500, sigma=1.5)


def test_filters_per_sequence(gpu_lib, dev):
    B = 48
    rng = np.random.default_rng(108)
    tk = rng.choice([0, 1, 5, 50], size=B).astype(np.int64)
    tp = rng.choice([1.0, 0.95, 0.8, 0.3], size=B)
    # The top-p boundary band (F3) is wider than F1 / F2: a few per batch.
    _case(gpu_lib, dev, 108, B, mixed_parents(108, B, 8), 4001, sigma=1.0, top_k=tk, top_p=tp,
          max_flag=12)


def test_llama8b_vocab(gpu_lib, dev):
    _case(gpu_lib, dev, 109, 16, mixed_parents(109, 16, 15), 128256, sigma=0.51)


def test_shared_tree_is_the_tree_call(gpu_lib, dev):
    # Every sequence with the same [2,2,2] tree: bit-identical to
    # spec_reject_sample_tree on the same inputs (flagged or not).
    par = tree_parents((2, 2, 2))
    B, V = 32, 6000
    inp = gen.make_tree_reject_inputs(seed=110, B=B, parent=par, V=V, draft_sigma=1.0)
    kv0 = np.full(B, 700, np.int32)
    per = _run(gpu_lib, inp, np.tile(par, (B, 1)), kv0, dev)
    kv = to_device(kv0, dev)
    ot, on, n = gpu_lib.reject_sample_tree(
        to_device(inp["target"], dev), to_device(inp["draft"], dev), par,
        to_device(inp["tokens"], dev), to_device(inp["uniforms"], dev),
        to_device(inp["temperature"], dev), kv)
    shared = (from_device(ot), from_device(on), from_device(n), from_device(kv))
    for a, b in zip(per, shared):
        assert np.array_equal(a, b)


def test_parent_outside_range_reads_as_previous_node(gpu_lib, dev):
    # parents[b][i] outside [0, i) is read as i - 1: the oracle on the
    # repaired arrays gives the reference.
    B, N, V = 16, 7, 900
    rng = np.random.default_rng(111)
    good = np.stack([random_parents(rng, N) for _ in range(B)])
    bad = good.copy()
    bad[::2, 3] = 5          # not before node 3
    bad[1::4, 5] = -2
    fixed = good.copy()
    fixed[::2, 3] = 2
    fixed[1::4, 5] = 4
    inp = gen.make_tree_reject_inputs(seed=111, B=B, parent=fixed, V=V, draft_sigma=1.0)
    kv0 = np.full(B, 40, np.int32)
    got = _run(gpu_lib, inp, bad, kv0, dev)
    ref = otr.reject_sample_tree(inp["target"], inp["draft"], fixed, inp["tokens"],
                                 inp["uniforms"], inp["temperature"])
    _compare(ref, got, inp, fixed, kv0, "repaired parents")
