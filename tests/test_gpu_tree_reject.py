"""GPU parity of spec_reject_sample_tree against the CPU oracle.

As for the chain: accepted paths, emitted tokens and the committed kv_len are
bit-exact with oracle.tree.reject_sample_tree (float64), except sequences the
oracle flags as boundary trials (F1: |u - ratio| < 1e-5 at an examined
test, siblings included; F2: the final draw within 1e-10 of probability mass
of a CDF edge), which are counted and checked for validity only.  Greedy
sequences are bit-exact always.  A chain-shaped tree must give exactly the
outputs of spec_reject_sample.
"""

import numpy as np
import pytest

from oracle import tree as otr
from synth import gen, CONFIGS
from synth.tree import chain_parents, tree_parents
from synth.device import to_device, from_device

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def dev(gpu_lib):
    return "cuda:0"


def _run(sv, inp, kv0, dev, with_draft=True, counters=None):
    kv = to_device(kv0, dev)
    ot, on, n = sv.reject_sample_tree(to_device(inp["target"], dev),
                                      to_device(inp["draft"], dev) if with_draft else None,
                                      inp["parent"], to_device(inp["tokens"], dev),
                                      to_device(inp["uniforms"], dev),
                                      to_device(inp["temperature"], dev), kv, counters=counters)
    return from_device(ot), from_device(on), from_device(n), from_device(kv)


def _valid_path(parent, tokens, nodes, toks, n, V):
    """A flagged sequence's outputs still describe a root path of the tree."""
    prev = 0
    for j in range(n):
        c = nodes[j]
        assert 0 < c < len(parent) and parent[c] == prev
        assert toks[j] == tokens[c]
        prev = c
    assert 0 <= toks[n] < V
    assert (toks[n + 1:] == -1).all() and (nodes[n:] == -1).all()


def _compare(ref, got, inp, kv0, idx, label):
    ot, on, n, kv = got
    sel = slice(None) if idx is None else idx
    ot, on, n, kv, k0 = ot[sel], on[sel], n[sel], kv[sel], kv0[sel]
    tok = inp["tokens"][sel]
    V = inp["target"].shape[-1]
    flag = ref["flag_accept"] | ref["flag_sample"]
    ok = ~flag
    assert (n >= 0).all(), label + ": a walk did not finish"
    assert np.array_equal(n[ok], ref["num_accepted"][ok]), label
    assert np.array_equal(on[ok], ref["out_nodes"][ok]), label
    assert np.array_equal(ot[ok], ref["out_tokens"][ok]), label
    assert np.array_equal(kv, k0 + n + 1), label
    for b in np.nonzero(flag)[0]:
        _valid_path(inp["parent"], tok[b], on[b], ot[b], n[b], V)
    _say("%s: %d sequences, mean accepted %.2f, flagged F1=%d F2=%d"
         % (label, len(n), n.mean(), ref["flag_accept"].sum(), ref["flag_sample"].sum()))
    # F1 / F2 are rare for every tree (2e-5 per examined test, ~1e-4 per
    # draw): a few flags at most, never a systematic exclusion.
    assert int(flag.sum()) <= 2 + len(n) // 1000, (label, int(flag.sum()))
    return int(flag.sum())


def _case(sv, dev, seed, B, parent, V, dtype="bf16", sigma=0.51, temp=1.0, std=2.0, idx=None,
          with_draft=True):
    parent = np.asarray(parent, dtype=np.int32)
    label = "tree reject seed=%d B=%d N=%d V=%d %s T=%s sigma=%s" % (seed, B, len(parent), V, dtype,
                                                                     temp, sigma)
    _say(label)
    inp = gen.make_tree_reject_inputs(seed=seed, B=B, parent=parent, V=V, dtype=dtype,
                                      logit_std=std, draft_sigma=sigma, temperature=temp)
    kv0 = np.random.default_rng(seed).integers(100, 5000, size=B).astype(np.int32)
    got = _run(sv, inp, kv0, dev, with_draft=with_draft)
    sel = slice(None) if idx is None else idx
    ref = otr.reject_sample_tree(inp["target"][sel], inp["draft"][sel] if with_draft else None,
                                 parent, inp["tokens"][sel], inp["uniforms"][sel],
                                 inp["temperature"][sel])
    flagged = _compare(ref, got, inp, kv0, idx, label)
    return inp, ref, got, flagged


def test_tiny_fp32_tree(gpu_lib, dev):
    _case(gpu_lib, dev, 1, 64, tree_parents((2, 2)), 300, dtype="f32", sigma=1.0)


@pytest.mark.parametrize("shape", [(2, 2, 2), (3, 2), (4,), (2, 1, 2), (1, 1, 1, 1)])
@pytest.mark.parametrize("sigma", [0.5, 2.0])
def test_shapes_vs_oracle(gpu_lib, dev, shape, sigma):
    # sigma 2.0: the draft is far from the target, so most first children are
    # rejected and the sibling tests against the residual carry the walk.
    _case(gpu_lib, dev, 10 + len(shape), 48, tree_parents(shape), 5000, sigma=sigma)


@pytest.mark.parametrize("temp", [0.6, 1.5])
def test_temperatures(gpu_lib, dev, temp):
    _case(gpu_lib, dev, 21, 32, tree_parents((2, 2, 2)), 20000, sigma=1.0, temp=temp)


def test_wide_root_every_round(gpu_lib, dev):
    # Root with 8 children and a far draft: walks reject up to all 8 siblings
    # (8 rounds of exact passes, each with a larger residual coefficient).
    _, ref, got, _ = _case(gpu_lib, dev, 31, 64, tree_parents((8,)), 4000, sigma=3.0)
    assert (got[2] == 0).sum() > 0


def test_max_nodes(gpu_lib, dev):
    _case(gpu_lib, dev, 41, 24, tree_parents((16,)), 3000, sigma=2.5)      # 16 rounds
    _case(gpu_lib, dev, 42, 24, chain_parents(17), 3000, sigma=0.3)         # 17-node chain


def test_root_only(gpu_lib, dev):
    # No drafts at all: the bonus draw from q_0 (sampling) or argmax (greedy).
    _case(gpu_lib, dev, 51, 16, [-1], 7000)
    _case(gpu_lib, dev, 52, 16, [-1], 7000, temp=0.0, with_draft=False)


def test_non_bfs_order(gpu_lib, dev):
    # Children of a node need not be contiguous: 0 -> {1, 3, 5}, 1 -> {2, 4}, 3 -> {6}.
    _case(gpu_lib, dev, 61, 48, [-1, 0, 1, 0, 1, 0, 3], 6000, sigma=1.5)


@pytest.mark.parametrize("shape", [(2, 2, 2), (3, 1), (1, 1, 1, 1, 1, 1, 1)])
def test_greedy(gpu_lib, dev, shape):
    _case(gpu_lib, dev, 71, 32, tree_parents(shape), 9000, temp=0.0, sigma=0.3,
          with_draft=False)


def test_mixed_temperatures_in_one_batch(gpu_lib, dev):
    temps = np.tile(np.array([0.0, 0.7, 1.0, -1.0, 1.3], dtype=np.float32), 8)
    _case(gpu_lib, dev, 81, 40, tree_parents((2, 2)), 8000, sigma=1.0, temp=temps)


@pytest.mark.parametrize("V,dtype", [(1001, "f32"), (33001, "bf16")])
def test_ragged_vocab(gpu_lib, dev, V, dtype):
    _case(gpu_lib, dev, 91, 32, tree_parents((2, 2)), V, dtype=dtype, sigma=1.5)


@pytest.mark.parametrize("V", [524288, 700001])
def test_large_vocab(gpu_lib, dev, V):
    """64 and 86 chunks of 8192 entries: the round's step reads every chunk's
    sums in one wave at 2^19 entries, in two wave segments past it."""
    _case(gpu_lib, dev, 95, 6, tree_parents((2, 2)), V, sigma=1.5)


def test_llama8b_vocab_tree_sampled(gpu_lib, dev):
    # 64 sequences over the full 128256-entry vocabulary with a [2,2,2] tree;
    # the oracle checks every 4th sequence.
    c = CONFIGS["llama8b_b64"]
    _case(gpu_lib, dev, 101, c.B, tree_parents((2, 2, 2)), c.V, sigma=1.0,
          idx=list(range(0, c.B, 4)))


def _chain_as_tree(inp):
    """Inputs of the chain call recast as a chain-shaped tree call."""
    tgt, drf = inp["target"], inp["draft"]
    B, K, V = drf.shape
    drf_t = np.concatenate([drf, drf[:, :1]], axis=1)              # leaf row: never read
    tok = np.zeros((B, K + 1), dtype=np.int32)
    tok[:, 1:] = inp["draft_tokens"]
    u = np.empty((B, K + 1), dtype=np.float32)
    u[:, 1:] = inp["uniforms"][:, :K]
    u[:, 0] = inp["uniforms"][:, K]
    return {"target": tgt, "draft": drf_t, "tokens": tok, "uniforms": u,
            "parent": chain_parents(K + 1), "temperature": inp["temperature"]}


@pytest.mark.parametrize("sigma,temp", [(0.51, 1.0), (2.0, 0.8), (0.3, 0.0)])
def test_chain_tree_is_the_chain_call(gpu_lib, dev, sigma, temp):
    import torch
    K, V, B = 7, 32000, 64
    _say("chain-as-tree K=%d V=%d sigma=%s T=%s" % (K, V, sigma, temp))
    inp = gen.make_reject_inputs(seed=111, B=B, K=K, V=V, dtype="bf16", logit_std=2.0,
                                 draft_sigma=sigma, temperature=temp)
    kv0 = np.arange(B, dtype=np.int32) + 100
    kv_c = to_device(kv0, dev)
    out_c, n_c = gpu_lib.reject_sample(to_device(inp["target"], dev), to_device(inp["draft"], dev),
                                       to_device(inp["draft_tokens"], dev),
                                       to_device(inp["uniforms"], dev),
                                       to_device(inp["temperature"], dev), kv_c)
    ot, on, n, kv = _run(gpu_lib, _chain_as_tree(inp), kv0, dev)
    assert np.array_equal(n, from_device(n_c))
    assert np.array_equal(ot, from_device(out_c))
    assert np.array_equal(kv, from_device(kv_c))
    for b in range(B):
        assert np.array_equal(on[b, :n[b]], np.arange(1, n[b] + 1))
        assert (on[b, n[b]:] == -1).all()
    _say("chain-as-tree: mean accepted %.2f" % n.mean())
    del torch


def test_counters_and_determinism(gpu_lib, dev):
    import torch
    par = tree_parents((2, 2, 2))
    inp = gen.make_tree_reject_inputs(seed=121, B=32, parent=par, V=12000, draft_sigma=1.0)
    kv0 = np.full(32, 1000, dtype=np.int32)
    cnt = torch.zeros(2, dtype=torch.int64, device=dev)
    a = _run(gpu_lib, inp, kv0, dev, counters=cnt)
    b = _run(gpu_lib, inp, kv0, dev)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    c = from_device(cnt)
    assert c[0] == 32 * (len(par) - 1)
    assert c[1] == a[2].sum()


def test_empty_batch_is_noop(gpu_lib, dev):
    import torch
    t = torch.zeros((0, 3, 100), dtype=torch.bfloat16, device=dev)
    z = torch.zeros((0, 3), dtype=torch.int32, device=dev)
    ot, on, n = gpu_lib.reject_sample_tree(t, t, [-1, 0, 0], z, z.float(),
                                           torch.zeros(0, device=dev),
                                           torch.zeros(0, dtype=torch.int32, device=dev))
    assert ot.numel() == 0 and n.numel() == 0
