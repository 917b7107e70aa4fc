"""Pins of the tree-verification oracle (no GPU).

Verifier:
  * a chain-shaped tree is exactly the chain verifier (itself pinned by
    brute-force enumeration, losslessness and the closed-form mean);
  * one tree per sequence ([B, N] parents): each sequence is its own
    one-sequence call, and the chain-shaped ones are the chain verifier;
  * losslessness: the first emitted token has the law q_root, and after the
    path descends into a child c the next emitted token has the law q_c
    (empirically, 2e5 trials at V = 16);
  * the sibling residual step, worked by hand on a point-mass draft;
  * greedy tree verification emits exactly the target's own greedy stream.
Attention:
  * a chain-shaped mask is the window-causal verify attention;
  * every node's output equals plain causal attention over its root path,
    evaluated on a separately built cache holding just that path;
  * keys of non-ancestors do not change any output.
"""

import zlib

import numpy as np
import pytest

from oracle import attention as oat
from oracle import reject as orj
from oracle import tree as otr
from oracle.reject import widen
from synth import gen
from synth.tree import ancestor_bits, chain_parents, children, mixed_parents, tree_parents


def _probs(logits, t=1.0):
    # Test-side softmax used only to build expected laws.
    z = np.asarray(logits, dtype=np.float64) / t
    z = z - z.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=-1, keepdims=True)


def test_tree_helpers():
    # The input encoders (synth.tree) and the oracle's own path walk, by hand.
    par = tree_parents((2, 2, 2))
    assert par.tolist() == [-1, 0, 0, 1, 1, 2, 2, 3, 3, 4, 4, 5, 5, 6, 6]
    anc = ancestor_bits(par)
    assert int(anc[0]) == 0b1
    assert int(anc[9]) == (1 << 9) | (1 << 4) | (1 << 1) | 1
    assert children(par)[2] == [5, 6] and otr.children_of(par)[2] == [5, 6]
    assert chain_parents(4).tolist() == [-1, 0, 1, 2]
    assert otr.path_to_root(par, 9) == [0, 1, 4, 9]
    assert otr.path_to_root(par, 0) == [0]
    # The bit sets and the walked paths agree on every node of several shapes.
    for shape in [(2, 2, 2), (3, 1, 2), (16,), (1, 1, 1, 1)]:
        p = tree_parents(shape)
        bits = ancestor_bits(p)
        for i in range(len(p)):
            assert [j for j in range(len(p)) if (int(bits[i]) >> j) & 1] == otr.path_to_root(p, i)
    with pytest.raises(ValueError):
        ancestor_bits(np.array([-1, 2, 0]))
    with pytest.raises(ValueError):
        otr.path_to_root(np.array([-1, 2, 0]), 1)


# --------------------------------------------------------------------------
# A chain is the chain verifier.
# --------------------------------------------------------------------------

@pytest.mark.parametrize("seed,B,K,V,temps", [
    (1, 40, 4, 50, 1.0),
    (2, 40, 7, 300, np.array([0.0, 0.6, 1.0, 1.2] * 10, np.float32)),
    (3, 30, 1, 20, 0.8),
])
def test_chain_tree_is_the_chain_verifier(seed, B, K, V, temps):
    r = gen.make_reject_inputs(seed=seed, B=B, K=K, V=V, dtype="bf16",
                               draft_sigma=1.0, temperature=temps)
    chain = orj.reject_sample(r["target"], r["draft"], r["draft_tokens"], r["uniforms"],
                              r["temperature"])
    n = K + 1
    draft = np.zeros((B, n, V), dtype=r["draft"].dtype)
    draft[:, :K] = r["draft"]                     # node i's children law = chain row i
    tokens = np.zeros((B, n), np.int32)
    tokens[:, 1:] = r["draft_tokens"]
    u = np.zeros((B, n), np.float32)
    u[:, 1:] = r["uniforms"][:, :K]
    u[:, 0] = r["uniforms"][:, K]
    tr = otr.reject_sample_tree(r["target"], draft, chain_parents(n), tokens, u,
                                r["temperature"])
    assert np.array_equal(tr["out_tokens"], chain["out_tokens"])
    assert np.array_equal(tr["num_accepted"], chain["num_accepted"])
    assert np.array_equal(tr["flag_accept"], chain["flag_accept"])
    assert np.array_equal(tr["flag_sample"], chain["flag_sample"])
    nodes = tr["out_nodes"]
    for b in range(B):
        m = tr["num_accepted"][b]
        assert nodes[b, :m].tolist() == list(range(1, m + 1))


# --------------------------------------------------------------------------
# One tree per sequence.
# --------------------------------------------------------------------------

_KEYS = ("out_tokens", "out_nodes", "num_accepted", "flag_accept", "flag_sample")


@pytest.mark.parametrize("seed,B,N,V", [(11, 12, 8, 60), (12, 8, 5, 40)])
def test_per_sequence_trees_are_independent_calls(seed, B, N, V):
    par = mixed_parents(seed, B, N)
    temps = np.array([1.0, 0.0, 0.7, 1.3] * (B // 4), np.float32)
    r = gen.make_tree_reject_inputs(seed, B, par, V, dtype="bf16", draft_sigma=1.0,
                                    temperature=temps)
    batch = otr.reject_sample_tree(r["target"], r["draft"], par, r["tokens"], r["uniforms"],
                                   r["temperature"])
    for b in range(B):
        one = otr.reject_sample_tree(r["target"][b:b + 1], r["draft"][b:b + 1], par[b],
                                     r["tokens"][b:b + 1], r["uniforms"][b:b + 1],
                                     r["temperature"][b:b + 1])
        for k in _KEYS:
            assert np.array_equal(batch[k][b], one[k][0]), (b, k)
    # The shapes differ, so the walks do: stars never accept two nodes.
    stars = [b for b in range(B) if (par[b, 1:] == 0).all()]
    assert stars and all(batch["num_accepted"][b] <= 1 for b in stars)


def test_chain_sequences_of_a_mixed_batch_are_the_chain_verifier():
    B, N, V = 16, 8, 80
    K = N - 1
    par = mixed_parents(21, B, N)
    r = gen.make_tree_reject_inputs(21, B, par, V, dtype="bf16", draft_sigma=1.0,
                                    temperature=np.array([1.0, 0.8] * (B // 2), np.float32))
    tr = otr.reject_sample_tree(r["target"], r["draft"], par, r["tokens"], r["uniforms"],
                                r["temperature"])
    rows = [b for b in range(B) if np.array_equal(par[b], chain_parents(N))]
    assert len(rows) == B // 4
    u = np.zeros((len(rows), N), np.float32)
    u[:, :K] = r["uniforms"][rows, 1:]
    u[:, K] = r["uniforms"][rows, 0]
    chain = orj.reject_sample(r["target"][rows], r["draft"][rows, :K], r["tokens"][rows, 1:], u,
                              r["temperature"][rows])
    assert np.array_equal(tr["out_tokens"][rows], chain["out_tokens"])
    assert np.array_equal(tr["num_accepted"][rows], chain["num_accepted"])


# --------------------------------------------------------------------------
# The sibling residual step, by hand.
# --------------------------------------------------------------------------

def test_sibling_residual_point_mass_draft():
    # Root with two leaf children, draft a point mass on token a = 2: both
    # children draft a.  Child 1 passes with probability q(a).  After its
    # rejection the residual (q - p)_+ is q without a, renormalised, so child 2
    # (also a) has ratio 0 and is rejected; the final token is drawn from
    # q / (1 - q(a)) restricted to tokens != a.  Net law of the first token: q.
    v = 5
    tgt = np.log(np.array([0.1, 0.2, 0.3, 0.15, 0.25]))[None, None, :].repeat(3, axis=1)
    drf = np.full((1, 3, v), -np.inf)
    drf[0, 0, 2] = 0.0
    par = np.array([-1, 0, 0], np.int32)
    toks = np.array([[0, 2, 2]], np.int32)
    for u1, u0, expect in [(0.29, 0.5, [2, -1]),          # child 1 accepted (0.29 < 0.3)
                           (0.31, 0.0, [0, -1]),          # rejected; u0 = 0 -> first token != a
                           (0.31, 0.5, [3, -1])]:         # q' = [.1,.2,0,.15,.25]/.7: C = .143,.429,.429,.643
        u = np.array([[u0, u1, 0.0]], np.float32)
        res = otr.reject_sample_tree(tgt, drf, par, toks, u, np.array([1.0]))
        out = res["out_tokens"][0, :2].tolist()
        if expect[0] == 2:
            # accepted child 1 (a leaf): the bonus is drawn from q_1 with u0.
            assert res["num_accepted"][0] == 1 and out[0] == 2
        else:
            assert res["num_accepted"][0] == 0 and out == expect
    # The accepted-first-child probability is q(a) exactly: u1 just below and
    # just above q(a) switch the outcome.
    for u1, n in [(0.2999, 1), (0.3001, 0)]:
        res = otr.reject_sample_tree(tgt, drf, par, toks, np.array([[0.5, u1, 0.0]], np.float32),
                                     np.array([1.0]))
        assert res["num_accepted"][0] == n


def test_zero_draft_probability_accepts_in_a_tree():
    v = 6
    rng = np.random.default_rng(3)
    tgt = rng.standard_normal((1, 3, v))
    drf = rng.standard_normal((1, 3, v))
    drf[0, 0, 4] = -np.inf                         # p_root(4) = 0
    res = otr.reject_sample_tree(tgt, drf, np.array([-1, 0, 0]), np.array([[0, 4, 1]]),
                                 np.array([[0.3, 0.999, 0.999]]), np.array([1.0]))
    assert res["num_accepted"][0] == 1 and res["out_nodes"][0, 0] == 1


# --------------------------------------------------------------------------
# Losslessness, empirically.
# --------------------------------------------------------------------------

def test_tree_losslessness_first_and_second_token():
    par = tree_parents((2, 2))                 # 7 nodes
    v, trials = 16, 200_000
    inp = gen.make_tree_reject_inputs(seed=77, B=trials, parent=par, V=v, dtype="f32",
                                      logit_std=1.0, draft_sigma=1.0, temperature=1.0,
                                      shared_rows=True)
    q = _probs(inp["target"][0])
    res = otr.reject_sample_tree(inp["target"], inp["draft"], par, inp["tokens"],
                                 inp["uniforms"], inp["temperature"])
    out, nodes = res["out_tokens"], res["out_nodes"]
    first = np.bincount(out[:, 0], minlength=v) / trials
    tv0 = 0.5 * np.abs(first - q[0]).sum()
    assert tv0 < 0.01, tv0                         # expected sampling TV ~0.004
    for c in (1, 2):                               # descended into child c
        m = nodes[:, 0] == c
        frac = m.mean()
        assert frac > 0.1
        second = np.bincount(out[m, 1], minlength=v) / m.sum()
        tv = 0.5 * np.abs(second - q[c]).sum()
        assert tv < 0.01 / np.sqrt(frac), (c, tv)
    # Testing the second sibling against q_v instead of the residual (no
    # update between siblings) raises tv0 to about 0.2 on these inputs.
    assert res["num_accepted"].max() == 2          # depth of the tree


# --------------------------------------------------------------------------
# Greedy: identical to target-only decoding.
# --------------------------------------------------------------------------

V_TOY = 12


def _toy(prefix, salt):
    h = zlib.crc32(np.asarray(prefix, dtype=np.int64).tobytes() + salt)
    x = np.random.default_rng(h).standard_normal(V_TOY).astype(np.float32)
    return gen.bf16_to_f32(gen.bf16_bits(np.round(x * 2) / 2))


def _target(prefix):
    return _toy(prefix, b"target")


def _draft(prefix):
    noise = np.random.default_rng(zlib.crc32(np.asarray(prefix).tobytes() + b"n")).standard_normal(V_TOY)
    return (_target(prefix).astype(np.float64) + 0.8 * noise).astype(np.float32)


@pytest.mark.parametrize("shape", [(2, 2), (3, 1, 1), (1, 1, 1, 1)])
def test_greedy_tree_equals_target_only_decoding(shape):
    par = tree_parents(shape)
    kids = children(par)
    n = len(par)
    prompt = [5, 1, 7]
    n_tokens = 120
    plain = list(prompt)
    while len(plain) < len(prompt) + n_tokens:
        plain.append(int(np.argmax(_target(plain))))
    seq = list(prompt)
    calls = 0
    while len(seq) < len(prompt) + n_tokens:
        # Greedy drafter: a node's children take its draft's top-ranked tokens.
        path_of = {0: []}
        toks = np.zeros(n, np.int32)
        for vtx in range(n):
            order = np.argsort(-_draft(seq + path_of[vtx]), kind="stable")
            for r, c in enumerate(kids[vtx]):
                toks[c] = order[r]
                path_of[c] = path_of[vtx] + [int(order[r])]
        tgt = np.stack([_target(seq + path_of[vtx]) for vtx in range(n)])[None]
        res = otr.reject_sample_tree(gen.bf16_bits(tgt), None, par, toks[None],
                                     np.zeros((1, n)), np.array([0.0]))
        m = int(res["num_accepted"][0])
        seq.extend(int(x) for x in res["out_tokens"][0, :m + 1])
        calls += 1
    assert seq[:len(plain)] == plain
    assert calls < n_tokens


# --------------------------------------------------------------------------
# Attention.
# --------------------------------------------------------------------------

def _attn_case(seed, B, N, Hq, Hkv, D, ctx, dtype="f32"):
    return gen.make_attn_inputs(seed=seed, B=B, K=N - 1, Hq=Hq, Hkv=Hkv, D=D, ctx=ctx, dtype=dtype)


def test_chain_mask_is_verify_attention():
    inp = _attn_case(11, 2, 6, 4, 2, 32, (10, 40))
    a = otr.tree_attention(inp["q"], inp["k_cache"], inp["v_cache"], inp["block_table"],
                           inp["kv_len"], chain_parents(6))
    b = oat.verify_attention(inp["q"], inp["k_cache"], inp["v_cache"], inp["block_table"],
                             inp["kv_len"])
    assert np.max(np.abs(a - b)) < 1e-12


def _chain_cache(keys, vals):
    """f32 paged caches [1 page per 16 tokens] holding keys / vals [L, Hkv, D] in order."""
    L, hkv, d = keys.shape
    x = 4
    nb = (L + 15) // 16
    kc = np.zeros((nb, hkv, d // x, 16, x), np.float32)
    vc = np.zeros((nb, hkv, d, 16), np.float32)
    for j in range(L):
        kc[j // 16, :, :, j % 16, :] = keys[j].reshape(hkv, d // x, x)
        vc[j // 16, :, :, j % 16] = vals[j]
    return kc, vc, np.arange(nb, dtype=np.int32)[None]


@pytest.mark.parametrize("shape", [(2, 2), (3, 2), (1, 3)])
def test_every_node_is_causal_attention_over_its_path(shape):
    par = tree_parents(shape)
    n = len(par)
    inp = _attn_case(21, 2, n, 4, 2, 32, (5, 30))
    anc = ancestor_bits(par)
    out = otr.tree_attention(inp["q"], inp["k_cache"], inp["v_cache"], inp["block_table"],
                             inp["kv_len"], par)
    for b in range(2):
        l0 = int(inp["kv_len"][b])
        keys, vals = oat.gather_kv(inp["k_cache"], inp["v_cache"], inp["block_table"], b, l0 + n)
        for i in range(n):
            path = [j for j in range(n) if (int(anc[i]) >> j) & 1]      # root .. i, in order
            sel = np.concatenate([np.arange(l0), l0 + np.asarray(path)])
            kc, vc, bt = _chain_cache(keys[sel], vals[sel])
            qk = np.asarray(widen(inp["q"]), np.float32)[b, i][None, None]   # [1, 1, Hq, D]
            ref = oat.verify_attention(qk, kc, vc, bt, np.array([l0 + len(path) - 1]))
            assert np.max(np.abs(out[b, i] - ref[0, 0])) < 1e-12, (b, i)


def test_non_ancestor_keys_do_not_matter():
    par = tree_parents((2, 2))
    n = len(par)
    inp = _attn_case(31, 1, n, 2, 1, 32, 20)
    a = otr.tree_attention(inp["q"], inp["k_cache"], inp["v_cache"], inp["block_table"],
                           inp["kv_len"], par)
    kc, vc = inp["k_cache"].copy(), inp["v_cache"].copy()
    l0 = int(inp["kv_len"][0])
    for j in (2, 5, 6):                                   # not ancestors of node 4
        pos = l0 + j
        blk = inp["block_table"][0, pos // 16]
        kc[blk, :, :, pos % 16, :] = 7.0
        vc[blk, :, :, pos % 16] = -3.0
    b = otr.tree_attention(inp["q"], kc, vc, inp["block_table"], inp["kv_len"], par)
    for i in (0, 1, 3, 4):
        assert np.max(np.abs(a[0, i] - b[0, i])) < 1e-12
    assert np.max(np.abs(a[0, 5] - b[0, 5])) > 1e-6       # node 5 does see node 2


def test_tree_f1_band_on_sibling_tests():
    # Root with two children (parent -1, 0, 0).  q_root = (0.5, 0.3, 0.2),
    # p_root = (0.2, 0.2, 0.6).  Node 1 drafts token 2: r = 0.2 / 0.6 = 1/3.
    # After it is rejected the residual is (0.3, 0.1, 0) / 0.4, so node 2's
    # token 2 has r = 0 (always rejected): |u - 0| < 1e-5 is the band there.
    q = np.array([0.5, 0.3, 0.2])
    p = np.array([0.2, 0.2, 0.6])
    tgt = np.log(np.stack([q, q, q]))[None]
    drf = np.log(np.stack([p, p, p]))[None]
    par = [-1, 0, 0]
    toks = np.array([[0, 2, 2]])

    def run(u1, u2):
        return otr.reject_sample_tree(tgt, drf, par, toks, np.array([[0.5, u1, u2]]),
                                      np.array([1.0]))

    # Node 1 rejected, node 2 examined and inside the band: flagged.
    res = run(0.9, 0.5e-5)
    assert res["num_accepted"][0] == 0 and res["flag_accept"][0]
    res = run(0.9, 1.01e-5)
    assert res["num_accepted"][0] == 0 and not res["flag_accept"][0]
    # Node 1 inside its band: flagged whichever way it goes.
    assert run(1 / 3 + 0.5e-5, 0.5)["flag_accept"][0]
    assert run(1 / 3 - 0.5e-5, 0.5)["flag_accept"][0]
    assert not run(1 / 3 - 1.01e-5, 0.5)["flag_accept"][0]
    # Node 1 accepted (a leaf: the bonus draw follows), so node 2 is never
    # examined: its uniform inside the band does not flag.
    res = run(0.1, 0.5e-5)
    assert res["num_accepted"][0] == 1 and list(res["out_nodes"][0, :1]) == [1]
    assert not res["flag_accept"][0]
