"""GPU parity of spec_reject_sample against the CPU oracle.

Accepted lengths, emitted tokens and the committed kv_len must be bit-exact
with the float64 oracle, except sequences the oracle flags as boundary
trials: F1 (|u - q/p| < 1e-5 at an examined accept test) or F2 (the final
draw's u*Z within 1e-10 probability mass of a CDF edge).  Flagged sequences
are excluded from the exact comparison, counted and printed, and still
checked for validity.  Greedy sequences have no flags: bit-exact always,
lowest index on ties.
"""

import numpy as np
import pytest

from oracle import reject as orj
from synth import gen, CONFIGS, SIGMA_FOR_ALPHA
from synth.device import to_device, from_device

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _run_gpu(sv, inp, kv0, dev, counters=None, with_draft=True):
    t = to_device(inp["target"], dev)
    d = to_device(inp["draft"], dev) if with_draft else None
    kv = to_device(kv0, dev)
    out, n = sv.reject_sample(t, d, to_device(inp["draft_tokens"], dev),
                              to_device(inp["uniforms"], dev),
                              to_device(inp["temperature"], dev), kv, counters=counters)
    return from_device(out), from_device(n), from_device(kv)


def max_flagged(n_seq):
    """Bound on the sequences a case may leave out of the exact comparison.

    F1 flags an examined accept test with probability 2e-5 (u uniform in a
    band of width 2e-5) and F2 a final draw with probability about
    2e-10 V / Z (1e-4 at V = 128K and residual mass 0.2), so a few in 1e4
    sequences at most; the bound sits far above that and far below a
    systematic exclusion."""
    return 2 + n_seq // 1000


def _compare(ref, out, n, kv_new, kv0, inp, idx=None, label=""):
    """Exact on unflagged sequences; validity on flagged ones.  Returns #flagged."""
    d = inp["draft_tokens"] if idx is None else inp["draft_tokens"][idx]
    k = d.shape[1]
    v = inp["target"].shape[-1]
    if idx is not None:
        out, n, kv_new, kv0 = out[idx], n[idx], kv_new[idx], kv0[idx]
    flag = ref["flag_accept"] | ref["flag_sample"]
    ok = ~flag
    assert np.array_equal(n[ok], ref["num_accepted"][ok]), label
    assert np.array_equal(out[ok], ref["out_tokens"][ok]), label
    assert np.array_equal(kv_new, kv0 + n + 1), label
    assert (n >= 0).all() and (n <= k).all()
    for b in np.nonzero(flag)[0]:
        nb = n[b]
        assert np.array_equal(out[b, :nb], d[b, :nb])
        assert 0 <= out[b, nb] < v
        assert (out[b, nb + 1:] == -1).all()
    _say("%s: %d sequences, flagged F1=%d F2=%d" % (label, len(n), ref["flag_accept"].sum(),
                                                     ref["flag_sample"].sum()))
    assert int(flag.sum()) <= max_flagged(len(n)), (label, int(flag.sum()))
    return int(flag.sum())


def _case(sv, dev, seed, B, K, V, dtype="bf16", sigma=0.51, temp=1.0, std=2.0,
          shared=False, idx=None):
    label = "reject seed=%d B=%d K=%d V=%d %s T=%s sigma=%s" % (seed, B, K, V, dtype, temp, sigma)
    _say(label)
    inp = gen.make_reject_inputs(seed=seed, B=B, K=K, V=V, dtype=dtype, logit_std=std,
                                 draft_sigma=sigma, temperature=temp, shared_rows=shared)
    kv0 = np.random.default_rng(seed).integers(100, 5000, size=B).astype(np.int32)
    out, n, kv_new = _run_gpu(sv, inp, kv0, dev)
    sel = slice(None) if idx is None else idx
    ref = orj.reject_sample(inp["target"][sel], inp["draft"][sel], inp["draft_tokens"][sel],
                            inp["uniforms"][sel], inp["temperature"][sel])
    flagged = _compare(ref, out, n, kv_new, kv0, inp, idx=idx, label=label)
    return inp, ref, out, n, flagged


@pytest.fixture(scope="module")
def dev(gpu_lib):
    return "cuda:0"


def test_tiny_1e5_trials_t1(gpu_lib, dev):
    c = CONFIGS["tiny"]
    _, ref, out, n, flagged = _case(gpu_lib, dev, 101, 100_000, c.K, c.V, "f32",
                                    sigma=c.draft_sigma, temp=1.0, std=c.logit_std, shared=True)
    assert flagged < 50


def test_tiny_greedy_fresh_logits(gpu_lib, dev):
    c = CONFIGS["tiny"]
    _, ref, out, n, flagged = _case(gpu_lib, dev, 102, 1000, c.K, c.V, "f32",
                                    sigma=c.draft_sigma, temp=0.0, std=c.logit_std)
    assert flagged == 0
    assert 0 < ref["num_accepted"].mean() < c.K


@pytest.mark.parametrize("K", [2, 4, 6, 8])
@pytest.mark.parametrize("temp", [0.0, 1.0])
def test_qwen_b1(gpu_lib, dev, K, temp):
    c = CONFIGS["qwen_b1"]
    _case(gpu_lib, dev, 200 + K, 1, K, c.V, sigma=c.draft_sigma, temp=temp)


@pytest.mark.parametrize("alpha", sorted(SIGMA_FOR_ALPHA))
def test_qwen_alpha_sweep(gpu_lib, dev, alpha):
    c = CONFIGS["qwen_b1"]
    # 16 sequences per alpha so both rejections and bonus draws occur.
    _case(gpu_lib, dev, 300 + int(alpha * 10), 16, 8, c.V, sigma=SIGMA_FOR_ALPHA[alpha], temp=1.0)


@pytest.mark.parametrize("B", [1, 2, 4, 8])
@pytest.mark.parametrize("temp", [0.0, 0.6, 1.0, 1.2])
def test_lowconc(gpu_lib, dev, B, temp):
    c = CONFIGS["lowconc"]
    _case(gpu_lib, dev, 400 + B, B, c.K, c.V, sigma=c.draft_sigma, temp=temp)


@pytest.mark.parametrize("temp", [1.0, 0.0])
def test_llama8b_b64_full(gpu_lib, dev, temp):
    c = CONFIGS["llama8b_b64"]
    _, ref, out, n, flagged = _case(gpu_lib, dev, 500, c.B, c.K, c.V, sigma=c.draft_sigma, temp=temp)
    assert flagged <= 1


@pytest.mark.parametrize("alpha", [0.6, 0.8, 0.9])
def test_llama70b_b256_sampled(gpu_lib, dev, alpha):
    c = CONFIGS["llama70b_b256"]
    idx = np.arange(0, c.B, 8)                       # 32 of the 256 sequences
    _case(gpu_lib, dev, 600 + int(alpha * 10), c.B, c.K, c.V, sigma=SIGMA_FOR_ALPHA[alpha],
          temp=1.0, idx=idx)


def test_llama70b_b256_greedy_sampled(gpu_lib, dev):
    c = CONFIGS["llama70b_b256"]
    _case(gpu_lib, dev, 650, c.B, c.K, c.V, sigma=c.draft_sigma, temp=0.0,
          idx=np.arange(3, c.B, 8))


def test_mixed_temperatures_in_one_batch(gpu_lib, dev):
    temps = np.array([0.0, 1.0, 0.6, 0.0, 1.2, 1.0, 0.0, 0.3], dtype=np.float32)
    _case(gpu_lib, dev, 700, 8, 7, 32000, sigma=0.51, temp=temps)


@pytest.mark.parametrize("V", [1, 7, 1003, 8191, 8193, 50257])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ragged_vocab(gpu_lib, dev, V, dtype):
    for temp in (1.0, 0.0):
        _case(gpu_lib, dev, 800 + V, 6, 3, V, dtype=dtype, sigma=0.8, temp=temp)


@pytest.mark.parametrize("V", [524_288, 600_000, 2_200_000])
@pytest.mark.parametrize("sigma", [0.25, 1.05])
def test_large_vocab(gpu_lib, dev, V, sigma):
    # 2^19 entries: 64 residual chunks, the most whose sums one wave holds
    # (the draw is made in the pass kernel); past it the draw is a kernel of
    # its own, the chunk scan spans several wave segments and, at 2.2M, more
    # than 256 chunks (chunk sums read in place).
    # sigma 0.25 accepts nearly every draft, so the bonus row is drawn too.
    _case(gpu_lib, dev, 950 + V // 100_000, 3, 2, V, sigma=sigma, temp=1.0)


@pytest.mark.parametrize("K", [1, 16])
def test_k_extremes(gpu_lib, dev, K):
    for temp in (1.0, 0.0):
        _case(gpu_lib, dev, 900 + K, 5, K, 4096, sigma=0.4, temp=temp)


def test_greedy_ties_lowest_index(gpu_lib, dev):
    # Coarse bf16 logits make ties at the maximum common.
    rng = np.random.default_rng(5)
    B, K, V = 32, 5, 20000
    x = np.round(rng.standard_normal((B, K + 1, V)).astype(np.float32) * 2) / 2
    tgt = gen.bf16_bits(x)
    am = np.argmax(gen.bf16_to_f32(tgt), axis=-1)
    d = am[:, :K].copy()
    d[::3, 2] = (d[::3, 2] + 1) % V                   # force some mismatches
    inp = {"target": tgt, "draft": tgt[:, :K].copy(), "draft_tokens": d.astype(np.int32),
           "uniforms": np.zeros((B, K + 1), np.float32),
           "temperature": np.zeros(B, np.float32)}
    ties = (gen.bf16_to_f32(tgt) == gen.bf16_to_f32(tgt).max(-1, keepdims=True)).sum(-1) > 1
    assert ties.any()
    kv0 = np.zeros(B, np.int32)
    ref = orj.reject_sample(inp["target"], None, inp["draft_tokens"], inp["uniforms"],
                            inp["temperature"])
    for with_draft in (True, False):
        out, n, kv_new = _run_gpu(gpu_lib, inp, kv0, dev, with_draft=with_draft)
        assert np.array_equal(out, ref["out_tokens"])
        assert np.array_equal(n, ref["num_accepted"])
        assert np.array_equal(kv_new, kv0 + n + 1)


@pytest.mark.parametrize("B,K,V", [(64, 7, 128256), (4, 3, 600_000)])
def test_greedy_without_draft_logits(gpu_lib, dev, B, K, V):
    # No draft logits: every sequence greedy, grids sized to the target rows
    # (and past 2^19 entries no separate draw kernel); the argmax stream of
    # the oracle, bit for bit.
    _say("greedy without draft logits B=%d K=%d V=%d" % (B, K, V))
    inp = gen.make_reject_inputs(seed=77 + K, B=B, K=K, V=V, draft_sigma=0.3, temperature=0.0)
    kv0 = np.full(B, 10, np.int32)
    ref = orj.reject_sample(inp["target"], None, inp["draft_tokens"], inp["uniforms"],
                            inp["temperature"])
    out, n, kv_new = _run_gpu(gpu_lib, inp, kv0, dev, with_draft=False)
    assert np.array_equal(out, ref["out_tokens"])
    assert np.array_equal(n, ref["num_accepted"])
    assert np.array_equal(kv_new, kv0 + n + 1)


def test_draft_prob_zero_and_residual_edges(gpu_lib, dev):
    # Draft logit -inf at the drafted token: always accepted.  Target -inf at
    # the drafted token: always rejected.
    B, K, V = 4, 2, 64
    rng = np.random.default_rng(9)
    tgt = rng.standard_normal((B, K + 1, V)).astype(np.float32)
    drf = rng.standard_normal((B, K, V)).astype(np.float32)
    d = np.array([[3, 5], [7, 9], [11, 13], [1, 2]], dtype=np.int32)
    drf[0, 0, 3] = -np.inf
    drf[1, 0, 7] = -np.inf
    tgt[2, 0, 11] = -np.inf
    u = np.full((B, K + 1), 0.999, np.float32)
    u[3] = 0.0
    inp = {"target": tgt, "draft": drf, "draft_tokens": d, "uniforms": u,
           "temperature": np.ones(B, np.float32)}
    kv0 = np.arange(B, dtype=np.int32) * 10
    ref = orj.reject_sample(tgt, drf, d, u, inp["temperature"])
    out, n, kv_new = _run_gpu(gpu_lib, inp, kv0, dev)
    assert n[0] >= 1 and n[1] >= 1 and n[2] == 0
    _compare(ref, out, n, kv_new, kv0, inp, label="edges")


def test_counters_and_determinism(gpu_lib, dev):
    import torch
    inp = gen.make_reject_inputs(seed=1000, B=64, K=7, V=128256, draft_sigma=0.51)
    kv0 = np.full(64, 2048, np.int32)
    cnt = torch.zeros(2, dtype=torch.int64, device=dev)
    o1, n1, _ = _run_gpu(gpu_lib, inp, kv0, dev, counters=cnt)
    o2, n2, _ = _run_gpu(gpu_lib, inp, kv0, dev, counters=cnt)
    assert np.array_equal(o1, o2) and np.array_equal(n1, n2)
    c = from_device(cnt)
    assert c[0] == 2 * 64 * 7 and c[1] == 2 * int(n1.sum())


def test_empty_batch_is_noop(gpu_lib, dev):
    import torch
    t = torch.zeros((0, 5, 100), dtype=torch.bfloat16, device=dev)
    out, n = gpu_lib.reject_sample(t, torch.zeros((0, 4, 100), dtype=torch.bfloat16, device=dev),
                                   torch.zeros((0, 4), dtype=torch.int32, device=dev),
                                   torch.zeros((0, 5), dtype=torch.float32, device=dev),
                                   torch.zeros((0,), dtype=torch.float32, device=dev),
                                   torch.zeros((0,), dtype=torch.int32, device=dev))
    assert out.shape == (0, 5) and n.shape == (0,)


def test_multi_step_commit_loop(gpu_lib, dev):
    """Several verify calls in a row on one kv_len buffer: each call commits
    L0 + n + 1 and the next call reads the new length."""
    import torch
    B, K, V = 16, 4, 5000
    kv = torch.full((B,), 100, dtype=torch.int32, device=dev)
    expect = np.full(B, 100, np.int64)
    for step in range(5):
        inp = gen.make_reject_inputs(seed=1100 + step, B=B, K=K, V=V, draft_sigma=0.5)
        out, n = gpu_lib.reject_sample(to_device(inp["target"], dev), to_device(inp["draft"], dev),
                                       to_device(inp["draft_tokens"], dev),
                                       to_device(inp["uniforms"], dev),
                                       to_device(inp["temperature"], dev), kv)
        ref = orj.reject_sample(inp["target"], inp["draft"], inp["draft_tokens"],
                                inp["uniforms"], inp["temperature"])
        ok = ~(ref["flag_accept"] | ref["flag_sample"])
        assert int((~ok).sum()) <= max_flagged(B)
        nn = from_device(n)
        assert np.array_equal(nn[ok], ref["num_accepted"][ok])
        expect += nn + 1
        assert np.array_equal(from_device(kv), expect)


def test_residual_classification_near_tied_rows(gpu_lib, dev):
    """Draft rows equal to the target except a few entries, built so that the
    two normalisers differ by 1e-8 .. 2e-7 of their value: then every tied
    entry has q slightly above p, its residual weight is ~1e-8 q, and which
    side of q = p it falls on must be decided exactly (the fp32 sweep
    statistics cannot resolve it).  Per sequence, at row 0 (V = 128256, K = 1,
    T = 1): the logits of entries a1 < a2 are swapped with smaller ones b1,
    b2 (so the residual holds a1, a2 and the tied entries), and entry c is
    raised by delta, which sets Sp - Sq; d_1 = c is rejected (u_0 = 0.99)."""
    B, K, V = 64, 1, 128256
    rng = np.random.default_rng(4242)
    x = (rng.standard_normal((B, K + 1, V)) * 2).astype(np.float32)
    tgt = gen.bf16_bits(x)
    xt = gen.bf16_to_f32(tgt).astype(np.float64)
    drf = tgt[:, :K].copy()
    d = np.zeros((B, K), np.int32)
    eps_grid = [1e-8, 2e-8, 4e-8, 8e-8, 1.6e-7, 3.2e-7]
    for b in range(B):
        row = xt[b, 0]
        S = np.exp(row).sum()
        # a1, a2 with logits near -1.5 (mass ~1e-7 each), b1, b2 about one lower.
        cand = np.nonzero((row > -1.6) & (row < -1.4))[0]
        a1 = int(cand[cand < V // 2][b % 7])
        a2 = int(cand[cand > V // 2][b % 5])
        low = np.nonzero((row > -2.6) & (row < -2.4))[0]
        b1, b2 = int(low[3 + b % 3]), int(low[-4 - b % 3])
        for a, bb in ((a1, b1), (a2, b2)):
            drf[b, 0, a], drf[b, 0, bb] = tgt[b, 0, bb], tgt[b, 0, a]
        # c with logit near -4: raise it so that (e^{x_c'} - e^{x_c}) / S ~ eps.
        cs = np.nonzero((row > -4.1) & (row < -3.9))[0]
        c = int(cs[b % len(cs)])
        eps = eps_grid[b % len(eps_grid)]
        new = np.log(np.exp(row[c]) + eps * S)
        drf[b, 0, c] = gen.bf16_bits(np.float32([new]))[0]
        d[b, 0] = c
    u = np.full((B, K + 1), 0.99, np.float32)
    u[:, K] = gen.uniforms24(rng, B)
    inp = {"target": tgt, "draft": drf, "draft_tokens": d, "uniforms": u,
           "temperature": np.ones(B, np.float32)}
    kv0 = np.full(B, 1000, np.int32)
    ref = orj.reject_sample(tgt, drf, d, u, inp["temperature"])
    assert (ref["num_accepted"] == 0).all()
    out, n, kv_new = _run_gpu(gpu_lib, inp, kv0, dev)
    # Many of these draws land among the tied entries, whose CDF edges are
    # ~1e-14 apart, so F2 flags them; the rest must agree exactly.
    flag = ref["flag_accept"] | ref["flag_sample"]
    ok = ~flag
    _say("near-tied rows: %d of %d unflagged" % (int(ok.sum()), B))
    assert ok.sum() >= B // 4
    assert np.array_equal(n[ok], ref["num_accepted"][ok])
    assert np.array_equal(out[ok], ref["out_tokens"][ok])
    assert np.array_equal(kv_new, kv0 + n + 1)
