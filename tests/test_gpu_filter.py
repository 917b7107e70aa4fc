"""GPU parity of spec_reject_sample_filtered against oracle.filter.

Exact on sequences the oracle does not flag (F1, F2 as for the plain
verifier; F3: a top-p boundary within 1e-6 of the mass).  The drafts are
drawn from the filtered draft law, as a filtering drafter would."""

import numpy as np
import pytest

from oracle import filter as of
from synth import gen, CONFIGS
from synth.device import to_device, from_device

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def dev(gpu_lib):
    return "cuda:0"


def _filtered_drafts(inp, top_k, top_p, seed):
    """Drafts d_i ~ filtered softmax(draft row i / T) by the Gumbel-max trick."""
    rng = np.random.default_rng(seed)
    B, K, V = inp["draft"].shape
    toks = inp["draft_tokens"].copy()
    for b in range(B):
        t = float(inp["temperature"][b])
        if t <= 0:
            continue
        df, _ = of.filtered_logits(inp["draft"][b], t, int(top_k[b]), float(top_p[b]))
        g = -np.log(-np.log(rng.random((K, V)) * (1 - 2e-16) + 1e-16))
        toks[b] = np.argmax(df / t + g, axis=-1)
    return toks.astype(np.int32)


def _case(sv, dev, seed, B, K, V, top_k, top_p, dtype="bf16", temp=1.0, sigma=0.8, idx=None,
          std=2.0, spikes=None, max_f3=None, ws="window"):
    """One filtered call against the oracle.  F1 / F2 may exclude a few
    sequences at most (as for the plain verifier); F3 at most ``max_f3``
    (default 2 + B // 50): a row's top-p edge lies within 1e-6 of top_p only
    when the entries at the edge carry little mass, which the cases that
    allow more say why.  ws "window": the binding's workspace (room for the
    sweep's window); "plain": spec_reject_sample_workspace_bytes only, so
    every row takes the filter's radix passes."""
    top_k = np.broadcast_to(np.asarray(top_k, np.int32), (B,)).copy()
    top_p = np.broadcast_to(np.asarray(top_p, np.float32), (B,)).copy()
    label = "filter seed=%d B=%d K=%d V=%d %s k=%s p=%s" % (seed, B, K, V, dtype,
                                                           np.unique(top_k).tolist(),
                                                           np.unique(top_p).tolist())
    _say(label)
    inp = gen.make_reject_inputs(seed=seed, B=B, K=K, V=V, dtype=dtype, draft_sigma=sigma,
                                 temperature=temp, logit_std=std)
    if spikes:
        # Fixed logits at fixed entries of every target row and every draft row.
        pos, tv, dv = spikes
        for name, vals in (("target", tv), ("draft", dv)):
            x = inp[name].copy()
            for i, v in zip(pos, vals):
                x[..., i] = gen._encode(np.float32([v]), dtype)[0]
            inp[name] = x
    inp["draft_tokens"] = _filtered_drafts(inp, top_k, top_p, seed + 1)
    kv0 = np.full(B, 500, np.int32)
    t = {k: to_device(v, dev) for k, v in inp.items()}
    kv = to_device(kv0, dev)
    workspace = None
    if ws == "plain":
        import torch
        workspace = torch.empty(sv.reject_sample_workspace_bytes(B, K, V), dtype=torch.uint8,
                                device=dev)
    out, n = sv.reject_sample(t["target"], t["draft"], t["draft_tokens"], t["uniforms"],
                              t["temperature"], kv, top_k=to_device(top_k, dev),
                              top_p=to_device(top_p, dev), workspace=workspace)
    out, n = from_device(out), from_device(n)
    sel = slice(None) if idx is None else idx
    ref = of.reject_sample_filtered(inp["target"][sel], inp["draft"][sel], inp["draft_tokens"][sel],
                                    inp["uniforms"][sel], inp["temperature"][sel], top_k[sel],
                                    top_p[sel].astype(np.float64))
    flag = ref["flag_accept"] | ref["flag_sample"] | ref["flag_filter"]
    ok = ~flag
    assert np.array_equal(n[sel][ok], ref["num_accepted"][ok]), label
    assert np.array_equal(out[sel][ok], ref["out_tokens"][ok]), label
    assert np.array_equal(from_device(kv), kv0 + n + 1)
    _say("%s: mean accepted %.2f, flagged F1=%d F2=%d F3=%d" % (
        label, n.mean(), ref["flag_accept"].sum(), ref["flag_sample"].sum(),
        ref["flag_filter"].sum()))
    n_seq = int(ref["num_accepted"].shape[0])
    f12 = int((ref["flag_accept"] | ref["flag_sample"]).sum())
    assert f12 <= 2 + n_seq // 1000, (label, f12)
    f3_bound = 2 + n_seq // 50 if max_f3 is None else max_f3
    assert int(ref["flag_filter"].sum()) <= f3_bound, (label, int(ref["flag_filter"].sum()))
    return n


@pytest.mark.parametrize("top_k", [1, 5, 50, 999])
def test_top_k(gpu_lib, dev, top_k):
    _case(gpu_lib, dev, 1, 48, 4, 1000, top_k, 1.0)


@pytest.mark.parametrize("top_p", [0.3, 0.8, 0.95, 0.999])
def test_top_p(gpu_lib, dev, top_p):
    # At 0.95 and 0.999 the edge of the kept set falls among tail entries of
    # ~1e-6 .. 1e-5 mass each (V = 3000), so the 1e-6 band catches a row of
    # 9 now and then (0.95: a few of 48 sequences) or often (0.999: about
    # half).  Those sequences are still checked for validity.
    bound = {0.95: 8, 0.999: 36}.get(top_p)
    _case(gpu_lib, dev, 2, 48, 4, 3000, 0, top_p, max_f3=bound)


def test_both_and_mixed_per_sequence(gpu_lib, dev):
    rng = np.random.default_rng(3)
    B = 64
    top_k = rng.choice([0, 3, 20, 200], size=B)
    top_p = rng.choice([1.0, 0.5, 0.9], size=B)
    temps = rng.choice([0.0, 0.7, 1.0, 1.3], size=B).astype(np.float32)
    _case(gpu_lib, dev, 3, B, 6, 5000, top_k, top_p, temp=temps)


@pytest.mark.parametrize("V,dtype", [(777, "f32"), (4001, "bf16"), (2048, "f32")])
def test_dtypes_and_ragged(gpu_lib, dev, V, dtype):
    _case(gpu_lib, dev, 4, 32, 3, V, 10, 0.9, dtype=dtype)


def test_llama8b_vocab(gpu_lib, dev):
    c = CONFIGS["llama8b_b64"]
    _case(gpu_lib, dev, 5, 16, c.K, c.V, 50, 0.9)


@pytest.mark.parametrize("ws", ["window", "plain"])
@pytest.mark.parametrize("top_k,top_p,temp", [(50, 1.0, 1.0), (0, 0.9, 1.0), (20, 0.8, 0.6),
                                               (0, 0.9, 1.3), (0, 0.5, 1.0), (1, 1.0, 1.0),
                                               (501, 1.0, 1.0), (502, 1.0, 1.0), (0, 0.99, 0.25)])
def test_llama8b_vocab_window_and_radix(gpu_lib, dev, top_k, top_p, temp, ws):
    """The serving vocabulary through both ways of taking the thresholds:
    counted in the sweep's window (the thresholds of these rows fall inside
    it) and the filter's radix passes (the plain workspace).  k = 501 and
    502 sit on either side of V / 256, where the top-k window changes from
    one binade under the sample's largest entry to all 512 keys under the
    top; T = 0.25 puts the top-p edge next to the largest entries."""
    c = CONFIGS["llama8b_b64"]
    _case(gpu_lib, dev, 13, 16, c.K, c.V, top_k, top_p, temp=temp, ws=ws)


def test_off_settings_equal_the_plain_call(gpu_lib, dev):
    import torch
    inp = gen.make_reject_inputs(seed=6, B=32, K=5, V=4000, draft_sigma=0.8)
    t = {k: to_device(v, dev) for k, v in inp.items()}
    kv_a, kv_b = to_device(np.zeros(32, np.int32), dev), to_device(np.zeros(32, np.int32), dev)
    a, na = gpu_lib.reject_sample(t["target"], t["draft"], t["draft_tokens"], t["uniforms"],
                                  t["temperature"], kv_a)
    off_k = torch.zeros(32, dtype=torch.int32, device=dev)
    off_p = torch.ones(32, dtype=torch.float32, device=dev)
    b, nb = gpu_lib.reject_sample(t["target"], t["draft"], t["draft_tokens"], t["uniforms"],
                                  t["temperature"], kv_b, top_k=off_k, top_p=off_p)
    assert torch.equal(a, b) and torch.equal(na, nb)


def test_deterministic(gpu_lib, dev):
    import torch
    inp = gen.make_reject_inputs(seed=7, B=32, K=4, V=6000, draft_sigma=0.8)
    t = {k: to_device(v, dev) for k, v in inp.items()}
    tk = torch.full((32,), 40, dtype=torch.int32, device=dev)
    tp = torch.full((32,), 0.9, dtype=torch.float32, device=dev)
    outs = []
    for _ in range(3):
        kv = torch.zeros(32, dtype=torch.int32, device=dev)
        o, n = gpu_lib.reject_sample(t["target"], t["draft"], t["draft_tokens"], t["uniforms"],
                                     t["temperature"], kv, top_k=tk, top_p=tp)
        outs.append((o.clone(), n.clone()))
    for o, n in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(n, outs[0][1])



# Entries outside the sampled vectors of the top-k bound.  A bf16 row of V
# entries has ceil(V / 8) vectors; the bound reads vector floor(t * nvec / 512)
# for t < 512, so at V = 32000 (or 32003) vectors 1..6 are never read.  The
# bulk is N(0, 0.01) (draft: plus N(0, 0.005)), so the laws over the spikes
# stay far from one-hot and the draft's reversed spikes force rejections.
_POS = (9, 20, 30)


@pytest.mark.parametrize("V", [32000, 32003])
def test_top_k_bound_far_below_the_kth(gpu_lib, dev, V):
    """Three spikes at 0.20..0.22, none of them in the sample: the sampled
    bound sits in the bulk (~0.03), more than 16 first-digit bins under the
    k-th largest value, so the first pass's window misses and the chosen
    bin's values come from the extra pass."""
    sp = (_POS, (0.20, 0.21, 0.22), (0.22, 0.21, 0.20))
    for seed, k in ((8, 3), (9, 2)):
        n = _case(gpu_lib, dev, seed, 32, 3, V, k, 1.0, sigma=0.005, std=0.01, spikes=sp)
        assert n.min() < 3                       # some drafts rejected


def test_top_p_over_top_k_far_above_the_kth(gpu_lib, dev):
    """Top-p over a top-200 set with most of its mass in three spikes at
    5.0..6.0: the top-p boundary bin is far above the 200th value's bin
    (where the window starts)."""
    sp = (_POS, (5.0, 5.5, 6.0), (6.0, 5.5, 5.0))
    for seed, p in ((10, 0.5), (11, 0.75)):
        n = _case(gpu_lib, dev, seed, 32, 3, 32000, 200, p, sigma=0.005, std=0.01, spikes=sp)
        assert n.min() < 3


def test_top_p_alone_with_spikes(gpu_lib, dev):
    # Top-p at 0.5 cuts through the bulk: ~2250 distinct bf16 values, so the
    # mass steps ~1e-4 at the edge and a row is F3-flagged with probability
    # ~2e-6 / 1e-4; with 7 rows per sequence about 15% of the sequences.
    sp = (_POS, (5.0, 5.5, 6.0), (6.0, 5.5, 5.0))
    _case(gpu_lib, dev, 12, 32, 3, 32003, 0, 0.5, sigma=0.005, std=0.01, spikes=sp, max_f3=12)
