"""Validation mode (SPECVERIFY_VALIDATE=1) through the C ABI.

Valid inputs give exactly the results of the unchecked calls.  An input that
breaks a stated precondition is refused with SV_ERR_BAD_INPUT before anything
is launched: the outputs and kv_len keep their previous contents.  Every bad
input here is caught on the host, so no kernel ever sees it.
"""

import numpy as np
import pytest

from synth import gen
from synth.device import to_device, from_device

pytestmark = pytest.mark.gpu

BAD_INPUT = -6


def _say(msg):
    print(msg, flush=True)


def _refused(sv, fn, *args, **kw):
    with pytest.raises(sv.SpecVerifyError) as ei:
        fn(*args, **kw)
    assert ei.value.status == BAD_INPUT, ei.value


def _attn_inputs(dev, seed=11, B=3, K=4, ctx=(40, 300)):
    inp = gen.make_attn_inputs(seed=seed, B=B, K=K, Hq=8, Hkv=2, D=128, ctx=ctx)
    return inp, {k: to_device(v, dev) for k, v in inp.items()}


def test_attention_valid_and_refused(gpu_lib, monkeypatch):
    import torch
    sv, dev = gpu_lib, "cuda:0"
    inp, t = _attn_inputs(dev)
    _say("validate attention B=3 K=4 Hq=8 Hkv=2 D=128")
    ref = sv.verify_attn(t["q"], t["k_cache"], t["v_cache"], t["block_table"], t["kv_len"])
    torch.cuda.synchronize()
    monkeypatch.setenv("SPECVERIFY_VALIDATE", "1")
    out = sv.verify_attn(t["q"], t["k_cache"], t["v_cache"], t["block_table"], t["kv_len"])
    assert torch.equal(out, ref)
    nb = inp["k_cache"].shape[0]
    L = int(inp["kv_len"][1])
    sentinel = torch.full_like(ref, 7.0)
    # A page the call reads (the one holding position L0 + K) out of range.
    bt = inp["block_table"].copy()
    bt[1, (L + 4) // 16] = nb
    _refused(sv, sv.verify_attn, t["q"], t["k_cache"], t["v_cache"], to_device(bt, dev),
             t["kv_len"], out=sentinel)
    bt[1, (L + 4) // 16] = -1
    _refused(sv, sv.verify_attn, t["q"], t["k_cache"], t["v_cache"], to_device(bt, dev),
             t["kv_len"], out=sentinel)
    # A page past the window is not read: garbage there is accepted.
    bt = inp["block_table"].copy()
    last = (int(inp["kv_len"].max()) + 4) // 16 + 1
    if last < bt.shape[1]:
        bt[:, last:] = nb + 100
        out = sv.verify_attn(t["q"], t["k_cache"], t["v_cache"], to_device(bt, dev), t["kv_len"])
        assert torch.equal(out, ref)
    # Lengths: negative, and above max_kv_len.
    kv = inp["kv_len"].copy()
    kv[0] = -1
    _refused(sv, sv.verify_attn, t["q"], t["k_cache"], t["v_cache"], t["block_table"],
             to_device(kv, dev), out=sentinel)
    _refused(sv, sv.verify_attn, t["q"], t["k_cache"], t["v_cache"], t["block_table"],
             t["kv_len"], out=sentinel, max_kv_len=int(inp["kv_len"].max()) - 1)
    torch.cuda.synchronize()
    assert bool((sentinel == 7.0).all()), "a refused call launched a kernel"


def _reject_case(dev, seed=21, B=6, K=4, V=3000):
    temps = np.array([1.0, 0.0, 0.7, 1.0, 1.3, 0.0], dtype=np.float32)[:B]
    r = gen.make_reject_inputs(seed=seed, B=B, K=K, V=V, temperature=temps)
    return r, {k: to_device(v, dev) for k, v in r.items()}


def _run_reject(sv, d, kv0, **kw):
    import torch
    kv = kv0.clone()
    tok, n = sv.reject_sample(d["target"], d["draft"], d["draft_tokens"], d["uniforms"],
                              d["temperature"], kv, **kw)
    torch.cuda.synchronize()
    return from_device(tok), from_device(n), from_device(kv)


def test_reject_valid_and_refused(gpu_lib, monkeypatch):
    import torch
    sv, dev = gpu_lib, "cuda:0"
    r, d = _reject_case(dev)
    B, K1, V = r["target"].shape
    K = K1 - 1
    kv0 = to_device(np.full(B, 500, dtype=np.int32), dev)
    _say("validate reject B=%d K=%d V=%d" % (B, K, V))
    ref = _run_reject(sv, d, kv0)
    ref_f = _run_reject(sv, d, kv0, top_k=to_device(np.full(B, 20, np.int32), dev),
                        top_p=to_device(np.full(B, 0.9, np.float32), dev))
    monkeypatch.setenv("SPECVERIFY_VALIDATE", "1")
    got = _run_reject(sv, d, kv0)
    for a, b in zip(got, ref):
        assert np.array_equal(a, b)
    got_f = _run_reject(sv, d, kv0, top_k=to_device(np.full(B, 20, np.int32), dev),
                        top_p=to_device(np.full(B, 0.9, np.float32), dev))
    for a, b in zip(got_f, ref_f):
        assert np.array_equal(a, b)

    def refused(**over):
        dd = dict(d)
        dd.update({k: to_device(v, dev) for k, v in over.items() if k in d})
        kv = kv0.clone()
        tok = torch.full((B, K1), -7, dtype=torch.int32, device=dev)
        extra = {k: to_device(v, dev) for k, v in over.items() if k in ("top_k", "top_p")}
        _refused(sv, sv.reject_sample, dd["target"], dd["draft"], dd["draft_tokens"],
                 dd["uniforms"], dd["temperature"], kv, out_tokens=tok, **extra)
        torch.cuda.synchronize()
        assert bool((kv == kv0).all()) and bool((tok == -7).all()), "refused call launched"

    dt = r["draft_tokens"].copy(); dt[2, 1] = V
    refused(draft_tokens=dt)
    dt = r["draft_tokens"].copy(); dt[0, 0] = -1
    refused(draft_tokens=dt)
    u = r["uniforms"].copy(); u[3, K] = 1.0
    refused(uniforms=u)
    t = r["temperature"].copy(); t[4] = np.nan
    refused(temperature=t)
    x = r["target"].copy(); x[1, 2, 17] = 0x7FC0          # bf16 NaN
    refused(target=x)
    x = r["target"].copy(); x[5, 0, 0] = 0x7F80           # bf16 +inf
    refused(target=x)
    x = r["draft"].copy(); x[0, 3, :] = 0xFF80            # a draft row of -inf only
    refused(draft=x)
    refused(top_p=np.array([0.9, np.nan, 0.9, 0.9, 0.9, 0.9], np.float32))
    # -inf entries are allowed.
    x = r["target"].copy(); x[:, :, 5] = 0xFF80
    d2 = dict(d); d2["target"] = to_device(x, dev)
    _run_reject(sv, d2, kv0)


def test_tree_reject_and_commit(gpu_lib, monkeypatch):
    import torch
    sv, dev = gpu_lib, "cuda:0"
    parent = [-1, 0, 0, 1, 1, 2, 2]
    B, N, V = 4, len(parent), 1000
    r = gen.make_tree_reject_inputs(seed=31, B=B, parent=parent, V=V,
                                    temperature=np.array([1.0, 0.0, 1.0, 0.5], np.float32))
    d = {k: to_device(v, dev) for k, v in r.items()}
    kv0 = to_device(np.full(B, 300, dtype=np.int32), dev)
    _say("validate tree reject B=%d N=%d V=%d" % (B, N, V))

    def run(tokens):
        kv = kv0.clone()
        out = sv.reject_sample_tree(d["target"], d["draft"], parent, tokens, d["uniforms"],
                                    d["temperature"], kv)
        torch.cuda.synchronize()
        return [from_device(o) for o in out] + [from_device(kv)]

    ref = run(d["tokens"])
    monkeypatch.setenv("SPECVERIFY_VALIDATE", "1")
    tok = r["tokens"].copy(); tok[:, 0] = 123456            # entry 0 is not used
    got = run(to_device(tok, dev))
    for a, b in zip(got, ref):
        assert np.array_equal(a, b)
    tok = r["tokens"].copy(); tok[2, 3] = V
    _refused(sv, sv.reject_sample_tree, d["target"], d["draft"], parent, to_device(tok, dev),
             d["uniforms"], d["temperature"], kv0.clone())

    # spec_kv_commit over the tree's outputs.
    inp, t = _attn_inputs(dev, seed=41, B=B, K=N - 1, ctx=(30, 200))
    kv_after = to_device(from_device(t["kv_len"]) + ref[2] + 1, dev)
    nacc, nodes = to_device(ref[2], dev), to_device(ref[1], dev)
    sv.kv_commit(t["k_cache"], t["v_cache"], t["block_table"], kv_after, nacc, nodes=nodes)
    bad = ref[2].copy(); bad[0] = N
    _refused(sv, sv.kv_commit, t["k_cache"], t["v_cache"], t["block_table"], kv_after,
             to_device(bad, dev), nodes=nodes)
    bt = inp["block_table"].copy(); bt[1, 0] = inp["k_cache"].shape[0]
    _refused(sv, sv.kv_commit, t["k_cache"], t["v_cache"], to_device(bt, dev), kv_after, nacc,
             nodes=nodes)
