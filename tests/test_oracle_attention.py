"""Pins of the verify-attention oracle (no GPU).

(i)   agreement with an independent dense reference: the pages are un-paged
      by inverting the block table (a different route from the oracle's
      per-token lookup) and torch's scaled_dot_product_attention runs in
      float64 on the CPU with an explicit window-causal mask;
(ii)  closed forms: q = 0 gives the mean of the visible values; a single
      visible key gives its value;
(iii) invariances: relabelling physical pages, changing keys the causal mask
      hides, and GQA == MHA with repeated KV heads.
"""

import numpy as np
import pytest
import torch

from oracle import attention as oat
from oracle.reject import widen
from synth import gen


def _dense_by_inverse_table(inp, dtype):
    """[B, Lmax, Hkv, D] keys / values by walking physical pages once."""
    kc, vc = widen(inp["k_cache"]), widen(inp["v_cache"])
    nb, hkv, dx, blk, x = kc.shape
    d = dx * x
    bt = inp["block_table"]
    kv_len = inp["kv_len"]
    b_sz = bt.shape[0]
    k1 = inp["q"].shape[1]
    lmax = int(kv_len.max()) + k1
    keys = np.zeros((b_sz, lmax, hkv, d))
    vals = np.zeros((b_sz, lmax, hkv, d))
    for b in range(b_sz):
        n_pages = (int(kv_len[b]) + k1 + blk - 1) // blk
        for pg in range(n_pages):
            phys = bt[b, pg]
            kpage = np.transpose(kc[phys], (2, 0, 1, 3)).reshape(blk, hkv, d)   # [16,Hkv,D]
            vpage = np.transpose(vc[phys], (2, 0, 1))                            # [16,Hkv,D]
            lo = pg * blk
            hi = min(lo + blk, lmax)
            keys[b, lo:hi] = kpage[: hi - lo]
            vals[b, lo:hi] = vpage[: hi - lo]
    return keys, vals


def _sdpa_reference(inp):
    q = widen(inp["q"])                          # [B, K+1, Hq, D]
    b_sz, k1, hq, d = q.shape
    keys, vals = _dense_by_inverse_table(inp, None)
    hkv = keys.shape[2]
    out = np.zeros_like(q)
    for b in range(b_sz):
        l0 = int(inp["kv_len"][b])
        L = l0 + k1
        kk = torch.from_numpy(keys[b, :L]).permute(1, 0, 2)      # [Hkv, L, D]
        vv = torch.from_numpy(vals[b, :L]).permute(1, 0, 2)
        kk = kk.repeat_interleave(hq // hkv, dim=0)               # [Hq, L, D]
        vv = vv.repeat_interleave(hq // hkv, dim=0)
        qq = torch.from_numpy(q[b]).permute(1, 0, 2)              # [Hq, K+1, D]
        pos = torch.arange(L)[None, :]
        qpos = l0 + torch.arange(k1)[:, None]
        mask = pos <= qpos                                        # [K+1, L]
        o = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, attn_mask=mask)
        out[b] = o.permute(1, 0, 2).numpy()
    return out


@pytest.mark.parametrize("dtype,B,K,Hq,Hkv,D,ctx", [
    ("f32", 1, 4, 1, 1, 64, 128),
    ("bf16", 3, 7, 8, 2, 64, (5, 40)),
    ("bf16", 2, 2, 4, 4, 128, (17, 33)),
    ("f32", 2, 3, 6, 3, 32, (0, 20)),
])
def test_matches_dense_sdpa(dtype, B, K, Hq, Hkv, D, ctx):
    inp = gen.make_attn_inputs(seed=7, B=B, K=K, Hq=Hq, Hkv=Hkv, D=D, ctx=ctx, dtype=dtype)
    ref = _sdpa_reference(inp)
    out = oat.verify_attention(inp["q"], inp["k_cache"], inp["v_cache"],
                               inp["block_table"], inp["kv_len"])
    assert np.max(np.abs(out - ref)) < 1e-10


def test_zero_query_gives_mean_of_visible_values():
    inp = gen.make_attn_inputs(seed=3, B=2, K=3, Hq=4, Hkv=2, D=32, ctx=(9, 30), dtype="f32")
    inp["q"] = np.zeros_like(inp["q"])
    out = oat.verify_attention(inp["q"], inp["k_cache"], inp["v_cache"],
                               inp["block_table"], inp["kv_len"])
    for b in range(2):
        l0 = int(inp["kv_len"][b])
        _, vals = oat.gather_kv(inp["k_cache"], inp["v_cache"], inp["block_table"], b, l0 + 4)
        for i in range(4):
            for h in range(4):
                g = h // 2
                assert np.allclose(out[b, i, h], vals[: l0 + i + 1, g].mean(axis=0), atol=1e-12)


def test_single_visible_key_gives_its_value():
    inp = gen.make_attn_inputs(seed=4, B=1, K=2, Hq=2, Hkv=1, D=16, ctx=0, dtype="f32")
    out = oat.verify_attention(inp["q"], inp["k_cache"], inp["v_cache"],
                               inp["block_table"], inp["kv_len"])
    blk = inp["block_table"][0, 0]
    v0 = inp["v_cache"][blk, 0, :, 0]
    assert np.allclose(out[0, 0, 0], v0, atol=1e-12)
    assert np.allclose(out[0, 0, 1], v0, atol=1e-12)


def test_page_relabelling_is_invisible():
    inp = gen.make_attn_inputs(seed=5, B=2, K=4, Hq=4, Hkv=2, D=32, ctx=(20, 50), dtype="bf16")
    base = oat.verify_attention(inp["q"], inp["k_cache"], inp["v_cache"],
                                inp["block_table"], inp["kv_len"])
    nb = inp["k_cache"].shape[0]
    perm = np.random.default_rng(1).permutation(nb)          # new slot of old block
    kc2 = np.empty_like(inp["k_cache"])
    vc2 = np.empty_like(inp["v_cache"])
    kc2[perm] = inp["k_cache"]
    vc2[perm] = inp["v_cache"]
    bt2 = perm[inp["block_table"]].astype(np.int32)
    out = oat.verify_attention(inp["q"], kc2, vc2, bt2, inp["kv_len"])
    assert np.array_equal(out, base)


def test_masked_keys_do_not_matter():
    inp = gen.make_attn_inputs(seed=6, B=1, K=5, Hq=2, Hkv=1, D=16, ctx=37, dtype="f32")
    base = oat.verify_attention(inp["q"], inp["k_cache"], inp["v_cache"],
                                inp["block_table"], inp["kv_len"])
    l0 = int(inp["kv_len"][0])
    # Change the K/V of window position 3 (absolute l0 + 3): queries 0..2 must not move.
    j = l0 + 3
    blk, slot = inp["block_table"][0, j // 16], j % 16
    kc, vc = inp["k_cache"].copy(), inp["v_cache"].copy()
    kc[blk, :, :, slot, :] += 5.0
    vc[blk, :, :, slot] -= 3.0
    out = oat.verify_attention(inp["q"], kc, vc, inp["block_table"], inp["kv_len"])
    assert np.array_equal(out[:, :3], base[:, :3])
    assert not np.allclose(out[:, 3:], base[:, 3:])


def test_gqa_equals_mha_with_repeated_heads():
    inp = gen.make_attn_inputs(seed=8, B=2, K=3, Hq=6, Hkv=2, D=32, ctx=(10, 25), dtype="f32")
    gqa = oat.verify_attention(inp["q"], inp["k_cache"], inp["v_cache"],
                               inp["block_table"], inp["kv_len"])
    rep = 3
    kc = np.repeat(inp["k_cache"], rep, axis=1)
    vc = np.repeat(inp["v_cache"], rep, axis=1)
    mha = oat.verify_attention(inp["q"], kc, vc, inp["block_table"], inp["kv_len"])
    assert np.max(np.abs(gqa - mha)) < 1e-12
