"""GPU parity of spec_verify_attn_tree against the CPU oracle.

Tolerances as for spec_verify_attn: bf16 |gpu - ref| <= 2e-2 + 1e-2 |ref|,
fp32 1e-4 + 1e-4 |ref|, against oracle.tree.tree_attention in float64.  A
chain-shaped tree must give exactly the bits of spec_verify_attn.
"""

import numpy as np
import pytest

from oracle import tree as otr
from synth import gen, CONFIGS
from synth.tree import ancestor_bits, chain_parents, tree_parents
from synth.device import to_device, from_device, make_attn_inputs_device

pytestmark = pytest.mark.gpu

BF16_ATOL, BF16_RTOL = 2e-2, 1e-2
F32_ATOL, F32_RTOL = 1e-4, 1e-4


def _say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def dev(gpu_lib):
    return "cuda:0"


def _check(gpu, ref, dtype, label):
    atol, rtol = (BF16_ATOL, BF16_RTOL) if dtype == "bf16" else (F32_ATOL, F32_RTOL)
    err = np.abs(gpu - ref)
    bad = err > atol + rtol * np.abs(ref)
    _say("%s: max abs err %.3g, violations %d of %d" % (label, err.max(), bad.sum(), bad.size))
    assert not bad.any(), label


def _widen(x, dtype):
    return gen.bf16_to_f32(x).astype(np.float64) if dtype == "bf16" else x.astype(np.float64)


def _anc_batch(parents):
    """[B, N] int32 view of the uint32 ancestor sets of one parent[] per sequence."""
    return np.stack([ancestor_bits(p).astype(np.uint32) for p in parents]).view(np.int32)


def _case(sv, dev, seed, B, parents, Hq, Hkv, D, ctx, dtype="bf16", q_scale=1.0, idx=None):
    n = len(parents[0])
    label = "tree attn seed=%d B=%d N=%d Hq=%d Hkv=%d D=%d ctx=%s %s" % (seed, B, n, Hq, Hkv, D,
                                                                        ctx, dtype)
    _say(label)
    inp = gen.make_attn_inputs(seed=seed, B=B, K=n - 1, Hq=Hq, Hkv=Hkv, D=D, ctx=ctx, dtype=dtype,
                               q_scale=q_scale)
    anc = _anc_batch(parents)
    t = {k: to_device(v, dev) for k, v in inp.items()}
    out = sv.verify_attn_tree(t["q"], t["k_cache"], t["v_cache"], t["block_table"], t["kv_len"],
                              to_device(anc, dev))
    gpu = _widen(from_device(out), dtype)
    ref = otr.tree_attention(inp["q"], inp["k_cache"], inp["v_cache"], inp["block_table"],
                             inp["kv_len"], np.stack(parents), batch_indices=idx)
    sel = slice(None) if idx is None else idx
    _check(gpu[sel], ref[sel], dtype, label)
    return inp, t, gpu


def test_tiny_fp32_tree(gpu_lib, dev):
    par = tree_parents((2, 2))
    _case(gpu_lib, dev, 1, 2, [par, par], 1, 1, 64, (40, 130), dtype="f32")


@pytest.mark.parametrize("shape", [(2, 2), (3, 2), (2, 2, 2), (4,), (1, 1, 1, 1, 1, 1, 1)])
def test_llama8b_shaped_trees(gpu_lib, dev, shape):
    # 32 q / 8 kv heads: G (N) rows per KV head, one 32-row tile up to N = 8,
    # two tiles up to N = 16.
    par = tree_parents(shape)
    c = CONFIGS["llama8b_b64"]
    _case(gpu_lib, dev, 100 + len(par), 6, [par] * 6, c.Hq, c.Hkv, c.D, (300, 2500))


def test_different_tree_per_sequence(gpu_lib, dev):
    shapes = [(2, 2), (1, 1, 1, 1, 1, 1), (3, 1), (6,)]           # all 7 nodes
    pars = [tree_parents(s) for s in shapes]
    assert len({len(p) for p in pars}) == 1
    _case(gpu_lib, dev, 7, 4, pars, 16, 8, 128, (0, 600))


def test_fp32_tree_shapes(gpu_lib, dev):
    par = tree_parents((2, 1, 2))
    _case(gpu_lib, dev, 8, 3, [par] * 3, 8, 2, 128, (10, 200), dtype="f32")


def test_chain_tree_is_bitwise_verify_attn(gpu_lib, dev):
    import torch
    c = CONFIGS["llama8b_b64"]
    K = c.K
    t = make_attn_inputs_device(2024, 16, K, c.Hq, c.Hkv, c.D, (100, 3000), dev)
    anc = _anc_batch([chain_parents(K + 1)] * 16)
    a = gpu_lib.verify_attn(t["q"], t["k_cache"], t["v_cache"], t["block_table"], t["kv_len"])
    b = gpu_lib.verify_attn_tree(t["q"], t["k_cache"], t["v_cache"], t["block_table"],
                                 t["kv_len"], to_device(anc, dev))
    assert torch.equal(a, b)


def test_llama8b_b64_tree_sampled(gpu_lib, dev):
    # Full-size batch with a [2,2,2] tree (15 nodes, two tiles per KV head);
    # the oracle checks every 8th sequence.
    c = CONFIGS["llama8b_b64"]
    par = tree_parents((2, 2, 2))
    n = len(par)
    _say("tree attn llama8b_b64 [2,2,2] device-drawn")
    t = make_attn_inputs_device(2025, c.B, n - 1, c.Hq, c.Hkv, c.D, c.ctx, dev)
    anc = _anc_batch([par] * c.B)
    out = gpu_lib.verify_attn_tree(t["q"], t["k_cache"], t["v_cache"], t["block_table"],
                                   t["kv_len"], to_device(anc, dev))
    idx = list(range(0, c.B, 8))
    kvl = from_device(t["kv_len"])
    bt = from_device(t["block_table"])
    import torch
    for b in idx:
        pages = bt[b, :(int(kvl[b]) + n + 15) // 16]
        sel = torch.from_numpy(pages.astype(np.int64)).to(dev)
        kc = from_device(t["k_cache"][sel])
        vc = from_device(t["v_cache"][sel])
        ref = otr.tree_attention(from_device(t["q"][b:b + 1]), kc, vc,
                                 np.arange(len(pages), dtype=np.int32)[None],
                                 kvl[b:b + 1], par)
        gpu = _widen(from_device(out[b:b + 1]), "bf16")
        _check(gpu, ref, "bf16", "llama8b tree seq %d" % b)
