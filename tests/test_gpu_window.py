"""GPU parity of the window calls: spec_verify_attn_window (append and
scratch modes), spec_kv_commit, and the page pool driving a multi-step loop.

The cache after an append must equal oracle.kv.append_window bit for bit,
and the attention output must equal spec_verify_attn (or _tree) run on that
appended cache bit for bit (the same bf16 operands reach the same MFMAs), and
the float64 oracle within the attention tolerance.  Scratch mode leaves the
cache untouched.  spec_kv_commit equals oracle.kv.commit bit for bit.
"""

import numpy as np
import pytest

from oracle import attention as oat
from oracle import kv as okv
from oracle import tree as otr
from synth import gen, CONFIGS
from synth.tree import ancestor_bits, chain_parents, children, tree_parents
from synth.device import to_device, from_device

pytestmark = pytest.mark.gpu

BF16_ATOL, BF16_RTOL = 2e-2, 1e-2
F32_ATOL, F32_RTOL = 1e-4, 1e-4


def _say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def dev(gpu_lib):
    return "cuda:0"


def _widen(x, dtype):
    return gen.bf16_to_f32(x).astype(np.float64) if dtype == "bf16" else x.astype(np.float64)


def _tol(gpu, ref, dtype, label):
    atol, rtol = (BF16_ATOL, BF16_RTOL) if dtype == "bf16" else (F32_ATOL, F32_RTOL)
    err = np.abs(gpu - ref)
    bad = err > atol + rtol * np.abs(ref)
    _say("%s: max abs err %.3g, violations %d" % (label, err.max(), bad.sum()))
    assert not bad.any(), label


def _case(sv, dev, seed, B, N, Hq, Hkv, D, ctx, dtype="bf16", parents=None, check_oracle=True):
    label = "window seed=%d B=%d N=%d Hq=%d Hkv=%d D=%d ctx=%s %s %s" % (
        seed, B, N, Hq, Hkv, D, ctx, dtype, "tree" if parents is not None else "chain")
    _say(label)
    inp = gen.make_attn_inputs(seed=seed, B=B, K=N - 1, Hq=Hq, Hkv=Hkv, D=D, ctx=ctx, dtype=dtype)
    kn, vn = gen.make_window_kv(seed + 1, B, N, Hkv, D, dtype)
    anc = None
    if parents is not None:
        anc = np.stack([ancestor_bits(p).astype(np.uint32) for p in parents]).view(np.int32)
    k_ref, v_ref = okv.append_window(inp["k_cache"], inp["v_cache"], inp["block_table"],
                                     inp["kv_len"], kn, vn)
    t = {k: to_device(v, dev) for k, v in inp.items()}
    d_anc = None if anc is None else to_device(anc, dev)
    d_kn, d_vn = to_device(kn, dev), to_device(vn, dev)
    # Reference on the device: the plain call on the oracle-appended cache.
    kr, vr = to_device(k_ref, dev), to_device(v_ref, dev)
    if anc is None:
        ref_out = sv.verify_attn(t["q"], kr, vr, t["block_table"], t["kv_len"])
    else:
        ref_out = sv.verify_attn_tree(t["q"], kr, vr, t["block_table"], t["kv_len"], d_anc)
    # Scratch mode: cache untouched, same output.
    kc0, vc0 = t["k_cache"].clone(), t["v_cache"].clone()
    out_r = sv.verify_attn_window(t["q"], d_kn, d_vn, kc0, vc0, t["block_table"], t["kv_len"],
                                  anc=d_anc, mode=sv.SV_WINDOW_READ)
    assert np.array_equal(from_device(kc0), inp["k_cache"]), label + " scratch wrote K"
    assert np.array_equal(from_device(vc0), inp["v_cache"]), label + " scratch wrote V"
    assert np.array_equal(from_device(out_r), from_device(ref_out)), label + " scratch out"
    # Append mode: cache = oracle append, same output.
    out_a = sv.verify_attn_window(t["q"], d_kn, d_vn, t["k_cache"], t["v_cache"],
                                  t["block_table"], t["kv_len"], anc=d_anc,
                                  mode=sv.SV_WINDOW_APPEND)
    assert np.array_equal(from_device(t["k_cache"]), k_ref), label + " append K"
    assert np.array_equal(from_device(t["v_cache"]), v_ref), label + " append V"
    assert np.array_equal(from_device(out_a), from_device(ref_out)), label + " append out"
    if check_oracle:
        if anc is None:
            ref = oat.verify_attention(inp["q"], k_ref, v_ref, inp["block_table"], inp["kv_len"])
        else:
            ref = otr.tree_attention(inp["q"], k_ref, v_ref, inp["block_table"], inp["kv_len"],
                                     np.stack(parents))
        _tol(_widen(from_device(out_a), dtype), ref, dtype, label)


def test_llama8b_shape_chain(gpu_lib, dev):
    c = CONFIGS["llama8b_b64"]
    # 24 sequences with L0 spread over every offset in a page pair: the window
    # starts anywhere and straddles pages and pairs.
    _case(gpu_lib, dev, 1, 24, c.K + 1, c.Hq, c.Hkv, c.D, (33, 700))


@pytest.mark.parametrize("N", [2, 5, 17])
def test_window_sizes(gpu_lib, dev, N):
    Hq = 2 * 8 if N * 2 <= 64 else 8
    _case(gpu_lib, dev, 10 + N, 12, N, Hq, 8, 128, (0, 300))


def test_two_tiles_and_d64(gpu_lib, dev):
    _case(gpu_lib, dev, 21, 8, 12, 32, 8, 128, (40, 900))         # 48 rows: two tiles
    _case(gpu_lib, dev, 22, 8, 8, 32, 8, 64, (40, 900))           # D = 64


def test_tree_window(gpu_lib, dev):
    par = tree_parents((2, 2, 2))
    c = CONFIGS["llama8b_b64"]
    _case(gpu_lib, dev, 31, 6, len(par), c.Hq, c.Hkv, c.D, (100, 2000), parents=[par] * 6)


def test_fp32_window(gpu_lib, dev):
    _case(gpu_lib, dev, 41, 4, 6, 8, 2, 64, (10, 200), dtype="f32")
    par = tree_parents((2, 2))
    _case(gpu_lib, dev, 42, 3, len(par), 8, 2, 128, (5, 90), dtype="f32", parents=[par] * 3)


@pytest.mark.parametrize("B,Hq", [(300, 64), (520, 32)])
def test_large_batch_prologue(gpu_lib, dev, B, Hq):
    # Past the thread count of a workgroup (256 two-tile, 512 one-tile): the
    # looped prologue; outputs and caches against the plain call on the
    # oracle-appended cache (that call's own parity is checked above).
    _case(gpu_lib, dev, 60 + B, B, 8, Hq, 8, 128, (16, 120), check_oracle=False)


def test_empty_context(gpu_lib, dev):
    _case(gpu_lib, dev, 51, 4, 8, 32, 8, 128, 0)                   # L0 = 0: the window alone


# ---- commit ---------------------------------------------------------------

def _paths(rng, parent, B):
    """A random root path per sequence: (num_accepted [B], nodes [B, N])."""
    kids = children(parent)
    n_out = np.zeros(B, np.int32)
    nodes = np.full((B, len(parent)), -1, np.int32)
    for b in range(B):
        v, path = 0, []
        while kids[v] and rng.random() < 0.8:
            v = int(rng.choice(kids[v]))
            path.append(v)
        n_out[b] = len(path)
        nodes[b, :len(path)] = path
    return n_out, nodes


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("mode", ["scratch_chain", "scratch_tree", "inplace_tree", "inplace_chain"])
def test_commit(gpu_lib, dev, dtype, mode):
    rng = np.random.default_rng(61)
    B, Hkv, D = 16, 4, 128
    par = tree_parents((2, 2, 2)) if "tree" in mode else chain_parents(8)
    N = len(par)
    inp = gen.make_attn_inputs(seed=62, B=B, K=N - 1, Hq=Hkv, Hkv=Hkv, D=D, ctx=(0, 100),
                               dtype=dtype)
    kn, vn = gen.make_window_kv(63, B, N, Hkv, D, dtype)
    if "tree" in mode:
        n, nodes = _paths(rng, par, B)
    else:
        n, nodes = rng.integers(0, N, size=B).astype(np.int32), None
    kv_after = (inp["kv_len"] + n + 1).astype(np.int32)
    scratch = mode.startswith("scratch")
    k_ref, v_ref = okv.commit(inp["k_cache"], inp["v_cache"], inp["block_table"], kv_after, n,
                              nodes=nodes, k_src=kn if scratch else None,
                              v_src=vn if scratch else None)
    kc, vc = to_device(inp["k_cache"], dev), to_device(inp["v_cache"], dev)
    gpu_lib.kv_commit(kc, vc, to_device(inp["block_table"], dev), to_device(kv_after, dev),
                      to_device(n, dev), nodes=None if nodes is None else to_device(nodes, dev),
                      k_src=to_device(kn, dev) if scratch else None,
                      v_src=to_device(vn, dev) if scratch else None, N=N)
    assert np.array_equal(from_device(kc), k_ref), mode
    assert np.array_equal(from_device(vc), v_ref), mode
    _say("commit %s %s: mean accepted %.2f" % (mode, dtype, n.mean()))


# ---- the loop: page pool -> append attention -> tree verifier -> commit -----

def test_multi_step_tree_loop_with_page_pool(gpu_lib, dev):
    """Several verify steps of a few sequences: the pool reserves the window
    pages, the attention appends the window in place, the tree verifier
    accepts a path, the commit compacts it and the pool frees the tail.  The
    cache must hold, at every committed position, the K/V row that the
    surviving path put there, and the pool must end with no page lost."""
    import torch
    rng = np.random.default_rng(71)
    B, Hq, Hkv, D, V = 4, 16, 4, 64, 4000
    par = tree_parents((2, 2))
    N = len(par)
    nb, mbps = 64, 12
    pool = gpu_lib.PagePool(nb, B, mbps)
    x = gen.kv_layout_x("bf16")
    kc = torch.zeros((nb, Hkv, D // x, 16, x), dtype=torch.bfloat16, device=dev)
    vc = torch.zeros((nb, Hkv, D, 16), dtype=torch.bfloat16, device=dev)
    kv_len = np.full(B, 5, np.int32)
    expect_k = [dict() for _ in range(B)]                  # position -> K row bits [Hkv, D]
    for b in range(B):
        pool.reserve(b, int(kv_len[b]))
        pool.commit(b, int(kv_len[b]))
    for step in range(6):
        for b in range(B):
            pool.reserve(b, int(kv_len[b]) + N)
        bt = to_device(pool.block_table(), dev)
        q = to_device(gen.bf16_bits(rng.standard_normal((B, N, Hq, D)).astype(np.float32)), dev)
        kn, vn = gen.make_window_kv(100 + step, B, N, Hkv, D)
        anc = to_device(np.stack([ancestor_bits(par).astype(np.uint32)] * B).view(np.int32), dev)
        d_len = to_device(kv_len, dev)
        gpu_lib.verify_attn_window(q, to_device(kn, dev), to_device(vn, dev), kc, vc, bt, d_len,
                                   anc=anc, mode=gpu_lib.SV_WINDOW_APPEND)
        rin = gen.make_tree_reject_inputs(seed=200 + step, B=B, parent=par, V=V,
                                          draft_sigma=0.5)
        ot, on, n = gpu_lib.reject_sample_tree(to_device(rin["target"], dev),
                                               to_device(rin["draft"], dev), par,
                                               to_device(rin["tokens"], dev),
                                               to_device(rin["uniforms"], dev),
                                               to_device(rin["temperature"], dev), d_len)
        gpu_lib.kv_commit(kc, vc, bt, d_len, n, nodes=on, N=N)
        n_h, on_h, new_len = from_device(n), from_device(on), from_device(d_len)
        for b in range(B):
            l0 = int(kv_len[b])
            assert new_len[b] == l0 + n_h[b] + 1
            rows = [0] + [int(v) for v in on_h[b, :n_h[b]]]
            for j, r in enumerate(rows):
                expect_k[b][l0 + j] = kn[b, r]
            for p in [p for p in expect_k[b] if p >= new_len[b]]:
                del expect_k[b][p]                     # rolled back
            pool.commit(b, int(new_len[b]))
        kv_len = new_len.astype(np.int32)
        assert pool.check() == 0
    # Every tracked position holds its row.
    k_all = from_device(kc)
    table = pool.block_table()
    for b in range(B):
        for p, row in expect_k[b].items():
            blk, tok = table[b, p // 16], p % 16
            assert np.array_equal(k_all[blk, :, :, tok, :].reshape(Hkv, D), row), (b, p)
    for b in range(B):
        pool.release(b)
    assert pool.free_count() == nb and pool.check() == 0
    _say("loop: final lengths %s" % kv_len.tolist())
