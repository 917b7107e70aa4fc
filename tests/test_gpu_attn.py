"""GPU parity of spec_verify_attn against the CPU oracle.

bf16: |gpu - ref| <= 2e-2 + 1e-2 * |ref| elementwise against the float64
oracle on the same bf16 inputs.  fp32: 1e-4 + 1e-4 * |ref| (fp32 scores and
sums over at most a few thousand keys carry ~1e-6 relative error).
"""

import numpy as np
import pytest

from oracle import attention as oat
from synth import gen, CONFIGS
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


def _case(sv, dev, seed, B, K, Hq, Hkv, D, ctx, dtype="bf16", q_scale=1.0, idx=None,
          max_kv_len=None):
    label = "attn seed=%d B=%d K=%d Hq=%d Hkv=%d D=%d ctx=%s %s qs=%s" % (
        seed, B, K, Hq, Hkv, D, ctx, dtype, q_scale)
    _say(label)
    inp = gen.make_attn_inputs(seed=seed, B=B, K=K, Hq=Hq, Hkv=Hkv, D=D, ctx=ctx, dtype=dtype,
                               q_scale=q_scale)
    t = {k: to_device(v, dev) for k, v in inp.items()}
    out = sv.verify_attn(t["q"], t["k_cache"], t["v_cache"], t["block_table"], t["kv_len"],
                         max_kv_len=max_kv_len)
    gpu = _widen(from_device(out), dtype)
    ref = oat.verify_attention(inp["q"], inp["k_cache"], inp["v_cache"], inp["block_table"],
                               inp["kv_len"], batch_indices=idx)
    sel = slice(None) if idx is None else idx
    _check(gpu[sel], ref[sel], dtype, label)
    return inp, gpu, ref


def test_tiny_fp32(gpu_lib, dev):
    c = CONFIGS["tiny"]
    _case(gpu_lib, dev, 11, 1, c.K, c.Hq, c.Hkv, c.D, c.ctx[0], dtype="f32")


@pytest.mark.parametrize("K", [2, 4, 6, 8])
def test_qwen_b1(gpu_lib, dev, K):
    c = CONFIGS["qwen_b1"]
    _case(gpu_lib, dev, 20 + K, 1, K, c.Hq, c.Hkv, c.D, c.ctx[0])


@pytest.mark.parametrize("B", [1, 2, 4, 8])
def test_lowconc(gpu_lib, dev, B):
    c = CONFIGS["lowconc"]
    _case(gpu_lib, dev, 30 + B, B, c.K, c.Hq, c.Hkv, c.D, c.ctx)


def test_llama8b_b64_full(gpu_lib, dev):
    c = CONFIGS["llama8b_b64"]
    _case(gpu_lib, dev, 40, c.B, c.K, c.Hq, c.Hkv, c.D, c.ctx)


def test_llama70b_b256_sampled(gpu_lib, dev):
    """Full-size cache (~21 GB, drawn on the device); the oracle checks 6
    sequences, including the shortest and the longest."""
    import torch
    c = CONFIGS["llama70b_b256"]
    _say("attn llama70b_b256 full size, device-drawn cache")
    t = make_attn_inputs_device(41, c.B, c.K, c.Hq, c.Hkv, c.D, c.ctx, dev)
    out = gpu_lib.verify_attn(t["q"], t["k_cache"], t["v_cache"], t["block_table"], t["kv_len"])
    kv = from_device(t["kv_len"])
    bt = from_device(t["block_table"])
    pick = sorted({int(np.argmin(kv)), int(np.argmax(kv)), 0, 77, 128, c.B - 1})
    for b in pick:
        pages = bt[b, :(kv[b] + c.K + 1 + 15) // 16]
        sub_k = from_device(t["k_cache"][torch.from_numpy(pages).long().to(dev)])
        sub_v = from_device(t["v_cache"][torch.from_numpy(pages).long().to(dev)])
        ref = oat.verify_attention(from_device(t["q"][b:b + 1]), sub_k, sub_v,
                                   np.arange(len(pages), dtype=np.int32)[None], kv[b:b + 1])
        gpu = _widen(from_device(out[b:b + 1]), "bf16")
        _check(gpu, ref, "bf16", "llama70b b=%d L0=%d" % (b, kv[b]))
    del t, out
    torch.cuda.empty_cache()


@pytest.mark.parametrize("q_scale", [4.0, 12.0])
def test_peaked_scores(gpu_lib, dev, q_scale):
    # Large q makes softmax nearly one-hot: stresses the max subtraction.
    _case(gpu_lib, dev, 50, 4, 7, 32, 8, 128, (100, 700), q_scale=q_scale)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("G,K", [(1, 1), (2, 16), (4, 7), (8, 7), (3, 5), (7, 8)])
def test_shapes(gpu_lib, dev, D, G, K):
    # Row tiles of 1..64 rows, ragged page pairs, contexts from 0.
    _case(gpu_lib, dev, 60 + G * 17 + K, 3, K, 2 * G, 2, D, (0, 300))


def test_fp32_shapes(gpu_lib, dev):
    _case(gpu_lib, dev, 70, 3, 3, 4, 2, 128, (0, 200), dtype="f32")
    _case(gpu_lib, dev, 71, 2, 6, 6, 3, 64, (15, 33), dtype="f32")


@pytest.mark.parametrize("B,Hq", [(300, 64), (600, 32), (1100, 32)])
def test_large_batch_prologue(gpu_lib, dev, B, Hq):
    """Batches larger than a workgroup's thread count (256 threads for the
    two-tile kernel at 64 rows, 512 for one tile at 32 rows): each workgroup
    finds its first sequence by a looped block scan over kv_len instead of a
    single one.  Short contexts keep the oracle fast; a spread of sequences,
    the first and the last included, is checked element by element."""
    idx = sorted(set(range(0, B, 23)) | {1, B // 2, B - 2, B - 1})
    _case(gpu_lib, dev, 90 + B, B, 7, Hq, 8, 128, (16, 200), idx=idx)


def test_split_boundaries(gpu_lib, dev):
    # Many sequences with lengths around split / pair boundaries.
    _case(gpu_lib, dev, 80, 24, 7, 32, 8, 128, (120, 2200))


def test_nan_in_unused_tail_slots(gpu_lib, dev):
    """Slots after the sequence end in its last page are never written by a
    real cache; NaN there must not reach the output."""
    inp = gen.make_attn_inputs(seed=90, B=3, K=4, Hq=8, Hkv=2, D=128, ctx=(33, 70))
    kc, vc = inp["k_cache"].copy(), inp["v_cache"].copy()
    for b in range(3):
        L = int(inp["kv_len"][b]) + 5
        for j in range(L, ((L + 31) // 32) * 32):
            pg = j // 16
            if pg < inp["block_table"].shape[1] and j < (L + 15) // 16 * 16:
                blk, slot = inp["block_table"][b, pg], j % 16
                kc[blk, :, :, slot, :] = 0x7FC0           # bf16 NaN
                vc[blk, :, :, slot] = 0x7FC0
    t = {k: to_device(v, dev) for k, v in inp.items()}
    out = gpu_lib.verify_attn(t["q"], to_device(kc, dev), to_device(vc, dev), t["block_table"],
                              t["kv_len"])
    gpu = _widen(from_device(out), "bf16")
    assert np.isfinite(gpu).all()
    ref = oat.verify_attention(inp["q"], kc, vc, inp["block_table"], inp["kv_len"])
    _check(gpu, ref, "bf16", "nan tail")


def test_determinism(gpu_lib, dev):
    inp = gen.make_attn_inputs(seed=95, B=8, K=7, Hq=32, Hkv=8, D=128, ctx=(500, 3000))
    t = {k: to_device(v, dev) for k, v in inp.items()}
    o1 = from_device(gpu_lib.verify_attn(t["q"], t["k_cache"], t["v_cache"], t["block_table"], t["kv_len"]))
    o2 = from_device(gpu_lib.verify_attn(t["q"], t["k_cache"], t["v_cache"], t["block_table"], t["kv_len"]))
    assert np.array_equal(o1, o2)


def test_determinism_at_serving_size(gpu_lib, dev):
    """Three calls at the serving size (many partial segments merged by the
    combine kernel) give the same bits.  One tile (the chain) and two tiles
    (8 query heads per KV head)."""
    import torch
    c = CONFIGS["llama8b_b64"]
    for Hq in (c.Hq, 2 * c.Hq):
        _say("attn determinism B=%d Hq=%d" % (c.B, Hq))
        t = make_attn_inputs_device(43, c.B, c.K, Hq, c.Hkv, c.D, c.ctx, dev)
        outs = [gpu_lib.verify_attn(t["q"], t["k_cache"], t["v_cache"], t["block_table"],
                                    t["kv_len"]) for _ in range(3)]
        torch.cuda.synchronize()
        for o in outs[1:]:
            assert torch.equal(o, outs[0])
        del t, outs
        torch.cuda.empty_cache()


def test_empty_batch_and_errors(gpu_lib, dev):
    import torch
    q = torch.zeros((0, 8, 32, 128), dtype=torch.bfloat16, device=dev)
    kc = torch.zeros((1, 8, 16, 16, 8), dtype=torch.bfloat16, device=dev)
    vc = torch.zeros((1, 8, 128, 16), dtype=torch.bfloat16, device=dev)
    out = gpu_lib.verify_attn(q, kc, vc, torch.zeros((0, 1), dtype=torch.int32, device=dev),
                              torch.zeros((0,), dtype=torch.int32, device=dev), max_kv_len=0)
    assert out.shape == q.shape
    q2 = torch.zeros((1, 8, 32, 96), dtype=torch.bfloat16, device=dev)     # D = 96 unsupported
    kc2 = torch.zeros((1, 8, 12, 16, 8), dtype=torch.bfloat16, device=dev)
    vc2 = torch.zeros((1, 8, 96, 16), dtype=torch.bfloat16, device=dev)
    with pytest.raises(gpu_lib.SpecVerifyError):
        gpu_lib.verify_attn(q2, kc2, vc2, torch.zeros((1, 1), dtype=torch.int32, device=dev),
                            torch.zeros((1,), dtype=torch.int32, device=dev), max_kv_len=0)
    with pytest.raises(ValueError):                                       # q and caches disagree on D
        gpu_lib.verify_attn(q2, kc, vc, torch.zeros((1, 1), dtype=torch.int32, device=dev),
                            torch.zeros((1,), dtype=torch.int32, device=dev), max_kv_len=0)
