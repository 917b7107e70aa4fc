"""spec_reject_sample_noalloc -- the verifier with the library's own per-device
scratch array as its workspace -- against spec_reject_sample on the same
inputs.  Both run the same kernels, so the accepted counts, emitted tokens,
committed lengths and counters must be identical.  Two calls in a row, the
second with a smaller input, so the second one runs on the first one's
leftover scratch contents; then the first shape again.
"""

import numpy as np
import pytest

from synth import gen
from synth.device import to_device, from_device

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _case(sv, dev, seed, B, K, V, temps):
    import torch
    _say("noalloc seed=%d B=%d K=%d V=%d" % (seed, B, K, V))
    inp = gen.make_reject_inputs(seed=seed, B=B, K=K, V=V, dtype="bf16", logit_std=2.0,
                                 draft_sigma=0.51, temperature=temps)
    kv0 = np.random.default_rng(seed).integers(100, 5000, size=B).astype(np.int32)
    t = to_device(inp["target"], dev)
    d = to_device(inp["draft"], dev)
    tok = to_device(inp["draft_tokens"], dev)
    uni = to_device(inp["uniforms"], dev)
    tmp = to_device(inp["temperature"], dev)
    # The call with a caller workspace.
    kv_a = to_device(kv0, dev)
    cnt_a = torch.zeros(2, dtype=torch.int64, device=dev)
    out_a, n_a = sv.reject_sample(t, d, tok, uni, tmp, kv_a, counters=cnt_a)
    # The call on the library's scratch array; outputs pre-filled with junk.
    kv_b = to_device(kv0, dev)
    cnt_b = torch.zeros(2, dtype=torch.int64, device=dev)
    out_b = torch.full((B, K + 1), -7, dtype=torch.int32, device=dev)
    n_b = torch.full((B,), -7, dtype=torch.int32, device=dev)
    sv.reject_sample_noalloc(t, d, tok, uni, tmp, kv_b, out_b, n_b, counters=cnt_b)
    torch.cuda.synchronize()
    assert np.array_equal(from_device(n_b), from_device(n_a))
    assert np.array_equal(from_device(out_b), from_device(out_a))
    assert np.array_equal(from_device(kv_b), from_device(kv_a))
    assert np.array_equal(from_device(kv_b), kv0 + from_device(n_b) + 1)
    assert np.array_equal(from_device(cnt_b), from_device(cnt_a))
    n = from_device(n_b)
    assert (n >= 0).all() and (n <= K).all()


def test_noalloc_matches_workspace_call(gpu_lib):
    sv = gpu_lib
    dev = "cuda:0"
    # The serving batch (mixed sampling and greedy sequences), then a smaller
    # call with a ragged vocabulary (element-load path), then the first again.
    temps64 = np.array([1.0, 0.6, 0.0, 1.2] * 16, dtype=np.float32)
    need = sv.reject_sample_workspace_bytes(64, 7, 128256)
    assert 0 < need <= sv.NOALLOC_SCRATCH_BYTES
    _case(sv, dev, 71, 64, 7, 128256, temps64)
    _case(sv, dev, 72, 5, 3, 1001, np.array([1.0, 0.0, 0.7, 1.0, 2.0], dtype=np.float32))
    _case(sv, dev, 73, 64, 7, 128256, temps64)


def test_noalloc_refuses_oversized_call(gpu_lib):
    import torch
    sv = gpu_lib
    dev = "cuda:0"
    # Beyond the array's limit: SV_ERR_WORKSPACE before any launch, so the
    # outputs keep their contents.
    B, K, V = 4096, 16, 128256
    assert sv.reject_sample_workspace_bytes(B, K, V) > sv.NOALLOC_SCRATCH_BYTES
    z = torch.zeros(1, dtype=torch.bfloat16, device=dev)
    zi = torch.zeros(1, dtype=torch.int32, device=dev)
    zf = torch.zeros(1, dtype=torch.float32, device=dev)
    lib = sv.load()
    st = lib.spec_reject_sample_noalloc(z.data_ptr(), z.data_ptr(), zi.data_ptr(), zf.data_ptr(),
                                        zf.data_ptr(), zi.data_ptr(), zi.data_ptr(), zi.data_ptr(),
                                        None, B, K, V, sv.SV_BF16, None)
    assert st == -3
    torch.cuda.synchronize()
    assert int(zi.item()) == 0
