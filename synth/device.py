"""Moving generated inputs onto a torch device, and seeded on-device KV caches.

The KV caches of the largest workloads (tens of GB) are drawn on the device
with a seeded torch generator instead of numpy; the oracle then copies back
only the pages of the sequences it checks.  Only randomness and layout live
here, no verify arithmetic.
"""

import numpy as np

from .gen import BLOCK, kv_layout_x

__all__ = ["to_device", "from_device", "make_attn_inputs_device"]


def to_device(arr, device):
    """numpy -> torch on ``device``; uint16 arrays are bf16 bit patterns."""
    import torch
    a = np.ascontiguousarray(arr)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


def from_device(t):
    """torch -> numpy; bfloat16 comes back as uint16 bit patterns."""
    import torch
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def make_attn_inputs_device(seed, B, K, Hq, Hkv, D, ctx, device, dtype="bf16",
                            spare_blocks=7, q_scale=1.0):
    """Like ``gen.make_attn_inputs`` but draws q / K / V with torch on ``device``.

    Context lengths and the shuffled page table come from numpy streams of
    the same SeedSequence; q, k_cache and v_cache are N(0, 1) (q scaled by
    ``q_scale``) from a torch generator seeded from it, rounded to bf16.
    Returns torch tensors on ``device``.
    """
    import torch
    ss = np.random.SeedSequence(seed)
    s_l, s_p, s_t = ss.spawn(3)
    r_l, r_p = np.random.default_rng(s_l), np.random.default_rng(s_p)
    if np.isscalar(ctx):
        l0 = np.full(B, int(ctx), dtype=np.int64)
    else:
        l0 = r_l.integers(int(ctx[0]), int(ctx[1]) + 1, size=B)
    need = (l0 + K + 1 + BLOCK - 1) // BLOCK
    mbps = int(need.max())
    nb = int(need.sum()) + spare_blocks
    perm = r_p.permutation(nb).astype(np.int32)
    bt = np.zeros((B, mbps), dtype=np.int32)
    off = 0
    for b in range(B):
        bt[b, :need[b]] = perm[off:off + need[b]]
        off += need[b]
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    g = torch.Generator(device=device)
    g.manual_seed(int(s_t.generate_state(1)[0]))
    x = kv_layout_x(dtype)

    def randn(shape, scale=1.0):
        out = torch.empty(shape, dtype=tdt, device=device)
        flat = out.view(-1)
        step = 1 << 26
        for i in range(0, flat.numel(), step):
            n = min(step, flat.numel() - i)
            flat[i:i + n] = (torch.randn(n, generator=g, device=device, dtype=torch.float32)
                             * scale).to(tdt)
        return out

    q = randn((B, K + 1, Hq, D), q_scale)
    kc = randn((nb, Hkv, D // x, BLOCK, x))
    vc = randn((nb, Hkv, D, BLOCK))
    return {"q": q, "k_cache": kc, "v_cache": vc,
            "block_table": torch.from_numpy(bt).to(device),
            "kv_len": torch.from_numpy(l0.astype(np.int32)).to(device)}
