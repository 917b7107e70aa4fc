"""The draft-length controller driving the verifier on the GPU: each step the
bandit picks K, spec_reject_sample verifies K drafts, the library's counters
and the acceptance statistics of num_accepted feed the reward.  Checks the
bookkeeping (counters = sum of K B proposed and of n accepted; a_i and L as
the oracle computes them from the same outputs), not a speed-up: the draft
cost is a stated model here (the verify path has no drafter)."""

import numpy as np
import pytest

from oracle import bandit as ob
from synth import gen
from synth.device import to_device, from_device

pytestmark = pytest.mark.gpu


def test_bandit_drives_the_verifier(gpu_lib):
    import torch
    dev = "cuda:0"
    B, V = 16, 32000
    arms = (2, 4, 6, 8)
    inputs = {}
    for K in arms:
        inp = gen.make_reject_inputs(seed=300 + K, B=B, K=K, V=V, draft_sigma=0.51)
        inputs[K] = {k: to_device(v, dev) for k, v in inp.items()}
    bandit = gpu_lib.DraftLengthBandit(arms)
    rng = np.random.default_rng(9)
    counters = torch.zeros(2, dtype=torch.int64, device=dev)
    proposed = accepted = 0
    draft_us_per_token = 40.0                  # modelled drafter cost per drafted token
    for step in range(24):
        a = bandit.select(*rng.random(2))
        K = arms[a]
        t = inputs[K]
        kv = torch.full((B,), 1000, dtype=torch.int32, device=dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        _, n = gpu_lib.reject_sample(t["target"], t["draft"], t["draft_tokens"], t["uniforms"],
                                     t["temperature"], kv, counters=counters)
        e1.record()
        torch.cuda.synchronize()
        n_h = from_device(n)
        a_i, L = gpu_lib.accept_stats(n_h, K)
        a_o, L_o = ob.acceptance_stats(n_h, K)
        assert np.array_equal(a_i, a_o) and L == L_o
        assert np.array_equal(from_device(kv), 1000 + n_h + 1)
        proposed += K * B
        accepted += int(n_h.sum())
        seconds = (e0.elapsed_time(e1) * 1e3 + K * draft_us_per_token) * 1e-6
        bandit.update(a, B * L / seconds)
    c = from_device(counters)
    assert c[0] == proposed and c[1] == accepted
    pulls, means, tcount = bandit.stats()
    assert tcount == 24 and sum(pulls) == 24 and min(pulls) >= 2
    print("pulls %s, mean tokens/s %s" % (pulls, [round(m) for m in means]), flush=True)
    bandit.close()
