"""The seeded input generator: encodings, ranges and the alpha it produces."""

import numpy as np
import pytest

from oracle import reject as orj
from synth import gen, CONFIGS, SIGMA_FOR_ALPHA


def test_bf16_round_to_nearest_even():
    # 1 + 2^-8 is halfway between bf16 neighbours 1 and 1 + 2^-7: ties to even (1).
    x = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20],
                 dtype=np.float32)
    back = gen.bf16_to_f32(gen.bf16_bits(x))
    assert back[0] == 1.0
    assert back[1] == 1.0 + 2 ** -6          # 1 + 3*2^-8 -> tie, even neighbour
    assert back[2] == -1.0
    assert back[3] == 1.0 + 2 ** -7          # above the tie rounds up
    rng = np.random.default_rng(0)
    y = rng.standard_normal(100000).astype(np.float32) * 3
    b = gen.bf16_to_f32(gen.bf16_bits(y))
    assert np.all(np.abs(b - y) <= np.abs(y) * 2 ** -8 + 1e-30)
    assert np.array_equal(gen.bf16_bits(b), gen.bf16_bits(y))          # idempotent
    assert gen.bf16_bits(np.array([np.inf], np.float32))[0] == 0x7F80


def test_uniforms_grid_and_range():
    u = gen.uniforms24(np.random.default_rng(1), (1000, 9))
    assert u.dtype == np.float32
    assert u.min() >= 0.0 and u.max() < 1.0
    assert np.all((u.astype(np.float64) * 2 ** 24) % 1 == 0)


def test_reject_inputs_shapes_and_determinism():
    a = gen.make_reject_inputs(seed=5, B=3, K=4, V=1000, temperature=[1.0, 0.0, 0.6])
    b = gen.make_reject_inputs(seed=5, B=3, K=4, V=1000, temperature=[1.0, 0.0, 0.6])
    assert a["target"].shape == (3, 5, 1000) and a["target"].dtype == np.uint16
    assert a["draft"].shape == (3, 4, 1000)
    assert a["draft_tokens"].shape == (3, 4) and a["uniforms"].shape == (3, 5)
    for k in a:
        assert np.array_equal(a[k], b[k])
    assert a["draft_tokens"].min() >= 0 and a["draft_tokens"].max() < 1000
    # The greedy sequence's drafts are the draft rows' argmax.
    vals = gen.bf16_to_f32(a["draft"][1])
    assert np.array_equal(a["draft_tokens"][1], np.argmax(vals, axis=-1))


def test_attn_inputs_page_table_is_a_permutation():
    inp = gen.make_attn_inputs(seed=2, B=4, K=7, Hq=8, Hkv=2, D=64, ctx=(30, 90))
    bt, L = inp["block_table"], inp["kv_len"]
    used = np.concatenate([bt[b, :(L[b] + 8 + 15) // 16] for b in range(4)])
    assert len(set(used.tolist())) == used.size            # no page shared
    assert used.min() >= 0 and used.max() < inp["k_cache"].shape[0]
    assert inp["k_cache"].shape[1:] == (2, 8, 16, 8)
    assert inp["v_cache"].shape[1:] == (2, 64, 16)


@pytest.mark.parametrize("alpha", sorted(SIGMA_FOR_ALPHA))
def test_sigma_gives_target_alpha(alpha):
    # Measured with the oracle at T = 1 on N(0, 2) bf16 rows of a large vocabulary.
    inp = gen.make_reject_inputs(seed=int(alpha * 10), B=2, K=2, V=128256,
                                 draft_sigma=SIGMA_FOR_ALPHA[alpha])
    a = orj.acceptance_rate(inp["target"][:, :2], inp["draft"], 1.0)
    assert abs(a.mean() - alpha) < 0.02, a


def test_configs_are_consistent():
    for c in CONFIGS.values():
        assert c.Hq % c.Hkv == 0
        assert c.ctx[0] <= c.ctx[1]
    assert CONFIGS["llama8b_b64"].B == 64 and CONFIGS["llama8b_b64"].V == 128256
