"""The seeded input generator: bf16 rounding, reproducibility and mask structure."""
import numpy as np
import pytest
import torch

from flashattention_forward_attn_amd import inputs


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 100000),
                        np.array([0.0, -0.0, 1.0, -1.0, 3.0e38, -3.0e38, 1e-40, 65504.0], np.float32)]).astype(np.float32)
    ours = inputs.bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    # exact round trip for values that are already bf16
    np.testing.assert_array_equal(inputs.bf16_bits(inputs.bf16_to_f32(ours)), ours)


def test_ties_round_to_even():
    # 1 + 2^-8 lies halfway between bf16 neighbours 1 and 1 + 2^-7: even mantissa wins
    x = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8], np.float32)
    np.testing.assert_array_equal(inputs.bf16_to_f32(inputs.bf16_bits(x)), [1.0, 1 + 2 * 2.0 ** -7])


def test_reproducible_and_seed_dependent():
    w = inputs.custom("t", "bf16", 2, 3, 40, 64, False)
    a, b = inputs.generate(w), inputs.generate(w)
    assert a.digests() == b.digests()
    c = inputs.generate(w, seed=1)
    assert a.digests()["q"] != c.digests()["q"]


def test_f32_workload_first_draw():
    w = inputs.WORKLOADS["f32_b1h1n256d64"]
    x = inputs.generate(w)
    ref = np.random.default_rng(0).standard_normal((1, 1, 256, 64)).astype(np.float32)
    np.testing.assert_array_equal(x.q, ref)
    assert x.q_bits is None and x.kv_limit is None


def test_key_padding_structure():
    w = inputs.custom("kp", "bf16", 8, 2, 1024, 128, False, qk_mult=8.0, v_dist="uniform", key_padding=True)
    x = inputs.generate(w)
    assert x.kv_limit.shape == (8, 1024) and x.kv_limit.dtype == np.int32
    assert np.all((x.lengths >= 1) & (x.lengths <= 1024))
    q0, b = x.masked_q0, x.masked_batch
    assert q0 % inputs.MASKED_QUERY_BLOCK == 0
    assert np.all(x.kv_limit[b, q0:q0 + inputs.MASKED_QUERY_BLOCK] == 0)
    rest = np.ones((8, 1024), bool)
    rest[b, q0:q0 + inputs.MASKED_QUERY_BLOCK] = False
    assert np.all(x.kv_limit[rest] == np.repeat(x.lengths[:, None], 1024, axis=1)[rest])
    assert np.abs(x.v).max() <= 1.0
    # Q and K carry the factor 8: their spread is about 8
    assert 7.5 < x.q.std() < 8.5


@pytest.mark.parametrize("name", sorted(inputs.WORKLOADS))
def test_workload_table(name):
    w = inputs.WORKLOADS[name]
    assert w.d in (64, 128) and w.dtype in ("bf16", "f32")
    assert w.flops() == 4.0 * w.B * w.H * w.N ** 2 * w.d / (2 if w.causal else 1)
