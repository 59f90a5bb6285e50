"""Input generators: determinism, bf16 rounding and planted structure."""
import numpy as np

import synth


def test_bf16_round_to_nearest_even():
    x = np.array([1.0, 1.00390625, 1.01171875, -2.5, 0.0, -0.0, 3.0e38, 1e-40], np.float32)
    u = x.view(np.uint32)
    b = synth.bf16_bits(x)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: rounds to the even mantissa (1.0)
    assert b[0] == 0x3F80 and b[1] == 0x3F80
    # 1 + 3*2^-8 is a tie between 1+2^-7 and 1+2^-6: rounds up to even
    assert b[2] == 0x3F82
    assert b[3] == u[3] >> 16 and b[4] == 0 and b[5] == 0x8000
    np.testing.assert_array_equal(synth.bf16_to_f32(b)[[0, 3]], x[[0, 3]])
    r = np.random.default_rng(0).standard_normal(10000).astype(np.float32)
    back = synth.bf16_to_f32(synth.bf16_bits(r))
    assert np.all(np.abs(back - r) <= np.abs(r) * 2.0 ** -8)  # unit roundoff of an 8-bit significand


def test_generators_are_deterministic_and_head_local():
    a = synth.sparsemm_heads(head_subset=[3, 700])
    b = synth.sparsemm_heads(head_subset=[700])
    np.testing.assert_array_equal(a.k[1], b.k[0])
    np.testing.assert_array_equal(a.q_obs[:, 1], b.q_obs[:, 0])
    c = synth.tiny_mha()
    d = synth.tiny_mha()
    assert c.k.tobytes() == d.k.tobytes()
    e = synth.tiny_mha(trial=1)
    assert c.k.tobytes() != e.k.tobytes()


def test_workload_shapes_and_planting():
    w = synth.tiny_mha()
    assert w.k.shape == (8, 2048, 64) and w.k.dtype == np.float32
    assert len(w.extra["heavy"]) == round(0.02 * 2048)
    assert w.extra["heavy"].min() >= 4 and w.extra["heavy"].max() < 2048 - 32
    w = synth.llama_obs(n=4096)
    assert w.q_obs.shape == (32, 32, 128) and w.k_top == int(0.3 * 4096) - 68
    assert all(len(h) == round(0.01 * 4096) for h in w.extra["heavy"])
    w = synth.qwen_std(frames=4)
    assert w.k.shape == (4, 4 * 196 + 512 + 5, 128)
    assert w.extra["q_verify"].shape == (5, 28, 128)
    s = synth.sparsemm_heads(head_subset=[]).extra
    assert len(s["visual_heads"]) == round(0.05 * 1024) and s["total_budget"] == 262144
