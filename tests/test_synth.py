"""The seeded input generator: determinism, storage formats, and the recipe's structure."""
import numpy as np

from hash_hierarchical_top_amd import synth


def test_seeded_and_deterministic():
    a = synth.make_hhr_inputs(2, 8, 2, [100, 37], 112, "bf16", seed=5)
    b = synth.make_hhr_inputs(2, 8, 2, [100, 37], 112, "bf16", seed=5)
    for k in a:
        assert np.array_equal(a[k], b[k]), k
    c = synth.make_hhr_inputs(2, 8, 2, [100, 37], 112, "bf16", seed=6)
    assert not np.array_equal(a["K"], c["K"])


def test_bf16_round_trip_and_rounding():
    x = np.array([1.0, 1.00390625, 1.01171875, -3.5, 0.0, -0.0, 65504.0], np.float32)
    bits = synth.f32_to_bf16_bits(x)
    back = synth.bf16_bits_to_f32(bits)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7 -> even (1.0); 1 + 3*2^-8 -> 1 + 2^-6 (even)
    assert back.tolist() == [1.0, 1.0, 1.015625, -3.5, 0.0, -0.0, 65536.0]
    assert np.array_equal(synth.f32_to_bf16_bits(back), bits)


def test_recipe_structure():
    inp = synth.make_hhr_inputs(2, 8, 2, [100, 37], 112, "bf16", seed=5)
    assert inp["K"].shape == (2, 2, 112, 128) and inp["K"].dtype == np.uint16
    assert np.all(inp["K"][1, :, 37:] == 0) and np.all(inp["V"][0, :, 100:] == 0)
    assert inp["q"].dtype == np.float32
    assert np.array_equal(synth.round_to_bf16(inp["q"]), inp["q"])
    R = inp["R"].astype(np.float64)
    assert np.abs(np.einsum("gij,gkj->gik", R, R) - np.eye(128)).max() < 1e-6
    assert np.all(np.diff(inp["planted"], axis=-1) > 0)
    K = synth.kv_values(inp["K"][0, 0, :100], "bf16")
    std = K.std(axis=0)
    out = inp["outliers"][0]
    assert np.all(std[out] > 4.0) and np.median(std) < 1.5


def test_ragged_lengths_in_range():
    w = synth.WORKLOADS["llama8b_ragged_b16"]
    lens = synth.seq_lens_for(w)
    assert lens.shape == (16,) and lens.min() >= 8192 and lens.max() <= 65536
    assert len(set(lens.tolist())) > 1


def test_e4m3_storage():
    inp = synth.make_hisa_inputs(4, 50, 64, 2, 9, head_dim=32)
    assert inp["k8"].dtype == np.uint8 and inp["k8"].shape == (64, 32)
    assert np.all(inp["k_scale"][50:] == 0) and np.all(inp["k_scale"][:50] > 0)
    # the largest magnitude in each row is stored as +-448 (0x7E / 0xFE)
    assert np.all(np.max(inp["k8"][:50] & 0x7F, axis=1) == 0x7E)
