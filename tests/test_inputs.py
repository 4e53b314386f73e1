"""The seeded input generator: deterministic, right shapes, sentinel tail."""
import hashlib

import numpy as np
import pytest

from attention_block_amd.inputs import (CONFIGS, BlockConfig, algorithmic_bytes, bf16_bits_to_f32,
                                        f32_to_bf16_bits, make_inputs, positions)

SMALL = BlockConfig("small_gqa", 3, 64, 4, 2, 16, "bf16", 5e5, ragged=(5, 40))


def digest(inp):
    h = hashlib.sha256()
    for k in ("hidden", "norm_w", "w_qkv", "w_o", "k_cache", "v_cache", "pos"):
        h.update(np.ascontiguousarray(inp[k]).tobytes())
    return h.hexdigest()


def test_same_seed_same_bytes():
    assert digest(make_inputs(SMALL, 1)) == digest(make_inputs(SMALL, 1))
    assert digest(make_inputs(SMALL, 1)) != digest(make_inputs(SMALL, 2))


def test_shapes_and_sentinel():
    inp = make_inputs(SMALL, 0, cap=50)
    B, H, nq, nkv, D = 3, 64, 4, 2, 16
    assert inp["hidden"].shape == (B, H) and inp["hidden"].dtype == np.uint16
    assert inp["w_qkv"].shape == (H, (nq + 2 * nkv) * D)
    assert inp["w_o"].shape == (nq * D, H)
    assert inp["k_cache"].shape == (B, 50, nkv, D)
    pos = inp["pos"]
    assert np.array_equal(pos, positions(SMALL, 0))
    assert pos.min() >= 5 and pos.max() <= 40
    for b in range(B):
        k = bf16_bits_to_f32(inp["k_cache"][b])
        assert np.all(np.isfinite(k[: pos[b]]))
        assert np.all(np.isnan(k[pos[b]:]))


def test_ragged_lengths_match_config_range():
    cfg = CONFIGS["gqa_ragged_bs32"]
    for seed in (0, 1):
        p = positions(cfg, seed)
        assert p.shape == (32,) and p.min() >= 256 and p.max() <= 8192


def test_distributions():
    cfg = BlockConfig("d", 2, 1024, 8, 8, 64, "f32", 1e4, pos=64)
    inp = make_inputs(cfg, 3)
    assert abs(np.std(inp["w_qkv"]) - 1 / 32) < 1e-3          # variance 1/H
    assert abs(np.mean(inp["norm_w"]) - 1) < 0.02 and abs(np.std(inp["norm_w"]) - 0.1) < 0.01
    assert abs(np.std(inp["k_cache"][:, :64]) - 1) < 0.02


def test_bf16_round_trip():
    x = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, -2.5, np.nan, 3.0e38], dtype=np.float32)
    b = f32_to_bf16_bits(x)
    back = bf16_bits_to_f32(b)
    assert back[0] == 1.0 and back[1] == 1.0 and back[2] == 1 + 2 ** -6 and back[3] == -2.5
    assert np.isnan(back[4])


def test_headline_bytes():
    cfg = CONFIGS["llama2_7b_bs1_4k"]
    assert algorithmic_bytes(cfg, [4096]) == 201_367_556


def test_position_override_without_configured_length():
    cfg = BlockConfig("free", 2, 64, 2, 1, 64, "f32", 1e4)
    inp = make_inputs(cfg, 0, cap=9, pos=[0, 8])
    assert list(inp["pos"]) == [0, 8] and inp["k_cache"].shape == (2, 9, 1, 64)
    assert np.all(np.isnan(inp["k_cache"][0])) and np.all(np.isfinite(inp["k_cache"][1, :8]))
    with pytest.raises(ValueError):
        make_inputs(cfg, 0)
