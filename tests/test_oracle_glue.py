"""Pins of the oracle's glue: the exact decoding of stored values and the
code that slices the valid cache rows out of a stored input set.

`to_f64` is checked against torch's own bf16 -> float64 conversion (a
second implementation) over random bit patterns and every special class
(signed zeros, subnormals, infinities, NaNs).  `decode_step_from_inputs`
and `ffn_step_from_inputs` are checked against the plain fp64 steps called
on hand-built arrays: the cache rows at and beyond each position hold NaN
(and the capacity differs from the oracle's own padding), so a row read
past pos, a missed upcast or a shifted slice shows up as a NaN or a
mismatch.
"""
import types

import numpy as np
import torch

import oracle
from attention_block_amd.inputs import f32_to_bf16_bits


def test_to_f64_bf16_matches_torch_on_every_class():
    rng = np.random.default_rng(5)
    bits = rng.integers(0, 1 << 16, size=200000, dtype=np.uint32).astype(np.uint16)
    special = np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x007F, 0x807F, 0x0080, 0x8080, 0x7F7F, 0xFF7F,
                        0x7F80, 0xFF80, 0x7FC0, 0xFFC0, 0x7F81, 0x3F80, 0xBF80], dtype=np.uint16)
    bits = np.concatenate([bits, special])
    ours = oracle.to_f64(bits, "bf16")
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    # signs of zeros and infinities survive
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))
    # the subnormal 0x0001 is 2^-133, the largest finite 0x7F7F is (2 - 2^-7) * 2^127
    assert oracle.to_f64(np.array([0x0001], dtype=np.uint16), "bf16")[0] == 2.0 ** -133
    assert oracle.to_f64(np.array([0x7F7F], dtype=np.uint16), "bf16")[0] == (2 - 2 ** -7) * 2.0 ** 127


def test_to_f64_f32_is_exact():
    rng = np.random.default_rng(6)
    x = (rng.standard_normal(10000) * np.exp(rng.uniform(-80, 80, 10000))).astype(np.float32)
    x = np.concatenate([x, np.array([0.0, -0.0, np.inf, -np.inf, 1e-45, -1e-45], dtype=np.float32)])
    ours = oracle.to_f64(x, "f32")
    ref = torch.from_numpy(x).to(torch.float64).numpy()
    assert np.array_equal(ours, ref) and np.array_equal(np.signbit(ours), np.signbit(ref))


def _stored(values, dtype):
    v32 = np.asarray(values, dtype=np.float32)
    return f32_to_bf16_bits(v32) if dtype == "bf16" else v32


def test_decode_step_from_inputs_reads_only_the_valid_rows():
    for dtype in ("bf16", "f32"):
        rng = np.random.default_rng(7)
        B, H, nq, nkv, D, cap = 3, 16, 4, 2, 8, 9
        pos = np.array([0, 5, 8], dtype=np.int32)            # an empty history, a middle and a full cache
        cfg = types.SimpleNamespace(n_q_heads=nq, n_kv_heads=nkv, head_dim=D, rope_theta=500.0, eps=1e-6,
                                    dtype=dtype)
        vals = {"hidden": rng.standard_normal((B, H)), "norm_w": 1 + 0.1 * rng.standard_normal(H),
                "w_qkv": rng.standard_normal((H, (nq + 2 * nkv) * D)) / 4,
                "w_o": rng.standard_normal((nq * D, H)) / 4,
                "k_cache": rng.standard_normal((B, cap, nkv, D)), "v_cache": rng.standard_normal((B, cap, nkv, D))}
        stored = {k: _stored(v, dtype) for k, v in vals.items()}
        for b in range(B):                                   # rows >= pos hold NaN, as the generator leaves them
            for k in ("k_cache", "v_cache"):
                stored[k][b, pos[b]:] = _stored(np.full((cap - pos[b], nkv, D), np.nan), dtype)
        inp = dict(stored, pos=pos, cfg=cfg)
        got = oracle.decode_step_from_inputs(inp, want_probs=True)
        # the same step on arrays decoded by torch, with the cache rows past pos set to zero
        dec = {k: torch.from_numpy(v.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
               if dtype == "bf16" else v.astype(np.float64) for k, v in stored.items()}
        for b in range(B):
            for k in ("k_cache", "v_cache"):
                dec[k][b, pos[b]:] = 0.0
        want = oracle.decode_step_fp64(dec["hidden"], dec["norm_w"], dec["w_qkv"], dec["w_o"], dec["k_cache"],
                                       dec["v_cache"], pos, n_q_heads=nq, n_kv_heads=nkv, head_dim=D,
                                       rope_theta=500.0, eps=1e-6, storage=dtype, want_probs=True)
        for k in ("out", "y", "q", "k_new", "v_new", "k_row", "v_row", "a", "out_stored"):
            assert np.all(np.isfinite(got[k])), (dtype, k)
            assert np.array_equal(got[k], want[k]), (dtype, k)
        for b in range(B):
            assert got["probs"][b].shape == (nq, pos[b] + 1)
            assert np.array_equal(got["probs"][b], want["probs"][b])
        # sequence 0 has no history: every head attends to the new token alone, so a = v
        G = nq // nkv
        for h in range(nq):
            assert np.allclose(got["a"][0, h * D:(h + 1) * D], got["v_new"][0, h // G], rtol=0, atol=1e-15)


def test_ffn_step_from_inputs_decodes_every_tensor():
    for dtype in ("bf16", "f32"):
        rng = np.random.default_rng(8)
        B, H, F = 2, 16, 24
        cfg = types.SimpleNamespace(eps=1e-6, dtype=dtype)
        vals = {"hidden": rng.standard_normal((B, H)), "norm_w": 1 + 0.1 * rng.standard_normal(H),
                "w_gate": rng.standard_normal((H, F)) / 4, "w_up": rng.standard_normal((H, F)) / 4,
                "w_down": rng.standard_normal((F, H)) / 5}
        stored = {k: _stored(v, dtype) for k, v in vals.items()}
        got = oracle.ffn_step_from_inputs(dict(stored, cfg=cfg))
        dec = {k: torch.from_numpy(v.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
               if dtype == "bf16" else v.astype(np.float64) for k, v in stored.items()}
        want = oracle.ffn_step_fp64(dec["hidden"], dec["norm_w"], dec["w_gate"], dec["w_up"], dec["w_down"],
                                    eps=1e-6, storage=dtype)
        for k in ("out", "y", "m", "g", "u", "hh", "out_stored"):
            assert np.array_equal(got[k], want[k]), (dtype, k)
        # gate and up are not swapped, and the weights are used as [in, out]
        g = torch.nn.functional.linear(torch.from_numpy(got["hh"]), torch.from_numpy(dec["w_gate"]).T).numpy()
        assert np.allclose(got["g"], g, rtol=1e-13, atol=1e-13)
