"""Pins of the fp64 oracle against things other than itself.

Each pin ties one step of the oracle to a library routine, a closed form, an
invariant or the 50-digit brute-force twin.  `test_planted_mistakes_are_caught`
plants plausible mistakes in the oracle (on the CPU) and checks that the pins
fail for each of them, so the pins are known to be sensitive.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import oracle.decode_step as ods
from oracle.brute import decode_step_brute

RNG = np.random.default_rng(20261202)


def rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def rand_problem(B=1, H=16, nq=2, nkv=1, D=8, pos=(3,), theta=1e4, seed=0, scale_w=None):
    rng = np.random.default_rng(seed)
    N = (nq + 2 * nkv) * D
    sw = scale_w if scale_w is not None else 1 / math.sqrt(H)
    cap = max(pos) + 2
    return dict(
        hidden=rng.standard_normal((B, H)),
        norm_w=1 + 0.1 * rng.standard_normal(H),
        w_qkv=rng.standard_normal((H, N)) * sw,
        w_o=rng.standard_normal((nq * D, H)) * sw,
        k_cache=rng.standard_normal((B, cap, nkv, D)),
        v_cache=rng.standard_normal((B, cap, nkv, D)),
        pos=np.array(pos, dtype=np.int64),
        kw=dict(n_q_heads=nq, n_kv_heads=nkv, head_dim=D, rope_theta=theta),
    )


def run_oracle(pb, eps=1e-6, **extra):
    return ods.decode_step_fp64(pb["hidden"], pb["norm_w"], pb["w_qkv"], pb["w_o"],
                                pb["k_cache"], pb["v_cache"], pb["pos"], eps=eps, **pb["kw"], **extra)


# ---------------------------------------------------------------------------
# pin checks: each returns the worst relative error found (0 = exact)
# ---------------------------------------------------------------------------

def check_rms_norm_vs_torch():
    worst = 0.0
    for H, eps, sc in ((64, 1e-6, 1.0), (256, 0.25, 0.3), (33, 1.0, 0.05)):
        x = RNG.standard_normal(H) * sc
        w = 1 + 0.1 * RNG.standard_normal(H)
        ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (H,), torch.from_numpy(w), eps).numpy()
        worst = max(worst, rel(ods.rms_norm(x, w, eps), ref))
    return worst


def check_rms_norm_scale_invariance():
    # rms_norm(c x, w, c^2 eps) == rms_norm(x, w, eps) holds exactly only with eps inside the root
    worst = 0.0
    for c in (0.01, 3.0, 1000.0):
        x = RNG.standard_normal(48)
        w = 1 + 0.1 * RNG.standard_normal(48)
        worst = max(worst, rel(ods.rms_norm(c * x, w, c * c * 0.3), ods.rms_norm(x, w, 0.3)))
    return worst


def check_rms_norm_closed_form():
    # w = 1: mean(xh^2) = m / (m + eps), m = mean(x^2)
    worst = 0.0
    for eps in (1e-6, 0.5, 2.0):
        x = RNG.standard_normal(128)
        m = np.mean(x * x)
        xh = ods.rms_norm(x, np.ones(128), eps)
        worst = max(worst, abs(np.mean(xh * xh) - m / (m + eps)) / (m / (m + eps)))
    return worst


def check_rope_vs_transformers():
    from transformers import LlamaConfig
    from transformers.models.llama.modeling_llama import LlamaRotaryEmbedding, apply_rotary_pos_emb
    worst = 0.0
    for D, theta, p in ((8, 1e4, 3), (64, 1e4, 7), (128, 5e5, 2)):
        cfg = LlamaConfig(hidden_size=D, num_attention_heads=1, num_key_value_heads=1, head_dim=D,
                          rope_theta=theta)
        rot = LlamaRotaryEmbedding(cfg)
        # the library builds its inverse frequencies in fp32: compare them at fp32 precision
        inv = rot.inv_freq.double().numpy()
        ours = ods.rope_angles(1, D, theta)
        err = rel(ours, inv)
        worst = max(worst, 0.0 if err < 3e-7 else err)   # the library's table is fp32: allow its rounding
        # rotation convention with the library's apply_rotary_pos_emb, angles in fp64
        ang = np.concatenate([ods.rope_angles(p, D, theta)] * 2)
        cos = torch.from_numpy(np.cos(ang))[None, None]
        sin = torch.from_numpy(np.sin(ang))[None, None]
        z = RNG.standard_normal((1, 1, 1, D))
        zq, _ = apply_rotary_pos_emb(torch.from_numpy(z), torch.from_numpy(z), cos, sin)
        worst = max(worst, rel(ods.rope(z[0, 0, 0], p, theta), zq[0, 0, 0].numpy()))
    return worst


def check_rope_invariants():
    worst = 0.0
    D, theta = 16, 1e4
    z = RNG.standard_normal(D)
    # pair norms preserved
    r = ods.rope(z, 11, theta)
    worst = max(worst, rel(r[:8] ** 2 + r[8:] ** 2, z[:8] ** 2 + z[8:] ** 2))
    # position 0 is the identity
    worst = max(worst, rel(ods.rope(z, 0, theta), z))
    # <RoPE(q, m), RoPE(k, n)> depends only on m - n
    q, k = RNG.standard_normal(D), RNG.standard_normal(D)
    d1 = ods.rope(q, 9, theta) @ ods.rope(k, 4, theta)
    d2 = ods.rope(q, 105, theta) @ ods.rope(k, 100, theta)
    worst = max(worst, abs(d1 - d2) / abs(d1))
    # equals the complex product (z_j + i z_{j+D/2}) e^{i phi_j}
    phi = ods.rope_angles(11, D, theta)
    c = (z[:8] + 1j * z[8:]) * np.exp(1j * phi)
    worst = max(worst, rel(r, np.concatenate([c.real, c.imag])))
    return worst


def check_attention_vs_sdpa():
    worst = 0.0
    for nq, nkv, D, T in ((4, 4, 16, 9), (8, 2, 32, 33), (6, 3, 8, 1)):
        q = RNG.standard_normal((nq, D))
        K = RNG.standard_normal((T, nkv, D))
        V = RNG.standard_normal((T, nkv, D))
        o, _ = ods.attention(q, K, V)
        G = nq // nkv
        kt = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(G, dim=0)   # [nq, T, D]
        vt = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(G, dim=0)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q)[:, None, :], kt, vt, scale=1 / math.sqrt(D))[:, 0, :]
        worst = max(worst, rel(o, ref.numpy()))
    return worst


def check_attention_closed_forms():
    worst = 0.0
    D = 8
    # single token: output equals its value
    q = RNG.standard_normal((2, D))
    K = RNG.standard_normal((1, 1, D))
    V = RNG.standard_normal((1, 1, D))
    o, p = ods.attention(q, K, V)
    worst = max(worst, rel(o, np.repeat(V[0], 2, axis=0)), abs(p.sum() - 2))
    # equal keys: uniform weights, output = mean of values
    K = np.repeat(RNG.standard_normal((1, 1, D)), 7, axis=0)
    V = RNG.standard_normal((7, 1, D))
    o, p = ods.attention(q, K, V)
    worst = max(worst, rel(o, np.repeat(V[:, 0].mean(axis=0, keepdims=True), 2, axis=0)),
                float(np.max(np.abs(p - 1 / 7))))
    # one dominant logit: output -> that token's value
    K = RNG.standard_normal((5, 1, D)) * 1e-3
    K[3, 0] = q[0] * 1e3
    V = RNG.standard_normal((5, 1, D))
    o, _ = ods.attention(q[:1], K, V)
    worst = max(worst, rel(o[0], V[3, 0]))
    # weights sum to one; rows of the cache can be permuted (K and V together)
    K = RNG.standard_normal((12, 2, D))
    V = RNG.standard_normal((12, 2, D))
    q4 = RNG.standard_normal((4, D))
    o, p = ods.attention(q4, K, V)
    worst = max(worst, float(np.max(np.abs(p.sum(axis=1) - 1))))
    perm = RNG.permutation(12)
    o2, _ = ods.attention(q4, K[perm], V[perm])
    worst = max(worst, rel(o2, o))
    return worst


def check_full_layer_vs_transformers():
    """Whole step versus a Llama attention layer (fp64, eager) plus an explicit RMSNorm."""
    from transformers import LlamaConfig
    from transformers.models.llama.modeling_llama import LlamaAttention, LlamaRotaryEmbedding
    from transformers.cache_utils import DynamicCache
    worst = 0.0
    for (H, nq, nkv, D, p, theta) in ((32, 4, 2, 8, 5, 1e4), (64, 4, 4, 16, 0, 1e4), (48, 6, 2, 8, 9, 5e5)):
        pb = rand_problem(H=H, nq=nq, nkv=nkv, D=D, pos=(p,), theta=theta, seed=p + H)
        res = run_oracle(pb, eps=0.05)
        cfg = LlamaConfig(hidden_size=H, num_attention_heads=nq, num_key_value_heads=nkv, head_dim=D,
                          rope_theta=theta, attention_bias=False, max_position_embeddings=4096)
        cfg._attn_implementation = "eager"
        att = LlamaAttention(cfg, layer_idx=0).double()
        W = torch.from_numpy(pb["w_qkv"])
        with torch.no_grad():
            att.q_proj.weight.copy_(W[:, : nq * D].T)
            att.k_proj.weight.copy_(W[:, nq * D:(nq + nkv) * D].T)
            att.v_proj.weight.copy_(W[:, (nq + nkv) * D:].T)
            att.o_proj.weight.copy_(torch.from_numpy(pb["w_o"]).T)
        x = torch.from_numpy(pb["hidden"])[:, None, :]
        xh = torch.nn.functional.rms_norm(x, (H,), torch.from_numpy(pb["norm_w"]), 0.05)
        inv = LlamaRotaryEmbedding(cfg).inv_freq.double()
        ang = p * inv
        ang = torch.cat([ang, ang])[None, None, :]
        cos, sin = torch.cos(ang), torch.sin(ang)
        cache = DynamicCache()
        if p:
            kh = torch.from_numpy(pb["k_cache"][:, :p]).permute(0, 2, 1, 3).contiguous()
            vh = torch.from_numpy(pb["v_cache"][:, :p]).permute(0, 2, 1, 3).contiguous()
            cache.update(kh, vh, 0)
        with torch.no_grad():
            y, _ = att(xh, position_embeddings=(cos, sin), attention_mask=None,
                       past_key_values=cache if p else None)
        ref_out = (x + y)[:, 0].numpy()
        # the library's inverse frequencies are fp32: angle error <= p * 6e-8 rad
        worst = max(worst, rel(res["out"], ref_out), rel(res["y"], y[:, 0].numpy()))
    return worst


def check_identity_projection():
    """H = nq*D, nq = nkv, W_qkv = [I|I|I], W_o = I, w = 1: out = x + SDPA(RoPE(xh), ...)."""
    worst = 0.0
    nq = nkv = 2
    D = 8
    H = nq * D
    for p in (0, 4):
        x = RNG.standard_normal((1, H))
        I = np.eye(H)
        kc = RNG.standard_normal((1, p + 1, nkv, D))
        vc = RNG.standard_normal((1, p + 1, nkv, D))
        res = ods.decode_step_fp64(x, np.ones(H), np.concatenate([I, I, I], axis=1), I, kc, vc, [p],
                                   n_q_heads=nq, n_kv_heads=nkv, head_dim=D, rope_theta=1e4)
        xh = torch.nn.functional.rms_norm(torch.from_numpy(x), (H,), None, 1e-6).numpy()[0]
        if p == 0:
            # empty history: attention returns the new value, which is xh itself
            worst = max(worst, rel(res["out"][0], x[0] + xh))
            continue
        # rotation from the complex-product form, independent of ods.rope
        phi = p * 1e4 ** (-np.arange(D // 2) * 2.0 / D)
        heads = xh.reshape(nq, D)
        cz = (heads[:, :D // 2] + 1j * heads[:, D // 2:]) * np.exp(1j * phi)
        rq = np.concatenate([cz.real, cz.imag], axis=1)
        keys = np.concatenate([kc[0, :p], rq[None]], axis=0)      # [p+1, nkv, D]
        vals = np.concatenate([vc[0, :p], heads[None]], axis=0)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(rq)[:, None, :], torch.from_numpy(keys).permute(1, 0, 2),
            torch.from_numpy(vals).permute(1, 0, 2), scale=1 / math.sqrt(D))[:, 0, :].numpy()
        worst = max(worst, rel(res["out"][0], x[0] + ref.reshape(-1)))
    return worst


def check_brute_force():
    worst = 0.0
    for nkv in (1, 2):
        for p in (0, 1, 2, 3):
            pb = rand_problem(H=8, nq=2, nkv=nkv, D=4, pos=(p,), seed=10 * nkv + p)
            res = run_oracle(pb, eps=1e-6, want_probs=True)
            bf = decode_step_brute(pb["hidden"][0].tolist(), pb["norm_w"].tolist(), pb["w_qkv"].tolist(),
                                   pb["w_o"].tolist(), pb["k_cache"][0, :p].tolist(),
                                   pb["v_cache"][0, :p].tolist(), p, eps=1e-6, **pb["kw"])
            for key, rk in (("out", "out"), ("y", "y"), ("q", "q"), ("k", "k_new"), ("v", "v_new")):
                ref = np.array([[float(e) for e in r] for r in bf[key]]) if isinstance(bf[key][0], list) \
                    else np.array([float(e) for e in bf[key]])
                worst = max(worst, rel(res[rk][0], ref))
            probs = np.array([[float(e) for e in r] for r in bf["probs"]])
            worst = max(worst, rel(res["probs"][0], probs))
    return worst


def check_append():
    kc = RNG.standard_normal((6, 2, 4))
    vc = RNG.standard_normal((6, 2, 4))
    kn, vn = RNG.standard_normal((2, 4)), RNG.standard_normal((2, 4))
    k2, v2 = ods.append_kv(kc, vc, 3, kn, vn)
    bad = 0.0
    mask = np.ones(6, bool)
    mask[3] = False
    bad += float(np.any(k2[mask] != kc[mask])) + float(np.any(v2[mask] != vc[mask]))
    bad += float(np.any(k2[3] != kn)) + float(np.any(v2[3] != vn))
    return bad


PINS = {
    "rms_norm_vs_torch": (check_rms_norm_vs_torch, 1e-13),
    "rms_norm_scale_invariance": (check_rms_norm_scale_invariance, 1e-13),
    "rms_norm_closed_form": (check_rms_norm_closed_form, 1e-12),
    "rope_vs_transformers": (check_rope_vs_transformers, 1e-12),
    "rope_invariants": (check_rope_invariants, 1e-12),
    "attention_vs_sdpa": (check_attention_vs_sdpa, 1e-12),
    "attention_closed_forms": (check_attention_closed_forms, 1e-9),
    "full_layer_vs_transformers": (check_full_layer_vs_transformers, 1e-6),
    "identity_projection": (check_identity_projection, 1e-12),
    "brute_force": (check_brute_force, 1e-13),
    "append": (check_append, 0.5),
}


@pytest.mark.parametrize("name", list(PINS))
def test_pin(name):
    fn, tol = PINS[name]
    err = fn()
    assert err <= tol, f"{name}: {err:.3e} > {tol:.1e}"


def test_softmax_weights_sum_to_one_at_size():
    pb = rand_problem(H=64, nq=8, nkv=2, D=16, pos=(200,), seed=3)
    res = run_oracle(pb, want_probs=True)
    assert np.max(np.abs(res["probs"][0].sum(axis=1) - 1)) < 1e-13
    assert res["probs"][0].shape == (8, 201)


def test_single_cached_token_output_equals_v():
    """pos = 0: attention output equals the new token's v (per kv group)."""
    pb = rand_problem(H=32, nq=4, nkv=2, D=8, pos=(0,), seed=7)
    res = run_oracle(pb)
    a = res["a"][0].reshape(4, 8)
    v = res["v_new"][0]
    assert rel(a, np.repeat(v, 2, axis=0)) < 1e-14


def test_batch_rows_are_independent():
    pb = rand_problem(B=3, H=32, nq=4, nkv=2, D=8, pos=(2, 0, 5), seed=11)
    res = run_oracle(pb)
    for b in range(3):
        one = {k: (v[b:b + 1] if isinstance(v, np.ndarray) and k not in ("norm_w", "w_qkv", "w_o") else v)
               for k, v in pb.items()}
        r1 = run_oracle(one)
        assert rel(res["out"][b], r1["out"][0]) < 1e-15


def test_pos_out_of_range_raises():
    pb = rand_problem(pos=(3,))
    pb["pos"] = np.array([pb["k_cache"].shape[1]])
    with pytest.raises(ValueError):
        run_oracle(pb)


def test_bf16_rounding_matches_torch():
    x = RNG.standard_normal(20000) * np.exp(RNG.uniform(-20, 20, 20000))
    ours = ods.round_to_storage(x, "bf16")
    ref = torch.from_numpy(x.astype(np.float32).astype(np.float64)).to(torch.bfloat16).double().numpy()
    # double rounding through fp32 may differ from direct rounding only on near-ties
    mism = np.nonzero(ours != ref)[0]
    assert len(mism) <= 2
    # exact ties (representable in fp32): nearest-even
    ties = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 2 + 2 ** -7])
    assert list(ods.round_to_storage(ties, "bf16")) == [1.0, 1 + 2 ** -6, -1.0, 2.0]


def test_generator_upcast_agrees_with_oracle_decode():
    """The generator's storage bits decode identically in the oracle (exact)."""
    from attention_block_amd.inputs import CONFIGS, make_inputs, bf16_bits_to_f32
    inp = make_inputs(CONFIGS["tiny_mha_f32"].__class__(**{**CONFIGS["tiny_mha_f32"].__dict__,
                                                           "dtype": "bf16", "name": "t"}), 0)
    assert np.array_equal(ods.to_f64(inp["hidden"], "bf16"), bf16_bits_to_f32(inp["hidden"]).astype(np.float64))


# ---------------------------------------------------------------------------
# planted mistakes: each must make at least one pin fail
# ---------------------------------------------------------------------------

_ORIG = {name: getattr(ods, name) for name in ("attention", "qkv_project", "rope_angles")}


def _rms_eps_outside(x, w, eps):
    return x / (np.sqrt(np.mean(x * x)) + eps) * w


def _layernorm(x, w, eps):
    xc = x - x.mean()
    return xc / np.sqrt(np.mean(xc * xc) + eps) * w


def _rope_sign(z, pos, theta):
    d = z.shape[-1]
    phi = _ORIG["rope_angles"](pos, d, theta)
    c, s = np.cos(phi), np.sin(phi)
    lo, hi = z[..., : d // 2], z[..., d // 2:]
    return np.concatenate([lo * c + hi * s, hi * c - lo * s], axis=-1)


def _rope_interleaved(z, pos, theta):
    d = z.shape[-1]
    phi = _ORIG["rope_angles"](pos, d, theta)
    c, s = np.cos(phi), np.sin(phi)
    ev, od = z[..., 0::2], z[..., 1::2]
    out = np.empty_like(z)
    out[..., 0::2] = ev * c - od * s
    out[..., 1::2] = od * c + ev * s
    return out


def _rope_angles_wrong(pos, d, theta):
    j = np.arange(d // 2, dtype=np.float64)
    return float(pos) * theta ** (-j / d)


def _attention_scale_d(q, keys, values):
    # scores scaled by 1/D instead of 1/sqrt(D)
    return _ORIG["attention"](q / np.sqrt(q.shape[1]), keys, values)


def _attention_drop_new(q, keys, values):
    # attends to the history only, leaving out the new token
    if keys.shape[0] == 1:
        return _ORIG["attention"](q, keys, values)
    return _ORIG["attention"](q, keys[:-1], values[:-1])


def _attention_gqa_modulo(q, keys, values):
    # query head h reads kv head h % nkv instead of h // (nq / nkv)
    nq, d = q.shape
    nkv = keys.shape[1]
    o = np.empty((nq, d))
    probs = np.empty((nq, keys.shape[0]))
    for h in range(nq):
        g = h % nkv
        p = ods.softmax(keys[:, g, :] @ q[h] / np.sqrt(d))
        probs[h] = p
        o[h] = p @ values[:, g, :]
    return o, probs


def _qkv_swap_kv(xh, w, nq, nkv, d):
    q, k, v = _ORIG["qkv_project"](xh, w, nq, nkv, d)
    return q, v, k


def _out_no_residual(x, a, w_o):
    y = a @ w_o
    return y, y


def _out_transposed(x, a, w_o):
    y = a @ w_o.T
    return x + y, y


def _softmax_shifted_denominator(s):
    e = np.exp(s - np.max(s, axis=-1, keepdims=True))
    return e / (np.sum(e, axis=-1, keepdims=True) + 1e-3)


MUTATIONS = {
    "eps_outside_root": ("rms_norm", _rms_eps_outside),
    "layernorm_mean": ("rms_norm", _layernorm),
    "rope_sign": ("rope", _rope_sign),
    "rope_interleaved": ("rope", _rope_interleaved),
    "rope_freq": ("rope_angles", _rope_angles_wrong),
    "scale_1_over_d": ("attention", _attention_scale_d),
    "drop_new_token": ("attention", _attention_drop_new),
    "gqa_modulo": ("attention", _attention_gqa_modulo),
    "swap_k_v": ("qkv_project", _qkv_swap_kv),
    "no_residual": ("out_project", _out_no_residual),
    "w_o_transposed": ("out_project", _out_transposed),
    "softmax_denominator": ("softmax", _softmax_shifted_denominator),
}


@pytest.mark.parametrize("mutation", list(MUTATIONS))
def test_planted_mistakes_are_caught(mutation, monkeypatch):
    attr, fn = MUTATIONS[mutation]
    monkeypatch.setattr(ods, attr, fn)
    failed = []
    for name, (check, tol) in PINS.items():
        try:
            err = check()
        except Exception:  # a mistake that breaks shapes also counts as caught
            err = float("inf")
        if not err <= tol:
            failed.append(name)
    assert failed, f"planted mistake {mutation!r} passed every pin"
