"""Pins of the latent-attention oracle (oracle/mla_step.py) against things other than itself.

Each pin ties the oracle to torch's fp64 scaled dot product attention, to the
explicit per-head (un-absorbed) form of latent attention, to closed forms
(one token, a zero query), to invariants, or to the 50-digit twin in
oracle/brute.py.  `test_planted_mistakes_are_caught` plants plausible
mistakes in the oracle (on the CPU) and checks that some pin fails for each.

Reading of the pages: ClusterFusion page, section 5.2 (DeepSeek-MLA runs
through the fused decode step); the formulas are DeepSeek's latent attention
in its absorbed decode form, as stated in the oracle's header.
"""
import math

import numpy as np
import pytest
import torch

import oracle.mla_step as oms
from attention_block_amd.inputs import MLA_CONFIGS, MlaConfig, make_mla_inputs
from oracle.brute import mla_decode_brute
from oracle.decode_step import to_f64

RNG = np.random.default_rng(20261204)


def rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def rand_mla(B=2, nh=4, R=16, P=8, cap=12, pos=(7, 11), seed=0):
    rng = np.random.default_rng(seed)
    return dict(q_lat=rng.standard_normal((B, nh, R)) * 0.5, q_rope=rng.standard_normal((B, nh, P)),
                c_cache=rng.standard_normal((B, cap, R)), kr_cache=rng.standard_normal((B, cap, P)),
                c_new=rng.standard_normal((B, R)), kr_new=rng.standard_normal((B, P)),
                pos=np.asarray(pos, dtype=np.int64))


def run(pb, scale, want_probs=False):
    return oms.mla_decode_fp64(pb["q_lat"], pb["q_rope"], pb["c_cache"], pb["kr_cache"], pb["c_new"],
                               pb["kr_new"], pb["pos"], scale=scale, storage="f32", want_probs=want_probs)


# ---------------------------------------------------------------------------
# pin checks: each returns the worst relative error found (0 = exact)
# ---------------------------------------------------------------------------

def check_vs_sdpa():
    """One shared key/value head: key = [c_t | kr_t], value = c_t, query = [q_lat_h | q_rope_h]."""
    worst = 0.0
    for (B, nh, R, P, cap, pos, seed) in ((2, 4, 32, 8, 40, (33, 17), 1), (1, 16, 64, 16, 9, (8,), 2),
                                           (3, 2, 16, 4, 5, (0, 1, 4), 3)):
        pb = rand_mla(B, nh, R, P, cap, pos, seed)
        scale = 1.0 / math.sqrt(R // 2 + P)
        res = run(pb, scale)
        for b in range(B):
            p = int(pb["pos"][b])
            keys = np.concatenate([np.concatenate([pb["c_cache"][b, :p], pb["c_new"][b][None]]),
                                   np.concatenate([pb["kr_cache"][b, :p], pb["kr_new"][b][None]])], axis=1)
            vals = np.concatenate([pb["c_cache"][b, :p], pb["c_new"][b][None]])
            q = np.concatenate([pb["q_lat"][b], pb["q_rope"][b]], axis=1)
            o = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(q)[None], torch.from_numpy(keys)[None], torch.from_numpy(vals)[None],
                scale=scale)[0].numpy()
            worst = max(worst, rel(res["out"][b], o))
    return worst


def check_absorption_identity():
    """The explicit per-head form: head h's no-rope key and value are W_UK_h^T c_t and W_UV_h^T c_t; its
    query's no-rope part is q_nope_h.  Folding W_UK_h into the query (q_lat_h = W_UK_h q_nope_h) and
    applying W_UV_h^T after the latent sum gives the same output."""
    worst = 0.0
    for (nh, R, P, dn, dv, pos, seed) in ((4, 24, 8, 12, 10, 19, 4), (2, 16, 4, 16, 16, 6, 5)):
        rng = np.random.default_rng(seed)
        w_uk = rng.standard_normal((nh, R, dn)) / math.sqrt(R)
        w_uv = rng.standard_normal((nh, R, dv)) / math.sqrt(R)
        q_nope = rng.standard_normal((nh, dn))
        q_rope = rng.standard_normal((nh, P))
        c = rng.standard_normal((pos + 1, R))
        kr = rng.standard_normal((pos + 1, P))
        scale = 1.0 / math.sqrt(dn + P)
        explicit = []
        for h in range(nh):
            k_h = torch.from_numpy(np.concatenate([c @ w_uk[h], kr], axis=1))
            v_h = torch.from_numpy(c @ w_uv[h])
            q_h = torch.from_numpy(np.concatenate([q_nope[h], q_rope[h]]))
            pr = torch.softmax((k_h @ q_h) * scale, dim=0)
            explicit.append((pr[:, None] * v_h).sum(0).numpy())
        q_lat = np.stack([w_uk[h] @ q_nope[h] for h in range(nh)])
        res = oms.mla_decode_fp64(q_lat[None], q_rope[None], c[None], kr[None], c[pos][None],
                                  kr[pos][None], np.array([pos]), scale=scale, storage="f32")
        absorbed = np.stack([res["out"][0, h] @ w_uv[h] for h in range(nh)])
        worst = max(worst, rel(absorbed, np.stack(explicit)))
    return worst


def check_brute_force():
    worst = 0.0
    for (nh, R, P, pos, seed) in ((3, 8, 4, 5, 6), (2, 6, 2, 9, 7)):
        pb = rand_mla(1, nh, R, P, pos + 1, (pos,), seed)
        scale = 1.0 / math.sqrt(R + P)
        res = run(pb, scale, want_probs=True)
        br = mla_decode_brute(pb["q_lat"][0].tolist(), pb["q_rope"][0].tolist(), pb["c_cache"][0, :pos].tolist(),
                              pb["kr_cache"][0, :pos].tolist(), pb["c_new"][0].tolist(), pb["kr_new"][0].tolist(),
                              scale=scale)
        worst = max(worst, rel(res["out"][0], np.array([[float(v) for v in row] for row in br["out"]])),
                    rel(res["probs"][0], np.array([[float(v) for v in row] for row in br["probs"]])))
    return worst


def check_closed_forms():
    worst = 0.0
    pb = rand_mla(2, 4, 16, 8, 12, (7, 11), 8)
    # a zero query weighs every attended token equally: the output is the mean of the latent rows
    z = dict(pb, q_lat=np.zeros_like(pb["q_lat"]), q_rope=np.zeros_like(pb["q_rope"]))
    res = run(z, 0.3)
    for b in range(2):
        p = int(pb["pos"][b])
        mean = (pb["c_cache"][b, :p].sum(0) + pb["c_new"][b]) / (p + 1)
        worst = max(worst, rel(res["out"][b], np.broadcast_to(mean, res["out"][b].shape)))
    # one token (pos 0): every head's output is the new latent row, weight exactly 1
    one = dict(pb, pos=np.array([0, 0]))
    r1 = run(one, 0.3, want_probs=True)
    for b in range(2):
        worst = max(worst, float(np.max(np.abs(r1["out"][b] - pb["c_new"][b]))),
                    float(np.max(np.abs(r1["probs"][b] - 1.0))))
    # a query on the rotary part only, against two tokens whose rotary keys differ by d: the odds of
    # the two are exp(scale q_rope . d), written out with math.exp
    R, P = 16, 8
    qr = RNG.standard_normal(P)
    d = RNG.standard_normal(P)
    kr0 = RNG.standard_normal(P)
    c0, c1 = RNG.standard_normal(R), RNG.standard_normal(R)
    scale = 0.4
    r2 = oms.mla_decode_fp64(np.zeros((1, 1, R)), qr[None, None], np.stack([c0, c1])[None],
                             np.stack([kr0, kr0 + d])[None], c1[None],
                             (kr0 + d)[None], np.array([1]), scale=scale, storage="f32")
    w1 = 1.0 / (1.0 + math.exp(-scale * float(np.dot(qr, d))))
    worst = max(worst, rel(r2["out"][0, 0], (1 - w1) * c0 + w1 * c1))
    return worst


def check_invariants():
    worst = 0.0
    pb = rand_mla(2, 4, 16, 8, 12, (7, 11), 9)
    base = run(pb, 0.25)
    # one vector added to every token's rotary key shifts each head's scores by a constant: no change
    u = RNG.standard_normal(8)
    sh = dict(pb, kr_cache=pb["kr_cache"] + u, kr_new=pb["kr_new"] + u)
    worst = max(worst, rel(run(sh, 0.25)["out"], base["out"]))
    # the history is a set: permuting the cached tokens changes nothing
    perm = dict(pb, c_cache=pb["c_cache"].copy(), kr_cache=pb["kr_cache"].copy())
    for b in range(2):
        p = int(pb["pos"][b])
        idx = RNG.permutation(p)
        perm["c_cache"][b, :p] = pb["c_cache"][b, idx]
        perm["kr_cache"][b, :p] = pb["kr_cache"][b, idx]
    worst = max(worst, rel(run(perm, 0.25)["out"], base["out"]))
    # rows at and past pos are not read
    junk = dict(pb, c_cache=pb["c_cache"].copy(), kr_cache=pb["kr_cache"].copy())
    for b in range(2):
        junk["c_cache"][b, int(pb["pos"][b]):] = np.nan
        junk["kr_cache"][b, int(pb["pos"][b]):] = np.nan
    worst = max(worst, rel(run(junk, 0.25)["out"], base["out"]))
    # heads are independent, and so are sequences
    one_head = dict(pb, q_lat=pb["q_lat"][:, 2:3], q_rope=pb["q_rope"][:, 2:3])
    worst = max(worst, rel(run(one_head, 0.25)["out"][:, 0], base["out"][:, 2]))
    return worst


PINS = {
    "vs_sdpa": (check_vs_sdpa, 1e-13),
    "absorption_identity": (check_absorption_identity, 1e-13),
    "brute_force": (check_brute_force, 1e-13),
    "closed_forms": (check_closed_forms, 1e-14),
    "invariants": (check_invariants, 1e-13),
}


@pytest.mark.parametrize("name", list(PINS))
def test_pin(name):
    fn, tol = PINS[name]
    err = fn()
    assert err <= tol, f"{name}: {err:.3e} > {tol:.1e}"


def test_append_rows_and_stored_inputs():
    """The appended rows are the new token's rows in the storage type (bit-exact), and the stored-input
    glue upcasts only the cached rows below each position (the NaN tails never reach the result)."""
    cfg = MlaConfig("t", 3, 4, 9, kv_lora_rank=32, rope_dim=16)
    inp = make_mla_inputs(cfg, 11, cap=20, pos=[9, 0, 19])
    res = oms.mla_decode_from_inputs(inp, want_probs=True)
    assert np.all(np.isfinite(res["out"]))
    assert np.array_equal(res["c_row"], to_f64(inp["c_new"], "bf16"))
    assert np.array_equal(res["kr_row"], to_f64(inp["kr_new"], "bf16"))
    assert np.array_equal(res["out"][1], np.broadcast_to(to_f64(inp["c_new"], "bf16")[1], (4, 32)))
    for b, p in enumerate([9, 0, 19]):
        assert res["probs"][b].shape == (4, p + 1)
        assert np.allclose(res["probs"][b].sum(-1), 1.0, rtol=0, atol=1e-14)


def test_mla_configs_and_generator():
    cfg = MLA_CONFIGS["mla_tiny"]
    a = make_mla_inputs(cfg, 3)
    b = make_mla_inputs(cfg, 3)
    for k in ("q_lat", "q_rope", "c_new", "kr_new", "c_cache", "kr_cache"):
        assert np.array_equal(a[k], b[k], equal_nan=True)
    assert a["c_cache"].shape == (2, 101, 512) and a["kr_cache"].shape == (2, 101, 64)
    assert a["c_cache"].dtype == np.uint16
    v3 = MLA_CONFIGS["deepseek_v3_mla_bs1_4k"]
    assert (v3.n_heads, v3.kv_lora_rank, v3.rope_dim) == (128, 512, 64)
    assert abs(v3.softmax_scale - 1 / math.sqrt(192)) < 1e-15
    # q_lat has the std of a 128-wide N(0, 1) query through an N(0, 1/512) projection
    assert abs(float(np.std(a["q_lat"])) - 0.5) < 0.02


# ---------------------------------------------------------------------------
# planted mistakes
# ---------------------------------------------------------------------------

_ORIG = {name: getattr(oms, name) for name in ("mla_scores", "attended_rows", "mla_attention")}


def _scores_no_rope(q_lat, q_rope, kc, kr, scale):
    return (q_lat @ kc.T) * scale


def _scores_rope_sign(q_lat, q_rope, kc, kr, scale):
    return (q_lat @ kc.T - q_rope @ kr.T) * scale


def _scores_unscaled(q_lat, q_rope, kc, kr, scale):
    return q_lat @ kc.T + q_rope @ kr.T


def _scores_scale_rope_only(q_lat, q_rope, kc, kr, scale):
    return q_lat @ kc.T + (q_rope @ kr.T) * scale


def _rows_no_new(cache, new, pos):
    return cache[:max(pos, 1)]


def _rows_drop_last(cache, new, pos):
    return np.concatenate([cache[:max(pos - 1, 0)], new[None]], axis=0)


def _rows_one_extra(cache, new, pos):
    return np.concatenate([cache[:pos + 1], new[None]], axis=0)


def _attention_softmax_over_heads(q_lat, q_rope, kc, kr, scale):
    s = _ORIG["mla_scores"](q_lat, q_rope, kc, kr, scale)
    e = np.exp(s - s.max(axis=0, keepdims=True))
    p = e / e.sum(axis=0, keepdims=True)
    return p @ kc, p


def _attention_unnormalised(q_lat, q_rope, kc, kr, scale):
    s = _ORIG["mla_scores"](q_lat, q_rope, kc, kr, scale)
    p = np.exp(s - s.max(axis=-1, keepdims=True))
    return p @ kc, p


MUTATIONS = {
    "rope_term_dropped": ("mla_scores", _scores_no_rope),
    "rope_term_sign": ("mla_scores", _scores_rope_sign),
    "scale_dropped": ("mla_scores", _scores_unscaled),
    "scale_on_rope_only": ("mla_scores", _scores_scale_rope_only),
    "new_token_not_attended": ("attended_rows", _rows_no_new),
    "last_history_token_dropped": ("attended_rows", _rows_drop_last),
    "row_past_pos_read": ("attended_rows", _rows_one_extra),
    "softmax_over_heads": ("mla_attention", _attention_softmax_over_heads),
    "softmax_not_normalised": ("mla_attention", _attention_unnormalised),
}


def _any_pin_fails():
    failed = []
    for name, (fn, tol) in PINS.items():
        try:
            err = fn()
        except Exception:                      # a shape error is a failure too
            failed.append(name)
            continue
        if not err <= tol:
            failed.append(name)
    return failed


@pytest.mark.parametrize("mutation", list(MUTATIONS))
def test_planted_mistakes_are_caught(mutation, monkeypatch):
    target, fn = MUTATIONS[mutation]
    monkeypatch.setattr(oms, target, fn)
    failed = _any_pin_fails()
    assert failed, f"planted mistake {mutation} passed every pin"
