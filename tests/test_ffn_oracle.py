"""Pins of the FFN oracle (oracle/ffn_step.py) against things other than itself.

Each pin ties a step of the FFN oracle to torch's fp64 routines, a closed
form of silu, an invariant, or the 50-digit twin in oracle/brute.py.
`test_planted_mistakes_are_caught` plants plausible mistakes in the oracle
(on the CPU) and checks that some pin fails for each.
"""
import math

import numpy as np
import pytest
import torch

import oracle.ffn_step as ofs
from oracle.brute import ffn_step_brute

RNG = np.random.default_rng(20261203)


def rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def rand_ffn(B=2, H=16, F=24, seed=0):
    rng = np.random.default_rng(seed)
    return dict(hidden=rng.standard_normal((B, H)), norm_w=1 + 0.1 * rng.standard_normal(H),
                w_gate=rng.standard_normal((H, F)) / math.sqrt(H), w_up=rng.standard_normal((H, F)) / math.sqrt(H),
                w_down=rng.standard_normal((F, H)) / math.sqrt(F))


def run(pb, eps=1e-6):
    return ofs.ffn_step_fp64(pb["hidden"], pb["norm_w"], pb["w_gate"], pb["w_up"], pb["w_down"], eps=eps)


# ---------------------------------------------------------------------------
# pin checks: each returns the worst relative error found (0 = exact)
# ---------------------------------------------------------------------------

def check_silu_vs_torch():
    z = np.concatenate([np.linspace(-60, 60, 2401), RNG.standard_normal(500) * 4, [0.0, 700.0, -700.0]])
    ref = torch.nn.functional.silu(torch.from_numpy(z)).numpy()
    return rel(ofs.silu(z), ref)


def check_silu_closed_forms():
    worst = 0.0
    z = np.linspace(-30, 30, 601)
    # sigmoid(z) + sigmoid(-z) = 1, so silu(z) - silu(-z) = z
    worst = max(worst, rel(ofs.silu(z) - ofs.silu(-z), z))
    # sigmoid(ln 3) = 3/4 and sigmoid(-ln 3) = 1/4
    l3 = math.log(3.0)
    worst = max(worst, abs(float(ofs.silu(np.array([l3]))[0]) - 0.75 * l3) / l3)
    worst = max(worst, abs(float(ofs.silu(np.array([-l3]))[0]) + 0.25 * l3) / l3)
    # silu(0) = 0; silu(z) / z -> 1 for large z and -> 0 for large negative z
    worst = max(worst, abs(float(ofs.silu(np.array([0.0]))[0])))
    worst = max(worst, abs(float(ofs.silu(np.array([40.0]))[0]) / 40.0 - 1.0))
    worst = max(worst, abs(float(ofs.silu(np.array([-40.0]))[0])) / 40.0)
    return worst


def check_ffn_vs_torch():
    worst = 0.0
    for (B, H, F, eps, seed) in ((3, 64, 96, 1e-6, 1), (1, 32, 128, 0.5, 2), (2, 48, 40, 1e-6, 3)):
        pb = rand_ffn(B, H, F, seed)
        t = {k: torch.from_numpy(v) for k, v in pb.items()}
        hh = torch.nn.functional.rms_norm(t["hidden"], (H,), t["norm_w"], eps)
        g = torch.nn.functional.linear(hh, t["w_gate"].T.contiguous())
        u = torch.nn.functional.linear(hh, t["w_up"].T.contiguous())
        y = torch.nn.functional.linear(torch.nn.functional.silu(g) * u, t["w_down"].T.contiguous())
        res = run(pb, eps)
        worst = max(worst, rel(res["y"], y.numpy()), rel(res["out"], (t["hidden"] + y).numpy()),
                    rel(res["m"], (torch.nn.functional.silu(g) * u).numpy()))
    return worst


def check_brute_force():
    worst = 0.0
    for (H, F, seed) in ((8, 12, 4), (12, 8, 5)):
        pb = rand_ffn(1, H, F, seed)
        res = run(pb)
        br = ffn_step_brute(pb["hidden"][0].tolist(), pb["norm_w"].tolist(), pb["w_gate"].tolist(),
                            pb["w_up"].tolist(), pb["w_down"].tolist(), eps=1e-6)
        for key in ("out", "y", "m"):
            worst = max(worst, rel(res[key][0], np.array([float(v) for v in br[key]])))
    return worst


def check_invariants():
    worst = 0.0
    pb = rand_ffn(2, 32, 48, 6)
    base = run(pb, eps=0.0)
    # h -> 3h leaves the normalised input, hence m and y, unchanged (eps = 0)
    pb3 = dict(pb, hidden=3.0 * pb["hidden"])
    r3 = run(pb3, eps=0.0)
    worst = max(worst, rel(r3["y"], base["y"]), rel(r3["out"], 3.0 * pb["hidden"] + base["y"]))
    # no down projection: out = h exactly; no up projection: y = 0
    r0 = run(dict(pb, w_down=np.zeros_like(pb["w_down"])))
    worst = max(worst, float(np.max(np.abs(r0["out"] - pb["hidden"]))))
    ru = run(dict(pb, w_up=np.zeros_like(pb["w_up"])))
    worst = max(worst, float(np.max(np.abs(ru["y"]))))
    return worst


def check_gating_closed_form():
    # H = F, norm weight 1, W_gate = a I, W_up = I, W_down = I: y_i = silu(a hh_i) hh_i,
    # with hh = h / rms(h), each term written out with math.exp
    H, a = 16, 1.7
    h = RNG.standard_normal(H)
    eye = np.eye(H)
    res = ofs.ffn_step_fp64(h[None], np.ones(H), a * eye, eye, eye, eps=0.0)
    rms = math.sqrt(sum(float(v) * float(v) for v in h) / H)
    expect = []
    for v in h:
        x = float(v) / rms
        expect.append(a * x / (1.0 + math.exp(-a * x)) * x)
    return rel(res["y"][0], np.array(expect))


PINS = {
    "silu_vs_torch": (check_silu_vs_torch, 1e-15),
    "silu_closed_forms": (check_silu_closed_forms, 1e-15),
    "ffn_vs_torch": (check_ffn_vs_torch, 1e-13),
    "brute_force": (check_brute_force, 1e-13),
    "invariants": (check_invariants, 1e-13),
    "gating_closed_form": (check_gating_closed_form, 1e-14),
}


@pytest.mark.parametrize("name", list(PINS))
def test_pin(name):
    fn, tol = PINS[name]
    err = fn()
    assert err <= tol, f"{name}: {err:.3e} > {tol:.1e}"


def test_storage_rounding_and_batch_rows():
    pb = rand_ffn(3, 16, 24, 7)
    res = run(pb)
    for b in range(3):
        one = run({**pb, "hidden": pb["hidden"][b:b + 1]})
        assert np.array_equal(one["out"][0], res["out"][b])
    bf = ofs.ffn_step_fp64(pb["hidden"], pb["norm_w"], pb["w_gate"], pb["w_up"], pb["w_down"], storage="bf16")
    ref = torch.from_numpy(bf["out"]).to(torch.bfloat16).double().numpy()
    assert np.array_equal(bf["out_stored"], ref)


# ---------------------------------------------------------------------------
# planted mistakes
# ---------------------------------------------------------------------------

_ORIG = {name: getattr(ofs, name) for name in ("silu", "gated", "down", "rms_norm", "gate_up")}


def _silu_sigmoid_only(z):
    z = np.asarray(z, dtype=np.float64)
    return _ORIG["silu"](z) / np.where(z == 0, 1.0, z)


def _silu_sign(z):
    return -_ORIG["silu"](-np.asarray(z, dtype=np.float64))


def _gated_swapped(g, u):
    return _ORIG["silu"](u) * g


def _gated_both(g, u):
    return _ORIG["silu"](g) * _ORIG["silu"](u)


def _down_no_residual(h, m, w_down):
    y = m @ w_down
    return y, y


def _rms_eps_outside(x, w, eps):
    return x / (np.sqrt(np.mean(x * x)) + eps) * w


def _rms_no_weight(x, w, eps):
    return _ORIG["rms_norm"](x, np.ones_like(w), eps)


def _gate_up_same(hh, w_gate, w_up):
    g = hh @ w_gate
    return g, g


MUTATIONS = {
    "silu_sigmoid_only": ("silu", _silu_sigmoid_only),
    "silu_sign": ("silu", _silu_sign),
    "gate_up_swapped": ("gated", _gated_swapped),
    "silu_on_both": ("gated", _gated_both),
    "no_residual": ("down", _down_no_residual),
    "eps_outside_root": ("rms_norm", _rms_eps_outside),
    "norm_weight_dropped": ("rms_norm", _rms_no_weight),
    "up_reads_gate": ("gate_up", _gate_up_same),
}


@pytest.mark.parametrize("mutation", list(MUTATIONS))
def test_planted_mistakes_are_caught(mutation, monkeypatch):
    attr, fn = MUTATIONS[mutation]
    monkeypatch.setattr(ofs, attr, fn)
    failed = []
    for name, (check, tol) in PINS.items():
        try:
            err = check()
        except Exception:  # a mistake that breaks shapes also counts as caught
            err = float("inf")
        if not err <= tol:
            failed.append(name)
    assert failed, f"planted mistake {mutation!r} passed every pin"
