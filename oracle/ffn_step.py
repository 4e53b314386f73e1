"""fp64 CPU oracle of the FFN half of the decoder layer.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package's smoke check and
the benchmark's CPU-baseline leg may import this module.  It shares no code
with the HIP library and imports nothing from it.

The operator-fusion page ("LayerNorm + Attention" CUDA kernel article),
section 1, lists the parts of each LLaMA-style transformer block: after the
attention block's O projection and residual come a second RMS norm and the
FFN.  The pages do not write the FFN out.  The reading taken here is the
FFN of the LLaMA architecture the page names, a SiLU-gated one, per
sequence, in float64 on values upcast exactly from the stored bits:

  F1  RMSNorm       r = (mean_i h_i^2 + eps)^(-1/2);  hh = h * r * w
                    (the same norm as the attention block's first step)
  F2  gate and up   g = hh @ W_gate,  u = hh @ W_up   (W [H, F], [in, out])
  F3  gating        m = silu(g) * u,  silu(z) = z * sigmoid(z) = z / (1 + e^-z)
  F4  down          y = m @ W_down  (W_down [F, H]);  out = h + y

The intermediate size F is not on the pages either: the workloads use the
published sizes of the models the pages benchmark (Llama-2-7B: 11008;
Llama-3-8B: 14336).  Every function is pinned by the CPU tests against
torch's fp64 routines, closed forms of silu, invariants and the 50-digit
twin in oracle/brute.py.
"""
from __future__ import annotations

import numpy as np

from .decode_step import rms_norm, round_to_storage, to_f64


def silu(z: np.ndarray) -> np.ndarray:
    """F3's gate: z * sigmoid(z), with the exponential taken of -|z| only (no overflow)."""
    z = np.asarray(z, dtype=np.float64)
    e = np.exp(-np.abs(z))                      # in (0, 1]
    sig = np.where(z >= 0, 1.0 / (1.0 + e), e / (1.0 + e))
    return z * sig


def gate_up(hh: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray):
    """F2: g = hh @ W_gate, u = hh @ W_up."""
    return hh @ w_gate, hh @ w_up


def gated(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    """F3: m = silu(g) * u (the gate goes through silu, the up projection does not)."""
    return silu(g) * u


def down(h: np.ndarray, m: np.ndarray, w_down: np.ndarray):
    """F4: y = m @ W_down, out = h + y."""
    y = m @ w_down
    return h + y, y


def ffn_step_fp64(hidden, norm_w, w_gate, w_up, w_down, *, eps: float = 1e-6, storage: str = "f32") -> dict:
    """The FFN half for every sequence of a batch, in float64.

    Arrays (float64 values): hidden [B, H], norm_w [H], w_gate and w_up
    [H, F], w_down [F, H].  Returns out [B, H] (unrounded), out_stored (out
    rounded to `storage`), y [B, H], m, g, u [B, F] and hh [B, H].
    """
    hidden = np.asarray(hidden, dtype=np.float64)
    res = {k: [] for k in ("out", "y", "m", "g", "u", "hh")}
    for b in range(hidden.shape[0]):
        h = hidden[b]
        hh = rms_norm(h, norm_w, eps)
        g, u = gate_up(hh, w_gate, w_up)
        m = gated(g, u)
        out, y = down(h, m, w_down)
        for name, val in (("out", out), ("y", y), ("m", m), ("g", g), ("u", u), ("hh", hh)):
            res[name].append(val)
    out = {k: np.stack(v) if v else np.zeros((0,)) for k, v in res.items()}
    out["out_stored"] = round_to_storage(out["out"], storage)
    return out


def ffn_step_from_inputs(inp: dict) -> dict:
    """Run `ffn_step_fp64` on a stored FFN input set (see the seeded generator)."""
    cfg = inp["cfg"]
    st = cfg.dtype
    return ffn_step_fp64(to_f64(inp["hidden"], st), to_f64(inp["norm_w"], st), to_f64(inp["w_gate"], st),
                         to_f64(inp["w_up"], st), to_f64(inp["w_down"], st), eps=cfg.eps, storage=st)
