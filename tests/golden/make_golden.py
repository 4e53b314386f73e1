"""Write tests/golden/brute_*.json from the 50-digit brute-force oracle twin.

The pages print no worked numeric example for the decode block, so the
stored values here come from oracle/brute.py alone (never from the HIP
library).  Inputs are drawn from a fixed seed with numpy and stored next to
the expected outputs, so the fixture stands by itself.

    python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle.brute import decode_step_brute, ffn_step_brute  # noqa: E402

FFN_CASES = [
    # H, F
    (8, 12),
]

CASES = [
    # H, nq, nkv, D, pos, theta
    (8, 2, 1, 4, 3, 1e4),
    (12, 4, 2, 2, 5, 5e5),
]


def main():
    for (H, nq, nkv, D, p, theta) in CASES:
        rng = np.random.default_rng(1000 + H + p)
        N = (nq + 2 * nkv) * D
        inp = {
            "hidden": rng.standard_normal(H).round(6).tolist(),
            "norm_w": (1 + 0.1 * rng.standard_normal(H)).round(6).tolist(),
            "w_qkv": (rng.standard_normal((H, N)) / np.sqrt(H)).round(6).tolist(),
            "w_o": (rng.standard_normal((nq * D, H)) / np.sqrt(H)).round(6).tolist(),
            "k_hist": rng.standard_normal((p, nkv, D)).round(6).tolist(),
            "v_hist": rng.standard_normal((p, nkv, D)).round(6).tolist(),
        }
        res = decode_step_brute(inp["hidden"], inp["norm_w"], inp["w_qkv"], inp["w_o"],
                                inp["k_hist"], inp["v_hist"], p, n_q_heads=nq, n_kv_heads=nkv,
                                head_dim=D, rope_theta=theta, eps=1e-6)
        expect = {
            "out": [str(v) for v in res["out"]],
            "y": [str(v) for v in res["y"]],
            "q": [[str(v) for v in r] for r in res["q"]],
            "k": [[str(v) for v in r] for r in res["k"]],
            "v": [[str(v) for v in r] for r in res["v"]],
        }
        doc = {
            "source": "oracle/brute.py (mpmath, 50 digits); written by tests/golden/make_golden.py",
            "shape": {"hidden": H, "n_q_heads": nq, "n_kv_heads": nkv, "head_dim": D,
                      "pos": p, "rope_theta": theta, "eps": 1e-6},
            "inputs": inp,
            "expected": expect,
        }
        name = f"brute_h{H}_nq{nq}_nkv{nkv}_d{D}_p{p}.json"
        with open(os.path.join(HERE, name), "w") as f:
            json.dump(doc, f, indent=1)
        print("wrote", name)
    for (H, F) in FFN_CASES:
        rng = np.random.default_rng(2000 + H + F)
        inp = {
            "hidden": rng.standard_normal(H).round(6).tolist(),
            "norm_w": (1 + 0.1 * rng.standard_normal(H)).round(6).tolist(),
            "w_gate": (rng.standard_normal((H, F)) / np.sqrt(H)).round(6).tolist(),
            "w_up": (rng.standard_normal((H, F)) / np.sqrt(H)).round(6).tolist(),
            "w_down": (rng.standard_normal((F, H)) / np.sqrt(F)).round(6).tolist(),
        }
        res = ffn_step_brute(inp["hidden"], inp["norm_w"], inp["w_gate"], inp["w_up"], inp["w_down"], eps=1e-6)
        doc = {
            "source": "oracle/brute.py ffn_step_brute (mpmath, 50 digits); written by tests/golden/make_golden.py",
            "shape": {"hidden": H, "intermediate": F, "eps": 1e-6},
            "inputs": inp,
            "expected": {k: [str(v) for v in res[k]] for k in ("out", "y", "m")},
        }
        name = f"ffn_brute_h{H}_f{F}.json"
        with open(os.path.join(HERE, name), "w") as f:
            json.dump(doc, f, indent=1)
        print("wrote", name)


if __name__ == "__main__":
    main()
