"""The numpy oracle against stored 50-digit brute-force results (tests/golden)."""
import glob
import json
import os

import numpy as np
import pytest

import oracle.decode_step as ods
import oracle.ffn_step as ofs

FILES = sorted(glob.glob(os.path.join(os.path.dirname(__file__), "golden", "brute_*.json")))


@pytest.mark.parametrize("path", FILES, ids=[os.path.basename(p) for p in FILES])
def test_oracle_matches_stored_brute_force(path):
    doc = json.load(open(path))
    s, inp, exp = doc["shape"], doc["inputs"], doc["expected"]
    H, nq, nkv, D, p = s["hidden"], s["n_q_heads"], s["n_kv_heads"], s["head_dim"], s["pos"]
    kc = np.zeros((1, p + 1, nkv, D))
    vc = np.zeros((1, p + 1, nkv, D))
    if p:
        kc[0, :p] = np.array(inp["k_hist"])
        vc[0, :p] = np.array(inp["v_hist"])
    res = ods.decode_step_fp64(np.array([inp["hidden"]]), np.array(inp["norm_w"]), np.array(inp["w_qkv"]),
                               np.array(inp["w_o"]), kc, vc, [p], n_q_heads=nq, n_kv_heads=nkv, head_dim=D,
                               rope_theta=s["rope_theta"], eps=s["eps"])
    for key, rk in (("out", "out"), ("y", "y"), ("q", "q"), ("k", "k_new"), ("v", "v_new")):
        ref = np.array(exp[key], dtype=np.float64)
        got = res[rk][0]
        assert np.max(np.abs(got - ref)) <= 1e-13 * max(1.0, np.max(np.abs(ref))), key


FFN_FILES = sorted(glob.glob(os.path.join(os.path.dirname(__file__), "golden", "ffn_brute_*.json")))


@pytest.mark.parametrize("path", FFN_FILES, ids=[os.path.basename(p) for p in FFN_FILES])
def test_ffn_oracle_matches_stored_brute_force(path):
    doc = json.load(open(path))
    inp, exp = doc["inputs"], doc["expected"]
    res = ofs.ffn_step_fp64(np.array([inp["hidden"]]), np.array(inp["norm_w"]), np.array(inp["w_gate"]),
                            np.array(inp["w_up"]), np.array(inp["w_down"]), eps=doc["shape"]["eps"])
    for key in ("out", "y", "m"):
        ref = np.array([float(v) for v in exp[key]])
        got = res[key][0]
        assert np.max(np.abs(got - ref)) <= 1e-13 * max(1.0, np.max(np.abs(ref))), key
