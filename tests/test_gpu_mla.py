"""GPU parity of the latent-attention (MLA) decode path against the fp64 oracle.

Every case runs the HIP kernels through the C ABI (attention_block_amd's
ctypes binding) on seeded inputs of oracle/mla_step.py's reading, then checks:
  - the output o [B, nh, R] per sequence and head: relative L2 <= 1e-2 (bf16
    operands, fp32 accumulation);
  - the append: cache row pos[b] holds the new token's rows bit for bit, and
    every other row of both caches (the NaN-filled tails included) is
    unchanged bit for bit.
Shapes span one chunk and many (fixed chunk lengths of 32..256 and the
automatic rule), ragged batches with pos = 0, 16 / 64 / 128 heads, and the
full DeepSeek-V3 attention shapes at 4K and 16K tokens (batch 1 and 16),
whose oracle runs whole on the CPU in seconds.  Planted dominant keys put
half of a head's weight on each of two tokens that straddle a chunk
boundary, the ends of the history, or the last history token and the new
token, so that a token dropped or counted twice moves that head's output by
O(1).

Reading of the pages: ClusterFusion page, section 5.2 (latent attention run
through the split-and-merge decode step); section 3.2 (the online softmax
with merged statistics equals softmax over all tokens).
"""
import sys

import numpy as np
import pytest

import oracle
from attention_block_amd.inputs import MLA_CONFIGS, MlaConfig, f32_to_bf16_bits, make_mla_inputs
from gpu_util import RECORD, rel_rows

pytestmark = pytest.mark.gpu

TOL = 1e-2


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(inp):
    import torch

    def bits(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()

    return dict(q_lat=torch.from_numpy(np.ascontiguousarray(inp["q_lat"], dtype=np.float32)).cuda(),
                q_rope=torch.from_numpy(np.ascontiguousarray(inp["q_rope"], dtype=np.float32)).cuda(),
                c_new=bits(inp["c_new"]), kr_new=bits(inp["kr_new"]), c_cache=bits(inp["c_cache"]),
                kr_cache=bits(inp["kr_cache"]), pos=torch.from_numpy(inp["pos"].astype(np.int32)).cuda())


def host_bits(t):
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def run_case(label, inp, kv_chunk=0, ref=None):
    import torch
    import attention_block_amd as ab
    cfg = inp["cfg"]
    say(f"[mla] {label}: B={cfg.batch} nh={cfg.n_heads} cap={inp['cap']} pos={list(inp['pos'][:8])} "
        f"kv_chunk={kv_chunk}")
    dev = to_device(inp)
    before_c, before_k = host_bits(dev["c_cache"]), host_bits(dev["kr_cache"])
    out = ab.mla_decode_attn(dev["q_lat"], dev["q_rope"], dev["c_new"], dev["kr_new"], dev["c_cache"],
                             dev["kr_cache"], dev["pos"], cfg.softmax_scale, kv_chunk=kv_chunk)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    if ref is None:
        ref = oracle.mla_decode_from_inputs(inp)
    B, nh = cfg.batch, cfg.n_heads
    per_head = rel_rows(got.reshape(B * nh, -1), ref["out"].reshape(B * nh, -1))
    errs = {"out": float(np.max(per_head)) if per_head.size else 0.0,
            "out_all": float(np.linalg.norm(got - ref["out"]) / max(np.linalg.norm(ref["out"]), 1e-300))}
    # the append, bit for bit, and nothing else written
    after_c, after_k = host_bits(dev["c_cache"]), host_bits(dev["kr_cache"])
    exp_c, exp_k = before_c.copy(), before_k.copy()
    for b in range(B):
        p = int(inp["pos"][b])
        exp_c[b, p] = inp["c_new"][b]
        exp_k[b, p] = inp["kr_new"][b]
    append_ok = bool(np.array_equal(after_c, exp_c) and np.array_equal(after_k, exp_k))
    say(f"[mla] {label}: worst head rel-L2 {errs['out']:.2e}, whole {errs['out_all']:.2e}, append exact "
        f"{append_ok}")
    RECORD.append((f"MLA {label}", "bf16", dict(errs)))
    assert np.all(np.isfinite(got)), f"{label}: non-finite output"
    assert append_ok, f"{label}: cache rows differ from the expected append"
    assert errs["out"] <= TOL, f"{label}: worst head rel-L2 {errs['out']:.3e} > {TOL:.0e}"
    return got, ref


def cfg_of(name, B, nh, pos, **kw):
    return MlaConfig(name, B, nh, pos, **kw)


CASES = [
    # (label, cfg, cap, pos list or None, kv_chunk)
    ("tiny one chunk", MLA_CONFIGS["mla_tiny"], None, None, 0),
    ("tiny 32-token chunks", MLA_CONFIGS["mla_tiny"], 130, [100, 37], 32),
    ("16 heads ragged with pos 0", cfg_of("r16", 4, 16, 0), 300, [0, 299, 31, 32], 0),
    ("16 heads chunks of 96", cfg_of("r16b", 3, 16, 0), 700, [699, 0, 350], 96),
    ("64 heads chunks of 64", cfg_of("h64", 2, 64, 0), 500, [499, 130], 64),
    ("64 heads auto", cfg_of("h64a", 3, 64, 0), 1200, [1199, 257, 1], 0),
    ("128 heads one tile", cfg_of("h128s", 2, 128, 0), 40, [0, 31], 0),
    ("128 heads chunks of 32, ragged tail", cfg_of("h128c", 2, 128, 0), 300, [290, 33], 32),
    ("128 heads chunks of 256", cfg_of("h128d", 1, 128, 0), 1100, [1000], 256),
    ("128 heads auto, batch 5", cfg_of("h128e", 5, 128, 0), 1000, [999, 1, 500, 256, 257], 0),
    # 1152 (sequence, head) pairs: partial rows in bf16, one-head merge; ragged, with a one-chunk sequence
    ("128 heads batch 9, bf16 partials", cfg_of("h128f", 9, 128, 0), 900, [899, 0, 450, 64, 63, 700, 129, 300, 31],
     64),
    ("V2-Lite 16 heads bs1 4K", MLA_CONFIGS["deepseek_v2_lite_mla_bs1_4k"], None, None, 0),
    ("V3 128 heads bs1 4K", MLA_CONFIGS["deepseek_v3_mla_bs1_4k"], None, None, 0),
    ("V3 128 heads bs1 4K chunks of 64", MLA_CONFIGS["deepseek_v3_mla_bs1_4k"], None, None, 64),
    ("V3 128 heads bs1 16K", MLA_CONFIGS["deepseek_v3_mla_bs1_16k"], None, None, 0),
    ("V3 128 heads bs16 4K", MLA_CONFIGS["deepseek_v3_mla_bs16_4k"], None, None, 0),
    ("V3 128 heads bs1 4K in a 16K cache", MLA_CONFIGS["deepseek_v3_mla_bs1_4k"], 16385, None, 0),
]


@pytest.mark.parametrize("label,cfg,cap,pos,kv_chunk", CASES, ids=[c[0] for c in CASES])
def test_mla_parity(label, cfg, cap, pos, kv_chunk):
    inp = make_mla_inputs(cfg, 7, cap=cap, pos=pos)
    run_case(label, inp, kv_chunk)


def test_mla_repeat_is_deterministic():
    """Two calls on the same inputs (the append rewrites the same row) give identical bits."""
    import torch
    import attention_block_amd as ab
    inp = make_mla_inputs(cfg_of("det", 2, 128, 0), 3, cap=600, pos=[599, 200])
    dev = to_device(inp)
    outs = []
    for _ in range(2):
        outs.append(ab.mla_decode_attn(dev["q_lat"], dev["q_rope"], dev["c_new"], dev["kr_new"], dev["c_cache"],
                                       dev["kr_cache"], dev["pos"], inp["cfg"].softmax_scale, kv_chunk=64).clone())
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])


# ---------------------------------------------------------------------------
# planted dominant keys
# ---------------------------------------------------------------------------

def plant(inp, b, h, t1, t2, score=12.0):
    """Tokens t1 and t2 of sequence b score `score` above zero for head h, equally: both get the rotary key
    along q_rope_h that adds `score`, and t2's latent row is t1's moved orthogonally to q_lat_h (so the
    two latent scores agree, yet the rows, the values, differ).  t2 == pos plants the new token's rows.
    A lift of 12 (e^12 against ~600 tokens of score ~N(0, 1)) already puts half the weight on each; a
    larger one would only scale the shared rotary key, whose product with the bf16-rounded query of the
    other 127 heads then errs in proportion (0.014 in log2 units at a lift of 40)."""
    cfg = inp["cfg"]
    qr, ql = inp["q_rope"][b, h].astype(np.float64), inp["q_lat"][b, h].astype(np.float64)
    kr = f32_to_bf16_bits((score / cfg.softmax_scale * qr / np.dot(qr, qr)).astype(np.float32))
    rng = np.random.default_rng(1000 + t1 + 7 * t2)
    c1 = rng.standard_normal(cfg.kv_lora_rank)
    r = rng.standard_normal(cfg.kv_lora_rank)
    c2 = r - (np.dot(ql, r) - np.dot(ql, c1)) * ql / np.dot(ql, ql)
    c1b, c2b = f32_to_bf16_bits(c1.astype(np.float32)), f32_to_bf16_bits(c2.astype(np.float32))
    p = int(inp["pos"][b])
    inp["c_cache"][b, t1], inp["kr_cache"][b, t1] = c1b, kr
    if t2 == p:
        inp["c_new"][b], inp["kr_new"][b] = c2b, kr
    else:
        inp["c_cache"][b, t2], inp["kr_cache"][b, t2] = c2b, kr


PLANTS = [
    # (label, cfg, cap, pos, kv_chunk, [(b, h, t1, t2)])
    ("chunk boundary 64", cfg_of("pa", 2, 128, 0), 700, [600, 333], 64, [(0, 5, 63, 64), (1, 77, 255, 256)]),
    ("tile boundary inside a chunk", cfg_of("pb", 1, 64, 0), 700, [600], 256, [(0, 40, 31, 32)]),
    ("first and last history", cfg_of("pc", 2, 128, 0), 700, [600, 333], 96, [(0, 0, 0, 599), (1, 127, 0, 332)]),
    ("last history and new token", cfg_of("pd", 2, 128, 0), 700, [600, 333], 0, [(0, 64, 599, 600), (1, 3, 332, 333)]),
    ("16 heads, new token in its own chunk", cfg_of("pe", 1, 16, 0), 300, [256], 128, [(0, 9, 255, 256)]),
]


@pytest.mark.parametrize("label,cfg,cap,pos,kv_chunk,plants", PLANTS, ids=[c[0] for c in PLANTS])
def test_mla_planted(label, cfg, cap, pos, kv_chunk, plants):
    inp = make_mla_inputs(cfg, 19, cap=cap, pos=pos)
    for b, h, t1, t2 in plants:
        plant(inp, b, h, t1, t2)
    ref = oracle.mla_decode_from_inputs(inp, want_probs=True)
    R = cfg.kv_lora_rank
    for b, h, t1, t2 in plants:
        pr = ref["probs"][b][h]
        assert abs(pr[t1] - 0.5) < 5e-2 and abs(pr[t2] - 0.5) < 5e-2, (b, h, pr[t1], pr[t2])
        vals = oracle.to_f64(inp["c_cache"][b], "bf16")
        v1 = vals[t1]
        o = ref["out"][b, h]
        assert np.linalg.norm(o - v1) / np.linalg.norm(o) > 0.3    # one token dropped would be this far off
    got, _ = run_case(f"planted {label}", inp, kv_chunk, ref=ref)
    for b, h, _, _ in plants:
        e = float(rel_rows(got[b, h][None], ref["out"][b, h][None])[0])
        assert e <= TOL, f"planted head ({b}, {h}): {e:.3e}"
