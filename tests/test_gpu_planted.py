"""Planted dominant keys: a dropped or doubled token must fail by O(1).

With random keys every token carries a weight of about 1/1500 at 4K tokens,
so a token lost or counted twice at a split-KV chunk boundary moves the
attention output by far less than the 1e-2 gate.  Here two keys of one kv
head are made dominant, with equal scores (about 40 above the rest) for the
group's first query head h, so that head's softmax puts weight 1/2 on each:
the correct output is the mean of the two value rows, one token dropped
gives one value row, one counted twice gives a 2:1 mixture.  Each case is
gated per sequence and query head on the attention output a (read through
the library's test tap) against the fp64 oracle run on the same planted
caches, and the oracle itself is checked to put half the weight on each
planted token (the plant did what it should).

Plants: the last token of one chunk with the first of the next, the first
history token with the last one, and the last history token with the new
token (whose key is known only after the projection: the planted key is the
new token's appended key, and every other history key of the group is
pushed 30 below it).  Paths: one query head per kv head (bf16 and fp32),
grouped heads over a bf16 cache (the pair dot products) and in fp32,
matrix-core panels (a bf16 batch of 9), the one-launch attention +
projection schedule, and the merge in a kernel of its own (many chunks).

Reading of the pages: ClusterFusion page, section 3.2 (the online softmax
with merged statistics is exactly softmax over all tokens).
"""
import sys

import numpy as np
import pytest

import oracle
from attention_block_amd.inputs import f32_to_bf16_bits, make_inputs
from gpu_util import check_errs, compare, rel_rows, run_gpu, small_cfg, storage_bits, to_device

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def store(values, dtype):
    v32 = np.asarray(values, dtype=np.float32)
    return f32_to_bf16_bits(v32) if dtype == "bf16" else v32


def decode(bits, dtype):
    return oracle.to_f64(bits, dtype)


def key_direction(ref0, b, g, G):
    """The part of head g*G's rotated q orthogonal to the other query heads of its group: a key along it
    scores for the target head only, so the group's other heads see the planted keys as ordinary
    tokens (score ~0) and their outputs keep their usual conditioning."""
    q = ref0["q"][b, g * G]
    others = ref0["q"][b, g * G + 1:(g + 1) * G]
    if len(others) == 0:
        return q
    basis, _ = np.linalg.qr(others.T)
    return q - basis @ (basis.T @ q)


def plant_pair(inp, ref0, b, t1, t2, score=40.0):
    """K[b, t1, g] = K[b, t2, g] = a key scoring `score` for head g * G, for every kv group g."""
    cfg = inp["cfg"]
    G, D = cfg.group, cfg.head_dim
    for g in range(cfg.n_kv_heads):
        q, k = ref0["q"][b, g * G], key_direction(ref0, b, g, G)
        key = store(score * np.sqrt(D) * k / np.dot(q, k), cfg.dtype)
        inp["k_cache"][b, t1, g] = key
        inp["k_cache"][b, t2, g] = key
    return [(b, g * G, (t1, t2)) for g in range(cfg.n_kv_heads)]


def plant_with_new(inp, ref0, b, below=30.0):
    """K[b, pos-1, g] = the new token's appended key; every earlier history key of group g scores `below`
    under the new token's score for head g * G."""
    cfg = inp["cfg"]
    G, D = cfg.group, cfg.head_dim
    p = int(inp["pos"][b])
    for g in range(cfg.n_kv_heads):
        q, k = ref0["q"][b, g * G], key_direction(ref0, b, g, G)
        k_new = decode(store(ref0["k_new"][b, g], cfg.dtype), cfg.dtype)
        s_new = float(np.dot(q, k_new)) / np.sqrt(D)
        low = store((s_new - below) * np.sqrt(D) * k / np.dot(q, k), cfg.dtype)
        inp["k_cache"][b, :p - 1, g] = low
        inp["k_cache"][b, p - 1, g] = store(k_new, cfg.dtype)
    return [(b, g * G, (p - 1, p)) for g in range(cfg.n_kv_heads)]


def planted_case(label, cfg, cap, pos, kv_chunk, schedule, plants, seed=17):
    label = f"planted {label} [{schedule}, kv_chunk {kv_chunk}]"
    say(f"[planted] {label}: B={cfg.batch} H={cfg.hidden} {cfg.n_q_heads}q/{cfg.n_kv_heads}kv x {cfg.head_dim} "
        f"{cfg.dtype} pos={pos}")
    inp = make_inputs(cfg, seed, cap=cap, pos=pos)
    ref0 = oracle.decode_step_from_inputs(inp)          # q' and the new k: they do not depend on the cache
    targets = []
    for kind, b, *ts in plants:
        if kind == "pair":
            targets += plant_pair(inp, ref0, b, *ts)
        else:
            targets += plant_with_new(inp, ref0, b)
    ref = oracle.decode_step_from_inputs(inp, want_probs=True)
    D = cfg.head_dim
    # the plant did what it should: half of head h's weight on each planted token
    for b, h, (t1, t2) in targets:
        pr = ref["probs"][b][h]
        assert abs(pr[t1] - 0.5) < 2e-2 and abs(pr[t2] - 0.5) < 2e-2, (b, h, pr[t1], pr[t2])
        vals = decode(inp["v_cache"][b], cfg.dtype)
        v1 = vals[t1, h // cfg.group]
        v2 = ref["v_new"][b, h // cfg.group] if t2 == int(inp["pos"][b]) else vals[t2, h // cfg.group]
        a_h = ref["a"][b, h * D:(h + 1) * D]
        # one token dropped or doubled would sit this far from the correct output
        assert np.linalg.norm(a_h - v1) / np.linalg.norm(a_h) > 0.3
        assert np.linalg.norm(a_h - (2 * v1 + v2) / 3) / np.linalg.norm(a_h) > 0.1
    dev = to_device(inp)
    before = (storage_bits(dev["k_cache"]), storage_bits(dev["v_cache"]))
    out, dbg, a = run_gpu(dev, cfg, kv_chunk=kv_chunk, schedule=schedule, want_a=True)
    errs = compare(inp, ref, dev, out, dbg, before, a=a)
    got = a.cpu().numpy()
    worst = max(float(rel_rows(got[b, h * D:(h + 1) * D], ref["a"][b, h * D:(h + 1) * D]))
                for b, h, _ in targets)
    errs["a_planted"] = worst
    say(f"[planted] {label}: " + ", ".join(f"{k}={v:.2e}" if isinstance(v, float) else f"{k}={v}"
                                           for k, v in errs.items()))
    check_errs(errs, cfg.dtype, label)


T = 128
BOUNDARY = [("pair", 0, T - 1, T), ("pair", 1, 2 * T - 1, 2 * T)]     # last of a chunk + first of the next
ENDS = [("pair", 0, 0, 599), ("new", 1)]                              # first + last history; last + new

CASES = [
    # (label, cfg, cap, pos, kv_chunk, schedule, plants)
    ("mha bf16 chunk boundary", small_cfg("pl1", 2, 512, 4, 4, 128, "bf16"), 700, [600, 333], T, "phased",
     BOUNDARY),
    ("mha bf16 ends", small_cfg("pl1", 2, 512, 4, 4, 128, "bf16"), 700, [600, 333], T, "phased", ENDS),
    ("mha f32 chunk boundary", small_cfg("pl2", 2, 512, 4, 4, 128, "f32"), 700, [600, 333], T, "phased",
     BOUNDARY),
    ("mha f32 ends", small_cfg("pl2", 2, 512, 4, 4, 128, "f32"), 700, [600, 333], T, "phased", ENDS),
    ("gqa4 bf16 pair dot, chunk boundary", small_cfg("pl3", 2, 512, 8, 2, 128, "bf16", 5e5), 700, [600, 333], T,
     "phased", BOUNDARY),
    ("gqa4 bf16 pair dot, ends", small_cfg("pl3", 2, 512, 8, 2, 128, "bf16", 5e5), 700, [600, 333], T, "phased",
     ENDS),
    ("gqa4 f32 ends", small_cfg("pl4", 2, 512, 8, 2, 128, "f32", 5e5), 700, [600, 333], T, "phased", ENDS),
    ("gqa8 d64 bf16 ends", small_cfg("pl5", 2, 512, 16, 2, 64, "bf16", 5e5), 700, [600, 333], T, "phased",
     ENDS),
    ("mfma batch 9 boundary + ends", small_cfg("pl6", 9, 1024, 8, 2, 128, "bf16", 5e5), 700,
     [600, 333, 300, 256, 400, 500, 290, 280, 599], T, "phased",
     [("pair", 0, T - 1, T), ("new", 8), ("pair", 4, 0, 399)]),
    ("one launch attn+oproj, boundary + new", small_cfg("pl7", 1, 512, 32, 32, 128, "bf16"), 700, [600], T,
     "attn_oproj", [("pair", 0, T - 1, T)]),
    ("one launch attn+oproj, new", small_cfg("pl7", 1, 512, 32, 32, 128, "bf16"), 700, [600], T,
     "attn_oproj", [("new", 0)]),
    ("one launch qkv+attn, new", small_cfg("pl8", 1, 4096, 32, 8, 128, "bf16", 5e5), 700, [600], T,
     "qkv_attn", [("new", 0)]),
    ("whole step one launch, boundary", small_cfg("pl7", 1, 512, 32, 32, 128, "bf16"), 700, [600], T,
     "fused", [("pair", 0, T - 1, T)]),
    ("whole step one launch, new", small_cfg("pl7", 1, 512, 32, 32, 128, "bf16"), 700, [600], T,
     "fused", [("new", 0)]),
    ("whole step one launch gqa4 batch 2, ends", small_cfg("pl10", 2, 1024, 32, 8, 128, "bf16", 5e5), 700,
     [600, 333], T, "fused", ENDS),
    # 63 chunks of 32 tokens with a group of 4: the merge runs as a kernel of its own
    ("merge kernel, boundary", small_cfg("pl9", 1, 512, 8, 2, 128, "bf16", 5e5), 2100, [2000], 32, "phased",
     [("pair", 0, 31 * 32 - 1, 31 * 32)]),
    ("merge kernel, new", small_cfg("pl9", 1, 512, 8, 2, 128, "bf16", 5e5), 2100, [2000], 32, "phased",
     [("new", 0)]),
]


@pytest.mark.parametrize("label,cfg,cap,pos,kv_chunk,schedule,plants", CASES, ids=[c[0] for c in CASES])
def test_planted_dominant_keys(label, cfg, cap, pos, kv_chunk, schedule, plants):
    planted_case(label, cfg, cap, pos, kv_chunk, schedule, plants)
