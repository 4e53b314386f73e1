"""HIP path versus the fp64 oracle, element by element, on seeded inputs.

Gates (relative L2 per sequence, the worst sequence counting): out, the
fp32 pre-residual tap y, the appended K rows and V rows; and per sequence
and query head the attention output a (read from the workspace through
the library's test tap); <= 1e-2 with bf16 storage and fp32 accumulation,
<= 1e-5 in fp32 mode.  Every cache element other than the appended rows
must keep its exact bits, including the NaN sentinel tail beyond each
sequence's position.
"""
import sys

import numpy as np
import pytest

import oracle
from attention_block_amd.inputs import CONFIGS, BlockConfig, make_inputs
from gpu_util import (RECORD, check_errs, compare, rel_l2, run_gpu, small_cfg, storage_bits, storage_values, tol_for,
                      to_device)

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def parity_case(cfg: BlockConfig, seed: int, *, cap=None, pos=None, kv_chunk=0, label="", schedule="auto"):
    label = (label or f"{cfg.name} seed={seed} cap={cap} pos={pos} kv_chunk={kv_chunk}") + f" [{schedule}]"
    say(f"[parity] {label}")
    inp = make_inputs(cfg, seed, cap=cap, pos=pos)
    ref = oracle.decode_step_from_inputs(inp)
    dev = to_device(inp)
    before = (storage_bits(dev["k_cache"]), storage_bits(dev["v_cache"]))
    out, dbg, a = run_gpu(dev, cfg, kv_chunk=kv_chunk, schedule=schedule, want_a=True)
    errs = compare(inp, ref, dev, out, dbg, before, a=a)
    say(f"[parity] {label}: " + ", ".join(f"{k}={v:.2e}" if isinstance(v, float) else f"{k}={v}"
                                          for k, v in errs.items()))
    check_errs(errs, cfg.dtype, label)
    return errs


# ---------------------------------------------------------------------------
# the workload configurations, full size
# ---------------------------------------------------------------------------

SCHEDULES = ["phased", "attn_oproj", "qkv_attn", "fused"]


def applies(cfg: BlockConfig, schedule: str) -> bool:
    """The one-launch kernels are built for groups 1, 2, 4, 8 and a projection of whole K-blocks (a
    multiple of 4096 bf16 / 2048 fp32 values): the output projection's K = nq * D for attn_oproj and
    fused, the QKV projection's K = H for qkv_attn; fused also for batches of up to 4 whose fp32 input
    rows fit one workgroup's 64 KB of LDS in both projections."""
    if schedule in ("auto", "phased"):
        return True
    kblock = 4096 if cfg.dtype == "bf16" else 2048
    k = cfg.hidden if schedule == "qkv_attn" else cfg.n_q_heads * cfg.head_dim
    ok = cfg.group in (1, 2, 4, 8) and k % kblock == 0
    if schedule == "fused":
        nb = 1 if cfg.batch <= 1 else 2 if cfg.batch == 2 else 4
        ok = ok and cfg.batch <= 4 and nb * max(cfg.hidden, cfg.n_q_heads * cfg.head_dim) * 4 <= 65536
    return ok


@pytest.mark.parametrize("schedule", ["auto"] + SCHEDULES)
@pytest.mark.parametrize("seed", [0, 1])
@pytest.mark.parametrize("name", list(CONFIGS))
def test_config_parity(name, seed, schedule):
    if not applies(CONFIGS[name], schedule):
        pytest.skip(f"{schedule} is not built for this shape")
    parity_case(CONFIGS[name], seed, schedule=schedule)


def test_auto_takes_attn_oproj_for_mha_at_small_batch():
    import attention_block_amd as ab
    for name, cfg in CONFIGS.items():
        c = ab.make_config(batch=cfg.batch, hidden=cfg.hidden, n_q_heads=cfg.n_q_heads, n_kv_heads=cfg.n_kv_heads,
                           head_dim=cfg.head_dim, cache_capacity=8193, dtype=cfg.dtype, rope_theta=cfg.rope_theta)
        fused = applies(cfg, "attn_oproj") and cfg.group == 1 and cfg.batch <= 4
        want = ["qkv_rmsnorm_rope_append", "attention_oproj_residual"] if fused else \
            ["qkv_rmsnorm_rope_append", "attention_split_kv", "oproj_residual"]
        # (the phased schedule adds a merge kernel where the chunks need more than one merge round)
        assert [n for n in ab.phase_names(c) if n != "attention_merge"] == want, name


# ---------------------------------------------------------------------------
# edge cases: several tiles, ragged tails, degenerate positions
# ---------------------------------------------------------------------------

EDGE = [
    # (label, cfg, cap, pos, kv_chunk)
    ("single token, empty history", small_cfg("e1", 1, 256, 4, 4, 64, "f32"), 4, [0], 0),
    ("single token bf16 gqa", small_cfg("e2", 2, 512, 8, 2, 128, "bf16"), 3, [0, 0], 0),
    ("chunk multiple", small_cfg("e3", 1, 256, 4, 2, 64, "f32"), 200, [127], 64),
    ("chunk multiple + 1", small_cfg("e4", 1, 256, 4, 2, 64, "f32"), 200, [128], 64),
    ("odd cap stride", small_cfg("e5", 3, 320, 3, 1, 64, "f32", 5e5), 301, [5, 299, 64], 64),
    ("partial slabs H=320 bf16", small_cfg("e6", 5, 320, 3, 1, 64, "bf16", 5e5), 97, [96, 1, 63, 64, 65], 0),
    ("group 8", small_cfg("e7", 2, 1024, 16, 2, 64, "bf16", 1e4), 600, [599, 300], 128),
    ("batch 9 groups", small_cfg("e8", 9, 512, 4, 4, 128, "bf16"), 130, list(range(0, 129, 16)), 64),
    ("fp32 d128 gqa", small_cfg("e9", 3, 512, 8, 2, 128, "f32", 5e5), 1100, [1099, 512, 3], 0),
    ("many chunks", small_cfg("e10", 1, 256, 2, 1, 128, "bf16"), 4097 * 2, [8000], 64),
    # bf16 batches of 8 or more with K a multiple of 1024 take the MFMA panels
    ("mfma batch 9, one padded tile", small_cfg("m1", 9, 1024, 8, 2, 128, "bf16", 5e5), 300,
     [299, 0, 17, 256, 1, 128, 64, 200, 33], 0),
    ("mfma batch 20, two tiles", small_cfg("m2", 20, 2048, 16, 4, 128, "bf16"), 130, list(range(3, 130, 6))[:20], 0),
    ("mfma d64 group 8", small_cfg("m3", 8, 1024, 16, 2, 64, "bf16", 5e5), 90, [89, 0, 5, 64, 33, 80, 12, 1], 32),
    # 6144 QKV rows: 256 panels of 24 rows (three half tiles of 4 RoPE pairs, some panels across two
    # heads) with 32 sequences (batch 20) and with 16 sequences at D 64
    ("mfma batch 20, 24-row QKV panels of 32 sequences", small_cfg("m4", 20, 1024, 32, 8, 128, "bf16", 5e5), 150,
     [149, 0, 7, 100, 1, 64, 33, 120, 17, 90, 3, 140, 50, 12, 77, 128, 99, 5, 60, 145], 0),
    ("mfma batch 16, 24-row QKV panels, D 64", small_cfg("m5", 16, 1024, 64, 16, 64, "bf16", 5e5), 120,
     [119, 0, 3, 64, 1, 100, 33, 110, 17, 90, 5, 115, 50, 12, 77, 96], 0),
    # caches far larger than the contexts: the grid is sized for the capacity, each sequence's chunks
    # for its own position
    ("large cap mha bf16", small_cfg("lc1", 2, 512, 4, 4, 128, "bf16"), 20000, [1000, 37], 0),
    ("large cap gqa bf16", small_cfg("lc2", 3, 512, 8, 2, 128, "bf16", 5e5), 12000, [3000, 0, 700], 0),
    ("large cap f32 d64", small_cfg("lc3", 2, 256, 4, 2, 64, "f32"), 9000, [8999, 5], 0),
    # groups of 5, 6 and 7 (merge rounds of 6, 5 and 4 chunks per thread), in bf16 (pair dot products)
    # and fp32, with the merge inside the attention kernel and in a kernel of its own (63 chunks)
    ("group 5 bf16", small_cfg("g5b", 2, 640, 10, 2, 64, "bf16", 5e5), 300, [299, 150], 32),
    ("group 5 f32", small_cfg("g5f", 2, 640, 10, 2, 64, "f32", 5e5), 300, [299, 150], 32),
    ("group 6 bf16 merge kernel", small_cfg("g6b", 1, 768, 12, 2, 128, "bf16", 5e5), 2100, [2000], 32),
    ("group 6 f32", small_cfg("g6f", 2, 768, 12, 2, 128, "f32"), 300, [299, 1], 64),
    ("group 7 bf16", small_cfg("g7b", 2, 896, 14, 2, 64, "bf16"), 300, [299, 0], 32),
    ("group 7 f32 merge kernel", small_cfg("g7f", 1, 896, 14, 2, 64, "f32", 5e5), 2100, [2000], 32),
    # the merge kernel over ragged batches: 160 heads of 47 chunks (bf16), 144 heads of 79 chunks (fp32,
    # D 64: four chunk sums per output)
    ("merge kernel ragged bf16", small_cfg("mk1", 5, 512, 32, 8, 128, "bf16", 5e5), 3000,
     [2999, 100, 2048, 1500, 64], 64),
    ("merge kernel ragged f32 d64", small_cfg("mk2", 9, 256, 16, 4, 64, "f32"), 2500,
     [2499, 0, 2048, 17, 1200, 2400, 2450, 33, 1600], 32),
]


@pytest.mark.parametrize("label,cfg,cap,pos,kv_chunk", EDGE, ids=[e[0] for e in EDGE])
def test_edge_parity(label, cfg, cap, pos, kv_chunk):
    parity_case(cfg, 7, cap=cap, pos=pos, kv_chunk=kv_chunk, label=label)


# shapes the one-launch kernels are built for, at small sizes
EDGE_ONE_LAUNCH = [
    ("mha f32", small_cfg("o1", 1, 256, 16, 16, 128, "f32"), 300, [299], 0),
    ("gqa f32 empty history", small_cfg("o2", 3, 512, 32, 8, 64, "f32", 5e5), 130, [0, 129, 64], 64),
    ("bf16 group 2 ragged", small_cfg("o3", 5, 512, 32, 16, 128, "bf16", 5e5), 700, [699, 1, 350, 64, 500], 0),
    ("bf16 group 8 batch 9", small_cfg("o4", 9, 1024, 64, 8, 64, "bf16"), 200, list(range(3, 200, 22)), 32),
    ("f32 H 2048 gqa ragged", small_cfg("o5", 3, 2048, 16, 4, 128, "f32", 5e5), 300, [299, 0, 150], 0),
    ("bf16 H 4096 batch 6", small_cfg("o6", 6, 4096, 32, 8, 128, "bf16", 5e5), 260, [259, 3, 128, 0, 200, 64], 0),
    ("f32 H 2048 d64 group 1", small_cfg("o7", 2, 2048, 32, 32, 64, "f32"), 90, [89, 17], 32),
    # 2048 chunks: every attention workgroup of the one-launch attention + projection takes several
    ("bf16 many chunks per workgroup", small_cfg("o8", 2, 4096, 32, 32, 128, "bf16"), 2000, [1999, 1000], 64),
]
EDGE_ONE_LAUNCH += [
    ("bf16 large cap", small_cfg("o12", 1, 4096, 32, 32, 128, "bf16"), 8192, [1000], 0),
    ("bf16 fused batch 3 ragged", small_cfg("o9", 3, 1024, 32, 8, 128, "bf16", 5e5), 900, [899, 0, 450], 64),
    ("f32 fused d64 group 2 batch 2", small_cfg("o10", 2, 2048, 32, 16, 64, "f32"), 260, [259, 100], 32),
    ("bf16 fused group 8 H 8192", small_cfg("o11", 1, 8192, 64, 8, 64, "bf16"), 520, [519], 0),
]
ONE_LAUNCH_CASES = [(sched, *e) for e in EDGE_ONE_LAUNCH for sched in ("attn_oproj", "qkv_attn", "fused")
                    if applies(e[1], sched)]


@pytest.mark.parametrize("schedule,label,cfg,cap,pos,kv_chunk", ONE_LAUNCH_CASES,
                         ids=[f"{c[0]}: {c[1]}" for c in ONE_LAUNCH_CASES])
def test_edge_parity_one_launch(schedule, label, cfg, cap, pos, kv_chunk):
    parity_case(cfg, 7, cap=cap, pos=pos, kv_chunk=kv_chunk, label=label, schedule=schedule)


def test_one_launch_edge_cases_cover_every_schedule():
    assert {c[0] for c in ONE_LAUNCH_CASES} == {"attn_oproj", "qkv_attn", "fused"}
    assert sum(c[0] == "qkv_attn" for c in ONE_LAUNCH_CASES) >= 3
    assert sum(c[0] == "fused" for c in ONE_LAUNCH_CASES) >= 6


def test_default_workspaces_follow_the_configuration():
    """Counters sit where the configuration puts them: a call with a second configuration must not see
    the counters a first one left (here the first one's merge counters lie where the second one's
    chunk-arrival counters for its last sequence go)."""
    first, second = EDGE_ONE_LAUNCH[1], EDGE_ONE_LAUNCH[2]
    for label, cfg, cap, pos, kv_chunk in (first, second, first, second):
        parity_case(cfg, 3, cap=cap, pos=pos, kv_chunk=kv_chunk, label="workspace reuse: " + label,
                    schedule="attn_oproj")


SAME_BITS = EDGE_ONE_LAUNCH[1:] + [
    ("7B 4K", CONFIGS["llama2_7b_bs1_4k"], None, None, 0),
    # 41 chunks of a group of 4: the phased schedule merges in a kernel of its own, the one-launch
    # schedules inside their attention workgroups, with the same arithmetic
    ("gqa 41 chunks, merge kernel", small_cfg("sb1", 1, 4096, 32, 8, 128, "bf16", 5e5), 2600, [2599], 64),
]


@pytest.mark.parametrize("label,cfg,cap,pos,kv_chunk", SAME_BITS, ids=[e[0] for e in SAME_BITS])
def test_schedules_give_identical_bits(label, cfg, cap, pos, kv_chunk):
    """Every schedule runs the same arithmetic in the same order for one chunk length: identical out, y
    and caches.  (The default chunk lengths differ between schedules, so the chunk length is fixed
    here; and bf16 batches of 8 or more take MFMA panels in the phased schedule, which round the
    projection inputs to bf16; there only the one-launch schedules are compared with each other.)"""
    import torch
    kv_chunk = kv_chunk or 128
    inp = make_inputs(cfg, 21, cap=cap, pos=pos)
    scheds = [s for s in SCHEDULES if applies(cfg, s)]
    if cfg.dtype == "bf16" and cfg.batch >= 8:
        scheds.remove("phased")
    say(f"[schedules] {label}: {scheds}")
    res = {}
    bits = torch.int16 if cfg.dtype == "bf16" else torch.int32
    for sched in scheds:
        dev = to_device(inp)
        out, dbg = run_gpu(dev, cfg, kv_chunk=kv_chunk, schedule=sched)
        res[sched] = (out.view(bits), dbg, dev["k_cache"].view(bits), dev["v_cache"].view(bits))
    for sched in scheds[1:]:
        for i in range(4):
            assert torch.equal(res[sched][i], res[scheds[0]][i]), (sched, scheds[0], i)


BATCH_INVARIANCE = [
    small_cfg("bi1", 5, 512, 8, 2, 128, "bf16", 5e5),    # batch groups of 4: one full, one padded
    small_cfg("bi2", 3, 256, 4, 4, 64, "f32"),
    small_cfg("bi3", 2, 4096, 32, 8, 128, "bf16", 5e5),  # full-width rows (whole K-blocks)
]


@pytest.mark.parametrize("cfg", BATCH_INVARIANCE, ids=[c.name for c in BATCH_INVARIANCE])
def test_sequence_alone_matches_its_batch(cfg):
    """Every sum of a sequence runs in one fixed order whatever batch group it lands in, so (at a fixed
    KV chunk) a sequence run alone gives the same bits as inside its batch: out, y and the appended rows.
    (Batches below 8, where both calls take the VALU panels; bf16 batches of 8 or more take MFMA panels,
    which round their inputs to bf16.)"""
    import torch
    pos = [(37 * b + 300) % 700 for b in range(cfg.batch)]
    inp = make_inputs(cfg, 13, cap=701, pos=pos)
    say(f"[batch invariance] {cfg.name}")
    dev = to_device(inp)
    out, dbg = run_gpu(dev, cfg, kv_chunk=64)
    for b in range(cfg.batch):
        one = BlockConfig(cfg.name + "_1", 1, cfg.hidden, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.dtype,
                          cfg.rope_theta)
        sub = {**inp, "hidden": inp["hidden"][b:b + 1], "k_cache": inp["k_cache"][b:b + 1],
               "v_cache": inp["v_cache"][b:b + 1], "pos": inp["pos"][b:b + 1], "cfg": one}
        d1 = to_device(sub)
        o1, y1 = run_gpu(d1, one, kv_chunk=64)
        assert torch.equal(o1[0], out[b]) and torch.equal(y1[0], dbg[b]), b
        p = pos[b]
        for k in ("k_cache", "v_cache"):   # raw bits: the caches hold NaN sentinels
            assert torch.equal(d1[k][0, p].view(torch.int16 if cfg.dtype == "bf16" else torch.int32),
                               dev[k][b, p].view(torch.int16 if cfg.dtype == "bf16" else torch.int32)), (b, k)


def test_tiny_fp32_tolerance_is_met_tightly():
    errs = parity_case(CONFIGS["tiny_mha_f32"], 3)
    assert errs["out"] < 1e-6 and errs["y"] < 1e-5


# ---------------------------------------------------------------------------
# properties of the HIP path
# ---------------------------------------------------------------------------

def test_split_count_invariance():
    """Different KV chunk sizes give the same result up to fp32 rounding."""
    import torch
    cfg = small_cfg("inv", 2, 512, 8, 2, 128, "f32", 5e5)
    inp = make_inputs(cfg, 11, cap=1500, pos=[1499, 700])
    say("[split invariance] chunks 64/128/256/1024/4096")
    outs = []
    for ch in (64, 128, 256, 1024, 4096):
        dev = to_device(inp)
        _, dbg = run_gpu(dev, cfg, kv_chunk=ch, schedule="phased")
        outs.append(dbg.cpu().numpy().astype(np.float64))
    for o in outs[1:]:
        assert np.linalg.norm(o - outs[0]) / np.linalg.norm(outs[0]) < 1e-6


def test_fused_counters_return_to_zero():
    """The whole step in one launch re-arms its counters itself (the last readers zero them): after a
    call, every word in front of the workspace's data (flags, chunk arrivals, ready counts and their
    reader counts, QKV panel counts) is zero again."""
    import torch
    import attention_block_amd as ab
    cfg = small_cfg("wsf", 3, 1024, 32, 8, 128, "bf16", 5e5)
    inp = make_inputs(cfg, 2, cap=300, pos=[299, 10, 150])
    dev = to_device(inp)
    c = ab.make_config(batch=3, hidden=1024, n_q_heads=32, n_kv_heads=8, head_dim=128, cache_capacity=300,
                       dtype="bf16", rope_theta=5e5, schedule="fused")
    ws = ab.Workspace(ab.workspace_size(c), dev["hidden"].device)
    say("[counters] fused: three calls, then inspect the counters")
    for _ in range(3):
        run_gpu(dev, cfg, workspace=ws, schedule="fused")
    torch.cuda.synchronize()

    def a256(n):
        return (n + 255) // 256 * 256
    B, nkv, nq = 3, 8, 32
    # the layout of the counter words (flags, arrivals, ready counts, their readers, panel counts)
    prefix = 256 + a256(4 * B * nkv) + 2 * a256(4 * B * 16 * 32) + a256(4 * B * (nq + 2 * nkv))
    raw = ws._buf[ws.ptr - ws._buf.data_ptr():][:prefix].cpu().numpy().view(np.int32)
    assert np.all(raw == 0), np.nonzero(raw)[0][:10]


@pytest.mark.parametrize("schedule", ["auto", "phased", "fused"])
def test_repeat_calls_are_bit_identical(schedule):
    """Deterministic merges, and counters back at zero after each call."""
    import torch
    cfg = BlockConfig("rep", 4, 4096, 32, 8, 128, "bf16", 5e5, pos=1000)
    inp = make_inputs(cfg, 5)
    dev = to_device(inp)
    say(f"[repeat] {schedule}: three calls on one workspace")
    res = []
    for _ in range(3):
        out, dbg = run_gpu(dev, cfg, schedule=schedule)
        res.append((out.clone(), dbg.clone()))
    for o, d in res[1:]:
        assert torch.equal(o, res[0][0]) and torch.equal(d, res[0][1])


def test_workspace_counters_return_to_zero():
    import torch
    import attention_block_amd as ab
    cfg = small_cfg("ws", 3, 512, 8, 2, 128, "bf16", 5e5)
    inp = make_inputs(cfg, 2, cap=300, pos=[299, 10, 150])
    dev = to_device(inp)
    c = ab.make_config(batch=3, hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=128, cache_capacity=300,
                       dtype="bf16", rope_theta=5e5)
    ws = ab.Workspace(ab.workspace_size(c), dev["hidden"].device)
    say("[counters] call then inspect workspace counters")
    run_gpu(dev, cfg, workspace=ws)
    torch.cuda.synchronize()
    raw = ws._buf[ws.ptr - ws._buf.data_ptr():][: 256 + 256].cpu().numpy().view(np.int32).copy()
    # the workspace starts with the flags words (256 bytes), then the
    # attention arrival counters (B * nkv = 6 of them at this shape)
    assert np.all(raw == 0)


BAD_POS = [(sched, small_cfg("badpos", 3, 2048, 16, 4, 128, "f32")) for sched in SCHEDULES] + [
    ("phased", small_cfg("badpos_mfma", 8, 1024, 8, 2, 128, "bf16"))]       # MFMA panels


@pytest.mark.parametrize("schedule,cfg", BAD_POS, ids=[f"{s}-{c.name}" for s, c in BAD_POS])
def test_bad_position_sets_flag_and_skips_sequence(schedule, cfg):
    import torch
    import attention_block_amd as ab
    inp = make_inputs(cfg, 4, cap=40, pos=[10 + 3 * b for b in range(cfg.batch)])
    dev = to_device(inp)
    dev["pos"][1] = 40                                 # == cap: out of range, seen only on the device
    before = (storage_bits(dev["k_cache"]), storage_bits(dev["v_cache"]))
    out = torch.full_like(dev["hidden"], 12345.0)
    say("[bad pos] sequence 1 at pos == cap")
    ab.read_device_error()                             # clear any earlier flag
    ab.decode_attn_block(dev["hidden"], dev["norm_w"], dev["w_qkv"], dev["w_o"], dev["k_cache"], dev["v_cache"],
                         dev["pos"], cfg.rope_theta, cfg.eps, out=out, schedule=schedule, weight_layout="out_in")
    flag = ab.read_device_error()
    assert flag == 1
    assert torch.all(out[1] == 12345.0)               # its output row was left unwritten
    kb, vb = storage_bits(dev["k_cache"]), storage_bits(dev["v_cache"])
    assert np.array_equal(kb[1], before[0][1]) and np.array_equal(vb[1], before[1][1])
    # the other sequences are still right
    ref = oracle.decode_step_from_inputs(inp)
    got = storage_values(out)
    for b in range(cfg.batch):
        if b != 1:
            assert np.linalg.norm(got[b] - ref["out"][b]) / np.linalg.norm(ref["out"][b]) < tol_for(cfg.dtype), b
    assert ab.read_device_error() == 0                 # reading cleared it


@pytest.mark.parametrize("schedule", SCHEDULES)
def test_graph_replay_matches_eager(schedule):
    import torch
    import attention_block_amd as ab
    cfg = small_cfg("graph", 2, 4096, 32, 8, 128, "bf16", 5e5)   # H = nq * D = 4096: every schedule applies
    inp = make_inputs(cfg, 9, cap=700, pos=[699, 333])
    dev = to_device(inp)
    say(f"[graph] {schedule}: eager, capture, 4 replays")
    eager, _ = run_gpu(dev, cfg, schedule=schedule)
    eager = eager.clone()
    out = torch.empty_like(dev["hidden"])
    c = ab.make_config(batch=2, hidden=4096, n_q_heads=32, n_kv_heads=8, head_dim=128, cache_capacity=700,
                       dtype="bf16", rope_theta=5e5, schedule=schedule)
    ws = ab.Workspace(ab.workspace_size(c), dev["hidden"].device)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm-up call outside capture
        ab.decode_attn_block(dev["hidden"], dev["norm_w"], dev["w_qkv"], dev["w_o"], dev["k_cache"],
                             dev["v_cache"], dev["pos"], cfg.rope_theta, cfg.eps, out=out, workspace=ws,
                             schedule=schedule, weight_layout="out_in")
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ab.decode_attn_block(dev["hidden"], dev["norm_w"], dev["w_qkv"], dev["w_o"], dev["k_cache"],
                             dev["v_cache"], dev["pos"], cfg.rope_theta, cfg.eps, out=out, workspace=ws,
                             schedule=schedule, weight_layout="out_in")
    for i in range(4):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i}"
        _ = (dev["hidden"].float() * 2).sum().item()   # unrelated eager work between replays


HINT = [("phased", small_cfg("hint_gqa", 4, 1024, 16, 4, 128, "bf16", 5e5)),
        ("attn_oproj", small_cfg("hint_mha", 2, 2048, 16, 16, 128, "f32"))]


@pytest.mark.parametrize("schedule,cfg", HINT, ids=[f"{s}-{c.name}" for s, c in HINT])
def test_max_position_hint(schedule, cfg):
    """A cache of 3000 rows with positions up to 299: with max_position = 299 the step is planned for 300
    tokens and every sequence matches the oracle; with a hint of 260 the sequence at 299 is rejected on
    the device (the flag, its output row and cache rows untouched) and the others stay right."""
    import torch
    import attention_block_amd as ab
    pos = [100, 299, 7, 250][:cfg.batch]
    inp = make_inputs(cfg, 11, cap=3000, pos=pos)
    ref = oracle.decode_step_from_inputs(inp)
    dev = to_device(inp)
    say(f"[hint] {schedule} {cfg.name}: cap 3000, pos {pos}, max_position {max(pos)}")
    ab.read_device_error()
    out = ab.decode_attn_block(dev["hidden"], dev["norm_w"], dev["w_qkv"], dev["w_o"], dev["k_cache"].clone(),
                               dev["v_cache"].clone(), dev["pos"], cfg.rope_theta, cfg.eps, schedule=schedule,
                               weight_layout="out_in", max_position=max(pos))
    assert ab.read_device_error() == 0
    got = storage_values(out)
    errs = [rel_l2(got[b], ref["out"][b]) for b in range(cfg.batch)]
    RECORD.append((f"hint {schedule} {cfg.name}", cfg.dtype, {"out": max(errs), "out_all": rel_l2(got, ref["out"])}))
    assert max(errs) <= tol_for(cfg.dtype), errs

    say(f"[hint] {schedule} {cfg.name}: max_position 260 with a sequence at 299")
    out = torch.full_like(dev["hidden"], 12345.0)
    before = (storage_bits(dev["k_cache"]), storage_bits(dev["v_cache"]))
    ab.decode_attn_block(dev["hidden"], dev["norm_w"], dev["w_qkv"], dev["w_o"], dev["k_cache"], dev["v_cache"],
                         dev["pos"], cfg.rope_theta, cfg.eps, out=out, schedule=schedule, weight_layout="out_in",
                         max_position=260)
    assert ab.read_device_error() == 1
    assert torch.all(out[1] == 12345.0)
    kb, vb = storage_bits(dev["k_cache"]), storage_bits(dev["v_cache"])
    assert np.array_equal(kb[1], before[0][1]) and np.array_equal(vb[1], before[1][1])
    got = storage_values(out)
    for b in range(cfg.batch):
        if b != 1:
            assert rel_l2(got[b], ref["out"][b]) <= tol_for(cfg.dtype), b
