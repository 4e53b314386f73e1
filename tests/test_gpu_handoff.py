"""Regression test of the in-launch hand-offs, bounded: many back-to-back calls, stop at the first mismatch.

The schedules pass partial results between workgroups of one launch: the
last chunk of a (sequence, kv head) merges the others' partials after an
arrival counter says they are all published; the one-launch schedules'
projection (and attention) workgroups poll ready counts before they read
the attention output (or q and the new k, v).  Those counters are re-armed
by the call itself, so consecutive calls on one workspace must not see each
other's counts.  Here each schedule runs CALLS calls back to back on one
stream and one workspace, with a copy of the result (another kernel) between
them and a single synchronisation at the end; every result must equal the
first bit for bit, the first must match the fp64 oracle, and the device
error flag (a bounded wait that gave up, bit 1) must stay clear.  Every wait
in the kernels is bounded, so a broken hand-off ends as a flag or a
mismatch, never as a hang.

Reading of the pages: ClusterFusion page, section 3.2 (partial softmax
states merged across the blocks of a cluster; here across workgroups).
"""
import sys

import numpy as np
import pytest

import oracle
from attention_block_amd.inputs import BlockConfig, make_inputs
from gpu_util import compare, check_errs, small_cfg, storage_bits, to_device

pytestmark = pytest.mark.gpu

CALLS = 64


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


CASES = [
    # (schedule, cfg, cap, pos, kv_chunk)
    ("phased", small_cfg("ho1", 4, 1024, 32, 8, 128, "bf16", 5e5), 1100, [1000, 3, 517, 1099], 64),
    ("phased", small_cfg("ho2", 2, 512, 8, 8, 128, "f32"), 700, [600, 333], 0),
    ("attn_oproj", BlockConfig("ho3", 1, 4096, 32, 32, 128, "bf16", 1e4, pos=1000), None, None, 0),
    ("qkv_attn", small_cfg("ho4", 2, 4096, 32, 8, 128, "bf16", 5e5), 900, [800, 41], 0),
    ("fused", BlockConfig("ho5", 1, 4096, 32, 32, 128, "bf16", 1e4, pos=1000), None, None, 0),
    ("fused", small_cfg("ho6", 3, 1024, 32, 8, 128, "bf16", 5e5), 400, [399, 10, 150], 0),
]


@pytest.mark.parametrize("schedule,cfg,cap,pos,kv_chunk", CASES, ids=[f"{c[0]}-{c[1].name}" for c in CASES])
def test_back_to_back_calls_agree(schedule, cfg, cap, pos, kv_chunk):
    import torch
    import attention_block_amd as ab
    inp = make_inputs(cfg, 31, cap=cap, pos=pos)
    ref = oracle.decode_step_from_inputs(inp)
    dev = to_device(inp)
    before = (storage_bits(dev["k_cache"]), storage_bits(dev["v_cache"]))
    say(f"[handoff] {schedule} {cfg.name}: B={cfg.batch} {cfg.n_q_heads}q/{cfg.n_kv_heads}kv {cfg.dtype}, "
        f"{CALLS} calls back to back")
    c = ab.make_config(batch=cfg.batch, hidden=cfg.hidden, n_q_heads=cfg.n_q_heads, n_kv_heads=cfg.n_kv_heads,
                       head_dim=cfg.head_dim, cache_capacity=dev["k_cache"].shape[1], dtype=cfg.dtype,
                       rope_theta=cfg.rope_theta, eps=cfg.eps, kv_chunk=kv_chunk, schedule=schedule)
    ws = ab.Workspace(ab.workspace_size(c), dev["hidden"].device)
    outs = torch.empty((CALLS,) + tuple(dev["hidden"].shape), dtype=dev["hidden"].dtype, device=dev["hidden"].device)
    ys = torch.empty((CALLS,) + tuple(dev["hidden"].shape), dtype=torch.float32, device=dev["hidden"].device)
    out = torch.empty_like(dev["hidden"])
    dbg = torch.empty(dev["hidden"].shape, dtype=torch.float32, device=dev["hidden"].device)
    for i in range(CALLS):          # no synchronisation between calls
        ab.decode_attn_block(dev["hidden"], dev["norm_w"], dev["w_qkv"], dev["w_o"], dev["k_cache"],
                             dev["v_cache"], dev["pos"], cfg.rope_theta, cfg.eps, out=out, dbg_y=dbg,
                             kv_chunk=kv_chunk, workspace=ws, schedule=schedule, weight_layout="out_in")
        outs[i].copy_(out)
        ys[i].copy_(dbg)
    torch.cuda.synchronize()
    first = (outs[0], ys[0])
    flag = ab.read_device_error(ws)
    assert flag == 0, f"device error flag {flag}"
    # the first call against the oracle (the cache append rewrote the same rows with the same bits since)
    errs = compare(inp, ref, dev, first[0], first[1], before)
    check_errs(errs, cfg.dtype, f"handoff {schedule} {cfg.name}")
    bits = torch.int16 if cfg.dtype == "bf16" else torch.int32
    o0, y0 = outs[0].view(bits), ys[0]
    for i in range(1, CALLS):
        if not (torch.equal(outs[i].view(bits), o0) and torch.equal(ys[i], y0)):
            pytest.fail(f"{schedule} {cfg.name}: call {i} differs from call 0")
    say(f"[handoff] {schedule} {cfg.name}: {CALLS} identical results, flag clear")
