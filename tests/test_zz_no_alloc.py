"""The allocation-free entry point (dab_decode_attn_block_noalloc) against the workspace entry point.

Two calls in a row through the C ABI, the second with a smaller input and another configuration (so the
scratch holds the first call's counters and partials when the second starts): each must give the same
bits as dab_decode_attn_block on the same inputs (out, the y tap, both caches), on every schedule that
applies to the shapes."""
import sys

import numpy as np
import pytest

from attention_block_amd.inputs import make_inputs
from gpu_util import run_gpu, small_cfg, storage_bits, to_device

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


CALLS = [
    # (cfg, cap, pos, schedule): large first, smaller second
    (small_cfg("na1", 3, 4096, 32, 8, 128, "bf16", 5e5), 1500, [1499, 700, 3], "phased"),
    (small_cfg("na2", 1, 512, 4, 4, 128, "bf16"), 200, [150], "auto"),
    (small_cfg("na3", 2, 4096, 32, 32, 128, "bf16"), 900, [899, 450], "attn_oproj"),
    (small_cfg("na4", 1, 4096, 32, 32, 128, "bf16"), 300, [100], "fused"),
    (small_cfg("na5", 9, 1024, 8, 2, 128, "bf16", 5e5), 400, list(range(10, 400, 44)), "phased"),
    (small_cfg("na6", 1, 256, 4, 4, 64, "f32"), 129, [128], "auto"),
]


def noalloc_call(dev, cfg, schedule):
    import torch
    import attention_block_amd as ab
    out = torch.empty_like(dev["hidden"])
    dbg = torch.empty(dev["hidden"].shape, dtype=torch.float32, device=dev["hidden"].device)
    ab.decode_attn_block_noalloc(dev["hidden"], dev["norm_w"], dev["w_qkv"], dev["w_o"], dev["k_cache"],
                                 dev["v_cache"], dev["pos"], cfg.rope_theta, cfg.eps, out=out, dbg_y=dbg,
                                 schedule=schedule)
    torch.cuda.synchronize()
    return out, dbg


@pytest.mark.parametrize("first,second", [(0, 1), (2, 3), (4, 5), (1, 0)])
def test_noalloc_matches_the_workspace_entry_point(first, second):
    import torch
    for idx in (first, second):
        cfg, cap, pos, schedule = CALLS[idx]
        say(f"[noalloc] {cfg.name} B={cfg.batch} H={cfg.hidden} pos={pos} [{schedule}]")
        inp = make_inputs(cfg, 31 + idx, cap=cap, pos=pos)
        d_ref, d_na = to_device(inp), to_device(inp)
        ref_out, ref_y = run_gpu(d_ref, cfg, schedule=schedule)
        out, y = noalloc_call(d_na, cfg, schedule)
        bits = torch.int16 if cfg.dtype == "bf16" else torch.int32
        assert torch.equal(out.view(bits), ref_out.view(bits)), cfg.name
        assert torch.equal(y, ref_y), cfg.name
        for k in ("k_cache", "v_cache"):
            assert np.array_equal(storage_bits(d_na[k]), storage_bits(d_ref[k])), (cfg.name, k)
