"""The decoder layer in one call (dab_decode_layer) through the C ABI.

Every layer schedule must give the bits of the two calls it replaces
(dab_decode_attn_block, then dab_decode_ffn_block on its output): in the
overlapped one (where dab_layer_overlapped holds) every value is computed by
the same code in the same order, only h reaches the FFN panels through
device-coherent stores and loads inside one launch.
The two paths run on copies of the same inputs and caches; h, out and both
caches are compared bit for bit, and out against the two oracles composed
(the attention block's output in the storage dtype feeding the FFN).  Calls
follow one another on one pair of workspaces, so a ready flag or counter left
raised by one call would show in the next."""
import sys

import numpy as np
import pytest

import oracle
from attention_block_amd.inputs import f32_to_bf16_bits, layer_ffn, make_ffn_inputs, make_inputs
from gpu_util import RECORD, rel_l2, small_cfg, storage_bits, storage_values, to_device, tol_for
from test_gpu_ffn import ffn_to_device

pytestmark = pytest.mark.gpu

# (label, attention block, positions, cache capacity, overlapped)
LAYERS = [
    ("7B shape bs1 bf16", small_cfg("l1", 1, 4096, 32, 32, 128, "bf16"), [700], 1024, True),
    ("bf16 bs3 head dim 64, ragged", small_cfg("l2", 3, 4096, 64, 64, 64, "bf16"), [299, 0, 150], 300, True),
    ("bf16 bs2", small_cfg("l3", 2, 4096, 32, 32, 128, "bf16"), [1, 1000], 1001, True),
    ("f32 bs4 H 2048", small_cfg("l4", 4, 2048, 16, 16, 128, "f32"), [63, 64, 65, 500], 501, True),
    ("f32 bs1 H 2048 head dim 64", small_cfg("l5", 1, 2048, 32, 32, 64, "f32"), [128], 129, True),
    ("bf16 gqa, two calls", small_cfg("l6", 2, 1024, 16, 4, 64, "bf16", 5e5), [37, 200], 201, False),
]


def to_storage(values, dtype):
    v32 = np.asarray(values, dtype=np.float32)
    return f32_to_bf16_bits(v32) if dtype == "bf16" else v32


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("label,cfg,pos,cap,overlapped", LAYERS, ids=[c[0] for c in LAYERS])
def test_layer_matches_two_calls_and_oracle(label, cfg, pos, cap, overlapped):
    import torch
    import attention_block_amd as ab
    from attention_block_amd import _lib
    fcfg = layer_ffn(cfg)
    say(f"[layer] {label}: B={cfg.batch} H={cfg.hidden} {cfg.n_q_heads}q/{cfg.n_kv_heads}kv D={cfg.head_dim} "
        f"F={fcfg.intermediate} {cfg.dtype} pos={pos} cap={cap}")
    dt = _lib.DAB_BF16 if cfg.dtype == "bf16" else _lib.DAB_F32
    acfg = ab.make_config(batch=cfg.batch, hidden=cfg.hidden, n_q_heads=cfg.n_q_heads, n_kv_heads=cfg.n_kv_heads,
                          head_dim=cfg.head_dim, cache_capacity=cap, dtype=cfg.dtype, rope_theta=cfg.rope_theta,
                          eps=cfg.eps)
    ffn_c = _lib.DabFfnConfig(cfg.batch, cfg.hidden, fcfg.intermediate, dt, fcfg.eps)
    assert ab.layer_overlapped(acfg, ffn_c) == overlapped

    ws = ab.Workspace(ab.workspace_size(acfg), torch.device("cuda"))
    fws = ab.Workspace(ab.ffn_workspace_size(ffn_c), torch.device("cuda"))
    schedules = ["overlap", "sequential"] if overlapped else ["auto"]
    if not overlapped:
        inp = make_inputs(cfg, 99, pos=pos, cap=cap)
        dev = to_device(inp)
        fdev = ffn_to_device(make_ffn_inputs(fcfg, 199))
        with pytest.raises(ab.DabError):       # refused on the host: nothing is enqueued
            ab.decode_layer(dev["hidden"], dev["norm_w"], dev["w_qkv"], dev["w_o"], dev["k_cache"], dev["v_cache"],
                            dev["pos"], fdev["norm_w"], fdev["w_gate"], fdev["w_up"], fdev["w_down"],
                            cfg.rope_theta, cfg.eps, fcfg.eps, workspace=ws, ffn_workspace=fws,
                            layer_schedule="overlap", weight_layout="out_in")
    for call in range(3 * len(schedules)):
        sched = schedules[call % len(schedules)]
        inp = make_inputs(cfg, 100 + call, pos=pos, cap=cap)
        finp = make_ffn_inputs(fcfg, 200 + call)
        # the oracles composed: the block's output in the storage dtype feeds the FFN
        ref_a = oracle.decode_step_from_inputs(inp)
        finp["hidden"] = to_storage(ref_a["out_stored"], cfg.dtype)
        ref_f = oracle.ffn_step_from_inputs(finp)

        dev = to_device(inp)
        fdev = ffn_to_device(finp)
        kc, vc = dev["k_cache"].clone(), dev["v_cache"].clone()
        # the two calls
        h2 = ab.decode_attn_block(dev["hidden"], dev["norm_w"], dev["w_qkv"], dev["w_o"], kc, vc, dev["pos"],
                                  cfg.rope_theta, cfg.eps, weight_layout="out_in")
        out2 = ab.decode_ffn_block(h2, fdev["norm_w"], fdev["w_gate"], fdev["w_up"], fdev["w_down"], fcfg.eps,
                                   weight_layout="out_in")
        # the layer in one call
        h1, out1 = ab.decode_layer(dev["hidden"], dev["norm_w"], dev["w_qkv"], dev["w_o"], dev["k_cache"],
                                   dev["v_cache"], dev["pos"], fdev["norm_w"], fdev["w_gate"], fdev["w_up"],
                                   fdev["w_down"], cfg.rope_theta, cfg.eps, fcfg.eps, workspace=ws,
                                   ffn_workspace=fws, layer_schedule=sched, weight_layout="out_in")
        torch.cuda.synchronize()
        assert ab.read_device_error(ws) == 0
        same = {name: np.array_equal(storage_bits(x), storage_bits(y))
                for name, x, y in (("h", h1, h2), ("out", out1, out2), ("k_cache", dev["k_cache"], kc),
                                   ("v_cache", dev["v_cache"], vc))}
        err = rel_l2(storage_values(out1), ref_f["out"])
        errs_seq = [rel_l2(storage_values(out1)[b], ref_f["out"][b]) for b in range(cfg.batch)]
        say(f"[layer] {label}: call {call} ({sched}): identical {same}; rel-L2(out) {err:.2e}, "
            f"worst sequence {max(errs_seq):.2e}")
        if call < len(schedules):
            RECORD.append((f"layer {sched} {cfg.name}", cfg.dtype, {"out": max(errs_seq), "out_all": err}))
        assert all(same.values()), same
        assert np.all(np.isfinite(storage_values(out1)))
        assert max(errs_seq) <= tol_for(cfg.dtype), errs_seq


def test_layer_bad_position_completes_and_flags():
    """Sequence 1 at position == capacity in the overlapped layer: the projection panels still count it,
    so every FFN panel's wait ends (a wait that ran out would add bit 2 to the flag); its h row is left
    unwritten, the other sequences match the composed oracles, and the next call on the same workspaces
    gives the two calls' bits."""
    import torch
    import attention_block_amd as ab
    from attention_block_amd import _lib
    cfg = small_cfg("lbad", 3, 2048, 16, 16, 128, "f32")
    fcfg = layer_ffn(cfg)
    cap = 40
    acfg = ab.make_config(batch=3, hidden=2048, n_q_heads=16, n_kv_heads=16, head_dim=128, cache_capacity=cap,
                          dtype="f32", rope_theta=cfg.rope_theta, eps=cfg.eps)
    ffn_c = _lib.DabFfnConfig(3, 2048, fcfg.intermediate, _lib.DAB_F32, fcfg.eps)
    assert ab.layer_overlapped(acfg, ffn_c)
    ws = ab.Workspace(ab.workspace_size(acfg), torch.device("cuda"))
    fws = ab.Workspace(ab.ffn_workspace_size(ffn_c), torch.device("cuda"))

    inp = make_inputs(cfg, 4, cap=cap, pos=[10, 13, 16])
    finp = make_ffn_inputs(fcfg, 5)
    ref_a = oracle.decode_step_from_inputs(inp)
    finp["hidden"] = to_storage(ref_a["out_stored"], cfg.dtype)
    ref_f = oracle.ffn_step_from_inputs(finp)
    dev = to_device(inp)
    fdev = ffn_to_device(finp)
    dev["pos"][1] = cap                                  # out of range, seen only on the device
    h = torch.full_like(dev["hidden"], 12345.0)
    say("[layer] bad position: sequence 1 at pos == cap, overlapped schedule")
    ab.read_device_error(ws)                             # clear any earlier flag
    _, out = ab.decode_layer(dev["hidden"], dev["norm_w"], dev["w_qkv"], dev["w_o"], dev["k_cache"],
                             dev["v_cache"], dev["pos"], fdev["norm_w"], fdev["w_gate"], fdev["w_up"],
                             fdev["w_down"], cfg.rope_theta, cfg.eps, fcfg.eps, h=h, workspace=ws,
                             ffn_workspace=fws, layer_schedule="overlap", weight_layout="out_in")
    torch.cuda.synchronize()
    assert ab.read_device_error(ws) == 1
    assert torch.all(h[1] == 12345.0)
    got = storage_values(out)
    for b in (0, 2):
        assert rel_l2(got[b], ref_f["out"][b]) <= tol_for(cfg.dtype), b

    # a valid call after it, on the same workspaces
    inp = make_inputs(cfg, 6, cap=cap, pos=[39, 0, 20])
    finp = make_ffn_inputs(fcfg, 7)
    dev = to_device(inp)
    fdev = ffn_to_device(finp)
    kc, vc = dev["k_cache"].clone(), dev["v_cache"].clone()
    h2 = ab.decode_attn_block(dev["hidden"], dev["norm_w"], dev["w_qkv"], dev["w_o"], kc, vc, dev["pos"],
                              cfg.rope_theta, cfg.eps, weight_layout="out_in")
    out2 = ab.decode_ffn_block(h2, fdev["norm_w"], fdev["w_gate"], fdev["w_up"], fdev["w_down"], fcfg.eps,
                               weight_layout="out_in")
    h1, out1 = ab.decode_layer(dev["hidden"], dev["norm_w"], dev["w_qkv"], dev["w_o"], dev["k_cache"],
                               dev["v_cache"], dev["pos"], fdev["norm_w"], fdev["w_gate"], fdev["w_up"],
                               fdev["w_down"], cfg.rope_theta, cfg.eps, fcfg.eps, workspace=ws, ffn_workspace=fws,
                               layer_schedule="overlap", weight_layout="out_in")
    torch.cuda.synchronize()
    assert ab.read_device_error(ws) == 0
    assert np.array_equal(storage_bits(h1), storage_bits(h2))
    assert np.array_equal(storage_bits(out1), storage_bits(out2))
    say("[layer] bad position: flag 1, other sequences right, the next call identical to the two calls")
