"""HIP FFN half of the layer versus the fp64 FFN oracle, element by element.

Gates (relative L2 over the whole tensor): out and the fp32 pre-residual tap
y; <= 1e-2 with bf16 storage and fp32 accumulation, <= 1e-5 in fp32 mode.
The intermediate m is not exposed.  Shapes span several row panels, batch
groups with padding rows, widths that are not whole 4096-element K-blocks
(the bounds-checked weight loads), and the largest intermediate size.
"""
import sys

import numpy as np
import pytest

import oracle
from attention_block_amd.inputs import FFN_CONFIGS, FfnConfig, make_ffn_inputs
from gpu_util import rel_l2, storage_bits, storage_values, tol_for

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def ffn_to_device(inp: dict, device="cuda"):
    import torch
    cfg = inp["cfg"]

    def t(a):
        if cfg.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)

    # the oracle's [in, out] matrices, packed by the library into its [out, in] layout
    import attention_block_amd as ab
    return dict(hidden=t(inp["hidden"]), norm_w=t(inp["norm_w"]), w_gate=ab.pack_weight(t(inp["w_gate"])),
                w_up=ab.pack_weight(t(inp["w_up"])), w_down=ab.pack_weight(t(inp["w_down"])))


def run_ffn(dev: dict, cfg: FfnConfig, workspace=None):
    import torch
    import attention_block_amd as ab
    dbg = torch.empty(dev["hidden"].shape, dtype=torch.float32, device=dev["hidden"].device)
    out = ab.decode_ffn_block(dev["hidden"], dev["norm_w"], dev["w_gate"], dev["w_up"], dev["w_down"], cfg.eps,
                              dbg_y=dbg, workspace=workspace, weight_layout="out_in")
    torch.cuda.synchronize()
    return out, dbg


def ffn_case(cfg: FfnConfig, seed: int, label: str = ""):
    label = label or f"{cfg.name} seed={seed}"
    say(f"[ffn] {label}: B={cfg.batch} H={cfg.hidden} F={cfg.intermediate} {cfg.dtype}")
    inp = make_ffn_inputs(cfg, seed)
    ref = oracle.ffn_step_from_inputs(inp)
    dev = ffn_to_device(inp)
    out, dbg = run_ffn(dev, cfg)
    errs = {"out": rel_l2(storage_values(out), ref["out"]), "y": rel_l2(dbg.cpu().numpy(), ref["y"])}
    say(f"[ffn] {label}: " + ", ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    assert np.all(np.isfinite(storage_values(out))) and np.all(np.isfinite(dbg.cpu().numpy())), label
    tol = tol_for(cfg.dtype)
    for k, v in errs.items():
        assert v <= tol, f"{label}: rel-L2({k}) = {v:.3e} > {tol:.0e}"
    return dev, out, dbg


@pytest.mark.parametrize("name", list(FFN_CONFIGS))
def test_ffn_config_parity(name):
    ffn_case(FFN_CONFIGS[name], 0)


EDGE = [
    # batch groups of 4 with padding rows; H and F not whole K-blocks (bounds-checked loads)
    FfnConfig("e1", 3, 512, 320, "bf16"),
    FfnConfig("e2", 5, 2112, 4160, "bf16"),
    FfnConfig("e3", 2, 1024, 2112, "f32"),
    # smallest widths; one panel of the down projection
    FfnConfig("e4", 1, 64, 64, "f32"),
    # the largest intermediate size (its fp32 row fills the 64 KB of LDS)
    FfnConfig("e5", 2, 256, 16384, "bf16"),
    # a batch of 9: three groups, the last with one sequence
    FfnConfig("e6", 9, 4096, 1088, "bf16"),
    # H of whole K-blocks with a ragged F
    FfnConfig("e7", 1, 4096, 11008 + 64, "bf16"),
    # MFMA panels (bf16, batch >= 8, H and F multiples of 256): one group of 8; two groups, the second
    # with one sequence; the down projection with two tiles (H / 32 panels >= 192) and with one
    FfnConfig("m1", 8, 2048, 5120, "bf16"),
    FfnConfig("m2", 17, 1024, 1280, "bf16"),
    FfnConfig("m3", 12, 8192, 2816, "bf16"),
    # the streamed panels: gate/up over H of 1024 and 2048, down over F of 14336 (one tile, 14 windows a
    # wave) and 8192 with 32 sequences a workgroup (a batch of 20: 12 padding rows)
    FfnConfig("s1", 8, 1024, 14336, "bf16"),
    FfnConfig("s2", 20, 2048, 8192, "bf16"),
]


@pytest.mark.parametrize("cfg", EDGE, ids=[c.name for c in EDGE])
def test_ffn_edge_parity(cfg):
    ffn_case(cfg, 3)


def test_ffn_batch_zero_touches_nothing():
    import torch
    import attention_block_amd as ab
    cfg = FfnConfig("z", 0, 256, 512, "bf16")
    inp = make_ffn_inputs(FfnConfig("z1", 1, 256, 512, "bf16"), 0)
    dev = ffn_to_device(inp)
    hidden = dev["hidden"][:0]
    out = torch.full((0, 256), 7.0, dtype=torch.bfloat16, device="cuda")
    ab.decode_ffn_block(hidden, dev["norm_w"], dev["w_gate"], dev["w_up"], dev["w_down"], cfg.eps, out=out, weight_layout="out_in")
    torch.cuda.synchronize()
    assert out.shape == (0, 256)


def test_ffn_is_deterministic_and_rows_are_independent():
    """Two calls give identical bits, and a sequence gets the same bits alone as in a batch of 6
    (its batch group changes, the arithmetic order does not)."""
    import torch
    cfg = FfnConfig("det", 6, 1024, 1536, "bf16")
    inp = make_ffn_inputs(cfg, 5)
    dev = ffn_to_device(inp)
    out1, _ = run_ffn(dev, cfg)
    bits1 = storage_bits(out1.clone())
    out2, _ = run_ffn(dev, cfg)
    assert np.array_equal(storage_bits(out2), bits1)
    for b in (0, 4, 5):
        one = dict(dev, hidden=dev["hidden"][b:b + 1].contiguous())
        o, _ = run_ffn(one, FfnConfig("det1", 1, 1024, 1536, "bf16"))
        assert np.array_equal(storage_bits(o)[0], bits1[b]), b
    torch.cuda.synchronize()


def test_ffn_graph_replay_matches_eager():
    import torch
    import attention_block_amd as ab
    cfg = FfnConfig("graph", 2, 4096, 11008, "bf16")
    inp = make_ffn_inputs(cfg, 9)
    dev = ffn_to_device(inp)
    eager, _ = run_ffn(dev, cfg)
    eager_bits = storage_bits(eager)
    out = torch.empty_like(dev["hidden"])
    ws = ab.Workspace(ab.ffn_workspace_size(ab.DabFfnConfig(2, 4096, 11008, ab.DAB_BF16, cfg.eps)), out.device)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        ab.decode_ffn_block(dev["hidden"], dev["norm_w"], dev["w_gate"], dev["w_up"], dev["w_down"], cfg.eps,
                            out=out, workspace=ws, weight_layout="out_in")
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ab.decode_ffn_block(dev["hidden"], dev["norm_w"], dev["w_gate"], dev["w_up"], dev["w_down"], cfg.eps,
                            out=out, workspace=ws, weight_layout="out_in")
    for rep in range(3):
        out.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(storage_bits(out), eager_bits), rep
