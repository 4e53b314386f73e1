"""The weight-layout conversion on the GPU (dab_pack_weight) and the pages'
[in, out] layout at the Python boundary.

pack_weight must copy every bit to its transposed place, for shapes that
are not whole 64 x 64 tiles too; a call that names weight_layout="in_out"
and hands over the oracle's [in, out] matrices must give the same bits as a
call on weights packed once beforehand."""
import sys

import numpy as np
import pytest

from attention_block_amd.inputs import FFN_CONFIGS, make_ffn_inputs, make_inputs
from gpu_util import run_gpu, small_cfg, storage_bits, to_device

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", [(4096, 12288), (4096, 4096), (333, 70), (1, 1), (64, 65), (130, 1)])
def test_pack_weight_is_a_bit_exact_transpose(dtype, shape):
    import torch
    import attention_block_amd as ab
    say(f"[pack] {dtype} {shape}")
    g = torch.Generator(device="cuda").manual_seed(3)
    w = torch.randn(*shape, generator=g, device="cuda", dtype=torch.float32)
    w[0, 0] = float("nan")
    w = w.to(torch.bfloat16 if dtype == "bf16" else torch.float32)
    out = ab.pack_weight(w)
    torch.cuda.synchronize()
    bits = torch.int16 if dtype == "bf16" else torch.int32
    assert out.shape == (shape[1], shape[0])
    assert torch.equal(out.view(bits), w.t().contiguous().view(bits))


@pytest.mark.parametrize("schedule", ["phased", "attn_oproj"])
def test_in_out_layout_gives_the_packed_bits(schedule):
    import torch
    import attention_block_amd as ab
    cfg = small_cfg("lay", 2, 4096, 32, 32, 128, "bf16")
    inp = make_inputs(cfg, 4, cap=300, pos=[299, 77])
    say(f"[layout] in_out vs packed, {schedule}")
    dev = to_device(inp)
    out_packed, y_packed = run_gpu(dev, cfg, schedule=schedule)
    out_packed, y_packed = out_packed.clone(), y_packed.clone()

    def t(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()

    dev2 = to_device(inp)
    y = torch.empty_like(y_packed)
    out = ab.decode_attn_block(dev2["hidden"], dev2["norm_w"], t(inp["w_qkv"]), t(inp["w_o"]), dev2["k_cache"],
                               dev2["v_cache"], dev2["pos"], cfg.rope_theta, cfg.eps, dbg_y=y, schedule=schedule,
                               weight_layout="in_out")
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out_packed.view(torch.int16))
    assert torch.equal(y, y_packed)
    assert np.array_equal(storage_bits(dev2["k_cache"]), storage_bits(dev["k_cache"]))
    # a square W_o in the wrong layout is not caught by its shape: the layout argument is what decides
    with pytest.raises(ValueError):
        ab.decode_attn_block(dev2["hidden"], dev2["norm_w"], dev2["w_qkv"], dev2["w_o"], dev2["k_cache"],
                             dev2["v_cache"], dev2["pos"], cfg.rope_theta, cfg.eps, weight_layout="in-out")


def test_ffn_in_out_layout_gives_the_packed_bits():
    import torch
    import attention_block_amd as ab
    from test_gpu_ffn import ffn_to_device, run_ffn
    cfg = FFN_CONFIGS["tiny_ffn_f32"]
    inp = make_ffn_inputs(cfg, 2)
    say("[layout] ffn in_out vs packed")
    dev = ffn_to_device(inp)
    out_p, y_p = run_ffn(dev, cfg)
    f = {k: torch.from_numpy(np.ascontiguousarray(inp[k], dtype=np.float32)).cuda()
         for k in ("w_gate", "w_up", "w_down")}
    y = torch.empty_like(y_p)
    out = ab.decode_ffn_block(dev["hidden"], dev["norm_w"], f["w_gate"], f["w_up"], f["w_down"], cfg.eps, dbg_y=y,
                              weight_layout="in_out")
    torch.cuda.synchronize()
    assert torch.equal(out, out_p) and torch.equal(y, y_p)
