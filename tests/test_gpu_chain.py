"""A chain of decoder layers (attention block, then its FFN, per layer) through the C ABI, against the
oracles composed layer by layer.  Each layer has its own weights and caches; layer l's output, stored in
the storage dtype, is layer l + 1's input on both sides."""
import sys

import numpy as np
import pytest

import oracle
from attention_block_amd.inputs import layer_ffn, make_ffn_inputs, make_inputs
from gpu_util import RECORD, rel_l2, small_cfg, storage_values, to_device, tol_for
from test_gpu_ffn import ffn_to_device

pytestmark = pytest.mark.gpu

CHAINS = [
    ("bf16 gqa, 3 layers", small_cfg("c1", 2, 512, 8, 2, 64, "bf16", 5e5), [37, 100], 3),
    ("f32 mha, 2 layers", small_cfg("c2", 1, 256, 4, 4, 64, "f32"), [50], 2),
]


@pytest.mark.parametrize("label,cfg,pos,n_layers", CHAINS, ids=[c[0] for c in CHAINS])
def test_layer_chain_parity(label, cfg, pos, n_layers):
    import torch
    import attention_block_amd as ab
    print(f"[chain] {label}", flush=True)
    sys.stdout.flush()
    fcfg = layer_ffn(cfg)
    ref_x = None
    gpu_x = None
    for layer in range(n_layers):
        inp = make_inputs(cfg, 10 + layer, pos=pos, cap=max(pos) + 3)
        finp = make_ffn_inputs(fcfg, 50 + layer)
        if ref_x is not None:
            inp["hidden"] = ref_x
        # oracle: attention block, its output in storage precision, then the FFN
        ref_a = oracle.decode_step_from_inputs(inp)
        finp["hidden"] = to_storage(ref_a["out_stored"], cfg.dtype)
        ref_f = oracle.ffn_step_from_inputs(finp)
        ref_x = to_storage(ref_f["out_stored"], cfg.dtype)
        # GPU: the same weights and caches; the input is the previous layer's GPU output
        dev = to_device(inp)
        fdev = ffn_to_device(finp)
        x = dev["hidden"] if gpu_x is None else gpu_x
        h = ab.decode_attn_block(x, dev["norm_w"], dev["w_qkv"], dev["w_o"], dev["k_cache"], dev["v_cache"],
                                 dev["pos"], cfg.rope_theta, cfg.eps, weight_layout="out_in")
        gpu_x = ab.decode_ffn_block(h, fdev["norm_w"], fdev["w_gate"], fdev["w_up"], fdev["w_down"], fcfg.eps,
                                    weight_layout="out_in")
        torch.cuda.synchronize()
        err = rel_l2(storage_values(gpu_x), ref_f["out"])
        print(f"[chain] {label}: layer {layer}: rel-L2(out) = {err:.2e}", flush=True)
        if layer == n_layers - 1:
            RECORD.append((f"chain {cfg.name}, layer {layer}", cfg.dtype, {"out": err, "out_all": err}))
        assert np.all(np.isfinite(storage_values(gpu_x)))
        assert err <= tol_for(cfg.dtype), (layer, err)


def to_storage(values, dtype):
    """fp64 values already representable in the storage dtype -> the generator's storage form."""
    from attention_block_amd.inputs import f32_to_bf16_bits
    v32 = np.asarray(values, dtype=np.float32)
    return f32_to_bf16_bits(v32) if dtype == "bf16" else v32
