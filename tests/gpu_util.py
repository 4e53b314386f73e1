"""Helpers shared by the GPU tests: move seeded inputs to the device, run the
HIP path, and compare with the oracle."""
import numpy as np

from attention_block_amd.inputs import BlockConfig, make_inputs


def tol_for(dtype: str) -> float:
    # relative-L2 gates: bf16 storage with fp32 accumulation, or fp32 throughout
    return 1e-2 if dtype == "bf16" else 1e-5


def rel_l2(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


def to_device(inp: dict, device="cuda"):
    import torch
    cfg = inp["cfg"]

    def t(a):
        if cfg.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)

    # the library takes weights one output feature per row: the transpose
    # of the [in, out] matrices the generator (and the oracle) use
    return dict(hidden=t(inp["hidden"]), norm_w=t(inp["norm_w"]), w_qkv=t(inp["w_qkv"].T), w_o=t(inp["w_o"].T),
                k_cache=t(inp["k_cache"]), v_cache=t(inp["v_cache"]),
                pos=torch.from_numpy(inp["pos"].astype(np.int32)).to(device))


def storage_bits(t):
    """Raw bits of a device tensor as a host numpy array (uint16 or uint32)."""
    import torch
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.view(torch.int32).cpu().numpy().view(np.uint32)


def storage_values(t):
    import torch
    return t.float().cpu().numpy().astype(np.float64) if t.dtype == torch.bfloat16 else \
        t.cpu().numpy().astype(np.float64)


def run_gpu(dev: dict, cfg: BlockConfig, kv_chunk=0, workspace=None, schedule="auto"):
    import torch
    import attention_block_amd as ab
    dbg = torch.empty(dev["hidden"].shape, dtype=torch.float32, device=dev["hidden"].device)
    out = ab.decode_attn_block(dev["hidden"], dev["norm_w"], dev["w_qkv"], dev["w_o"], dev["k_cache"],
                               dev["v_cache"], dev["pos"], cfg.rope_theta, cfg.eps, dbg_y=dbg,
                               kv_chunk=kv_chunk, workspace=workspace, schedule=schedule)
    torch.cuda.synchronize()
    return out, dbg


def compare(inp: dict, ref: dict, dev: dict, out, dbg, cache_bits_before):
    """Every gate of the parity check; returns a dict of measured errors.

    cache_bits_before: (k_bits, v_bits) raw bits of both caches before the call.
    """
    cfg = inp["cfg"]
    pos = inp["pos"]
    B = len(pos)
    errs = {
        "out": rel_l2(storage_values(out), ref["out"]),
        "y": rel_l2(dbg.cpu().numpy(), ref["y"]),
    }
    kb_after, vb_after = storage_bits(dev["k_cache"]), storage_bits(dev["v_cache"])
    kb0, vb0 = cache_bits_before
    kvals = storage_values(dev["k_cache"])
    vvals = storage_values(dev["v_cache"])
    errs["k_row"] = rel_l2(np.stack([kvals[b, pos[b]] for b in range(B)]), ref["k_row"])
    errs["v_row"] = rel_l2(np.stack([vvals[b, pos[b]] for b in range(B)]), ref["v_row"])
    # bit-exact append indices: exactly rows (b, pos_b) may differ
    mask = np.ones(kb0.shape[:2], dtype=bool)
    mask[np.arange(B), pos] = False
    errs["cache_untouched"] = bool(np.array_equal(kb_after[mask], kb0[mask]) and
                                   np.array_equal(vb_after[mask], vb0[mask]))
    errs["finite"] = bool(np.all(np.isfinite(storage_values(out))) and np.all(np.isfinite(dbg.cpu().numpy())))
    return errs


def check_errs(errs: dict, dtype: str, label: str = ""):
    tol = tol_for(dtype)
    assert errs["finite"], f"{label}: non-finite output"
    assert errs["cache_untouched"], f"{label}: cache changed outside the appended rows"
    for k in ("out", "y", "k_row", "v_row"):
        assert errs[k] <= tol, f"{label}: rel-L2({k}) = {errs[k]:.3e} > {tol:.0e}"


def small_cfg(name, B, H, nq, nkv, D, dtype, theta=1e4, ragged=None, pos=None):
    return BlockConfig(name, B, H, nq, nkv, D, dtype, theta, pos=pos, ragged=ragged)


__all__ = ["tol_for", "rel_l2", "to_device", "storage_bits", "storage_values", "run_gpu", "compare",
           "check_errs", "small_cfg", "make_inputs"]
