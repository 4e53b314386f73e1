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

    # the generator (and the oracle) hold the weights in the pages' [in, out]
    # layout; the library's pack kernel turns them into its own [out, in]
    import attention_block_amd as ab
    return dict(hidden=t(inp["hidden"]), norm_w=t(inp["norm_w"]), w_qkv=ab.pack_weight(t(inp["w_qkv"])),
                w_o=ab.pack_weight(t(inp["w_o"])), k_cache=t(inp["k_cache"]), v_cache=t(inp["v_cache"]),
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


def dab_config_for(dev: dict, cfg: BlockConfig, kv_chunk=0, schedule="auto"):
    """The C config a call on these device tensors builds (the binding derives it from the shapes)."""
    import attention_block_amd as ab
    B, cap, nkv, D = dev["k_cache"].shape
    return ab.make_config(batch=B, hidden=dev["hidden"].shape[1], n_q_heads=cfg.n_q_heads, n_kv_heads=nkv,
                          head_dim=D, cache_capacity=cap, dtype=cfg.dtype, rope_theta=cfg.rope_theta, eps=cfg.eps,
                          kv_chunk=kv_chunk, schedule=schedule)


def run_gpu(dev: dict, cfg: BlockConfig, kv_chunk=0, workspace=None, schedule="auto", want_a=False):
    """One call through the C ABI; returns (out, y tap) or, with want_a, (out, y tap, attention output a)."""
    import torch
    import attention_block_amd as ab
    dbg = torch.empty(dev["hidden"].shape, dtype=torch.float32, device=dev["hidden"].device)
    c = dab_config_for(dev, cfg, kv_chunk, schedule)
    ws = workspace if workspace is not None else ab.workspace_of(c, dev["hidden"].device)
    out = ab.decode_attn_block(dev["hidden"], dev["norm_w"], dev["w_qkv"], dev["w_o"], dev["k_cache"],
                               dev["v_cache"], dev["pos"], cfg.rope_theta, cfg.eps, dbg_y=dbg,
                               kv_chunk=kv_chunk, workspace=ws, schedule=schedule, weight_layout="out_in")
    a = ab.attention_output(c, ws) if want_a else None
    torch.cuda.synchronize()
    return (out, dbg, a) if want_a else (out, dbg)


def rel_rows(got, ref) -> np.ndarray:
    """Relative L2 of every row (last axis) of got against ref."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return np.linalg.norm(got - ref, axis=-1) / np.maximum(np.linalg.norm(ref, axis=-1), 1e-300)


def compare(inp: dict, ref: dict, dev: dict, out, dbg, cache_bits_before, a=None):
    """Every gate of the parity check; returns a dict of measured errors.

    out, y and the appended K and V rows are gated per sequence (the worst
    sequence's relative L2), the attention output a (when given) per
    sequence and query head; the whole-tensor figures are kept for the
    record.  cache_bits_before: (k_bits, v_bits) raw bits of both caches
    before the call.
    """
    cfg = inp["cfg"]
    pos = inp["pos"]
    B = len(pos)
    got_out, got_y = storage_values(out), dbg.cpu().numpy()
    errs = {
        "out": float(rel_rows(got_out, ref["out"]).max()) if B else 0.0,
        "y": float(rel_rows(got_y, ref["y"]).max()) if B else 0.0,
        "out_all": rel_l2(got_out, ref["out"]),
        "y_all": rel_l2(got_y, ref["y"]),
    }
    kb_after, vb_after = storage_bits(dev["k_cache"]), storage_bits(dev["v_cache"])
    kb0, vb0 = cache_bits_before
    kvals = storage_values(dev["k_cache"])
    vvals = storage_values(dev["v_cache"])
    krows = np.stack([kvals[b, pos[b]] for b in range(B)]).reshape(B, -1)
    vrows = np.stack([vvals[b, pos[b]] for b in range(B)]).reshape(B, -1)
    errs["k_row"] = float(rel_rows(krows, ref["k_row"].reshape(B, -1)).max())
    errs["v_row"] = float(rel_rows(vrows, ref["v_row"].reshape(B, -1)).max())
    if a is not None:
        D = cfg.head_dim
        got_a = a.cpu().numpy().reshape(B, cfg.n_q_heads, D)
        errs["a"] = float(rel_rows(got_a, ref["a"].reshape(B, cfg.n_q_heads, D)).max())
    # bit-exact append indices: exactly rows (b, pos_b) may differ
    mask = np.ones(kb0.shape[:2], dtype=bool)
    mask[np.arange(B), pos] = False
    errs["cache_untouched"] = bool(np.array_equal(kb_after[mask], kb0[mask]) and
                                   np.array_equal(vb_after[mask], vb0[mask]))
    errs["finite"] = bool(np.all(np.isfinite(got_out)) and np.all(np.isfinite(got_y)) and
                          (a is None or bool(np.all(np.isfinite(a.cpu().numpy())))))
    return errs


# measured errors of every parity case of the session, for the record (see conftest.py)
RECORD = []


def check_errs(errs: dict, dtype: str, label: str = ""):
    RECORD.append((label, dtype, dict(errs)))
    tol = tol_for(dtype)
    assert errs["finite"], f"{label}: non-finite output"
    assert errs["cache_untouched"], f"{label}: cache changed outside the appended rows"
    for k in ("out", "y", "k_row", "v_row", "a"):
        if k in errs:
            assert errs[k] <= tol, f"{label}: rel-L2({k}) = {errs[k]:.3e} > {tol:.0e}"


def small_cfg(name, B, H, nq, nkv, D, dtype, theta=1e4, ragged=None, pos=None):
    return BlockConfig(name, B, H, nq, nkv, D, dtype, theta, pos=pos, ragged=ragged)


__all__ = ["tol_for", "rel_l2", "rel_rows", "to_device", "storage_bits", "storage_values", "run_gpu", "compare",
           "check_errs", "small_cfg", "make_inputs", "dab_config_for", "RECORD"]
