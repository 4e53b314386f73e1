"""attention_block_amd: the fused single-token decode attention block on MI355X.

The compute lives in libdab.so (hand-written HIP kernels for gfx950 behind
the C ABI of include/dab.h).  This module only marshals torch tensors into
that ABI: torch provides device memory and the current stream, nothing
else.  There is no CPU or torch fallback: without the built library every
call raises.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence

from . import _lib
from ._lib import DAB_BF16, DAB_F32, FFN_PHASES, MLA_PHASES, READ_PROBE_BLOCKS, DabConfig, DabFfnConfig, DabMlaConfig

__all__ = ["DabError", "DabConfig", "make_config", "workspace_size", "Workspace", "decode_attn_block",
           "decode_attn_block_timed", "read_device_error", "phase_names", "HipEvent", "lib_version",
           "DabFfnConfig", "FFN_PHASES", "ffn_workspace_size", "decode_ffn_block", "decode_ffn_block_timed",
           "decode_layer", "layer_overlapped",
           "read_probe", "READ_PROBE_BLOCKS", "pack_weight", "attention_output", "WEIGHT_LAYOUTS",
           "decode_attn_block_noalloc", "DabMlaConfig", "MLA_PHASES", "mla_workspace_size",
           "mla_decode_attn", "mla_decode_attn_timed"]

# Weight layouts a call may name: "out_in" is the library's own ([out_features, in_features], one
# output feature per row, as torch.nn.Linear stores its weight); "in_out" is the pages' ([in, out],
# y = x @ W), converted by the library's pack kernel into temporaries on every call.  The layout is a
# required argument because a square matrix (W_o of an MHA layer with nq * D == H) has the same shape
# in both.
WEIGHT_LAYOUTS = ("out_in", "in_out")


class DabError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        lib = _lib.load()
        msg = lib.dab_status_string(status).decode()
        if status == _lib.DAB_ERR_HIP:
            msg += f" [{lib.dab_last_hip_error().decode()}]"
        super().__init__(f"{where}: {msg} (status {status})")


def _check(status: int, where: str) -> None:
    if status != _lib.DAB_OK:
        raise DabError(status, where)


def lib_version() -> str:
    return _lib.load().dab_version().decode()


def make_config(*, batch: int, hidden: int, n_q_heads: int, n_kv_heads: int, head_dim: int,
                cache_capacity: int, dtype: str, rope_theta: float, eps: float = 1e-6,
                kv_chunk: int = 0, schedule: str = "auto", max_position: int = 0) -> DabConfig:
    """Build the C config struct.  dtype is "bf16" or "f32"; schedule one of _lib.SCHEDULES;
    max_position the largest position a call's sequences hold (0: not given)."""
    if dtype not in ("bf16", "f32"):
        raise ValueError(f"dtype must be 'bf16' or 'f32', not {dtype!r}")
    if schedule not in _lib.SCHEDULES:
        raise ValueError(f"schedule must be one of {sorted(_lib.SCHEDULES)}")
    return DabConfig(batch, hidden, n_q_heads, n_kv_heads, head_dim, cache_capacity,
                     DAB_BF16 if dtype == "bf16" else DAB_F32, rope_theta, eps, kv_chunk,
                     _lib.SCHEDULES[schedule], max_position)


def workspace_size(cfg: DabConfig) -> int:
    n = _lib.load().dab_workspace_size(ctypes.byref(cfg))
    if n == 0:
        raise DabError(_lib.DAB_ERR_INVALID_ARG, "dab_workspace_size")
    return n


def phase_names(cfg: DabConfig) -> list:
    lib = _lib.load()
    return [lib.dab_phase_name(ctypes.byref(cfg), i).decode() for i in range(lib.dab_phase_count(ctypes.byref(cfg)))]


class Workspace:
    """Device scratch for the library (partials, counters, error flag).

    Allocated once with torch and zeroed once by dab_workspace_init.  Every
    call re-arms the counters it uses, so one workspace serves any number of
    calls with ONE configuration on one stream at a time.  Where the
    counters sit depends on the configuration: a workspace used with another
    configuration must be zeroed again first (reset()).
    """

    def __init__(self, nbytes: int, device):
        import torch
        self.nbytes = int(nbytes)
        self._buf = torch.empty(self.nbytes + 256, dtype=torch.uint8, device=device)
        base = self._buf.data_ptr()
        self.ptr = (base + 255) // 256 * 256
        self.device = self._buf.device
        self.reset()

    def reset(self) -> None:
        """Zero the workspace (on the current stream), as before its first call."""
        _check(_lib.load().dab_workspace_init(ctypes.c_void_p(self.ptr), self.nbytes, _stream_ptr(self.device)),
               "dab_workspace_init")


# Default workspaces, one per device and configuration (the counters of a
# workspace sit where its configuration puts them); the most recent few are kept.
_default_ws = {}
_DEFAULT_WS_KEEP = 8


def _config_key(cfg: DabConfig) -> tuple:
    return tuple(getattr(cfg, name) for name, _ in DabConfig._fields_)


def _workspace_for(cfg: DabConfig, device) -> Workspace:
    key = (device.type, device.index, _config_key(cfg))
    ws = _default_ws.pop(key, None)
    if ws is None:
        ws = Workspace(workspace_size(cfg), device)
        while len(_default_ws) >= _DEFAULT_WS_KEEP:
            _default_ws.pop(next(iter(_default_ws)))
    _default_ws[key] = ws          # most recently used last
    return ws


def _stream_ptr(device) -> ctypes.c_void_p:
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t) -> ctypes.c_void_p:
    return ctypes.c_void_p(t.data_ptr() if t is not None else 0)


def pack_weight(w, out=None):
    """[in_features, out_features] -> [out_features, in_features] on the device (dab_pack_weight).

    w: a contiguous 2-D bfloat16 or float32 GPU tensor in the pages' layout (y = x @ w).  Returns (or
    fills `out`, contiguous, same dtype and device) the library's layout, bit for bit; asynchronous on
    the current stream.  Pack static weights once at load time."""
    import torch
    if w.dim() != 2 or not w.is_cuda or not w.is_contiguous() or w.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("pack_weight: a contiguous 2-D bfloat16 or float32 GPU tensor is required")
    n_in, n_out = w.shape
    if out is None:
        out = torch.empty((n_out, n_in), dtype=w.dtype, device=w.device)
    elif out.shape != (n_out, n_in) or out.dtype != w.dtype or out.device != w.device or not out.is_contiguous():
        raise ValueError(f"pack_weight: out must be a contiguous [{n_out}, {n_in}] {w.dtype} tensor on {w.device}")
    _check(_lib.load().dab_pack_weight(_ptr(w), _ptr(out), n_in, n_out,
                                       DAB_BF16 if w.dtype == torch.bfloat16 else DAB_F32, _stream_ptr(w.device)),
           "dab_pack_weight")
    return out


def _layout(weight_layout: str) -> None:
    if weight_layout not in WEIGHT_LAYOUTS:
        raise ValueError(f"weight_layout must be one of {WEIGHT_LAYOUTS}, not {weight_layout!r}")


def _prepare(hidden, norm_w, w_qkv, w_o, k_cache, v_cache, pos, rope_theta, eps, out, dbg_y, kv_chunk,
             schedule, weight_layout, max_position=0):
    import torch
    _layout(weight_layout)
    if hidden.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("hidden must be bfloat16 or float32")
    dt = hidden.dtype
    dev = hidden.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU device")
    named = dict(hidden=hidden, norm_w=norm_w, w_qkv=w_qkv, w_o=w_o, k_cache=k_cache, v_cache=v_cache)
    for name, t in named.items():
        if t.dtype != dt or t.device != dev or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {dt} tensor on {dev}")
    if pos.dtype != torch.int32 or pos.device != dev or not pos.is_contiguous():
        raise ValueError(f"pos must be a contiguous int32 tensor on {dev}")
    if hidden.dim() != 2 or k_cache.dim() != 4 or k_cache.shape != v_cache.shape:
        raise ValueError("hidden must be [B, H]; k_cache and v_cache [B, cap, nkv, D] of one shape")
    B, H = hidden.shape
    _, cap, nkv, D = k_cache.shape
    if k_cache.shape[0] != B or pos.shape != (B,) or norm_w.shape != (H,):
        raise ValueError("batch or hidden size mismatch")
    if w_qkv.dim() != 2 or w_o.dim() != 2:
        raise ValueError("w_qkv and w_o must be 2-D")
    if weight_layout == "in_out":
        n_qkv = w_qkv.shape[1]
        if w_qkv.shape[0] != H or n_qkv % D or n_qkv // D <= 2 * nkv:
            raise ValueError("w_qkv must be [H, (nq + 2 nkv) D] (weight_layout='in_out')")
        nq = n_qkv // D - 2 * nkv
        if w_o.shape != (nq * D, H):
            raise ValueError(f"w_o must be [{nq * D}, {H}] (weight_layout='in_out')")
        w_qkv, w_o = pack_weight(w_qkv), pack_weight(w_o)
    n_qkv = w_qkv.shape[0]
    if w_qkv.shape[1] != H or n_qkv % D or n_qkv // D <= 2 * nkv:
        raise ValueError("w_qkv must be [(nq + 2 nkv) D, H] (one output feature per row)")
    nq = n_qkv // D - 2 * nkv
    if w_o.shape != (H, nq * D):
        raise ValueError(f"w_o must be [{H}, {nq * D}] (one output feature per row)")
    if out is None:
        out = torch.empty_like(hidden)
    elif out.shape != hidden.shape or out.dtype != dt or out.device != dev or not out.is_contiguous():
        raise ValueError("out must match hidden")
    if dbg_y is not None and (dbg_y.shape != hidden.shape or dbg_y.dtype != torch.float32
                              or dbg_y.device != dev or not dbg_y.is_contiguous()):
        raise ValueError("dbg_y must be a contiguous float32 [B, H] tensor")
    cfg = make_config(batch=B, hidden=H, n_q_heads=nq, n_kv_heads=nkv, head_dim=D, cache_capacity=cap,
                      dtype="bf16" if dt == torch.bfloat16 else "f32", rope_theta=rope_theta, eps=eps,
                      kv_chunk=kv_chunk, schedule=schedule, max_position=max_position)
    return cfg, out, w_qkv, w_o


def decode_attn_block(hidden, norm_w, w_qkv, w_o, k_cache, v_cache, pos, rope_theta: float, eps: float = 1e-6,
                      out=None, dbg_y=None, workspace: Optional[Workspace] = None, kv_chunk: int = 0,
                      schedule: str = "auto", *, weight_layout: str, max_position: int = 0):
    """One decode step on the current stream; returns `out`.

    Shapes: hidden [B, H]; norm_w [H]; k_cache, v_cache [B, cap, nkv, D] (row
    pos[b] is written); pos int32 [B]; all but pos in one dtype (bfloat16 or
    float32) on one GPU.  weight_layout (required) names the layout of w_qkv
    and w_o: "out_in", the library's (w_qkv [(nq+2nkv)D, H], w_o [H, nq D],
    one output feature per row, as torch.nn.Linear stores its weight), or
    "in_out", the pages' (w_qkv [H, (nq+2nkv)D], w_o [nq D, H]), packed by the
    library's kernel into temporaries on every call (pack once with
    pack_weight for repeated calls).  dbg_y (optional, float32 [B, H])
    receives the pre-residual attention-output projection.
    schedule: "phased" (one kernel per phase), "attn_oproj" (attention and
    the output projection in one launch), "qkv_attn" (QKV and attention in
    one launch) or "auto" (the fastest that applies).  max_position (optional): the largest
    position in pos, so that the work is sized for the tokens in use rather than the capacity; a
    sequence beyond it is rejected on the device (the error flag) like one past the capacity.
    """
    cfg, out, w_qkv, w_o = _prepare(hidden, norm_w, w_qkv, w_o, k_cache, v_cache, pos, rope_theta, eps, out, dbg_y,
                                    kv_chunk, schedule, weight_layout, max_position)
    ws = workspace if workspace is not None else _workspace_for(cfg, hidden.device)
    _check(_lib.load().dab_decode_attn_block(
        ctypes.byref(cfg), _ptr(hidden), _ptr(norm_w), _ptr(w_qkv), _ptr(w_o), _ptr(k_cache), _ptr(v_cache),
        _ptr(pos), _ptr(out), _ptr(dbg_y), ctypes.c_void_p(ws.ptr), ws.nbytes, _stream_ptr(hidden.device)),
        "dab_decode_attn_block")
    return out


def attention_output(cfg: DabConfig, workspace: Workspace, out=None):
    """The attention output a [B, nq * D] (float32, head-major) that the last call with configuration `cfg`
    left in `workspace` (dab_attention_output): a test tap, copied on the current stream."""
    import torch
    n = cfg.batch * cfg.n_q_heads * cfg.head_dim
    if out is None:
        out = torch.empty((cfg.batch, cfg.n_q_heads * cfg.head_dim), dtype=torch.float32, device=workspace.device)
    elif out.numel() != n or out.dtype != torch.float32 or not out.is_contiguous():
        raise ValueError("attention_output: out must be a contiguous float32 tensor of B * nq * D elements")
    _check(_lib.load().dab_attention_output(ctypes.byref(cfg), ctypes.c_void_p(workspace.ptr), workspace.nbytes,
                                            _ptr(out), _stream_ptr(workspace.device)), "dab_attention_output")
    return out


def workspace_of(cfg: DabConfig, device) -> Workspace:
    """The default workspace calls without a `workspace` argument use for this configuration and device."""
    return _workspace_for(cfg, device)


def decode_attn_block_noalloc(hidden, norm_w, w_qkv, w_o, k_cache, v_cache, pos, rope_theta: float,
                              eps: float = 1e-6, out=None, dbg_y=None, kv_chunk: int = 0, schedule: str = "auto",
                              max_position: int = 0):
    """decode_attn_block through dab_decode_attn_block_noalloc: the library's own per-GPU scratch serves
    as the workspace, so the call allocates nothing on the device (give `out`, and the weights in the
    library's [out, in] layout, for a call that allocates nothing at all).  Calls that overlap in time
    on one GPU race on that scratch."""
    cfg, out, w_qkv, w_o = _prepare(hidden, norm_w, w_qkv, w_o, k_cache, v_cache, pos, rope_theta, eps, out, dbg_y,
                                    kv_chunk, schedule, "out_in", max_position)
    _check(_lib.load().dab_decode_attn_block_noalloc(
        ctypes.byref(cfg), _ptr(hidden), _ptr(norm_w), _ptr(w_qkv), _ptr(w_o), _ptr(k_cache), _ptr(v_cache),
        _ptr(pos), _ptr(out), _ptr(dbg_y), _stream_ptr(hidden.device)), "dab_decode_attn_block_noalloc")
    return out


class HipEvent:
    """A raw hipEvent_t (timing only), so phases can be timed on the stream they run on."""

    _hip = None

    @classmethod
    def _rt(cls):
        if cls._hip is None:
            import torch  # noqa: F401  (loads the HIP runtime torch links against)
            hip = ctypes.CDLL("libamdhip64.so")
            hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
            hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
            cls._hip = hip
        return cls._hip

    def __init__(self):
        h = ctypes.c_void_p()
        if self._rt().hipEventCreate(ctypes.byref(h)) != 0:
            raise RuntimeError("hipEventCreate failed")
        self.handle = h

    def record(self, stream_ptr) -> None:
        if self._rt().hipEventRecord(self.handle, stream_ptr) != 0:
            raise RuntimeError("hipEventRecord failed")

    def synchronize(self) -> None:
        self._rt().hipEventSynchronize(self.handle)

    def elapsed_ms(self, end: "HipEvent") -> float:
        ms = ctypes.c_float()
        if self._rt().hipEventElapsedTime(ctypes.byref(ms), self.handle, end.handle) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def __del__(self):
        try:
            if self._hip is not None and self.handle:
                self._hip.hipEventDestroy(self.handle)
        except Exception:
            pass


def decode_attn_block_timed(events: Sequence[HipEvent], hidden, norm_w, w_qkv, w_o, k_cache, v_cache, pos,
                            rope_theta: float, eps: float = 1e-6, out=None, dbg_y=None,
                            workspace: Optional[Workspace] = None, kv_chunk: int = 0, schedule: str = "auto", *,
                            weight_layout: str, max_position: int = 0):
    """decode_attn_block that also records events[2i], events[2i + 1] at the start and end of kernel i
    (2 * len(phase_names) events; taken by each kernel's own dispatch)."""
    cfg, out, w_qkv, w_o = _prepare(hidden, norm_w, w_qkv, w_o, k_cache, v_cache, pos, rope_theta, eps, out, dbg_y,
                                    kv_chunk, schedule, weight_layout, max_position)
    ws = workspace if workspace is not None else _workspace_for(cfg, hidden.device)
    arr = (ctypes.c_void_p * len(events))(*[e.handle.value for e in events])
    _check(_lib.load().dab_decode_attn_block_timed(
        ctypes.byref(cfg), _ptr(hidden), _ptr(norm_w), _ptr(w_qkv), _ptr(w_o), _ptr(k_cache), _ptr(v_cache),
        _ptr(pos), _ptr(out), _ptr(dbg_y), ctypes.c_void_p(ws.ptr), ws.nbytes, _stream_ptr(hidden.device),
        arr, len(events)), "dab_decode_attn_block_timed")
    return out


# ---------------------------------------------------------------------------
# the FFN half of the layer
# ---------------------------------------------------------------------------

def ffn_workspace_size(cfg: DabFfnConfig) -> int:
    n = _lib.load().dab_ffn_workspace_size(ctypes.byref(cfg))
    if n == 0:
        raise DabError(_lib.DAB_ERR_INVALID_ARG, "dab_ffn_workspace_size")
    return n


_ffn_ws = {}


def _prepare_ffn(hidden, norm_w, w_gate, w_up, w_down, eps, out, dbg_y, workspace, weight_layout):
    import torch
    _layout(weight_layout)
    if hidden.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("hidden must be bfloat16 or float32")
    dt, dev = hidden.dtype, hidden.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU device")
    for name, t in dict(hidden=hidden, norm_w=norm_w, w_gate=w_gate, w_up=w_up, w_down=w_down).items():
        if t.dtype != dt or t.device != dev or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {dt} tensor on {dev}")
    if hidden.dim() != 2 or w_gate.dim() != 2:
        raise ValueError("hidden must be [B, H] and w_gate [F, H]")
    B, H = hidden.shape
    if weight_layout == "in_out":
        F = w_gate.shape[1]
        if w_gate.shape != (H, F) or w_up.shape != (H, F) or w_down.shape != (F, H):
            raise ValueError("need w_gate and w_up [H, F], w_down [F, H] (weight_layout='in_out')")
        w_gate, w_up, w_down = pack_weight(w_gate), pack_weight(w_up), pack_weight(w_down)
    F = w_gate.shape[0]
    if norm_w.shape != (H,) or w_gate.shape != (F, H) or w_up.shape != (F, H) or w_down.shape != (H, F):
        raise ValueError("need norm_w [H], w_gate and w_up [F, H], w_down [H, F] (one output feature per row)")
    if out is None:
        out = torch.empty_like(hidden)
    elif out.shape != hidden.shape or out.dtype != dt or out.device != dev or not out.is_contiguous():
        raise ValueError("out must match hidden")
    if dbg_y is not None and (dbg_y.shape != hidden.shape or dbg_y.dtype != torch.float32
                              or dbg_y.device != dev or not dbg_y.is_contiguous()):
        raise ValueError("dbg_y must be a contiguous float32 [B, H] tensor")
    cfg = DabFfnConfig(B, H, F, DAB_BF16 if dt == torch.bfloat16 else DAB_F32, eps)
    if workspace is None:
        key = (dev.type, dev.index, B, F)
        workspace = _ffn_ws.get(key)
        if workspace is None:
            workspace = _ffn_ws[key] = Workspace(ffn_workspace_size(cfg), dev)
    return cfg, out, workspace, w_gate, w_up, w_down


def decode_ffn_block(hidden, norm_w, w_gate, w_up, w_down, eps: float = 1e-6, out=None, dbg_y=None,
                     workspace: Optional[Workspace] = None, *, weight_layout: str):
    """The FFN half of the layer on the current stream; returns `out` = h + silu(g) * u @ W_down^T.

    Shapes: hidden [B, H]; norm_w [H]; with weight_layout "out_in" w_gate and
    w_up [F, H], w_down [H, F] (one output feature per row), with "in_out" (the
    pages' layout, packed into temporaries on every call) w_gate and w_up
    [H, F], w_down [F, H]; one dtype (bfloat16 or float32) on one GPU.  dbg_y
    (optional, float32 [B, H]) receives the pre-residual projection.
    """
    cfg, out, ws, w_gate, w_up, w_down = _prepare_ffn(hidden, norm_w, w_gate, w_up, w_down, eps, out, dbg_y,
                                                      workspace, weight_layout)
    _check(_lib.load().dab_decode_ffn_block(
        ctypes.byref(cfg), _ptr(hidden), _ptr(norm_w), _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(out),
        _ptr(dbg_y), ctypes.c_void_p(ws.ptr), ws.nbytes, _stream_ptr(hidden.device)), "dab_decode_ffn_block")
    return out


def decode_ffn_block_timed(events: Sequence[HipEvent], hidden, norm_w, w_gate, w_up, w_down, eps: float = 1e-6,
                           out=None, dbg_y=None, workspace: Optional[Workspace] = None, *, weight_layout: str):
    """decode_ffn_block that records events[0..3] at the start and end of its two kernels."""
    cfg, out, ws, w_gate, w_up, w_down = _prepare_ffn(hidden, norm_w, w_gate, w_up, w_down, eps, out, dbg_y,
                                                      workspace, weight_layout)
    arr = (ctypes.c_void_p * len(events))(*[e.handle.value for e in events])
    _check(_lib.load().dab_decode_ffn_block_timed(
        ctypes.byref(cfg), _ptr(hidden), _ptr(norm_w), _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ptr(out),
        _ptr(dbg_y), ctypes.c_void_p(ws.ptr), ws.nbytes, _stream_ptr(hidden.device), arr, len(events)),
        "dab_decode_ffn_block_timed")
    return out


def layer_overlapped(cfg: DabConfig, ffn_cfg: DabFfnConfig) -> bool:
    """Whether decode_layer's "overlap" schedule is built for these configurations (dab_layer_overlapped)."""
    r = _lib.load().dab_layer_overlapped(ctypes.byref(cfg), ctypes.byref(ffn_cfg))
    if r < 0:
        raise DabError(_lib.DAB_ERR_INVALID_ARG, "dab_layer_overlapped")
    return r == 1


def decode_layer(hidden, attn_norm_w, w_qkv, w_o, k_cache, v_cache, pos, ffn_norm_w, w_gate, w_up, w_down,
                 rope_theta: float, eps: float = 1e-6, ffn_eps: Optional[float] = None, h=None, out=None,
                 workspace: Optional[Workspace] = None, ffn_workspace: Optional[Workspace] = None,
                 kv_chunk: int = 0, schedule: str = "auto", layer_schedule: str = "auto", *, weight_layout: str,
                 max_position: int = 0):
    """One decoder layer (dab_decode_layer): the attention block into `h`, its FFN into `out`; returns
    (h, out).  The arguments are those of decode_attn_block and decode_ffn_block (ffn_eps defaults to
    eps).  layer_schedule: "sequential" (the two blocks' kernels one after the other), "overlap" (the
    FFN's weight stream started under the attention block, where layer_overlapped(...) holds) or
    "auto" (sequential, the faster on MI355X).  Every schedule gives the bits of those two calls.  The
    FFN workspace is zeroed on allocation (Workspace), as "overlap" needs."""
    if layer_schedule not in _lib.LAYER_SCHEDULES:
        raise ValueError(f"layer_schedule must be one of {sorted(_lib.LAYER_SCHEDULES)}, not {layer_schedule!r}")
    h_cfg, h, w_qkv, w_o = _prepare(hidden, attn_norm_w, w_qkv, w_o, k_cache, v_cache, pos, rope_theta, eps, h,
                                    None, kv_chunk, schedule, weight_layout, max_position)
    f_cfg, out, fws, w_gate, w_up, w_down = _prepare_ffn(h, ffn_norm_w, w_gate, w_up, w_down,
                                                         eps if ffn_eps is None else ffn_eps, out, None,
                                                         ffn_workspace, weight_layout)
    ws = workspace if workspace is not None else _workspace_for(h_cfg, hidden.device)
    _check(_lib.load().dab_decode_layer(
        ctypes.byref(h_cfg), ctypes.byref(f_cfg), _ptr(hidden), _ptr(attn_norm_w), _ptr(w_qkv), _ptr(w_o),
        _ptr(k_cache), _ptr(v_cache), _ptr(pos), _ptr(ffn_norm_w), _ptr(w_gate), _ptr(w_up), _ptr(w_down),
        _ptr(h), _ptr(out), ctypes.c_void_p(ws.ptr), ws.nbytes, ctypes.c_void_p(fws.ptr), fws.nbytes,
        _lib.LAYER_SCHEDULES[layer_schedule], _stream_ptr(hidden.device)), "dab_decode_layer")
    return h, out


# latent attention (MLA) decode over a latent cache
# ---------------------------------------------------------------------------

def mla_workspace_size(cfg: DabMlaConfig) -> int:
    n = _lib.load().dab_mla_workspace_size(ctypes.byref(cfg))
    if n == 0:
        raise DabError(_lib.DAB_ERR_INVALID_ARG, "dab_mla_workspace_size")
    return n


_mla_ws = {}


def _prepare_mla(q_lat, q_rope, c_new, kr_new, c_cache, kr_cache, pos, softmax_scale, kv_chunk, out, workspace):
    import torch
    dev = q_lat.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU device")
    need = dict(q_lat=(q_lat, torch.float32), q_rope=(q_rope, torch.float32), c_new=(c_new, torch.bfloat16),
                kr_new=(kr_new, torch.bfloat16), c_cache=(c_cache, torch.bfloat16),
                kr_cache=(kr_cache, torch.bfloat16), pos=(pos, torch.int32))
    for name, (t, dt) in need.items():
        if t.dtype != dt or t.device != dev or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {dt} tensor on {dev}")
    if q_lat.dim() != 3 or c_cache.dim() != 3:
        raise ValueError("q_lat must be [B, nh, R] and c_cache [B, cap, R]")
    B, nh, R = q_lat.shape
    cap = c_cache.shape[1]
    P = q_rope.shape[-1]
    if (q_rope.shape != (B, nh, P) or c_new.shape != (B, R) or kr_new.shape != (B, P)
            or c_cache.shape != (B, cap, R) or kr_cache.shape != (B, cap, P) or pos.shape != (B,)):
        raise ValueError("need q_lat [B, nh, R], q_rope [B, nh, P], c_new [B, R], kr_new [B, P], "
                         "c_cache [B, cap, R], kr_cache [B, cap, P], pos [B]")
    if out is None:
        out = torch.empty((B, nh, R), dtype=torch.float32, device=dev)
    elif out.shape != (B, nh, R) or out.dtype != torch.float32 or out.device != dev or not out.is_contiguous():
        raise ValueError("out must be a contiguous float32 [B, nh, R] tensor")
    cfg = DabMlaConfig(B, nh, R, P, cap, softmax_scale, kv_chunk)
    if workspace is None:
        key = (dev.type, dev.index, B, nh, R, P, cap, kv_chunk)
        workspace = _mla_ws.get(key)
        if workspace is None:
            workspace = _mla_ws[key] = Workspace(mla_workspace_size(cfg), dev)
    return cfg, out, workspace


def mla_decode_attn(q_lat, q_rope, c_new, kr_new, c_cache, kr_cache, pos, softmax_scale: float, kv_chunk: int = 0,
                    out=None, workspace: Optional[Workspace] = None):
    """Latent attention decode on the current stream; returns `out` (float32 [B, nh, R]), the softmax-weighted
    latent rows of each head, and appends c_new / kr_new at row pos[b] of the caches.

    q_lat [B, nh, R] and q_rope [B, nh, P] float32; c_new [B, R], kr_new [B, P], c_cache [B, cap, R],
    kr_cache [B, cap, P] bfloat16; pos int32 [B]; R = 512, P = 64, nh a multiple of 16.
    """
    cfg, out, ws = _prepare_mla(q_lat, q_rope, c_new, kr_new, c_cache, kr_cache, pos, softmax_scale, kv_chunk,
                                out, workspace)
    _check(_lib.load().dab_mla_decode_attn(
        ctypes.byref(cfg), _ptr(q_lat), _ptr(q_rope), _ptr(c_new), _ptr(kr_new), _ptr(c_cache), _ptr(kr_cache),
        _ptr(pos), _ptr(out), ctypes.c_void_p(ws.ptr), ws.nbytes, _stream_ptr(q_lat.device)), "dab_mla_decode_attn")
    return out


def mla_decode_attn_timed(events: Sequence[HipEvent], q_lat, q_rope, c_new, kr_new, c_cache, kr_cache, pos,
                          softmax_scale: float, kv_chunk: int = 0, out=None, workspace: Optional[Workspace] = None):
    """mla_decode_attn that records events[0..3] at the start and end of its two kernels."""
    cfg, out, ws = _prepare_mla(q_lat, q_rope, c_new, kr_new, c_cache, kr_cache, pos, softmax_scale, kv_chunk,
                                out, workspace)
    arr = (ctypes.c_void_p * len(events))(*[e.handle.value for e in events])
    _check(_lib.load().dab_mla_decode_attn_timed(
        ctypes.byref(cfg), _ptr(q_lat), _ptr(q_rope), _ptr(c_new), _ptr(kr_new), _ptr(c_cache), _ptr(kr_cache),
        _ptr(pos), _ptr(out), ctypes.c_void_p(ws.ptr), ws.nbytes, _stream_ptr(q_lat.device), arr, len(events)),
        "dab_mla_decode_attn_timed")
    return out


def read_probe(buffer, out) -> None:
    """One plain stream over `buffer` (a contiguous device tensor, 16-byte aligned, a whole number of
    16-byte vectors) with the step's 16-byte non-temporal loads; `out` (a device tensor of at least
    READ_PROBE_BLOCKS 32-bit words) receives each workgroup's XOR of the words it read.  Asynchronous
    on the current stream: time it with events to get the HBM read bandwidth a plain stream attains."""
    import torch
    lib = _lib.load()
    if not (buffer.is_cuda and out.is_cuda and buffer.is_contiguous() and out.is_contiguous()):
        raise ValueError("read_probe: contiguous device tensors required")
    nbytes = buffer.numel() * buffer.element_size()
    st = lib.dab_read_probe(ctypes.c_void_p(buffer.data_ptr()), nbytes, ctypes.c_void_p(out.data_ptr()),
                            out.numel() * out.element_size(), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    _check(st, "dab_read_probe")


def read_device_error(workspace: Optional[Workspace] = None, device=None) -> int:
    """Read and clear the sticky device error flag (synchronises the stream).

    Without `workspace`: the flags of every default workspace of the device,
    OR-ed together (each is cleared)."""
    import torch
    if workspace is not None:
        spaces = [workspace]
    else:
        dev = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
        spaces = [ws for key, ws in _default_ws.items() if key[:2] == (dev.type, dev.index)]
    flags = 0
    for ws in spaces:
        flag = ctypes.c_int32()
        _check(_lib.load().dab_read_device_error(ctypes.c_void_p(ws.ptr), _stream_ptr(ws.device),
                                                 ctypes.byref(flag)), "dab_read_device_error")
        flags |= flag.value
    return flags
