"""ctypes view of libdab.so (declarations mirror include/dab.h)."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# DAB_LIBRARY names another build of the same library (e.g. to compare builds)
LIB_PATH = os.environ.get("DAB_LIBRARY") or os.path.join(HERE, "libdab.so")

DAB_OK, DAB_ERR_INVALID_ARG, DAB_ERR_UNSUPPORTED, DAB_ERR_WORKSPACE, DAB_ERR_HIP = range(5)
DAB_F32, DAB_BF16 = 0, 1
SCHEDULES = {"auto": 0, "phased": 1, "attn_oproj": 2, "qkv_attn": 3, "fused": 4}
LAYER_SCHEDULES = {"auto": 0, "sequential": 1, "overlap": 2}       # dab_layer_schedule

# every symbol include/dab.h declares
EXPORTS = (
    "dab_workspace_size", "dab_workspace_init", "dab_decode_attn_block", "dab_decode_attn_block_timed",
    "dab_phase_count", "dab_phase_name", "dab_read_device_error", "dab_status_string", "dab_version",
    "dab_last_hip_error", "dab_ffn_workspace_size", "dab_decode_ffn_block", "dab_decode_ffn_block_timed",
    "dab_read_probe", "dab_attention_output", "dab_pack_weight", "dab_decode_attn_block_noalloc",
    "dab_mla_workspace_size", "dab_mla_decode_attn", "dab_mla_decode_attn_timed", "dab_decode_layer",
    "dab_layer_overlapped",
)
NOALLOC_SCRATCH_BYTES = 16 << 20      # DAB_NOALLOC_SCRATCH_BYTES
READ_PROBE_BLOCKS = 2048      # DAB_READ_PROBE_BLOCKS
# names of the two FFN kernels, in launch order
FFN_PHASES = ("ffn_rmsnorm_gate_up_silu", "ffn_down_residual")


class DabConfig(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("hidden", ctypes.c_int32),
        ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("cache_capacity", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("rope_theta", ctypes.c_float),
        ("eps", ctypes.c_float),
        ("kv_chunk", ctypes.c_int32),
        ("schedule", ctypes.c_int32),
        ("max_position", ctypes.c_int32),
    ]


class DabFfnConfig(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("hidden", ctypes.c_int32),
        ("intermediate", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("eps", ctypes.c_float),
    ]


class DabMlaConfig(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("n_heads", ctypes.c_int32),
        ("kv_lora_rank", ctypes.c_int32),
        ("rope_dim", ctypes.c_int32),
        ("cache_capacity", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("kv_chunk", ctypes.c_int32),
    ]


# names of the two latent-attention kernels, in launch order
MLA_PHASES = ("mla_chunk", "mla_merge")

_lib = None


def load() -> ctypes.CDLL:
    """Load libdab.so once.  Raises if it has not been built: there is no fallback."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m attention_block_amd.build`")
    # torch ships its own HIP runtime under the same soname; load it first so
    # that the library and torch's streams and allocations share one runtime
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    vp, sz, i32, cfgp = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.POINTER(DabConfig)
    lib.dab_workspace_size.argtypes = [cfgp]
    lib.dab_workspace_size.restype = sz
    lib.dab_workspace_init.argtypes = [vp, sz, vp]
    lib.dab_workspace_init.restype = i32
    call = [cfgp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.dab_decode_attn_block.argtypes = call
    lib.dab_decode_attn_block.restype = i32
    lib.dab_decode_attn_block_timed.argtypes = call + [ctypes.POINTER(vp), i32]
    lib.dab_decode_attn_block_timed.restype = i32
    lib.dab_phase_count.argtypes = [cfgp]
    lib.dab_phase_count.restype = i32
    lib.dab_phase_name.argtypes = [cfgp, i32]
    lib.dab_phase_name.restype = ctypes.c_char_p
    lib.dab_read_device_error.argtypes = [vp, vp, ctypes.POINTER(ctypes.c_int32)]
    lib.dab_read_device_error.restype = i32
    lib.dab_status_string.argtypes = [i32]
    lib.dab_status_string.restype = ctypes.c_char_p
    lib.dab_version.argtypes = []
    lib.dab_version.restype = ctypes.c_char_p
    lib.dab_last_hip_error.argtypes = []
    lib.dab_last_hip_error.restype = ctypes.c_char_p
    lib.dab_read_probe.argtypes = [vp, sz, vp, sz, vp]
    lib.dab_read_probe.restype = i32
    lib.dab_attention_output.argtypes = [cfgp, vp, sz, vp, vp]
    lib.dab_attention_output.restype = i32
    lib.dab_pack_weight.argtypes = [vp, vp, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, vp]
    lib.dab_pack_weight.restype = i32
    lib.dab_decode_attn_block_noalloc.argtypes = [cfgp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.dab_decode_attn_block_noalloc.restype = i32
    ffnp = ctypes.POINTER(DabFfnConfig)
    lib.dab_ffn_workspace_size.argtypes = [ffnp]
    lib.dab_ffn_workspace_size.restype = sz
    ffn_call = [ffnp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.dab_decode_ffn_block.argtypes = ffn_call
    lib.dab_decode_ffn_block.restype = i32
    lib.dab_decode_ffn_block_timed.argtypes = ffn_call + [ctypes.POINTER(vp), i32]
    lib.dab_decode_ffn_block_timed.restype = i32
    lib.dab_decode_layer.argtypes = [cfgp, ffnp] + [vp] * 13 + [vp, sz, vp, sz, i32, vp]
    lib.dab_decode_layer.restype = i32
    lib.dab_layer_overlapped.argtypes = [cfgp, ffnp]
    lib.dab_layer_overlapped.restype = i32
    mlap = ctypes.POINTER(DabMlaConfig)
    lib.dab_mla_workspace_size.argtypes = [mlap]
    lib.dab_mla_workspace_size.restype = sz
    mla_call = [mlap, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.dab_mla_decode_attn.argtypes = mla_call
    lib.dab_mla_decode_attn.restype = i32
    lib.dab_mla_decode_attn_timed.argtypes = mla_call + [ctypes.POINTER(vp), i32]
    lib.dab_mla_decode_attn_timed.restype = i32
    _lib = lib
    return lib
