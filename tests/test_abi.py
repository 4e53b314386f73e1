"""The C ABI library: loads, exports what include/dab.h declares, and rejects
bad arguments on the host before any HIP call (no compute on the CPU)."""
import ctypes
import os
import re
import subprocess

import pytest

from attention_block_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dab.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from attention_block_amd.build import build
        build()
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dab_[a-z_]+)\s*\(", text)))


def test_header_declares_the_binding_exports():
    assert declared_functions() == sorted(_lib.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (dab_[a-z_]+)$", out, flags=re.M))
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_library_targets_gfx950(lib):
    # the embedded device code object names its target triple
    blob = open(_lib.LIB_PATH, "rb").read()
    assert b"amdgcn-amd-amdhsa--gfx950" in blob


def cfg(**kw):
    base = dict(batch=1, hidden=256, n_q_heads=4, n_kv_heads=4, head_dim=64, cache_capacity=129,
                dtype=_lib.DAB_F32, rope_theta=1e4, eps=1e-6, kv_chunk=0)
    base.update(kw)
    return _lib.DabConfig(**base)


@pytest.mark.parametrize("bad", [
    dict(hidden=0), dict(hidden=100), dict(head_dim=96), dict(n_q_heads=6, n_kv_heads=4),
    dict(n_q_heads=32, n_kv_heads=2), dict(dtype=7), dict(rope_theta=0.0), dict(eps=-1.0),
    dict(cache_capacity=0), dict(kv_chunk=100), dict(batch=-1), dict(rope_theta=float("inf")),
    dict(eps=float("nan")),
])
def test_invalid_configs_have_no_workspace(lib, bad):
    c = cfg(**bad)
    assert lib.dab_workspace_size(ctypes.byref(c)) == 0
    assert lib.dab_phase_count(ctypes.byref(c)) == 0


def test_workspace_size_valid(lib):
    c = cfg()
    n = lib.dab_workspace_size(ctypes.byref(c))
    assert n > 0 and n % 256 == 0
    big = cfg(batch=32, hidden=4096, n_q_heads=32, n_kv_heads=8, head_dim=128, cache_capacity=8193,
              dtype=_lib.DAB_BF16, rope_theta=5e5)
    assert lib.dab_workspace_size(ctypes.byref(big)) > n
    ph = cfg(schedule=1)
    assert lib.dab_phase_count(ctypes.byref(ph)) == 3
    assert [lib.dab_phase_name(ctypes.byref(ph), i) for i in range(4)] == [
        b"qkv_rmsnorm_rope_append", b"attention_split_kv", b"oproj_residual", None]


PHASED = [b"qkv_rmsnorm_rope_append", b"attention_split_kv", b"oproj_residual"]
PHASED_SPLIT = [b"qkv_rmsnorm_rope_append", b"attention_split_kv", b"attention_merge", b"oproj_residual"]
ATTN_OPROJ = [b"qkv_rmsnorm_rope_append", b"attention_oproj_residual"]
QKV_ATTN = [b"qkv_attention_split_kv", b"oproj_residual"]


def names(lib, c):
    return [lib.dab_phase_name(ctypes.byref(c), i) for i in range(lib.dab_phase_count(ctypes.byref(c)))]


def test_schedule_selection(lib):
    # a group of 3, or projections that are not whole K-blocks: auto is phased, one-launch schedules unsupported
    for c in (cfg(n_q_heads=6, n_kv_heads=2), cfg()):
        assert names(lib, c) == PHASED
        for sched in (2, 3):
            c.schedule = sched
            assert call(lib, c) == _lib.DAB_ERR_UNSUPPORTED
            assert lib.dab_phase_count(ctypes.byref(c)) == 0
    for bad in (-1, 5, 7):
        assert lib.dab_workspace_size(ctypes.byref(cfg(schedule=bad))) == 0
        assert call(lib, cfg(schedule=bad)) == _lib.DAB_ERR_INVALID_ARG
    # the 7B layer: auto takes attention + projection in one launch; every schedule is available
    head = dict(batch=1, hidden=4096, n_q_heads=32, n_kv_heads=32, head_dim=128, cache_capacity=4097,
                dtype=_lib.DAB_BF16)
    assert names(lib, cfg(**head)) == ATTN_OPROJ
    assert names(lib, cfg(**head, schedule=1)) == PHASED
    assert names(lib, cfg(**head, schedule=2)) == ATTN_OPROJ
    assert names(lib, cfg(**head, schedule=3)) == QKV_ATTN
    assert names(lib, cfg(**head, schedule=4)) == [b"decode_block_fused"]
    assert lib.dab_phase_name(ctypes.byref(cfg(**head)), 2) is None
    # the whole step in one launch: batches of up to 4, whole K-blocks in the output projection
    assert call(lib, cfg(**{**head, "batch": 5}, schedule=4)) == _lib.DAB_ERR_UNSUPPORTED
    assert names(lib, cfg(**{**head, "batch": 4, "n_kv_heads": 8}, schedule=4)) == [b"decode_block_fused"]
    assert call(lib, cfg(n_q_heads=6, n_kv_heads=2, schedule=4)) == _lib.DAB_ERR_UNSUPPORTED
    # four fp32 rows of H = 8192 do not fit the 64 KB of staged inputs
    assert call(lib, cfg(batch=4, hidden=8192, n_q_heads=16, n_kv_heads=16, head_dim=128, schedule=4)) == \
        _lib.DAB_ERR_UNSUPPORTED
    # grouped heads, or batch above 4: auto stays phased; a group of 4 at 4K tokens has 64 chunks of 64,
    # more than one merge round (8 chunks per thread and head) in the attention kernel, so the merge
    # runs as a kernel of its own; 16 sequences have 8 chunks each and merge in the attention kernel
    assert names(lib, cfg(**{**head, "n_kv_heads": 8})) == PHASED_SPLIT
    assert names(lib, cfg(**{**head, "n_kv_heads": 8, "batch": 16})) == PHASED
    assert names(lib, cfg(**{**head, "batch": 5})) == PHASED
    assert names(lib, cfg(**{**head, "batch": 4})) == ATTN_OPROJ
    # fp32: K a multiple of 2048 -- nq * D for attention + projection, H for QKV + attention
    assert names(lib, cfg(n_q_heads=16, n_kv_heads=16, head_dim=128)) == ATTN_OPROJ
    assert names(lib, cfg(n_q_heads=16, n_kv_heads=4, head_dim=128)) == PHASED
    assert names(lib, cfg(n_q_heads=16, n_kv_heads=4, head_dim=128, schedule=2)) == ATTN_OPROJ
    assert call(lib, cfg(n_q_heads=16, n_kv_heads=4, head_dim=128, schedule=3)) == _lib.DAB_ERR_UNSUPPORTED
    assert names(lib, cfg(hidden=2048, schedule=3)) == QKV_ATTN
    assert call(lib, cfg(hidden=2048, schedule=2)) == _lib.DAB_ERR_UNSUPPORTED


def test_gemv_width_limits(lib):
    # every GEMV workgroup keeps one fp32 input row in 64 KB of LDS
    assert lib.dab_workspace_size(ctypes.byref(cfg(hidden=16384, n_q_heads=256, n_kv_heads=32))) > 0
    assert call(lib, cfg(hidden=16384 + 64)) == _lib.DAB_ERR_UNSUPPORTED
    assert call(lib, cfg(n_q_heads=264, n_kv_heads=33)) == _lib.DAB_ERR_UNSUPPORTED


class FakePtrs:
    """Distinct, aligned, never-dereferenced addresses for the pointer checks."""

    def __init__(self):
        self.next = 1 << 40

    def take(self, nbytes, align=256):
        p = self.next
        self.next += (nbytes + 2 * align) // align * align + (1 << 30)
        return p


def call(lib, c, **over):
    f = FakePtrs()
    ptrs = dict(hidden=f.take(1 << 20), norm_w=f.take(1 << 20), w_qkv=f.take(1 << 24), w_o=f.take(1 << 24),
                k_cache=f.take(1 << 24), v_cache=f.take(1 << 24), pos=f.take(64), out=f.take(1 << 20),
                dbg_y=0, ws=f.take(1 << 26))
    ws_bytes = lib.dab_workspace_size(ctypes.byref(c))
    ptrs.update(over)
    ws_bytes = over.pop("ws_bytes", ws_bytes)
    vp = ctypes.c_void_p
    return lib.dab_decode_attn_block(ctypes.byref(c), vp(ptrs["hidden"]), vp(ptrs["norm_w"]), vp(ptrs["w_qkv"]),
                                     vp(ptrs["w_o"]), vp(ptrs["k_cache"]), vp(ptrs["v_cache"]), vp(ptrs["pos"]),
                                     vp(ptrs["out"]), vp(ptrs["dbg_y"]), vp(ptrs["ws"]), ws_bytes, None)


def test_null_and_misaligned_pointers(lib):
    c = cfg()
    for name in ("hidden", "norm_w", "w_qkv", "w_o", "k_cache", "v_cache", "pos", "out"):
        assert call(lib, c, **{name: 0}) == _lib.DAB_ERR_INVALID_ARG, name
    for name in ("hidden", "w_qkv", "out", "k_cache"):
        assert call(lib, c, **{name: (1 << 40) + 8}) == _lib.DAB_ERR_INVALID_ARG, name
    assert call(lib, c, pos=(1 << 41) + 2) == _lib.DAB_ERR_INVALID_ARG
    assert call(lib, c, dbg_y=(1 << 42) + 4) == _lib.DAB_ERR_INVALID_ARG


def test_read_probe_host_checks(lib):
    # checked on the host before anything is enqueued (the pointers are never touched)
    buf, out, n = (1 << 40), (1 << 41), 4096
    for args in ((0, n, out, 8192), (buf, n, 0, 8192), (buf + 8, n, out, 8192), (buf, n + 4, out, 8192),
                 (buf, n, out + 2, 8192), (buf, n, out, 4 * _lib.READ_PROBE_BLOCKS - 4)):
        assert lib.dab_read_probe(*args, None) == _lib.DAB_ERR_INVALID_ARG, args


def test_workspace_checks(lib):
    c = cfg()
    assert call(lib, c, ws=0) == _lib.DAB_ERR_WORKSPACE
    need = lib.dab_workspace_size(ctypes.byref(c))
    assert call(lib, c, ws_bytes=need - 256) == _lib.DAB_ERR_WORKSPACE
    assert call(lib, c, ws=(1 << 43) + 128) == _lib.DAB_ERR_INVALID_ARG


def test_output_aliasing_rejected(lib):
    c = cfg()
    f = FakePtrs()
    shared = f.take(1 << 20)
    assert call(lib, c, hidden=shared, out=shared) == _lib.DAB_ERR_INVALID_ARG
    assert call(lib, c, k_cache=shared, v_cache=shared + 256) == _lib.DAB_ERR_INVALID_ARG
    assert call(lib, c, out=shared, dbg_y=shared + 512) == _lib.DAB_ERR_INVALID_ARG


def test_unsupported_shapes(lib):
    assert call(lib, cfg(head_dim=96)) == _lib.DAB_ERR_UNSUPPORTED
    assert call(lib, cfg(n_q_heads=36, n_kv_heads=4)) == _lib.DAB_ERR_UNSUPPORTED


def test_batch_zero_is_a_no_op(lib):
    # nothing is enqueued, so this is safe without a device
    assert call(lib, cfg(batch=0)) == _lib.DAB_OK


def test_timed_variant_checks_events(lib):
    # two events per kernel (its own start and end); every check fails before anything is enqueued
    c = cfg()
    vp = ctypes.c_void_p
    f = FakePtrs()
    ptrs = [f.take(1 << 20), f.take(1 << 20), f.take(1 << 24), f.take(1 << 24), f.take(1 << 24), f.take(1 << 24),
            f.take(64), f.take(1 << 20)]
    args = [ctypes.byref(c)] + [vp(q) for q in ptrs] + [vp(0), vp(f.take(1 << 26)),
                                                      lib.dab_workspace_size(ctypes.byref(c)), None]
    assert lib.dab_decode_attn_block_timed(*args, None, 0) == _lib.DAB_ERR_INVALID_ARG
    n = lib.dab_phase_count(ctypes.byref(c))
    for count in (n + 1, 2 * n - 1, 2 * n + 1):        # the old one-between-kernels count is rejected too
        ev = (vp * count)(*[vp(8 * (i + 1)) for i in range(count)])
        assert lib.dab_decode_attn_block_timed(*args, ev, count) == _lib.DAB_ERR_INVALID_ARG, count
    ev = (vp * (2 * n))(*[vp(8 * (i + 1)) for i in range(2 * n - 1)] + [vp(0)])
    assert lib.dab_decode_attn_block_timed(*args, ev, 2 * n) == _lib.DAB_ERR_INVALID_ARG   # a null event


def test_status_strings(lib):
    for s in range(5):
        assert lib.dab_status_string(s)
    assert lib.dab_version().startswith(b"dab")


# ---------------------------------------------------------------------------
# the FFN entry points
# ---------------------------------------------------------------------------

def ffn_cfg(**kw):
    base = dict(batch=1, hidden=256, intermediate=512, dtype=_lib.DAB_BF16, eps=1e-6)
    base.update(kw)
    return _lib.DabFfnConfig(**base)


@pytest.mark.parametrize("bad", [
    dict(hidden=0), dict(intermediate=0), dict(hidden=100), dict(intermediate=96 + 8), dict(dtype=7),
    dict(eps=float("nan")), dict(eps=-1.0), dict(batch=-1), dict(hidden=16384 + 64), dict(intermediate=16384 + 64),
])
def test_ffn_invalid_configs_have_no_workspace(lib, bad):
    assert lib.dab_ffn_workspace_size(ctypes.byref(ffn_cfg(**bad))) == 0


def test_ffn_workspace_size(lib):
    n = lib.dab_ffn_workspace_size(ctypes.byref(ffn_cfg()))
    assert n > 0 and n % 256 == 0
    # m in fp32 and in bf16, per sequence
    assert lib.dab_ffn_workspace_size(ctypes.byref(ffn_cfg(batch=16, hidden=4096, intermediate=14336))) >= \
        16 * 14336 * 6


def ffn_call(lib, c, timed=None, **over):
    f = FakePtrs()
    ptrs = dict(hidden=f.take(1 << 20), norm_w=f.take(1 << 20), w_gate=f.take(1 << 24), w_up=f.take(1 << 24),
                w_down=f.take(1 << 24), out=f.take(1 << 20), dbg_y=0, ws=f.take(1 << 26))
    ws_bytes = lib.dab_ffn_workspace_size(ctypes.byref(c))
    ws_bytes = over.pop("ws_bytes", ws_bytes)
    ptrs.update(over)
    vp = ctypes.c_void_p
    args = [ctypes.byref(c)] + [vp(ptrs[k]) for k in ("hidden", "norm_w", "w_gate", "w_up", "w_down", "out",
                                                         "dbg_y", "ws")] + [ws_bytes, None]
    if timed is None:
        return lib.dab_decode_ffn_block(*args)
    events, n = timed
    return lib.dab_decode_ffn_block_timed(*args, events, n)


def test_ffn_host_checks(lib):
    c = ffn_cfg()
    for name in ("hidden", "norm_w", "w_gate", "w_up", "w_down", "out"):
        assert ffn_call(lib, c, **{name: 0}) == _lib.DAB_ERR_INVALID_ARG, name
        assert ffn_call(lib, c, **{name: (1 << 44) + 8}) == _lib.DAB_ERR_INVALID_ARG, name
    assert ffn_call(lib, c, dbg_y=(1 << 45) + 4) == _lib.DAB_ERR_INVALID_ARG
    assert ffn_call(lib, c, ws=0) == _lib.DAB_ERR_WORKSPACE
    assert ffn_call(lib, c, ws_bytes=lib.dab_ffn_workspace_size(ctypes.byref(c)) - 256) == _lib.DAB_ERR_WORKSPACE
    shared = FakePtrs().take(1 << 20)
    assert ffn_call(lib, c, hidden=shared, out=shared) == _lib.DAB_ERR_INVALID_ARG
    assert ffn_call(lib, c, w_gate=shared, out=shared + 256) == _lib.DAB_ERR_INVALID_ARG
    assert ffn_call(lib, ffn_cfg(hidden=96)) == _lib.DAB_ERR_UNSUPPORTED
    # nothing is enqueued for an empty batch, so this is safe without a device
    assert ffn_call(lib, ffn_cfg(batch=0)) == _lib.DAB_OK


def test_ffn_timed_variant_checks_events(lib):
    vp = ctypes.c_void_p
    c = ffn_cfg()
    assert ffn_call(lib, c, timed=(None, 0)) == _lib.DAB_ERR_INVALID_ARG
    for count in (2, 3, 5):
        ev = (vp * count)(*[vp(8 * (i + 1)) for i in range(count)])
        assert ffn_call(lib, c, timed=(ev, count)) == _lib.DAB_ERR_INVALID_ARG, count
    ev = (vp * 4)(vp(8), vp(16), vp(0), vp(32))
    assert ffn_call(lib, c, timed=(ev, 4)) == _lib.DAB_ERR_INVALID_ARG


# ---------------------------------------------------------------------------
# the weight-layout conversion and the attention-output tap: host checks
# ---------------------------------------------------------------------------

def test_pack_weight_host_checks(lib):
    src, dst = (1 << 40), (1 << 42)
    ok = dict(src=src, dst=dst, n_in=4096, n_out=12288, dtype=_lib.DAB_BF16)
    bad = [dict(src=0), dict(dst=0), dict(src=src + 8), dict(dst=dst + 2), dict(n_in=0), dict(n_out=-1),
           dict(n_in=65535 * 64 + 1), dict(dtype=5),
           dict(dst=src + 4096 * 2 * 100),            # dst starts inside src
           dict(src=dst + 16, dst=dst)]               # src starts inside dst
    for over in bad:
        a = {**ok, **over}
        st = lib.dab_pack_weight(ctypes.c_void_p(a["src"]), ctypes.c_void_p(a["dst"]), a["n_in"], a["n_out"],
                                 a["dtype"], None)
        assert st == _lib.DAB_ERR_INVALID_ARG, over


def test_attention_output_host_checks(lib):
    c = cfg()
    n = lib.dab_workspace_size(ctypes.byref(c))
    ws, dst = (1 << 40), (1 << 42)
    vp = ctypes.c_void_p
    assert lib.dab_attention_output(ctypes.byref(cfg(head_dim=96)), vp(ws), n, vp(dst), None) == \
        _lib.DAB_ERR_UNSUPPORTED
    assert lib.dab_attention_output(ctypes.byref(c), vp(0), n, vp(dst), None) == _lib.DAB_ERR_INVALID_ARG
    assert lib.dab_attention_output(ctypes.byref(c), vp(ws + 128), n, vp(dst), None) == _lib.DAB_ERR_INVALID_ARG
    assert lib.dab_attention_output(ctypes.byref(c), vp(ws), n, vp(0), None) == _lib.DAB_ERR_INVALID_ARG
    assert lib.dab_attention_output(ctypes.byref(c), vp(ws), n - 256, vp(dst), None) == _lib.DAB_ERR_WORKSPACE
    assert lib.dab_attention_output(ctypes.byref(c), vp(ws), n, vp(ws + 512), None) == _lib.DAB_ERR_INVALID_ARG
    # batch 0: nothing to copy, nothing enqueued
    assert lib.dab_attention_output(ctypes.byref(cfg(batch=0)), vp(ws), n, vp(dst), None) == _lib.DAB_OK


def test_python_wrapper_requires_a_weight_layout():
    import inspect
    import attention_block_amd as ab
    for f in (ab.decode_attn_block, ab.decode_attn_block_timed, ab.decode_ffn_block, ab.decode_ffn_block_timed):
        p = inspect.signature(f).parameters["weight_layout"]
        assert p.kind is inspect.Parameter.KEYWORD_ONLY and p.default is inspect.Parameter.empty, f.__name__


def test_noalloc_host_checks(lib):
    """The allocation-free entry point rejects what the workspace entry point rejects, and a configuration
    whose workspace exceeds its scratch, all before any device call (so this runs without a GPU)."""
    vp = ctypes.c_void_p
    f = FakePtrs()
    ptrs = dict(hidden=f.take(1 << 20), norm_w=f.take(1 << 20), w_qkv=f.take(1 << 24), w_o=f.take(1 << 24),
                k_cache=f.take(1 << 24), v_cache=f.take(1 << 24), pos=f.take(64), out=f.take(1 << 20), dbg_y=0)

    def na(c, **over):
        p = {**ptrs, **over}
        return lib.dab_decode_attn_block_noalloc(ctypes.byref(c), *[vp(p[k]) for k in (
            "hidden", "norm_w", "w_qkv", "w_o", "k_cache", "v_cache", "pos", "out", "dbg_y")], None)

    assert na(cfg(head_dim=96)) == _lib.DAB_ERR_UNSUPPORTED
    assert na(cfg(dtype=7)) == _lib.DAB_ERR_INVALID_ARG
    assert na(cfg(), hidden=0) == _lib.DAB_ERR_INVALID_ARG
    assert na(cfg(), out=ptrs["hidden"]) == _lib.DAB_ERR_INVALID_ARG
    assert na(cfg(batch=0)) == _lib.DAB_OK                       # nothing to do, nothing enqueued
    # a workspace larger than the scratch: 32 sequences of 64 chunks of 32 heads
    big = cfg(batch=32, hidden=4096, n_q_heads=32, n_kv_heads=32, head_dim=128, cache_capacity=1 << 16,
              dtype=_lib.DAB_BF16, rope_theta=1e4, kv_chunk=1024)
    assert lib.dab_workspace_size(ctypes.byref(big)) > _lib.NOALLOC_SCRATCH_BYTES
    assert na(big) == _lib.DAB_ERR_WORKSPACE


# the decoder layer (dab_decode_layer): selection of the overlapped schedule, host checks

def test_layer_overlapped_selection(lib):
    def ov(c, f):
        return lib.dab_layer_overlapped(ctypes.byref(c), ctypes.byref(f))
    bf, f32 = _lib.DAB_BF16, _lib.DAB_F32
    mha7b = dict(hidden=4096, n_q_heads=32, n_kv_heads=32, head_dim=128, cache_capacity=4097)
    # the 7B layer at batch 1 and 4 (bf16), an fp32 layer of 2048
    assert ov(cfg(dtype=bf, **mha7b), ffn_cfg(hidden=4096, intermediate=11008)) == 1
    assert ov(cfg(batch=4, dtype=bf, **mha7b), ffn_cfg(batch=4, hidden=4096, intermediate=11008)) == 1
    assert ov(cfg(hidden=2048, n_q_heads=32, n_kv_heads=32, head_dim=64, dtype=f32),
              ffn_cfg(hidden=2048, intermediate=4096, dtype=f32)) == 1
    # run as two calls: grouped heads (phased schedule), partial K-blocks, the FFN's MFMA panels at
    # batch 8, a schedule forced to phased
    assert ov(cfg(hidden=4096, n_q_heads=32, n_kv_heads=8, head_dim=128, dtype=bf),
              ffn_cfg(hidden=4096, intermediate=14336)) == 0
    assert ov(cfg(dtype=bf), ffn_cfg()) == 0
    assert ov(cfg(batch=8, dtype=bf, **mha7b), ffn_cfg(batch=8, hidden=4096, intermediate=11008)) == 0
    assert ov(cfg(dtype=bf, schedule=1, **mha7b), ffn_cfg(hidden=4096, intermediate=11008)) == 0
    # the two configurations disagree, or one is invalid
    assert ov(cfg(dtype=bf, **mha7b), ffn_cfg(batch=2, hidden=4096, intermediate=11008)) == -1
    assert ov(cfg(dtype=bf, **mha7b), ffn_cfg(hidden=2048, intermediate=11008)) == -1
    assert ov(cfg(dtype=f32, **mha7b), ffn_cfg(hidden=4096, intermediate=11008)) == -1
    assert ov(cfg(dtype=bf, head_dim=96), ffn_cfg()) == -1


def layer_call(lib, c, fc, schedule=0, **over):
    f = FakePtrs()
    names = ("hidden", "attn_norm_w", "w_qkv", "w_o", "k_cache", "v_cache", "pos", "ffn_norm_w", "w_gate", "w_up",
             "w_down", "h", "out")
    ptrs = {k: f.take(1 << 26) for k in names}
    ptrs["ws"] = f.take(1 << 26)
    ptrs["fws"] = f.take(1 << 26)
    ws_bytes = over.pop("ws_bytes", lib.dab_workspace_size(ctypes.byref(c)))
    fws_bytes = over.pop("fws_bytes", lib.dab_ffn_workspace_size(ctypes.byref(fc)))
    ptrs.update(over)
    vp = ctypes.c_void_p
    return lib.dab_decode_layer(ctypes.byref(c), ctypes.byref(fc), *[vp(ptrs[k]) for k in names],
                                vp(ptrs["ws"]), ws_bytes, vp(ptrs["fws"]), fws_bytes, schedule, None)


def test_layer_host_checks(lib):
    # every check fails before anything is enqueued (the pointers are never touched)
    c, fc = cfg(), ffn_cfg(dtype=_lib.DAB_F32)
    for name in ("hidden", "attn_norm_w", "w_qkv", "w_o", "k_cache", "v_cache", "pos", "ffn_norm_w", "w_gate",
                 "w_up", "w_down", "h", "out"):
        assert layer_call(lib, c, fc, **{name: 0}) == _lib.DAB_ERR_INVALID_ARG, name
    for name in ("hidden", "w_gate", "h", "out"):
        assert layer_call(lib, c, fc, **{name: (1 << 46) + 8}) == _lib.DAB_ERR_INVALID_ARG, name
    assert layer_call(lib, c, fc, ws=0) == _lib.DAB_ERR_WORKSPACE
    assert layer_call(lib, c, fc, fws=0) == _lib.DAB_ERR_WORKSPACE
    assert layer_call(lib, c, fc, fws_bytes=lib.dab_ffn_workspace_size(ctypes.byref(fc)) - 256) == \
        _lib.DAB_ERR_WORKSPACE
    # overlaps within a half and across the halves
    shared = FakePtrs().take(1 << 20) + (1 << 47)
    for a, b in (("hidden", "h"), ("h", "out"), ("h", "w_gate"), ("out", "w_qkv"), ("out", "k_cache"),
                 ("fws", "ws"), ("fws", "hidden"), ("v_cache", "w_down"), ("ws", "ffn_norm_w")):
        assert layer_call(lib, c, fc, **{a: shared, b: shared + 256}) == _lib.DAB_ERR_INVALID_ARG, (a, b)
    # inputs read by both halves may coincide
    assert layer_call(lib, cfg(batch=0), ffn_cfg(batch=0, dtype=_lib.DAB_F32),
                      w_up=shared, w_gate=shared) == _lib.DAB_OK
    # mismatched configurations
    assert layer_call(lib, c, ffn_cfg(batch=2, dtype=_lib.DAB_F32)) == _lib.DAB_ERR_INVALID_ARG
    assert layer_call(lib, c, ffn_cfg()) == _lib.DAB_ERR_INVALID_ARG          # bf16 FFN after an fp32 block
    # nothing is enqueued for an empty batch
    assert layer_call(lib, cfg(batch=0), ffn_cfg(batch=0, dtype=_lib.DAB_F32)) == _lib.DAB_OK
    # layer schedules: not a dab_layer_schedule; the overlapped one where it is not built (H 256)
    for bad in (-1, 3, 7):
        assert layer_call(lib, c, fc, schedule=bad) == _lib.DAB_ERR_INVALID_ARG, bad
    assert layer_call(lib, c, fc, schedule=_lib.LAYER_SCHEDULES["overlap"]) == _lib.DAB_ERR_UNSUPPORTED
    assert layer_call(lib, cfg(batch=0), ffn_cfg(batch=0, dtype=_lib.DAB_F32),
                      schedule=_lib.LAYER_SCHEDULES["sequential"]) == _lib.DAB_OK


def test_max_position_hint(lib):
    # the hint is the largest position a call's sequences hold: 0 (not given) up to cap - 1
    for bad in (-1, 129, 500):
        assert lib.dab_workspace_size(ctypes.byref(cfg(max_position=bad))) == 0, bad
    for ok in (0, 1, 64, 128):
        assert lib.dab_workspace_size(ctypes.byref(cfg(max_position=ok))) > 0, ok
    # grouped heads at batch 16 in a 16K cache with 4K tokens in use: the split-KV partials are sized
    # for the hint, as for a cache of 4097
    gqa = dict(batch=16, hidden=4096, n_q_heads=32, n_kv_heads=8, head_dim=128, dtype=_lib.DAB_BF16)
    big = lib.dab_workspace_size(ctypes.byref(cfg(cache_capacity=16384, **gqa)))
    hinted = lib.dab_workspace_size(ctypes.byref(cfg(cache_capacity=16384, max_position=4096, **gqa)))
    small = lib.dab_workspace_size(ctypes.byref(cfg(cache_capacity=4097, **gqa)))
    assert hinted == small < big
