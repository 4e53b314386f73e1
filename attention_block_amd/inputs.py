"""Seeded synthetic inputs for the single-token decode attention block.

This module produces inputs only.  It holds none of the block's arithmetic
(no norm, projection, rotation, softmax or merge): both the fp64 oracle and
the HIP path are fed from it, and nothing else is shared between them.

Workloads.  The pages benchmark a Llama2-7B decode block at 1K and 4K context
(ClusterFusion page, sections 1.1 and 5.1), a long-context build at 16K
tokens (same page, section 5.1, the MAX_SEQ_LEN build flag), and a fused
RMSNorm+QKV+attention kernel with 32 query heads, 8 KV heads and head_dim 128
(the operator-fusion page, section 3, its constants).  No trained weights or
datasets are used: every tensor is drawn from a seeded generator with the
distributions listed in CONFIGS, which stand in for the real models.

Storage.  bf16 tensors are carried as raw uint16 bit patterns (numpy has no
bf16 type); fp32 tensors as float32.  Draws are made in fp32 and rounded to
bf16 with round-to-nearest-even.  Cache rows at or beyond a sequence's
position are filled with a NaN sentinel so that any read past the valid
tokens poisons the result.

Draw order (fixed, so a seed names one input set):
  1. ragged configs only: per-sequence lengths, integers in [lo, hi] inclusive
  2. hidden [B, H] ~ N(0, 1)
  3. norm_w [H] = 1 + 0.1 * N(0, 1)
  4. w_qkv [H, (nq + 2 nkv) D] ~ N(0, 1/H)   (variance 1/H)
  5. w_o [nq D, H] ~ N(0, 1/H)
  6. for each sequence b: K_b [pos_b, nkv, D] ~ N(0, 1), then V_b likewise
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Sequence

import numpy as np

BF16_NAN = np.uint16(0x7FC0)


@dataclasses.dataclass(frozen=True)
class BlockConfig:
    """Shape and precision of one decode-block workload."""
    name: str
    batch: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    dtype: str                      # "f32" or "bf16": storage of every tensor
    rope_theta: float
    eps: float = 1e-6
    pos: Optional[int] = None       # tokens already cached (uniform batch)
    ragged: Optional[tuple] = None  # (lo, hi) inclusive range of per-sequence lengths

    @property
    def n_qkv(self) -> int:
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads


CONFIGS = {
    # Tiny MHA step, fp32 end to end.
    "tiny_mha_f32": BlockConfig("tiny_mha_f32", 1, 256, 4, 4, 64, "f32", 1e4, pos=128),
    # Llama-2-7B-shaped MHA layer at 1K and 4K context.
    "llama2_7b_bs1_1k": BlockConfig("llama2_7b_bs1_1k", 1, 4096, 32, 32, 128, "bf16", 1e4, pos=1024),
    "llama2_7b_bs1_4k": BlockConfig("llama2_7b_bs1_4k", 1, 4096, 32, 32, 128, "bf16", 1e4, pos=4096),
    # Llama-3-8B-shaped GQA layer, 16 sequences at 4K.
    "llama3_8b_gqa_bs16_4k": BlockConfig("llama3_8b_gqa_bs16_4k", 16, 4096, 32, 8, 128, "bf16", 5e5, pos=4096),
    # Long-context GQA, one sequence at 16K.
    "gqa_bs1_16k": BlockConfig("gqa_bs1_16k", 1, 4096, 32, 8, 128, "bf16", 5e5, pos=16384),
    # Ragged GQA batch: 32 sequences, lengths uniform in [256, 8192].
    "gqa_ragged_bs32": BlockConfig("gqa_ragged_bs32", 32, 4096, 32, 8, 128, "bf16", 5e5, ragged=(256, 8192)),
}

HEADLINE = "llama2_7b_bs1_4k"


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); return uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    rounded = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        rounded[nan] = BF16_NAN
    return rounded


def bf16_bits_to_f32(u: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 (exact)."""
    return (np.asarray(u, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _store(a32: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(a32) if dtype == "bf16" else np.ascontiguousarray(a32, dtype=np.float32)


def positions(cfg: BlockConfig, seed: int) -> np.ndarray:
    """Per-sequence token counts already in the cache (= the new token's index)."""
    if cfg.ragged is not None:
        rng = np.random.default_rng(seed)
        lo, hi = cfg.ragged
        return rng.integers(lo, hi, size=cfg.batch, endpoint=True).astype(np.int32)
    return np.full(cfg.batch, cfg.pos, dtype=np.int32)


def make_inputs(cfg: BlockConfig, seed: int, *, cap: Optional[int] = None,
                pos: Optional[Sequence[int]] = None, nan_tail: bool = True) -> dict:
    """Draw one seeded input set for `cfg`.

    Returns a dict of host arrays in storage form (uint16 bf16 bits or float32):
      hidden [B, H], norm_w [H], w_qkv [H, N_qkv], w_o [nq*D, H],
      k_cache, v_cache [B, cap, nkv, D], pos int32 [B], plus the config.
    `cap` defaults to max(pos) + 1.  `pos` overrides the configured lengths
    (used by edge-case tests); it must then be given for every sequence.
    Rows t >= pos[b] of both caches hold the NaN sentinel when `nan_tail`,
    else zeros.
    """
    rng = np.random.default_rng(seed)
    B, H, nq, nkv, D = cfg.batch, cfg.hidden, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    drawn = None
    if cfg.ragged is not None:
        lo, hi = cfg.ragged
        drawn = rng.integers(lo, hi, size=B, endpoint=True).astype(np.int32)
    elif cfg.pos is not None:
        drawn = np.full(B, cfg.pos, dtype=np.int32)
    if pos is None and drawn is None:
        raise ValueError(f"{cfg.name} has no configured length: pass pos")
    p = np.asarray(pos, dtype=np.int32) if pos is not None else drawn
    if p.shape != (B,):
        raise ValueError(f"pos must have shape ({B},)")
    if cap is None:
        cap = int(p.max()) + 1
    if int(p.max()) >= cap or int(p.min()) < 0:
        raise ValueError("every pos must lie in [0, cap)")

    std = 1.0 / np.sqrt(H)
    hidden = rng.standard_normal((B, H), dtype=np.float32)
    norm_w = (1.0 + 0.1 * rng.standard_normal(H, dtype=np.float32)).astype(np.float32)
    w_qkv = (rng.standard_normal((H, cfg.n_qkv), dtype=np.float32) * np.float32(std)).astype(np.float32)
    w_o = (rng.standard_normal((nq * D, H), dtype=np.float32) * np.float32(std)).astype(np.float32)

    sdt = np.uint16 if cfg.dtype == "bf16" else np.float32
    fill = BF16_NAN if cfg.dtype == "bf16" else np.float32(np.nan)
    if not nan_tail:
        fill = sdt(0)
    k_cache = np.full((B, cap, nkv, D), fill, dtype=sdt)
    v_cache = np.full((B, cap, nkv, D), fill, dtype=sdt)
    for b in range(B):
        n = int(p[b])
        kb = rng.standard_normal((n, nkv, D), dtype=np.float32)
        vb = rng.standard_normal((n, nkv, D), dtype=np.float32)
        k_cache[b, :n] = _store(kb, cfg.dtype)
        v_cache[b, :n] = _store(vb, cfg.dtype)

    return {
        "cfg": cfg,
        "hidden": _store(hidden, cfg.dtype),
        "norm_w": _store(norm_w, cfg.dtype),
        "w_qkv": _store(w_qkv, cfg.dtype),
        "w_o": _store(w_o, cfg.dtype),
        "k_cache": k_cache,
        "v_cache": v_cache,
        "pos": p,
        "cap": cap,
    }


# ---------------------------------------------------------------------------
# the FFN half of the layer
# ---------------------------------------------------------------------------
#
# Draw order: hidden [B, H] ~ N(0, 1); norm_w [H] = 1 + 0.1 N(0, 1);
# w_gate [H, F] ~ N(0, 1/H); w_up [H, F] ~ N(0, 1/H); w_down [F, H] ~ N(0, 1/F)
# (variances 1/fan-in, so g, u and y stay of order one).  The intermediate
# sizes are those of the models the pages benchmark (Llama-2-7B 11008,
# Llama-3-8B 14336); the pages do not give them.

@dataclasses.dataclass(frozen=True)
class FfnConfig:
    """Shape and precision of one FFN workload."""
    name: str
    batch: int
    hidden: int
    intermediate: int
    dtype: str
    eps: float = 1e-6


FFN_CONFIGS = {
    "tiny_ffn_f32": FfnConfig("tiny_ffn_f32", 1, 256, 704, "f32"),
    "llama2_7b_ffn_bs1": FfnConfig("llama2_7b_ffn_bs1", 1, 4096, 11008, "bf16"),
    "llama3_8b_ffn_bs16": FfnConfig("llama3_8b_ffn_bs16", 16, 4096, 14336, "bf16"),
}

FFN_HEADLINE = "llama2_7b_ffn_bs1"


def layer_ffn(cfg: BlockConfig) -> FfnConfig:
    """The FFN that follows `cfg`'s attention block in a full decoder layer (multi-layer chains).

    Intermediate size: Llama-3-8B's 14336 for its GQA shape (32 q / 8 kv heads at H 4096), else
    Llama-2's rule, 8H/3 rounded up to a multiple of 256 (11008 at H 4096)."""
    if (cfg.hidden, cfg.n_q_heads, cfg.n_kv_heads) == (4096, 32, 8):
        F = 14336
    else:
        F = 256 * -(-8 * cfg.hidden // 768)          # ceil(8H / 3 / 256) * 256
    return FfnConfig(cfg.name + "_ffn", cfg.batch, cfg.hidden, F, cfg.dtype, cfg.eps)


def make_ffn_inputs(cfg: FfnConfig, seed: int) -> dict:
    """Draw one seeded FFN input set (storage form, weights in the [in, out] orientation)."""
    rng = np.random.default_rng(seed)
    B, H, F = cfg.batch, cfg.hidden, cfg.intermediate
    hidden = rng.standard_normal((B, H), dtype=np.float32)
    norm_w = (1.0 + 0.1 * rng.standard_normal(H, dtype=np.float32)).astype(np.float32)
    sh, sf = np.float32(1.0 / np.sqrt(H)), np.float32(1.0 / np.sqrt(F))
    w_gate = (rng.standard_normal((H, F), dtype=np.float32) * sh).astype(np.float32)
    w_up = (rng.standard_normal((H, F), dtype=np.float32) * sh).astype(np.float32)
    w_down = (rng.standard_normal((F, H), dtype=np.float32) * sf).astype(np.float32)
    return {"cfg": cfg, "hidden": _store(hidden, cfg.dtype), "norm_w": _store(norm_w, cfg.dtype),
            "w_gate": _store(w_gate, cfg.dtype), "w_up": _store(w_up, cfg.dtype),
            "w_down": _store(w_down, cfg.dtype)}


def ffn_algorithmic_bytes(cfg: FfnConfig) -> int:
    """Three weight matrices once, the norm weight, hidden in and out."""
    s = 2 if cfg.dtype == "bf16" else 4
    return s * 3 * cfg.hidden * cfg.intermediate + s * cfg.hidden + 2 * s * cfg.batch * cfg.hidden


def ffn_algorithmic_flops(cfg: FfnConfig) -> int:
    return 2 * cfg.batch * 3 * cfg.hidden * cfg.intermediate


def algorithmic_bytes(cfg: BlockConfig, pos: Sequence[int]) -> int:
    """Bytes one decode step must move through HBM at minimum.

    Weights once, norm weight, the KV read of pos_b tokens per sequence, the
    appended K/V row, hidden in and out, and the position array.
    """
    s = 2 if cfg.dtype == "bf16" else 4
    B, H, nq, nkv, D = cfg.batch, cfg.hidden, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    total_pos = int(np.sum(np.asarray(pos, dtype=np.int64)))
    return (s * (H * cfg.n_qkv + nq * D * H) + s * H
            + s * 2 * nkv * D * total_pos + s * 2 * nkv * D * B
            + 2 * s * B * H + 4 * B)


def algorithmic_flops(cfg: BlockConfig, pos: Sequence[int]) -> int:
    """Multiply-adds x2 of the projections and of attention (scores and P.V)."""
    B, H, nq, D = cfg.batch, cfg.hidden, cfg.n_q_heads, cfg.head_dim
    total = int(np.sum(np.asarray(pos, dtype=np.int64) + 1))
    return 2 * B * H * cfg.n_qkv + 2 * B * nq * D * H + 4 * nq * D * total


# ---------------------------------------------------------------------------
# multi-head latent attention (MLA) decode over a latent cache
# ---------------------------------------------------------------------------
#
# The ClusterFusion page (section 5.2) runs DeepSeek's latent attention through
# the fused decode step at 4K and 16K tokens; these workloads take DeepSeek-V3's
# attention shape (128 heads, a 512-wide latent cache row and a 64-wide shared
# rotary key per token, softmax scale 1/sqrt(128 + 64)) and DeepSeek-V2-Lite's
# (16 heads, the same widths).  The query arrives already folded through the
# key up-projection.  No trained weights: synthetic stand-ins whose scores are
# of order one.  Draw order: (1) ragged lengths (none here); (2) q_lat
# [B, nh, R] ~ N(0, 1/4) (a 128-wide N(0, 1) query through an N(0, 1/512)
# projection); (3) q_rope [B, nh, P] ~ N(0, 1); (4) c_new [B, R], kr_new [B, P]
# ~ N(0, 1); (5) per sequence c_b [pos_b, R] then kr_b [pos_b, P] ~ N(0, 1).
# q in fp32; the cache rows and the new token's rows in the storage type.

@dataclasses.dataclass(frozen=True)
class MlaConfig:
    """Shape of one MLA decode-attention workload."""
    name: str
    batch: int
    n_heads: int
    pos: int
    kv_lora_rank: int = 512
    rope_dim: int = 64
    softmax_scale: float = 1.0 / np.sqrt(128 + 64)
    dtype: str = "bf16"


MLA_CONFIGS = {
    "mla_tiny": MlaConfig("mla_tiny", 2, 16, 100),
    "deepseek_v2_lite_mla_bs1_4k": MlaConfig("deepseek_v2_lite_mla_bs1_4k", 1, 16, 4096),
    "deepseek_v3_mla_bs1_4k": MlaConfig("deepseek_v3_mla_bs1_4k", 1, 128, 4096),
    "deepseek_v3_mla_bs1_16k": MlaConfig("deepseek_v3_mla_bs1_16k", 1, 128, 16384),
    "deepseek_v3_mla_bs16_4k": MlaConfig("deepseek_v3_mla_bs16_4k", 16, 128, 4096),
}


def make_mla_inputs(cfg: MlaConfig, seed: int, *, cap: Optional[int] = None,
                    pos: Optional[Sequence[int]] = None, nan_tail: bool = True) -> dict:
    """One seeded MLA input set: q_lat, q_rope (fp32), c_new [B, R], kr_new [B, P], caches c_cache
    [B, cap, R] and kr_cache [B, cap, P] (storage form; rows >= pos hold the NaN sentinel), pos [B]."""
    rng = np.random.default_rng(seed)
    B, nh, R, P = cfg.batch, cfg.n_heads, cfg.kv_lora_rank, cfg.rope_dim
    p = np.asarray(pos, dtype=np.int32) if pos is not None else np.full(B, cfg.pos, dtype=np.int32)
    if p.shape != (B,):
        raise ValueError(f"pos must have shape ({B},)")
    if cap is None:
        cap = int(p.max()) + 1
    if int(p.max()) >= cap or int(p.min()) < 0:
        raise ValueError("every pos must lie in [0, cap)")
    q_lat = (0.5 * rng.standard_normal((B, nh, R), dtype=np.float32)).astype(np.float32)
    q_rope = rng.standard_normal((B, nh, P), dtype=np.float32)
    c_new = rng.standard_normal((B, R), dtype=np.float32)
    kr_new = rng.standard_normal((B, P), dtype=np.float32)
    sdt = np.uint16 if cfg.dtype == "bf16" else np.float32
    fill = (BF16_NAN if cfg.dtype == "bf16" else np.float32(np.nan)) if nan_tail else sdt(0)
    c_cache = np.full((B, cap, R), fill, dtype=sdt)
    kr_cache = np.full((B, cap, P), fill, dtype=sdt)
    for b in range(B):
        n = int(p[b])
        c_cache[b, :n] = _store(rng.standard_normal((n, R), dtype=np.float32), cfg.dtype)
        kr_cache[b, :n] = _store(rng.standard_normal((n, P), dtype=np.float32), cfg.dtype)
    return {"cfg": cfg, "q_lat": q_lat, "q_rope": q_rope, "c_new": _store(c_new, cfg.dtype),
            "kr_new": _store(kr_new, cfg.dtype), "c_cache": c_cache, "kr_cache": kr_cache, "pos": p, "cap": cap}


def mla_algorithmic_bytes(cfg: MlaConfig, pos: Sequence[int]) -> int:
    """The latent cache rows of every cached token read once, the new rows read and appended, q (fp32) in
    and the latent output (fp32) out, and the positions."""
    s = 2 if cfg.dtype == "bf16" else 4
    B, nh, R, P = cfg.batch, cfg.n_heads, cfg.kv_lora_rank, cfg.rope_dim
    total = int(np.sum(np.asarray(pos, dtype=np.int64)))
    return s * (R + P) * total + 2 * s * (R + P) * B + 4 * B * nh * (R + P) + 4 * B * nh * R + 4 * B


def mla_algorithmic_flops(cfg: MlaConfig, pos: Sequence[int]) -> int:
    """Scores over R + P values and the weighted sum over R, per head and attended token."""
    total = int(np.sum(np.asarray(pos, dtype=np.int64) + 1))
    return 2 * cfg.n_heads * (2 * cfg.kv_lora_rank + cfg.rope_dim) * total
