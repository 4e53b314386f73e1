"""fp64 CPU oracle of multi-head latent attention (MLA) decode over a latent cache.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package's smoke check and
the benchmark's CPU-baseline leg may import this module.  It shares no code
with the HIP library and imports nothing from it.

The ClusterFusion page (section 5.2, DeepSeek-MLA) adapts the fused decode
step to latent attention by partitioning the latent key/value cache across
clusters and merging the partial softmax results with a sparse reduction; it
gives no formulas.  The reading adopted (listed with the others in the design
notes) is DeepSeek's latent attention in its absorbed decode form: every
cached token t holds one latent vector c_t (kv_lora_rank values, shared by all
heads) and one rotary key kr_t (rope_dim values, shared by all heads); head
h's query has been folded through the key up-projection into q_lat_h (same
width as c_t) and carries a rotary part q_rope_h; then

  M1  score   s_{h,t} = (q_lat_h . c_t + q_rope_h . kr_t) * scale
  M2  softmax over the tokens t = 0 .. pos (the history and the new token)
  M3  output  o_h = sum_t pi_{h,t} c_t          (a latent vector; the value
                                                  up-projection and the output
                                                  projection follow outside)

The new token's latent row and rotary key are appended to the caches at row
pos and take part in the softmax, as in the attention block's append-then-
attend order.  Pins (tests/test_mla_oracle.py): torch's scaled dot product
attention with one shared key/value head; the absorption identity against
explicit per-head keys and values; a single token; a 50-digit twin on tiny
shapes.
"""
from __future__ import annotations

import numpy as np

from .decode_step import round_to_storage, softmax, to_f64


def attended_rows(cache: np.ndarray, new_row: np.ndarray, pos: int) -> np.ndarray:
    """The rows one sequence attends to: its cached rows 0 .. pos-1, then the new token's row."""
    return np.concatenate([cache[:pos], new_row[None]], axis=0)


def mla_scores(q_lat: np.ndarray, q_rope: np.ndarray, keys_c: np.ndarray, keys_r: np.ndarray,
               scale: float) -> np.ndarray:
    """M1: s [nh, T], the latent part and the shared rotary part of every head's score, scaled."""
    return (q_lat @ keys_c.T + q_rope @ keys_r.T) * scale


def mla_attention(q_lat: np.ndarray, q_rope: np.ndarray, keys_c: np.ndarray, keys_r: np.ndarray,
                  scale: float):
    """M1-M3 for one sequence: q_lat [nh, R], q_rope [nh, P], keys_c [T, R], keys_r [T, P] (every token
    attended).  Returns (o [nh, R], probs [nh, T])."""
    p = softmax(mla_scores(q_lat, q_rope, keys_c, keys_r, scale))
    return p @ keys_c, p


def mla_decode_fp64(q_lat, q_rope, c_cache, kr_cache, c_new, kr_new, pos, *, scale: float,
                    storage: str = "bf16", want_probs: bool = False) -> dict:
    """MLA decode attention for every sequence of a batch, in float64.

    Arrays (float64 values): q_lat [B, nh, R], q_rope [B, nh, P], c_cache [B, cap, R], kr_cache
    [B, cap, P], c_new [B, R], kr_new [B, P]; pos int [B].  Rows t < pos[b] of the caches are read; the
    new token's rows enter as given (they are already storage values).  Returns out [B, nh, R], the
    appended rows c_row [B, R] and kr_row [B, P] (rounded to `storage`), and probs (list of [nh, pos+1])
    with want_probs.
    """
    B = q_lat.shape[0]
    cap = c_cache.shape[1]
    outs, probs, c_rows, kr_rows = [], [], [], []
    for b in range(B):
        p = int(pos[b])
        if not 0 <= p < cap:
            raise ValueError(f"pos[{b}] = {p} outside [0, {cap})")
        o, pr = mla_attention(q_lat[b], q_rope[b], attended_rows(c_cache[b], c_new[b], p),
                              attended_rows(kr_cache[b], kr_new[b], p), scale)
        outs.append(o)
        probs.append(pr)
        c_rows.append(round_to_storage(c_new[b], storage))
        kr_rows.append(round_to_storage(kr_new[b], storage))
    res = {"out": np.stack(outs) if B else np.zeros((0,) + q_lat.shape[1:]),
           "c_row": np.stack(c_rows) if B else np.zeros((0, c_cache.shape[2])),
           "kr_row": np.stack(kr_rows) if B else np.zeros((0, kr_cache.shape[2]))}
    if want_probs:
        res["probs"] = probs
    return res


def mla_decode_from_inputs(inp: dict, want_probs: bool = False) -> dict:
    """Run `mla_decode_fp64` on a stored MLA input set (see the seeded generator): q in fp32, the caches
    and the new token's rows in the storage type; only rows t < pos[b] of the caches are upcast."""
    cfg = inp["cfg"]
    st = cfg.dtype
    pos = np.asarray(inp["pos"])
    B = pos.shape[0]
    R, P = cfg.kv_lora_rank, cfg.rope_dim
    pmax = int(pos.max()) if B else 0
    cc = np.zeros((B, pmax + 1, R))
    kc = np.zeros((B, pmax + 1, P))
    for b in range(B):
        p = int(pos[b])
        cc[b, :p] = to_f64(inp["c_cache"][b, :p], st)
        kc[b, :p] = to_f64(inp["kr_cache"][b, :p], st)
    return mla_decode_fp64(np.asarray(inp["q_lat"], dtype=np.float64), np.asarray(inp["q_rope"], dtype=np.float64),
                           cc, kc, to_f64(inp["c_new"], st), to_f64(inp["kr_new"], st), pos,
                           scale=cfg.softmax_scale, storage=st, want_probs=want_probs)
