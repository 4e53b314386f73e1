"""fp64 CPU oracle of the single-token decode attention block.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package's smoke check and
the benchmark's CPU-baseline leg may import this module.  It shares no code
with the HIP library and imports nothing from it.

What it computes is the plain definition of the block, one sequence at a
time, in float64 on numbers upcast exactly from the stored bf16/fp32 bits:

  O1  RMSNorm            r = (mean_i x_i^2 + eps)^(-1/2);  xh = x * r * w
      The operator-fusion page ("LayerNorm + Attention" CUDA kernel article),
      section 3, stage 1 of its kernel, normalises by sqrt(sum_sq / hidden + 1e-6)
      and then multiplies by the norm weight; the one-shot all-reduce page,
      section 2.2, puts eps inside the root (rsqrt(mean_square + eps)) and
      defaults eps to 1e-6 (section 3.1).  There is no mean subtraction and no
      bias (the kernel signature carries neither).
  O2  QKV projection     u = xh @ W_qkv, W_qkv row-major [H, (nq+2nkv)D],
      columns packed [Q | K | V], head-major inside each part.  ClusterFusion
      page, section 1.1 pseudo-code (torch.mm(hidden, W_qkv)) and section 5.1
      (Q, K and V merged into one matrix product); operator-fusion page,
      section 3, stage 2 (q_weight indexed [row * (heads*head_dim) + col]).
  O3  RoPE               rotate-half pairing (j, j + D/2), angle
      pos * theta^(-2j/D); applied to q and to the new k, not to v.
      Operator-fusion page, section 1 (RoPE in the block) and section 3
      (rotate_half in registers).
  O4  KV append          the new (rotated) k and v go to cache row pos of
      their sequence; every other cache element is unchanged.  Operator-fusion
      page, section 3, stage 3 (K/V written straight into the cache) and the
      cache layout [max_seq_len, num_kv_heads, head_dim].
  O5  Attention          for each query head h (kv head g = h // (nq/nkv),
      the GQA mapping of the operator-fusion page, section 3), scores
      q'_h . key_t / sqrt(D) over every token t = 0..pos (the history and the
      new token), softmax, weighted sum of values.  ClusterFusion page,
      sections 3.2 (online softmax with reduced statistics) and 1.1 (flash
      attention over the cache).  Split-KV with a log-sum-exp merge is an
      exact rewrite of this softmax, so the oracle uses the plain one.
  O6  Output projection  y = a @ W_o (a = heads concatenated, head-major),
      out = x + y.  ClusterFusion page, section 1.1 pseudo-code
      (torch.mm(attn_out, W_out)); operator-fusion page, section 1 (O
      projection with residual connection).

Readings where the pages are silent or garbled (scale 1/sqrt(D), the RoPE
frequency formula, eps = 1e-6 everywhere, pos = number of cached tokens,
tokens 0..pos inclusive, unrounded new k/v inside attention) are listed with
their reasons in the design notes.  Every function here is pinned by the
CPU tests against library routines, closed forms, invariants and a
50-digit brute-force twin (oracle/brute.py).
"""
from __future__ import annotations

import numpy as np


# --------------------------------------------------------------------------
# storage decoding / encoding (the oracle's own; not shared with the library)
# --------------------------------------------------------------------------

def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact upcast of stored values: uint16 bf16 bits or float32 -> float64."""
    if dtype == "bf16":
        bits = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)


def round_to_storage(a: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 values to the storage type, nearest-even.

    bf16: the value is rounded directly from float64 to the 8-bit significand
    (not through float32), using numpy's own nearest-even rounding of the
    scaled significand.  Returns float64 values that are exactly
    representable in the storage type.
    """
    a = np.asarray(a, dtype=np.float64)
    if dtype == "f32":
        return a.astype(np.float32).astype(np.float64)
    if dtype != "bf16":
        raise ValueError(dtype)
    out = np.empty_like(a)
    finite = np.isfinite(a) & (a != 0)
    m, e = np.frexp(a[finite])            # a = m * 2**e, 0.5 <= |m| < 1
    # bf16 keeps 8 significant bits: scale |m| to [128, 256) and round half-even
    out[finite] = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)
    out[~finite] = a[~finite]
    return out


# --------------------------------------------------------------------------
# the steps, each on one sequence
# --------------------------------------------------------------------------

def rms_norm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """O1: x * (mean(x^2) + eps)^(-1/2) * w  (eps inside the root)."""
    ms = np.mean(x * x)
    r = 1.0 / np.sqrt(ms + eps)
    return x * r * w


def qkv_project(xh: np.ndarray, w_qkv: np.ndarray, nq: int, nkv: int, d: int):
    """O2: u = xh @ W_qkv split into q [nq, D], k [nkv, D], v [nkv, D]."""
    u = xh @ w_qkv
    q = u[: nq * d].reshape(nq, d)
    k = u[nq * d: (nq + nkv) * d].reshape(nkv, d)
    v = u[(nq + nkv) * d:].reshape(nkv, d)
    return q, k, v


def rope_angles(pos: int, d: int, theta: float) -> np.ndarray:
    """O3 angles: phi_j = pos * theta^(-2j/D) for j = 0 .. D/2-1."""
    j = np.arange(d // 2, dtype=np.float64)
    return float(pos) * theta ** (-2.0 * j / d)


def rope(z: np.ndarray, pos: int, theta: float) -> np.ndarray:
    """O3: rotate-half RoPE of rows z[..., D] at position pos.

    (z_j, z_{j+D/2}) -> (z_j cos phi_j - z_{j+D/2} sin phi_j,
                         z_{j+D/2} cos phi_j + z_j sin phi_j)
    """
    d = z.shape[-1]
    phi = rope_angles(pos, d, theta)
    c, s = np.cos(phi), np.sin(phi)
    lo, hi = z[..., : d // 2], z[..., d // 2:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)


def append_kv(k_cache: np.ndarray, v_cache: np.ndarray, pos: int,
              k_new: np.ndarray, v_new: np.ndarray):
    """O4: copies of one sequence's caches [cap, nkv, D] with row pos replaced."""
    kc, vc = k_cache.copy(), v_cache.copy()
    kc[pos] = k_new
    vc[pos] = v_new
    return kc, vc


def softmax(s: np.ndarray) -> np.ndarray:
    """Numerically safe softmax over the last axis."""
    e = np.exp(s - np.max(s, axis=-1, keepdims=True))
    return e / np.sum(e, axis=-1, keepdims=True)


def attention(q: np.ndarray, keys: np.ndarray, values: np.ndarray):
    """O5 for one sequence.

    q [nq, D]; keys, values [T, nkv, D] (all T tokens attended, the new one
    included).  Query head h reads kv head h // (nq // nkv).
    Returns (o [nq, D], probs [nq, T]).
    """
    nq, d = q.shape
    nkv = keys.shape[1]
    group = nq // nkv
    o = np.empty((nq, d))
    probs = np.empty((nq, keys.shape[0]))
    for h in range(nq):
        g = h // group
        s = keys[:, g, :] @ q[h] / np.sqrt(d)
        p = softmax(s)
        probs[h] = p
        o[h] = p @ values[:, g, :]
    return o, probs


def out_project(x: np.ndarray, a: np.ndarray, w_o: np.ndarray):
    """O6: y = a @ W_o, out = x + y."""
    y = a @ w_o
    return x + y, y


# --------------------------------------------------------------------------
# the whole step
# --------------------------------------------------------------------------

def decode_step_fp64(hidden, norm_w, w_qkv, w_o, k_cache, v_cache, pos, *,
                     n_q_heads: int, n_kv_heads: int, head_dim: int,
                     rope_theta: float, eps: float = 1e-6,
                     storage: str = "f32", want_probs: bool = False) -> dict:
    """One decode step for every sequence of a batch, in float64.

    All array arguments are float64 values (upcast with `to_f64`):
      hidden [B, H], norm_w [H], w_qkv [H, (nq+2nkv)D], w_o [nq D, H],
      k_cache, v_cache [B, cap, nkv, D]; pos int [B].
    Only rows t < pos[b] of the caches are read.  The new token's k and v
    enter attention unrounded; the rows the step writes into the caches are
    returned rounded to `storage`.

    Returns a dict of float64 arrays:
      out [B, H] (unrounded), out_stored [B, H] (rounded to storage),
      y [B, H], q [B, nq, D] (after RoPE), k_new [B, nkv, D] (after RoPE),
      v_new [B, nkv, D], k_row, v_row [B, nkv, D] (rounded, as appended),
      a [B, nq*D], and probs (list of [nq, pos_b+1]) when want_probs.
    """
    nq, nkv, d = n_q_heads, n_kv_heads, head_dim
    hidden = np.asarray(hidden, dtype=np.float64)
    B, H = hidden.shape
    cap = k_cache.shape[1]
    res = {k: [] for k in ("out", "y", "q", "k_new", "v_new", "k_row", "v_row", "a", "probs")}
    for b in range(B):
        p = int(pos[b])
        if not 0 <= p < cap:
            raise ValueError(f"pos[{b}] = {p} outside [0, {cap})")
        x = hidden[b]
        xh = rms_norm(x, norm_w, eps)
        q, k, v = qkv_project(xh, w_qkv, nq, nkv, d)
        q = rope(q, p, rope_theta)
        k = rope(k, p, rope_theta)
        keys = np.concatenate([k_cache[b, :p], k[None]], axis=0)
        vals = np.concatenate([v_cache[b, :p], v[None]], axis=0)
        o, probs = attention(q, keys, vals)
        a = o.reshape(-1)
        out, y = out_project(x, a, w_o)
        for name, val in (("out", out), ("y", y), ("q", q), ("k_new", k), ("v_new", v),
                          ("k_row", round_to_storage(k, storage)),
                          ("v_row", round_to_storage(v, storage)), ("a", a)):
            res[name].append(val)
        if want_probs:
            res["probs"].append(probs)
    result = {k: np.stack(v) for k, v in res.items() if k != "probs"}
    result["out_stored"] = round_to_storage(result["out"], storage)
    if want_probs:
        result["probs"] = res["probs"]
    return result


def decode_step_from_inputs(inp: dict, want_probs: bool = False) -> dict:
    """Convenience: run `decode_step_fp64` on a stored input set.

    `inp` holds storage arrays (see the seeded input generator) and a config
    object with n_q_heads, n_kv_heads, head_dim, rope_theta, eps and dtype.
    Only the first pos[b] rows of each cache are upcast.
    """
    cfg = inp["cfg"]
    st = cfg.dtype
    pos = np.asarray(inp["pos"])
    B = pos.shape[0]
    nkv, d = cfg.n_kv_heads, cfg.head_dim
    pmax = int(pos.max()) if B else 0
    kc = np.zeros((B, max(pmax, 1), nkv, d))
    vc = np.zeros((B, max(pmax, 1), nkv, d))
    for b in range(B):
        p = int(pos[b])
        kc[b, :p] = to_f64(inp["k_cache"][b, :p], st)
        vc[b, :p] = to_f64(inp["v_cache"][b, :p], st)
    # cache capacity seen by the oracle: enough rows for every pos
    kc = np.concatenate([kc, np.zeros((B, 1, nkv, d))], axis=1)
    vc = np.concatenate([vc, np.zeros((B, 1, nkv, d))], axis=1)
    return decode_step_fp64(
        to_f64(inp["hidden"], st), to_f64(inp["norm_w"], st),
        to_f64(inp["w_qkv"], st), to_f64(inp["w_o"], st), kc, vc, pos,
        n_q_heads=cfg.n_q_heads, n_kv_heads=nkv, head_dim=d,
        rope_theta=cfg.rope_theta, eps=cfg.eps, storage=st, want_probs=want_probs)
