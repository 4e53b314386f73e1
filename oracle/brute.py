"""50-digit brute-force twins of the decode-block and FFN oracles, for tiny shapes.

TEST INFRASTRUCTURE ONLY (imported by the CPU tests, never by the library).

Written independently of oracle/decode_step.py: explicit scalar loops over
mpmath numbers, no numpy arithmetic, no shared helpers.  It follows the same
statement of the block (RMSNorm with eps inside the root, one packed
[Q | K | V] projection, rotate-half RoPE with angle pos * theta^(-2j/D),
append of the new token, softmax attention with scale 1/sqrt(D) over the
history and the new token, output projection plus residual), as described
in the oracle's header, so that an indexing slip in either one shows up as a
disagreement.
"""
from __future__ import annotations

import mpmath

mp = mpmath.mp


def decode_step_brute(hidden, norm_w, w_qkv, w_o, k_hist, v_hist, pos, *,
                      n_q_heads, n_kv_heads, head_dim, rope_theta, eps, digits=50):
    """One sequence.  Plain nested lists (or anything indexable) of floats.

    hidden [H], norm_w [H], w_qkv [H][(nq+2nkv)D], w_o [nq*D][H],
    k_hist, v_hist [pos][nkv][D]  (the cached tokens before the new one).
    Returns dict of nested lists of mpf: out [H], y [H], q [nq][D] (rotated),
    k [nkv][D] (rotated), v [nkv][D], probs [nq][pos+1].
    """
    with mpmath.workdps(digits):
        f = mpmath.mpf
        H = len(hidden)
        nq, nkv, D = n_q_heads, n_kv_heads, head_dim
        x = [f(hidden[i]) for i in range(H)]

        # RMSNorm
        acc = f(0)
        for i in range(H):
            acc += x[i] * x[i]
        scale = 1 / mpmath.sqrt(acc / H + f(eps))
        xn = [x[i] * scale * f(norm_w[i]) for i in range(H)]

        # packed projection, column by column
        ncol = (nq + 2 * nkv) * D
        u = []
        for c in range(ncol):
            s = f(0)
            for i in range(H):
                s += xn[i] * f(w_qkv[i][c])
            u.append(s)
        q = [[u[h * D + e] for e in range(D)] for h in range(nq)]
        k = [[u[nq * D + g * D + e] for e in range(D)] for g in range(nkv)]
        v = [[u[(nq + nkv) * D + g * D + e] for e in range(D)] for g in range(nkv)]

        # rotate-half RoPE
        half = D // 2

        def rotate(vec):
            res = [None] * D
            for j in range(half):
                ang = f(pos) * mpmath.power(f(rope_theta), -f(2 * j) / D)
                c, s_ = mpmath.cos(ang), mpmath.sin(ang)
                a, b = vec[j], vec[j + half]
                res[j] = a * c - b * s_
                res[j + half] = b * c + a * s_
            return res

        q = [rotate(q[h]) for h in range(nq)]
        k = [rotate(k[g]) for g in range(nkv)]

        # attention over pos history tokens plus the new one
        group = nq // nkv
        att = []
        probs = []
        for h in range(nq):
            g = h // group
            scores = []
            for t in range(pos + 1):
                key = k[g] if t == pos else [f(k_hist[t][g][e]) for e in range(D)]
                dot = f(0)
                for e in range(D):
                    dot += q[h][e] * key[e]
                scores.append(dot / mpmath.sqrt(D))
            top = max(scores)
            ex = [mpmath.exp(s - top) for s in scores]
            tot = f(0)
            for e_ in ex:
                tot += e_
            pr = [e_ / tot for e_ in ex]
            probs.append(pr)
            o = []
            for e in range(D):
                s = f(0)
                for t in range(pos + 1):
                    val = v[g][e] if t == pos else f(v_hist[t][g][e])
                    s += pr[t] * val
                o.append(s)
            att.extend(o)

        # output projection and residual
        y = []
        for c in range(H):
            s = f(0)
            for r in range(nq * D):
                s += att[r] * f(w_o[r][c])
            y.append(s)
        out = [x[c] + y[c] for c in range(H)]
        return {"out": out, "y": y, "q": q, "k": k, "v": v, "probs": probs}


def ffn_step_brute(hidden, norm_w, w_gate, w_up, w_down, *, eps, digits=50):
    """The FFN half for one sequence, in explicit loops over mpmath numbers.

    hidden [H], norm_w [H], w_gate [H][F], w_up [H][F], w_down [F][H].
    Returns dict of lists of mpf: out [H], y [H], m [F].  The gate is
    written from its definition, z / (1 + e^-z).
    """
    with mpmath.workdps(digits):
        f = mpmath.mpf
        H, F = len(hidden), len(w_gate[0])
        h = [f(hidden[i]) for i in range(H)]
        sq = f(0)
        for i in range(H):
            sq += h[i] * h[i]
        r = 1 / mpmath.sqrt(sq / H + f(eps))
        hn = [h[i] * r * f(norm_w[i]) for i in range(H)]
        m = []
        for c in range(F):
            g = f(0)
            u = f(0)
            for i in range(H):
                g += hn[i] * f(w_gate[i][c])
                u += hn[i] * f(w_up[i][c])
            m.append(g / (1 + mpmath.exp(-g)) * u)
        y = []
        for c in range(H):
            s = f(0)
            for j in range(F):
                s += m[j] * f(w_down[j][c])
            y.append(s)
        return {"out": [h[c] + y[c] for c in range(H)], "y": y, "m": m}


def mla_decode_brute(q_lat, q_rope, c_hist, kr_hist, c_new, kr_new, *, scale, digits=50):
    """Latent attention decode for one sequence, in explicit loops over mpmath numbers.

    q_lat [nh][R], q_rope [nh][P], c_hist [pos][R], kr_hist [pos][P] (the cached tokens), c_new [R],
    kr_new [P].  Head h scores token t as (q_lat_h . c_t + q_rope_h . kr_t) * scale over the history and
    the new token, and returns the softmax-weighted sum of the latent rows c_t.
    Returns dict: out [nh][R], probs [nh][pos+1].
    """
    with mpmath.workdps(digits):
        f = mpmath.mpf
        nh, R, P = len(q_lat), len(c_new), len(kr_new)
        pos = len(c_hist)

        def row_c(t):
            return c_new if t == pos else c_hist[t]

        def row_r(t):
            return kr_new if t == pos else kr_hist[t]

        out, probs = [], []
        for h in range(nh):
            sc = []
            for t in range(pos + 1):
                s = f(0)
                ct, rt = row_c(t), row_r(t)
                for e in range(R):
                    s += f(q_lat[h][e]) * f(ct[e])
                for e in range(P):
                    s += f(q_rope[h][e]) * f(rt[e])
                sc.append(s * f(scale))
            top = max(sc)
            ex = [mpmath.exp(s - top) for s in sc]
            tot = f(0)
            for e_ in ex:
                tot += e_
            pr = [e_ / tot for e_ in ex]
            probs.append(pr)
            o = []
            for e in range(R):
                s = f(0)
                for t in range(pos + 1):
                    s += pr[t] * f(row_c(t)[e])
                o.append(s)
            out.append(o)
        return {"out": out, "probs": probs}
