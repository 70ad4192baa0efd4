"""Brute-force forward pass in pure Python float64 loops (test infrastructure).

Independent of ``oracle.py`` (no shared helpers, no NumPy arithmetic): every
dot product, norm, rotation and softmax is a Python loop over ``float``.  It
exists to pin the NumPy oracle on tiny shapes; it is far too slow for real
ones.  Only the test suite imports it.

Same definitions as the oracle (see its header for the page sections): token
embedding; per block RMSNorm, Q/K/V projection with ``[out, in]`` weights,
per-head RMSNorm of q and k, rotate-half RoPE, causal GQA softmax attention
scaled by 1/sqrt(head_dim), output projection and residual, RMSNorm, SwiGLU
FFN and residual; final RMSNorm of the last row and the tied head.
"""
from __future__ import annotations

import math


def _mat(a):
    return [[float(v) for v in row] for row in a]


def _vec(a):
    return [float(v) for v in a]


def _matvec(w, x):
    # w: list of rows [out][in]; returns w . x
    out = []
    for row in w:
        acc = 0.0
        for a, b in zip(row, x):
            acc += a * b
        out.append(acc)
    return out


def _rms(x, g, eps):
    ss = 0.0
    for v in x:
        ss += v * v
    inv = 1.0 / math.sqrt(ss / len(x) + eps)
    return [v * inv * gi for v, gi in zip(x, g)]


def _rotate(x, p, theta):
    d = len(x)
    half = d // 2
    out = list(x)
    for i in range(half):
        a = p * theta ** (-2.0 * i / d)
        c, s = math.cos(a), math.sin(a)
        out[i] = x[i] * c - x[i + half] * s
        out[i + half] = x[i + half] * c + x[i] * s
    return out


def brute_forward(shape, weights, token_ids, all_rows=False):
    """Last-token logits (or all rows) of the forward pass, in float64 loops."""
    H, nq, nkv, d = shape.hidden, shape.n_heads, shape.n_kv_heads, shape.head_dim
    eps, theta = shape.rms_eps, shape.rope_theta
    E = _mat(weights["embed"])
    rows = [list(E[int(t)]) for t in token_ids]
    S = len(rows)
    for lw in weights["layers"]:
        W = {k: (_mat(v) if getattr(v, "ndim", 1) == 2 else _vec(v)) for k, v in lw.items()}
        qs, ks, vs = [], [], []
        for p in range(S):
            xn = _rms(rows[p], W["attn_norm"], eps)
            q = _matvec(W["wq"], xn)
            k = _matvec(W["wk"], xn)
            v = _matvec(W["wv"], xn)
            qh = [_rotate(_rms(q[h * d:(h + 1) * d], W["q_norm"], eps), p, theta) for h in range(nq)]
            kh = [_rotate(_rms(k[j * d:(j + 1) * d], W["k_norm"], eps), p, theta) for j in range(nkv)]
            vh = [v[j * d:(j + 1) * d] for j in range(nkv)]
            qs.append(qh)
            ks.append(kh)
            vs.append(vh)
        new_rows = []
        for p in range(S):
            attn = []
            for h in range(nq):
                j = h // (nq // nkv)
                scores = []
                for u in range(p + 1):
                    dot = 0.0
                    for a, b in zip(qs[p][h], ks[u][j]):
                        dot += a * b
                    scores.append(dot / math.sqrt(d))
                m = max(scores)
                e = [math.exp(s - m) for s in scores]
                tot = sum(e)
                o = [0.0] * d
                for u in range(p + 1):
                    wgt = e[u] / tot
                    for i in range(d):
                        o[i] += wgt * vs[u][j][i]
                attn.extend(o)
            x = [a + b for a, b in zip(rows[p], _matvec(W["wo"], attn))]
            xn = _rms(x, W["mlp_norm"], eps)
            gt = _matvec(W["w_gate"], xn)
            up = _matvec(W["w_up"], xn)
            hmid = [(gv / (1.0 + math.exp(-gv))) * uv for gv, uv in zip(gt, up)]
            x = [a + b for a, b in zip(x, _matvec(W["w_down"], hmid))]
            new_rows.append(x)
        rows = new_rows
    gfin = _vec(weights["final_norm"])
    pick = rows if all_rows else [rows[-1]]
    out = []
    for r in pick:
        hn = _rms(r, gfin, eps)
        out.append(_matvec(E, hn))
    return out if all_rows else out[0]
