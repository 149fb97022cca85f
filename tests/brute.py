"""Scalar brute-force attention for tiny shapes (test helper).

Deliberately written with a different formula from the oracle, so that the
two agree only if both compute eq. (1) of nickwang.xyz "Lire « Attention Is
All You Need »" §3.2.1:

* the mask is a per-element predicate evaluated inside the loops (no boolean
  matrix);
* each weight is 1 / Σ_c' exp(s_c' − s_c) over the visible c' (no row max,
  no division of exponentials);
* the output is accumulated one visible key at a time with Python floats.
"""

import math


def _dot(a, b):
    t = 0.0
    for x, y in zip(a, b):
        t += float(x) * float(y)
    return t


def head(q, k, v, scale, causal, kv_len, window=None):
    n_q, n_k, d_v = len(q), len(k), len(v[0]) if len(v) else 0
    lim = n_k if kv_len is None else min(max(int(kv_len), 0), n_k)
    out = [[0.0] * d_v for _ in range(n_q)]
    for r in range(n_q):
        cols = [c for c in range(n_k) if c < lim and (not causal or c <= r)
                and (window is None or (abs(c - r) <= window[0] if c < r else c - r <= window[1]))]
        s = {c: scale * _dot(q[r], k[c]) for c in cols}
        for c in cols:
            w = 1.0 / sum(math.exp(s[c2] - s[c]) for c2 in cols)
            for j in range(d_v):
                out[r][j] += w * float(v[c][j])
    return out


def sdpa(Q, K, V, scale, causal=False, seq_lens=None, window=None):
    """Q, K, V nested lists or arrays [B][h][n][d]; returns nested lists.
    ``window`` (left, right): key c within left positions before or right
    positions after the query (restricted attention)."""
    out = []
    for b in range(len(Q)):
        kv_len = None if seq_lens is None else seq_lens[b]
        out.append([head(Q[b][i], K[b][i], V[b][i], scale, causal, kv_len, window)
                    for i in range(len(Q[b]))])
    return out


def mha(x_q, x_kv, Wq, Wk, Wv, Wo, h, causal=False, kv_lens=None):
    """Scalar multi-head attention with explicit index arithmetic."""
    x_kv = x_q if x_kv is None else x_kv
    d_model = len(Wq)
    d_k = len(Wq[0]) // h
    d_v = len(Wv[0]) // h
    scale = 1.0 / math.sqrt(d_k)

    def proj(x, W, col0, width):
        return [[sum(float(x[t][m]) * float(W[m][col0 + j]) for m in range(d_model))
                 for j in range(width)] for t in range(len(x))]

    out = []
    for b in range(len(x_q)):
        kv_len = None if kv_lens is None else kv_lens[b]
        n_q = len(x_q[b])
        d_out = len(Wo[0])
        acc = [[0.0] * d_out for _ in range(n_q)]
        for i in range(h):
            o = head(proj(x_q[b], Wq, i * d_k, d_k), proj(x_kv[b], Wk, i * d_k, d_k),
                     proj(x_kv[b], Wv, i * d_v, d_v), scale, causal, kv_len)
            # concat·Wo restricted to head i's rows of Wo
            for t in range(n_q):
                for c in range(d_out):
                    acc[t][c] += sum(o[t][j] * float(Wo[i * d_v + j][c]) for j in range(d_v))
        out.append(acc)
    return out
