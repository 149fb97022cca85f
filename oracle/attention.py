"""Scaled dot-product attention and multi-head attention in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

The functions are split into the steps of eq. (1) so that a reader can check
each against the pages, and so that the mutation tests can replace one step
at a time with a planted mistake:

    visible  -> scores -> (mask by setting -inf) -> softmax_rows -> weighted_sum

Inputs may be any real dtype; they are upcast exactly to float64 and nothing
is rounded afterwards.
"""

import numpy as np

MASK_NONE = 0
MASK_CAUSAL = 1


def visible(n_q, n_k, mask_kind=MASK_NONE, kv_len=None):
    """Boolean [n_q, n_k]: may query row r look at key column c?

    * Causal (decoder self-attention): a position sees the positions up to
      and including itself -- agi-iri.ru §3.2.1 ("позиции ≤ текущей") and
      nickwang.xyz "Trois usages de l'attention dans le modèle" (table row
      "Auto-attention du décodeur").  So c <= r.
    * Key padding: only the first ``kv_len`` keys of the sequence exist.  The
      pages are silent on padding; it is the plain reading of a batch of
      sequences of different valid lengths.  ``kv_len`` is clamped to
      [0, n_k].
    """
    r = np.arange(n_q)[:, None]
    c = np.arange(n_k)[None, :]
    vis = np.ones((n_q, n_k), dtype=bool)
    if mask_kind == MASK_CAUSAL:
        vis &= c <= r
    elif mask_kind != MASK_NONE:
        raise ValueError(f"unknown mask kind {mask_kind}")
    if kv_len is not None:
        n = min(max(int(kv_len), 0), n_k)
        vis &= c < n
    return vis


def band(n_q, n_k, left, right):
    """Boolean [n_q, n_k]: does key c lie in the neighbourhood of query r,
    r - left <= c <= r + right?

    nickwang.xyz §4 (Table 1, the "Auto-attention restreinte" row, and the
    text after it): for very long sequences, self-attention may be
    restricted to a neighbourhood of size r centred on the output position,
    at O(r·n·d) per layer.  The window is given here by its two reaches from
    the query position: the centred neighbourhood of size 2w + 1 is
    left = right = w; left >= n_k with right = 0 sees exactly what the causal
    mask lets through.  Positions are absolute indices of the query and key
    sequences.
    """
    if left < 0 or right < 0:
        raise ValueError("window reaches must be >= 0")
    r = np.arange(n_q)[:, None]
    c = np.arange(n_k)[None, :]
    return (c >= r - int(left)) & (c <= r + int(right))


def scores(q, k, scale):
    """S = scale · Q·Kᵀ for one head (nickwang.xyz, §3.2.1 eq. (1): the
    compatibility of each query with each key is their dot product, divided
    by √d_k; the divisor is passed in as ``scale`` = 1/√d_k)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    return scale * (q @ k.T)


def softmax_rows(s, vis):
    """Row-wise softmax where forbidden scores are *set* to -inf first.

    nickwang.xyz "Trois usages ...": before the softmax every forbidden
    connection's value is set to -inf, so its weight is exactly zero.  Each
    row is a separate softmax whose weights add up to 1 (the worked figure
    "L'attention dans une phrase").  Subtracting the row maximum is exact in
    real arithmetic and keeps exp() finite in float64.  A row with no visible
    key has no defined softmax; its weights are all zero here (a reading the
    pages leave open).
    """
    s = np.where(vis, s, -np.inf)
    p = np.zeros_like(s, dtype=np.float64)
    has_key = vis.any(axis=1)
    if not has_key.any():
        return p
    sv = s[has_key]
    m = sv.max(axis=1, keepdims=True)
    with np.errstate(invalid="ignore"):
        e = np.where(vis[has_key], np.exp(sv - m), 0.0)
    p[has_key] = e / e.sum(axis=1, keepdims=True)
    return p


def weighted_sum(p, vis, v):
    """O = P·V summed over visible columns only.

    The output is the sum of the values weighted by the softmax weights
    (nickwang.xyz §3.2, the definition of attention).  A masked key has
    weight exactly zero, so it contributes nothing at all -- even when its
    value vector holds NaN or Inf, whose product with 0 would otherwise be
    NaN.  Value rows that are all finite go through one matrix product; each
    non-finite row is added only to the rows that can see it.
    """
    v = np.asarray(v, dtype=np.float64)
    finite = np.isfinite(v).all(axis=1)
    out = p @ np.where(finite[:, None], v, 0.0)
    for c in np.nonzero(~finite)[0]:
        rows = vis[:, c]
        out[rows] += p[rows, c][:, None] * v[c][None, :]
    return out


def attention_head(q, k, v, scale, mask_kind=MASK_NONE, kv_len=None, window=None):
    """One head of eq. (1): returns (O [n_q, d_v], P [n_q, n_k]).  ``window``
    is None or (left, right): restricted attention, see ``band``."""
    n_q, n_k = q.shape[0], k.shape[0]
    vis = visible(n_q, n_k, mask_kind, kv_len)
    if window is not None:
        vis = vis & band(n_q, n_k, window[0], window[1])
    s = scores(q, k, scale)
    p = softmax_rows(s, vis)
    return weighted_sum(p, vis, v), p


def sdpa(Q, K, V, scale, mask_kind=MASK_NONE, seq_lens=None, window=None):
    """Batched scaled dot-product attention, float64.

    Q [B, h, n_q, d_k], K [B, h, n_k, d_k], V [B, h, n_k, d_v] (any real
    dtype, upcast exactly).  ``seq_lens`` is None or B integers: the valid key
    count of each batch entry.  ``window`` is None or (left, right), the
    restricted attention of ``band``.  Returns O [B, h, n_q, d_v] float64.
    Every (batch, head) pair is an independent eq. (1).
    """
    Q = np.asarray(Q)
    K = np.asarray(K)
    V = np.asarray(V)
    B, h, n_q, _ = Q.shape
    d_v = V.shape[3]
    out = np.zeros((B, h, n_q, d_v), dtype=np.float64)
    for b in range(B):
        kv_len = None if seq_lens is None else int(seq_lens[b])
        for i in range(h):
            out[b, i], _ = attention_head(Q[b, i], K[b, i], V[b, i], scale,
                                          mask_kind, kv_len, window)
    return out


def mha(x_q, x_kv, Wq, Wk, Wv, Wo, h, mask_kind=MASK_NONE, kv_lens=None):
    """Multi-head attention sublayer, float64.

    nickwang.xyz "Attention multi-têtes" (paper §3.2.2):
      MultiHead = Concat(head_1..head_h)·W^O,
      head_i    = Attention(x_q·W_i^Q, x_kv·W_i^K, x_kv·W_i^V),
    with W_i^Q, W_i^K ∈ R^{d_model×d_k}, W_i^V ∈ R^{d_model×d_v} and
    W^O ∈ R^{h·d_v×d_model}.  The h per-head matrices sit side by side as
    the column blocks of one [d_model, h·d] matrix, head i taking columns
    [i·d, (i+1)·d) (ml-canon "32 Transformer", the PyTorch sketch splits the
    projected rows into h pieces in order); W^O's row blocks follow the same
    head order, which is the order of the concat.  Queries come from x_q,
    keys and values from x_kv: x_kv is x_q for self-attention and the encoder
    output for encoder-decoder attention (nickwang.xyz "Trois usages ...").
    No bias, no dropout, no residual or normalisation: those are outside the
    sublayer's attention function.

    x_q [B, n_q, d_model]; x_kv [B, n_k, d_model] or None (self-attention);
    returns [B, n_q, d_model] float64.
    """
    x_q = np.asarray(x_q, dtype=np.float64)
    x_kv = x_q if x_kv is None else np.asarray(x_kv, dtype=np.float64)
    Wq = np.asarray(Wq, dtype=np.float64)
    Wk = np.asarray(Wk, dtype=np.float64)
    Wv = np.asarray(Wv, dtype=np.float64)
    Wo = np.asarray(Wo, dtype=np.float64)
    B, n_q, _ = x_q.shape
    d_k = Wq.shape[1] // h
    d_v = Wv.shape[1] // h
    scale = 1.0 / np.sqrt(d_k)
    out = np.zeros((B, n_q, Wo.shape[1]), dtype=np.float64)
    for b in range(B):
        q_all = x_q[b] @ Wq
        k_all = x_kv[b] @ Wk
        v_all = x_kv[b] @ Wv
        kv_len = None if kv_lens is None else int(kv_lens[b])
        heads = []
        for i in range(h):
            o, _ = attention_head(q_all[:, i * d_k:(i + 1) * d_k],
                                  k_all[:, i * d_k:(i + 1) * d_k],
                                  v_all[:, i * d_v:(i + 1) * d_v],
                                  scale, mask_kind, kv_len)
            heads.append(o)
        concat = np.concatenate(heads, axis=1)
        out[b] = concat @ Wo
    return out
