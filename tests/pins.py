"""Pins: facts the pages or mathematics fix about attention, as reusable
checks.

Each ``pin_*`` takes an implementation and raises AssertionError when it
disagrees with the fact.  The same pins check the fp64 oracle (tight
tolerance, ``tests/test_oracle_pins.py``), catch planted mistakes in copies
of the oracle (``tests/test_oracle_mutants.py``) and re-run through the HIP
library on the GPU (``tests/test_sdpa_gpu.py``, ``tests/test_mha_gpu.py``),
where the inputs are first rounded to the device dtype.

Implementation signatures:
  sdpa_fn(Q, K, V, scale, mask_kind, seq_lens) -> ndarray [B, h, n_q, d_v]
  mha_fn(x_q, x_kv, Wq, Wk, Wv, Wo, h, mask_kind, kv_lens) -> [B, n_q, d_model]
  add_norm_fn(x, sub, gamma, beta, eps) -> [rows, d]   (LayerNorm(x + sub))
  window_fn(Q, K, V, scale, left, right, seq_lens) -> [B, h, n_q, d_v]
      (restricted attention: key c visible to query r iff r-left <= c <= r+right)
Inputs are float64 numpy arrays; an implementation that stores lower
precision rounds them itself, and ``rnd`` (a function array -> array) lets a
pin build its expected value from the rounded inputs.

Page references (title, section):
  [N] nickwang.xyz, "Lire « Attention Is All You Need » : l'article original
      du Transformer"
  [A] agi-iri.ru, "Attention Is All You Need (на русском)"
  [M] ml-canon.vercel.app, "32 Transformer"
"""

import json
import math
import os

import numpy as np

NONE, CAUSAL = 0, 1
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _ident(x):
    return x


def _close(a, b, atol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} != {b.shape}"
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert np.all(np.isfinite(a)), f"{what}: non-finite output"
    assert err <= atol, f"{what}: max-abs error {err:.3g} > {atol:.3g}"


def worked_example():
    with open(os.path.join(GOLDEN, "worked_example_il.json"), encoding="utf-8") as f:
        return json.load(f)


# ----------------------------------------------------------------- SDPA pins

def pin_worked_example(sdpa_fn, pad_to=None, sum_atol=1e-12):
    """[N] "Attention par produit scalaire mis à l'échelle", figure
    "L'attention dans une phrase": query "il" = [2.2, 0] against seven 2-d
    keys, scores divided by √2.  With V = identity, the output row is the
    weight vector.  Checks the printed weights at their printed precision,
    and the printed scores through log(w_c / w_car) = s_c − s_car, s_car = 0.
    ``pad_to`` zero-pads q and k to that many dims (scores unchanged);
    ``sum_atol`` is how far from 1 the weights may add up."""
    g = worked_example()
    d = g["d_k"] if pad_to is None else pad_to
    n = len(g["keys"])
    Q = np.zeros((1, 1, 1, d))
    K = np.zeros((1, 1, n, d))
    Q[0, 0, 0, :2] = g["query"]
    K[0, 0, :, :2] = g["keys"]
    dv = max(n, d if pad_to else n)
    V = np.zeros((1, 1, n, dv))
    V[0, 0, :, :n] = np.eye(n)
    w = np.asarray(sdpa_fn(Q, K, V, g["scale"], NONE, None))[0, 0, 0, :n]
    pct = 100.0 * w
    for c in range(n):
        dec = g["printed_weights_decimals"][c]
        half = 0.5 * 10.0 ** (-dec)
        assert abs(pct[c] - g["printed_weights_percent"][c]) <= half + 1e-9, (
            f"weight of {g['words'][c]}: {pct[c]:.4f}% vs printed "
            f"{g['printed_weights_percent'][c]}%")
    car = g["words"].index("car")
    for c in range(n):
        s = math.log(w[c] / w[car])
        assert abs(s - g["printed_scores"][c]) <= 0.005 + 1e-9, (
            f"score of {g['words'][c]}: {s:.4f} vs printed {g['printed_scores'][c]}")
    assert abs(w.sum() - 1.0) <= sum_atol
    return w


def pin_worked_example_causal(sdpa_fn, sum_atol=1e-12):
    """The same figure with its causal toggle: the query "il" at position 4
    sees the first five words only ([A] §3.2.1: positions ≤ the current one).
    Its weights must be the printed unmasked weights of those five words,
    renormalised -- checked to the precision the printed percentages carry
    (relative error ≤ 0.5/2.9 on the smallest one)."""
    g = worked_example()
    n = len(g["keys"])
    qi = g["query_index"]
    Q = np.zeros((1, 1, n, 2))
    Q[0, 0, qi] = g["query"]
    K = np.zeros((1, 1, n, 2))
    K[0, 0] = g["keys"]
    V = np.zeros((1, 1, n, n))
    V[0, 0] = np.eye(n)
    w = np.asarray(sdpa_fn(Q, K, V, g["scale"], CAUSAL, None))[0, 0, qi]
    assert np.all(w[qi + 1:] == 0.0), "causal: a later word got weight"
    printed = np.asarray(g["printed_weights_percent"][:qi + 1], dtype=np.float64)
    expect = printed / printed.sum()
    rel = np.abs(w[:qi + 1] - expect) / expect
    assert np.all(rel <= 0.5 / 2.9 * 1.05), f"renormalised weights {w} vs {expect}"
    # each row of the causal figure is its own softmax over a prefix
    w_all = np.asarray(sdpa_fn(Q, K, V, g["scale"], CAUSAL, None))[0, 0]
    np.testing.assert_allclose(w_all.sum(axis=1), 1.0, atol=sum_atol)


def pin_saturation(sdpa_fn):
    """[N] same section: with d_k = 64 and two keys whose unscaled scores are
    8 and 0, the softmax gives ≈0.9997 (derivative p(1−p) ≈ 0.0003); divided
    by 8 the scores become 1 and 0 and the weights ≈0.73 / 0.27 (derivative
    ≈0.20).  Closed form: the weights are σ(8), σ(−8) and σ(1), σ(−1)."""
    d = 64
    Q = np.zeros((1, 1, 1, d))
    Q[0, 0, 0, 0] = 8.0
    K = np.zeros((1, 1, 2, d))
    K[0, 0, 0, 0] = 1.0   # q·k1 = 8
    K[0, 0, 1, 1] = 1.0   # q·k2 = 0
    V = np.zeros((1, 1, 2, d))
    V[0, 0, 0, 0] = 1.0
    V[0, 0, 1, 1] = 1.0
    sig = lambda x: 1.0 / (1.0 + math.exp(-x))  # noqa: E731
    p_raw = np.asarray(sdpa_fn(Q, K, V, 1.0, NONE, None))[0, 0, 0, :2]
    p_scl = np.asarray(sdpa_fn(Q, K, V, 1.0 / math.sqrt(d), NONE, None))[0, 0, 0, :2]
    np.testing.assert_allclose(p_raw, [sig(8), sig(-8)], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(p_scl, [sig(1), sig(-1)], rtol=1e-12)
    assert round(p_raw[0], 4) == 0.9997
    assert round(p_raw[0] * (1 - p_raw[0]), 4) == 0.0003
    assert (round(p_scl[0], 2), round(p_scl[1], 2)) == (0.73, 0.27)
    assert round(p_scl[0] * (1 - p_scl[0]), 2) == 0.20


def _rand(rs, *shape):
    return rs.standard_normal(shape)


def pin_rows_sum_to_one(sdpa_fn, atol=1e-12, rnd=_ident, shapes=((2, 3, 9, 9, 8),)):
    """Each row is a softmax that totals 100 % ([N] figure; [M] "строки
    суммируются в 1"): with V = 1 everywhere, O = 1 everywhere, for every
    mask and key length ≥ 1."""
    rs = np.random.default_rng(11)
    for (B, h, nq, nk, d) in shapes:
        Q, K = rnd(_rand(rs, B, h, nq, d)), rnd(_rand(rs, B, h, nk, d))
        V = np.ones((B, h, nk, d))
        for mask in (NONE, CAUSAL) if nq == nk else (NONE,):
            for lens in (None, rs.integers(1, nk + 1, size=B)):
                O = sdpa_fn(Q, K, V, 1.0 / math.sqrt(d), mask, lens)
                _close(O, np.ones_like(O), atol, f"V=1 mask={mask} lens={lens}")


def _visible_mean(V, mask, kv_len):
    n_k = V.shape[0]
    lim = n_k if kv_len is None else min(max(int(kv_len), 0), n_k)
    rows = []
    for r in range(V.shape[0] if mask == CAUSAL else 1):
        top = min(lim, r + 1) if mask == CAUSAL else lim
        rows.append(V[:top].mean(axis=0) if top > 0 else np.zeros(V.shape[1]))
    return np.stack(rows)


def pin_zero_query_is_mean(sdpa_fn, atol=1e-12, rnd=_ident):
    """Q = 0 (or scale = 0) makes every visible score equal, so the weights
    are uniform and O is the plain mean of the visible V rows: the prefix
    mean under the causal mask, the mean of the first len rows with key
    padding."""
    rs = np.random.default_rng(12)
    B, h, n, d = 3, 2, 10, 8
    K, V = rnd(_rand(rs, B, h, n, d)), rnd(_rand(rs, B, h, n, d))
    Qz = np.zeros((B, h, n, d))
    Qr = rnd(_rand(rs, B, h, n, d))
    lens = np.array([1, 7, 10])
    for mask in (NONE, CAUSAL):
        for ln in (None, lens):
            for (Q, scale) in ((Qz, 0.125), (Qr, 0.0)):
                O = np.asarray(sdpa_fn(Q, K, V, scale, mask, ln))
                for b in range(B):
                    for i in range(h):
                        m = _visible_mean(V[b, i], mask, None if ln is None else ln[b])
                        exp = np.broadcast_to(m, O[b, i].shape)
                        _close(O[b, i], exp, atol, f"uniform mask={mask} lens={ln}")


def pin_causal_row0(sdpa_fn, atol=0.0, rnd=_ident):
    """Under the causal mask the first position sees only itself ([A]
    §3.2.1), so its output is V[0] exactly."""
    rs = np.random.default_rng(13)
    B, h, n, d = 2, 2, 12, 8
    Q, K, V = (rnd(_rand(rs, B, h, n, d)) for _ in range(3))
    O = np.asarray(sdpa_fn(Q, K, V, 0.3, CAUSAL, None))
    _close(O[:, :, 0, :], V[:, :, 0, :], atol, "causal row 0")


def pin_permutation(sdpa_fn, atol=1e-12, rnd=_ident):
    """Without positional information attention sees a bag of tokens ([M],
    "Positional encodings" and the closing questions).  Unmasked
    self-attention: permuting the rows of Q, K and V permutes the output rows
    the same way.  Any unmasked attention: a joint permutation of the K and V
    rows leaves the output unchanged (also with n_q ≠ n_k)."""
    rs = np.random.default_rng(14)
    B, h, n, d = 2, 2, 11, 8
    Q, K, V = (rnd(_rand(rs, B, h, n, d)) for _ in range(3))
    perm = rs.permutation(n)
    O = np.asarray(sdpa_fn(Q, K, V, 0.35, NONE, None))
    Op = np.asarray(sdpa_fn(Q[:, :, perm], K[:, :, perm], V[:, :, perm], 0.35, NONE, None))
    _close(Op, O[:, :, perm], atol, "row permutation equivariance")
    Qc = rnd(_rand(rs, B, h, 5, d))
    Oc = np.asarray(sdpa_fn(Qc, K, V, 0.35, NONE, None))
    Ocp = np.asarray(sdpa_fn(Qc, K[:, :, perm], V[:, :, perm], 0.35, NONE, None))
    _close(Ocp, Oc, atol, "joint K/V permutation invariance")


def pin_one_hot(sdpa_fn, atol=1e-9, rnd=_ident, d=8):
    """Large scores push the softmax to a one-hot distribution ([N] §3.2.1
    discussion of saturation): with keys scaled up strongly and a unique
    best key by a clear margin, O tends to the V row of the best key."""
    rs = np.random.default_rng(15)
    B, h, nq, nk = 1, 2, 6, 9
    Q = rnd(_rand(rs, B, h, nq, d))
    K = rnd(_rand(rs, B, h, nk, d))
    V = rnd(_rand(rs, B, h, nk, d))
    c = 1.0
    while True:   # grow the key scale until every row's winner leads by ≥ 60
        Kc = rnd(K * c)
        s = np.einsum("bhqd,bhkd->bhqk", Q, Kc)
        srt = np.sort(s, axis=-1)
        margin = float((srt[..., -1] - srt[..., -2]).min())
        if margin >= 60.0 or c > 1e6:
            break
        c *= 2.0
    assert margin >= 60.0
    O = np.asarray(sdpa_fn(Q, Kc, V, 1.0, NONE, None))
    best = np.argmax(s, axis=-1)                         # [B, h, nq]
    exp = np.stack([[V[b, i][best[b, i]] for i in range(h)] for b in range(B)])
    _close(O, exp, atol, "one-hot limit")


def pin_mask_reduces(sdpa_fn, atol=1e-12, rnd=_ident):
    """Masking only removes keys: causal row r equals unmasked attention of
    q_r against K[:r+1], V[:r+1]; a padded entry equals unmasked attention
    against K[:len], V[:len]."""
    rs = np.random.default_rng(16)
    B, h, n, d = 2, 2, 9, 8
    Q, K, V = (rnd(_rand(rs, B, h, n, d)) for _ in range(3))
    Oc = np.asarray(sdpa_fn(Q, K, V, 0.4, CAUSAL, None))
    for r in range(n):
        Or = np.asarray(sdpa_fn(Q[:, :, r:r + 1], K[:, :, :r + 1], V[:, :, :r + 1], 0.4, NONE, None))
        _close(Oc[:, :, r:r + 1], Or, atol, f"causal row {r}")
    lens = np.array([3, 9])
    Op = np.asarray(sdpa_fn(Q, K, V, 0.4, NONE, lens))
    for b in range(B):
        L = lens[b]
        Ob = np.asarray(sdpa_fn(Q[b:b + 1], K[b:b + 1, :, :L], V[b:b + 1, :, :L], 0.4, NONE, None))
        _close(Op[b:b + 1], Ob, atol, f"padding len={L}")


def pin_masked_contents_ignored(sdpa_fn, atol=0.0, rnd=_ident):
    """A forbidden score is set to −∞ and gets weight exactly zero ([N]
    "Trois usages ..."), so whatever the masked K and V rows hold -- NaN and
    Inf included -- the output is unchanged and finite."""
    rs = np.random.default_rng(17)
    B, h, n, d = 2, 2, 10, 8
    Q, K, V = (rnd(_rand(rs, B, h, n, d)) for _ in range(3))
    lens = np.array([4, 7])
    O = np.asarray(sdpa_fn(Q, K, V, 0.3, NONE, lens))
    K2, V2 = K.copy(), V.copy()
    for b in range(B):
        K2[b, :, lens[b]:, ::2] = np.nan
        K2[b, :, lens[b]:, 1::2] = np.inf
        V2[b, :, lens[b]:] = np.nan
    O2 = np.asarray(sdpa_fn(Q, K2, V2, 0.3, NONE, lens))
    _close(O2, O, atol, "NaN in padded keys")


def pin_shift_invariance(sdpa_fn, atol=1e-10, rnd=_ident, big=1000.0):
    """Adding the same vector u to every key adds q·u to a whole row of
    scores, and a softmax does not change under a constant shift of its
    row.  A large shift (|q·u| ≈ ``big``) also checks that the softmax is
    evaluated without overflow."""
    rs = np.random.default_rng(18)
    B, h, n, d = 1, 2, 8, 8
    Q, K, V = (rnd(_rand(rs, B, h, n, d)) for _ in range(3))
    Q = np.abs(Q) + 0.5
    u = np.full(d, big / d)
    for mask in (NONE, CAUSAL):
        O = np.asarray(sdpa_fn(Q, K, V, 1.0, mask, None))
        Os = np.asarray(sdpa_fn(Q, K + u, V, 1.0, mask, None))
        _close(Os, O, atol, f"shift invariance mask={mask}")


def pin_linear_in_v(sdpa_fn, atol=1e-12, rnd=_ident):
    """O is linear in V: O(αV₁ + βV₂) = αO(V₁) + βO(V₂)."""
    rs = np.random.default_rng(19)
    B, h, n, d = 2, 2, 7, 8
    Q, K, V1, V2 = (rnd(_rand(rs, B, h, n, d)) for _ in range(4))
    a, b = 0.75, -2.5
    for mask in (NONE, CAUSAL):
        O1 = np.asarray(sdpa_fn(Q, K, V1, 0.3, mask, None))
        O2 = np.asarray(sdpa_fn(Q, K, V2, 0.3, mask, None))
        O12 = np.asarray(sdpa_fn(Q, K, a * V1 + b * V2, 0.3, mask, None))
        _close(O12, a * O1 + b * O2, atol, f"linearity mask={mask}")


def pin_empty_rows(sdpa_fn):
    """A key length of 0 leaves a row nothing to attend to; the pages are
    silent and the reading taken is an all-zero output (never NaN)."""
    rs = np.random.default_rng(20)
    Q, K, V = (_rand(rs, 2, 1, 4, 8) for _ in range(3))
    O = np.asarray(sdpa_fn(Q, K, V, 0.3, NONE, np.array([0, 4])))
    assert np.all(O[0] == 0.0), "len = 0 must give zero rows"
    assert np.all(np.isfinite(O[1]))


SDPA_PINS = [pin_worked_example, pin_worked_example_causal, pin_saturation,
             pin_rows_sum_to_one, pin_zero_query_is_mean, pin_causal_row0,
             pin_permutation, pin_one_hot, pin_mask_reduces,
             pin_masked_contents_ignored, pin_shift_invariance,
             pin_linear_in_v, pin_empty_rows]


# ------------------------------------------------------------------ MHA pins

def _mha_inputs(rs, B, n_q, n_k, d_model, cross):
    x_q = _rand(rs, B, n_q, d_model)
    x_kv = _rand(rs, B, n_k, d_model) if cross else None
    W = [_rand(rs, d_model, d_model) / math.sqrt(d_model) for _ in range(4)]
    return x_q, x_kv, W


def pin_mha_shapes(mha_fn):
    """[N] "Attention multi-têtes": a 10-token sentence, 10×512 in, eight
    heads of 10×64, concat back to 10×512, times the 512×512 W^O; the
    sublayer holds four 512×512 matrices = 1,048,576 weights."""
    rs = np.random.default_rng(30)
    x_q, _, W = _mha_inputs(rs, 1, 10, 10, 512, False)
    assert sum(w.size for w in W) == 1_048_576
    out = np.asarray(mha_fn(x_q, None, *W, 8, NONE, None))
    assert out.shape == (1, 10, 512)
    assert np.all(np.isfinite(out))


def pin_mha_head_blocks(mha_fn, sdpa_fn, atol=1e-10):
    """Concat(head_1..head_h)·W^O = Σ_i head_i·W^O[i·d_v:(i+1)·d_v, :], where
    head_i is attention on the i-th column blocks of the projections ([N]
    "Attention multi-têtes", eq. for MultiHead; [M] sketch splits columns in
    head order).  Pins the head order of both the split and the concat."""
    rs = np.random.default_rng(31)
    B, n, d_model, h = 2, 6, 32, 4
    d = d_model // h
    for cross in (False, True):
        n_k = 9 if cross else n
        x_q, x_kv, (Wq, Wk, Wv, Wo) = _mha_inputs(rs, B, n, n_k, d_model, cross)
        xkv = x_q if x_kv is None else x_kv
        out = np.asarray(mha_fn(x_q, x_kv, Wq, Wk, Wv, Wo, h, NONE, None))
        exp = np.zeros_like(out)
        for i in range(h):
            sl = slice(i * d, (i + 1) * d)
            Q = (x_q @ Wq[:, sl])[:, None]
            K = (xkv @ Wk[:, sl])[:, None]
            V = (xkv @ Wv[:, sl])[:, None]
            head = np.asarray(sdpa_fn(Q, K, V, 1.0 / math.sqrt(d), NONE, None))[:, 0]
            exp += head @ Wo[sl, :]
        _close(out, exp, atol, f"head block identity cross={cross}")


def pin_mha_head_permutation(mha_fn, atol=1e-10):
    """Relabelling the heads -- permuting the column blocks of W^Q, W^K, W^V
    and the row blocks of W^O together -- leaves the sublayer unchanged."""
    rs = np.random.default_rng(32)
    B, n, d_model, h = 2, 5, 32, 4
    d = d_model // h
    x_q, _, (Wq, Wk, Wv, Wo) = _mha_inputs(rs, B, n, n, d_model, False)
    perm = [2, 0, 3, 1]
    cols = np.concatenate([np.arange(p * d, (p + 1) * d) for p in perm])
    out = np.asarray(mha_fn(x_q, None, Wq, Wk, Wv, Wo, h, CAUSAL, None))
    outp = np.asarray(mha_fn(x_q, None, Wq[:, cols], Wk[:, cols], Wv[:, cols], Wo[cols, :],
                             h, CAUSAL, None))
    _close(outp, out, atol, "head relabelling")


def pin_mha_single_head(mha_fn, sdpa_fn, atol=1e-10):
    """[N] Table 3 rows (A): h = 1 is one head of full width d_k = d_model,
    so the sublayer is one attention with scale 1/√d_model, then W^O."""
    rs = np.random.default_rng(33)
    B, n, d_model = 2, 7, 16
    x_q, _, (Wq, Wk, Wv, Wo) = _mha_inputs(rs, B, n, n, d_model, False)
    out = np.asarray(mha_fn(x_q, None, Wq, Wk, Wv, Wo, 1, NONE, None))
    Q, K, V = ((x_q @ W)[:, None] for W in (Wq, Wk, Wv))
    o = np.asarray(sdpa_fn(Q, K, V, 1.0 / math.sqrt(d_model), NONE, None))[:, 0]
    _close(out, o @ Wo, atol, "h = 1")


MHA_PINS = [pin_mha_shapes, pin_mha_head_blocks, pin_mha_head_permutation,
            pin_mha_single_head]


# ---- restricted attention ([N] §4: Table 1's "Auto-attention restreinte"
# row and the text after it -- a neighbourhood of the output position)

def _qkv(rs, B, h, n_q, n_k, d, rnd):
    return (rnd(rs.standard_normal((B, h, n_q, d))), rnd(rs.standard_normal((B, h, n_k, d))),
            rnd(rs.standard_normal((B, h, n_k, d))))


def pin_window_covering_is_unmasked(window_fn, sdpa_fn, atol=1e-12, rnd=_ident):
    """A window that reaches every key is plain attention (with and without
    key padding)."""
    rs = np.random.RandomState(21)
    Q, K, V = _qkv(rs, 2, 2, 9, 13, 8, rnd)
    for lens in (None, [5, 13]):
        _close(window_fn(Q, K, V, 0.3, 13, 13, lens), sdpa_fn(Q, K, V, 0.3, NONE, lens), atol,
               f"covering window, lens {lens}")


def pin_window_left_unbounded_is_causal(window_fn, sdpa_fn, atol=1e-12, rnd=_ident):
    """Reaching back to the first key and not forward at all is the causal
    mask."""
    rs = np.random.RandomState(22)
    Q, K, V = _qkv(rs, 1, 3, 11, 11, 8, rnd)
    _close(window_fn(Q, K, V, 0.5, 11, 0, None), sdpa_fn(Q, K, V, 0.5, CAUSAL, None), atol,
           "window (n, 0)")


def pin_window_zero_width(window_fn, atol=1e-12, rnd=_ident):
    """Window (0, 0): query r sees key r alone, weight 1, so O[r] = V[r];
    query rows past the last key see nothing and give 0."""
    rs = np.random.RandomState(23)
    Q, K, V = _qkv(rs, 2, 1, 7, 5, 8, rnd)
    O = np.asarray(window_fn(Q, K, V, 0.7, 0, 0, None), dtype=np.float64)
    _close(O[:, :, :5], V, atol, "O[r] = V[r]")
    _close(O[:, :, 5:], np.zeros_like(O[:, :, 5:]), atol, "rows with no key")


def pin_window_rows_are_slices(window_fn, sdpa_fn, atol=1e-12, rnd=_ident):
    """Row r of the windowed attention is plain attention of q_r over the
    keys r - left .. r + right (clipped to the sequence)."""
    rs = np.random.RandomState(24)
    n, left, right = 12, 2, 3
    Q, K, V = _qkv(rs, 1, 1, n, n, 8, rnd)
    O = np.asarray(window_fn(Q, K, V, 0.4, left, right, None), dtype=np.float64)
    for r in (0, 1, 5, 9, 11):
        lo, hi = max(0, r - left), min(n, r + right + 1)
        o = sdpa_fn(Q[:, :, r:r + 1], K[:, :, lo:hi], V[:, :, lo:hi], 0.4, NONE, None)
        _close(O[:, :, r:r + 1], o, atol, f"row {r}")


def pin_window_outside_ignored(window_fn, atol=0.0, rnd=_ident):
    """Keys outside every query's window have no effect, NaN included."""
    rs = np.random.RandomState(25)
    Q, K, V = _qkv(rs, 1, 2, 5, 12, 8, rnd)
    clean = np.asarray(window_fn(Q, K, V, 0.6, 1, 1, None), dtype=np.float64)
    K2, V2 = K.copy(), V.copy()
    K2[:, :, 6:] = np.nan
    V2[:, :, 6:] = np.nan
    _close(window_fn(Q, K2, V2, 0.6, 1, 1, None), clean, atol, "NaN beyond every window")


WINDOW_PINS = [pin_window_covering_is_unmasked, pin_window_left_unbounded_is_causal,
               pin_window_zero_width, pin_window_rows_are_slices, pin_window_outside_ignored]


# ---- Add & Norm ([N], the section on the encoder and decoder stacks, paper
# §3.1): a sub-layer's output is LayerNorm(x + Sublayer(x)).  LayerNorm is
# not written out on the pages; the pins fix the standard per-position
# normalisation through values and properties, not through its formula.
# Inputs are multiples of 1/8 below 32 in magnitude, exact in bf16, fp16 and
# fp32, so every pin holds for a device implementation as it stands.

def _eighths(rs, *shape, scale=8):
    return np.round(rs.standard_normal(shape) * scale) / 8.0


def pin_ln_hand_values(add_norm_fn, atol=1e-12):
    """Rows whose mean and mean squared deviation are known by inspection."""
    d = 64
    g, b = np.ones(d), np.zeros(d)
    pm = np.tile([-1.0, 1.0], d // 2)[None]             # mean 0, mean square 1
    z4 = np.tile([0.0, 0.0, 0.0, 4.0], d // 4)[None]     # mean 1, deviations -1,-1,-1,3: mean square 3
    zero = np.zeros((1, d))
    _close(add_norm_fn(pm, zero, g, b, 0.0), pm, atol, "±1 row, eps 0")
    # eps sits under the square root: variance 1 + eps 1 -> 1/√2
    _close(add_norm_fn(pm, zero, g, b, 1.0), pm / math.sqrt(2.0), atol, "±1 row, eps 1")
    exp4 = np.tile([-1.0, -1.0, -1.0, 3.0], d // 4)[None] / math.sqrt(3.0)
    _close(add_norm_fn(z4, zero, g, b, 0.0), exp4, atol, "0,0,0,4 row")
    # the residual addition: x and sub add up to the same row
    _close(add_norm_fn(z4 - pm, pm, g, b, 0.0), exp4, atol, "row split over x and sub")


def pin_ln_moments(add_norm_fn, atol=1e-12, rows=6, d=128):
    """With gain 1, bias 0, eps 0 every output row has mean 0 and mean
    square 1 -- per row (position), whatever the row's own mean and spread."""
    rs = np.random.RandomState(11)
    x = _eighths(rs, rows, d) + np.arange(rows)[:, None]
    sub = _eighths(rs, rows, d) * (1 + np.arange(rows)[:, None] % 3)
    y = np.asarray(add_norm_fn(x, sub, np.ones(d), np.zeros(d), 0.0), dtype=np.float64)
    _close(y.mean(axis=1), np.zeros(rows), atol, "row means")
    _close((y * y).mean(axis=1), np.ones(rows), 4 * atol, "row mean squares")


def pin_ln_shift_and_scale(add_norm_fn, atol=1e-12, rows=4, d=64):
    """eps 0: adding a constant to a row changes nothing; scaling it by a > 0
    changes nothing, by -1 flips the sign of (y - beta)."""
    rs = np.random.RandomState(12)
    x, sub = _eighths(rs, rows, d), _eighths(rs, rows, d)
    g, b = 1 + _eighths(rs, d, scale=2) / 4, _eighths(rs, d, scale=2)
    y = np.asarray(add_norm_fn(x, sub, g, b, 0.0), dtype=np.float64)
    _close(add_norm_fn(x + 4.0, sub, g, b, 0.0), y, atol, "shift by 4")
    _close(add_norm_fn(2.0 * x, 2.0 * sub, g, b, 0.0), y, atol, "scale by 2")
    _close(add_norm_fn(-x, -sub, g, b, 0.0), 2 * b[None] - y, atol, "scale by -1")


def pin_ln_gain_bias(add_norm_fn, atol=1e-12, rows=3, d=64):
    """Gain and bias act per feature after the normalisation:
    y(g, b) = g * y(1, 0) + b."""
    rs = np.random.RandomState(13)
    x, sub = _eighths(rs, rows, d), _eighths(rs, rows, d)
    g, b = _eighths(rs, d, scale=2), _eighths(rs, d, scale=2)
    y0 = np.asarray(add_norm_fn(x, sub, np.ones(d), np.zeros(d), 1e-3), dtype=np.float64)
    _close(add_norm_fn(x, sub, g, b, 1e-3), g[None] * y0 + b[None], atol, "gain and bias")


def pin_ln_constant_row(add_norm_fn, atol=0.0, rows=3, d=64):
    """x + sub constant along a row: zero deviation, so the output is the
    bias exactly (eps > 0)."""
    rs = np.random.RandomState(14)
    x = _eighths(rs, rows, d)
    b = _eighths(rs, d, scale=2)
    y = add_norm_fn(x, 5.0 - x, _eighths(rs, d, scale=2), b, 1e-5)
    _close(y, np.broadcast_to(b, (rows, d)), atol, "constant row")


LN_PINS = [pin_ln_hand_values, pin_ln_moments, pin_ln_shift_and_scale, pin_ln_gain_bias,
           pin_ln_constant_row]
