"""Planted mistakes in copies of the oracle must each fail at least one pin.

This shows that the pins constrain every step: a dropped term, a wrong sign
or index, a transposed operand or a wrong mask boundary anywhere in the
oracle would be caught.  Every mistake is planted on the CPU, in a patched
copy of one oracle step (``monkeypatch`` restores the real one afterwards),
never in the HIP path.
"""

import math

import numpy as np
import pytest

import oracle
import oracle.attention as A
import pins

_real = {name: getattr(A, name) for name in ("visible", "scores", "softmax_rows", "weighted_sum")}


def _vis_exclusive(n_q, n_k, mask_kind=0, kv_len=None):
    v = _real["visible"](n_q, n_k, 0, kv_len)
    if mask_kind == 1:
        v &= np.arange(n_k)[None, :] < np.arange(n_q)[:, None]
    return v


def _vis_upper(n_q, n_k, mask_kind=0, kv_len=None):
    v = _real["visible"](n_q, n_k, 0, kv_len)
    if mask_kind == 1:
        v &= np.arange(n_k)[None, :] >= np.arange(n_q)[:, None]
    return v


def _vis_pad_off_by_one(n_q, n_k, mask_kind=0, kv_len=None):
    return _real["visible"](n_q, n_k, mask_kind, None if kv_len is None else kv_len + 1)


def _vis_no_padding(n_q, n_k, mask_kind=0, kv_len=None):
    return _real["visible"](n_q, n_k, mask_kind, None)


def _vis_no_mask(n_q, n_k, mask_kind=0, kv_len=None):
    return np.ones((n_q, n_k), dtype=bool)


def _scores_no_scale(q, k, scale):
    return _real["scores"](q, k, 1.0)


def _scores_sqrt_scale(q, k, scale):
    return _real["scores"](q, k, math.sqrt(scale) if scale > 0 else scale)


def _scores_neg(q, k, scale):
    return -_real["scores"](q, k, scale)


def _scores_first_dim_only(q, k, scale):
    return scale * np.outer(np.asarray(q, float)[:, 0], np.asarray(k, float)[:, 0])


def _softmax_no_max(s, vis):
    e = np.where(vis, np.exp(np.where(vis, s, -np.inf)), 0.0)
    d = e.sum(axis=1, keepdims=True)
    with np.errstate(invalid="ignore", divide="ignore"):
        return np.where(d > 0, e / np.where(d > 0, d, 1), 0.0)


def _softmax_columns(s, vis):
    s = np.where(vis, s, -np.inf)
    with np.errstate(invalid="ignore"):
        e = np.where(vis, np.exp(s - np.nanmax(np.where(vis, s, np.nan), axis=0, keepdims=True)), 0.0)
        d = e.sum(axis=0, keepdims=True)
        return np.where(d > 0, e / np.where(d > 0, d, 1), 0.0)


def _softmax_unnormalised(s, vis):
    s = np.where(vis, s, -np.inf)
    p = np.zeros_like(s)
    has = vis.any(axis=1)
    m = s[has].max(axis=1, keepdims=True)
    p[has] = np.where(vis[has], np.exp(s[has] - m), 0.0)
    return p


def _softmax_add_not_set(s, vis):
    # adds a finite penalty instead of setting -inf: masked keys keep a tiny weight
    return _real["softmax_rows"](np.where(vis, s, s - 8.0), np.ones_like(vis))


def _ws_plain(p, vis, v):
    return p @ np.asarray(v, float)


def _ws_reversed(p, vis, v):
    return p @ np.asarray(v, float)[::-1]


SDPA_MUTANTS = {
    "causal_excludes_diagonal": ("visible", _vis_exclusive),
    "causal_upper_triangle": ("visible", _vis_upper),
    "padding_off_by_one": ("visible", _vis_pad_off_by_one),
    "padding_ignored": ("visible", _vis_no_padding),
    "mask_ignored": ("visible", _vis_no_mask),
    "scale_dropped": ("scores", _scores_no_scale),
    "scale_sqrt": ("scores", _scores_sqrt_scale),
    "score_sign": ("scores", _scores_neg),
    "dot_product_truncated": ("scores", _scores_first_dim_only),
    "softmax_without_max": ("softmax_rows", _softmax_no_max),
    "softmax_over_columns": ("softmax_rows", _softmax_columns),
    "softmax_unnormalised": ("softmax_rows", _softmax_unnormalised),
    "mask_added_not_set": ("softmax_rows", _softmax_add_not_set),
    "nan_leaks_through_zero_weight": ("weighted_sum", _ws_plain),
    "value_rows_reversed": ("weighted_sum", _ws_reversed),
}


def _sdpa(Q, K, V, scale, mask, lens):
    return oracle.sdpa(Q, K, V, scale, mask, lens)


def _failing_sdpa_pins():
    import warnings
    failed = []
    for pin in pins.SDPA_PINS:
        try:
            with np.errstate(all="ignore"), warnings.catch_warnings():
                warnings.simplefilter("ignore", RuntimeWarning)
                pin(_sdpa)
        except (AssertionError, ValueError, FloatingPointError, IndexError):
            failed.append(pin.__name__)
    return failed


@pytest.mark.parametrize("name", sorted(SDPA_MUTANTS))
def test_sdpa_mutant_is_caught(name, monkeypatch):
    step, fn = SDPA_MUTANTS[name]
    monkeypatch.setattr(A, step, fn)
    failed = _failing_sdpa_pins()
    assert failed, f"mutant {name} passed every pin"


# ---- multi-head mutants: copies of oracle.mha with one planted mistake each

def _mha_variant(mistake):
    def mha(x_q, x_kv, Wq, Wk, Wv, Wo, h, mask_kind=0, kv_lens=None):
        x_q = np.asarray(x_q, float)
        x_kv = x_q if x_kv is None else np.asarray(x_kv, float)
        if mistake == "kv_from_queries":
            x_kv = x_q[:, :x_kv.shape[1]] if x_q.shape[1] >= x_kv.shape[1] else x_kv * 0 + x_q.mean()
        Wq, Wk, Wv, Wo = (np.asarray(w, float) for w in (Wq, Wk, Wv, Wo))
        if mistake == "wo_transposed":
            Wo = Wo.T
        if mistake == "wk_is_wq":
            Wk = Wq
        B, n_q, _ = x_q.shape
        d_k = Wq.shape[1] // h
        d_v = Wv.shape[1] // h
        scale = 1.0 / np.sqrt(Wq.shape[0] if mistake == "scale_by_d_model" else d_k)
        out = np.zeros((B, n_q, Wo.shape[1]))
        for b in range(B):
            q_all, k_all, v_all = x_q[b] @ Wq, x_kv[b] @ Wk, x_kv[b] @ Wv
            kv_len = None if kv_lens is None else int(kv_lens[b])
            heads = []
            for i in range(h):
                ki = (i + 1) % h if mistake == "k_head_shifted" else i
                o, _ = A.attention_head(q_all[:, i * d_k:(i + 1) * d_k],
                                        k_all[:, ki * d_k:(ki + 1) * d_k],
                                        v_all[:, i * d_v:(i + 1) * d_v], scale, mask_kind, kv_len)
                heads.append(o)
            if mistake == "concat_reversed":
                heads = heads[::-1]
            if mistake == "heads_interleaved":
                concat = np.stack(heads, axis=2).reshape(n_q, h * d_v)
            else:
                concat = np.concatenate(heads, axis=1)
            out[b] = concat @ Wo
        return out
    return mha


MHA_MUTANTS = ["wo_transposed", "wk_is_wq", "scale_by_d_model", "k_head_shifted",
               "concat_reversed", "heads_interleaved", "kv_from_queries"]


@pytest.mark.parametrize("name", MHA_MUTANTS)
def test_mha_mutant_is_caught(name):
    import inspect
    mutant = _mha_variant(name)
    failed = []
    for pin in pins.MHA_PINS:
        try:
            if "sdpa_fn" in inspect.signature(pin).parameters:
                pin(mutant, _sdpa)
            else:
                pin(mutant)
        except AssertionError:
            failed.append(pin.__name__)
    # the torch library comparison is a pin too
    if not failed:
        from test_oracle_pins import check_against_torch_mha
        for case in ("self", "causal", "cross_pad"):
            try:
                check_against_torch_mha(mutant, case)
            except AssertionError:
                failed.append(f"torch_mha_fp64[{case}]")
    assert failed, f"mutant {name} passed every pin"


def test_unmutated_copy_passes():
    """The copy used for the mutants, without a mistake, passes every pin
    (so a caught mutant is caught for its mistake, not for the copy)."""
    import inspect
    good = _mha_variant(None)
    for pin in pins.MHA_PINS:
        if "sdpa_fn" in inspect.signature(pin).parameters:
            pin(good, _sdpa)
        else:
            pin(good)


# ---- Add & Norm mutants: copies of oracle.add_norm with one planted mistake

def _add_norm_variant(mistake):
    def add_norm(x, sub, gamma, beta, eps):
        x, sub = np.asarray(x, float), np.asarray(sub, float)
        gamma, beta = np.asarray(gamma, float), np.asarray(beta, float)
        z = x if mistake == "no_residual" else x + sub
        if mistake == "norm_before_add":
            z = x  # normalise x alone, add sub afterwards
        d = z.shape[-1]
        axis = 0 if mistake == "wrong_axis" else -1
        mu = z.mean(axis=axis, keepdims=True)
        dev = z - mu
        denom = d - 1 if mistake == "unbiased_variance" else d
        var = (dev * dev).sum(axis=axis, keepdims=True) / (denom if axis == -1 else z.shape[0])
        if mistake == "raw_second_moment":
            var = (z * z).mean(axis=axis, keepdims=True)
        if mistake == "eps_outside_sqrt":
            y = dev / (np.sqrt(var) + eps)
        else:
            y = dev / np.sqrt(var + eps)
        if mistake == "no_centering":
            y = z / np.sqrt(var + eps)
        if mistake == "gain_bias_swapped":
            y = beta * y + gamma
        else:
            y = gamma * y + beta
        if mistake == "norm_before_add":
            y = y + sub
        return y
    return add_norm


LN_MUTANTS = ["no_residual", "norm_before_add", "wrong_axis", "unbiased_variance",
              "raw_second_moment", "eps_outside_sqrt", "no_centering", "gain_bias_swapped"]


@pytest.mark.parametrize("name", LN_MUTANTS)
def test_add_norm_mutant_is_caught(name):
    mutant = _add_norm_variant(name)
    failed = []
    for pin in pins.LN_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(mutant)
        except (AssertionError, ValueError, FloatingPointError):
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"


def test_add_norm_unmutated_copy_passes():
    good = _add_norm_variant(None)
    for pin in pins.LN_PINS:
        pin(good)


# ---- band mutants: the window step with one planted mistake each

_real_band = A.band


def _band_right_exclusive(n_q, n_k, left, right):
    r = np.arange(n_q)[:, None]
    c = np.arange(n_k)[None, :]
    return (c >= r - left) & (c < r + right)


def _band_swapped(n_q, n_k, left, right):
    return _real_band(n_q, n_k, right, left)


def _band_ignored(n_q, n_k, left, right):
    return np.ones((n_q, n_k), dtype=bool)


def _band_left_short(n_q, n_k, left, right):
    return _real_band(n_q, n_k, max(left - 1, 0), right)


BAND_MUTANTS = {"right_exclusive": _band_right_exclusive, "swapped": _band_swapped,
                "ignored": _band_ignored, "left_short": _band_left_short}


@pytest.mark.parametrize("name", sorted(BAND_MUTANTS))
def test_band_mutant_is_caught(name, monkeypatch):
    import inspect
    monkeypatch.setattr(A, "band", BAND_MUTANTS[name])

    def window(Q, K, V, scale, left, right, lens):
        return oracle.sdpa(Q, K, V, scale, 0, lens, window=(left, right))
    failed = []
    for pin in pins.WINDOW_PINS:
        try:
            with np.errstate(all="ignore"):
                if "sdpa_fn" in inspect.signature(pin).parameters:
                    pin(window, _sdpa)
                else:
                    pin(window)
        except (AssertionError, ValueError):
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"
