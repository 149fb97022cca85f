"""The fp64 oracle against what the pages and mathematics fix (CPU only).

Three kinds of evidence, none of which re-types the oracle's formula:
* the pins in ``tests/pins.py`` (printed worked example, closed forms,
  invariants);
* a scalar brute force written with a different formula (``tests/brute.py``)
  on tiny shapes, every mask, random key lengths;
* torch's own CPU float64 attention routines, an implementation written by
  others (``scaled_dot_product_attention`` and ``multi_head_attention_forward``).
"""

import math

import numpy as np
import pytest

import oracle
import pins
import brute

ATOL = 1e-12


def _sdpa(Q, K, V, scale, mask, lens):
    return oracle.sdpa(Q, K, V, scale, mask, lens)


def _mha(x_q, x_kv, Wq, Wk, Wv, Wo, h, mask, lens):
    return oracle.mha(x_q, x_kv, Wq, Wk, Wv, Wo, h, mask, lens)


@pytest.mark.parametrize("pin", pins.SDPA_PINS, ids=lambda p: p.__name__)
def test_sdpa_pin(pin):
    pin(_sdpa)


@pytest.mark.parametrize("pin", pins.MHA_PINS, ids=lambda p: p.__name__)
def test_mha_pin(pin):
    import inspect
    if "sdpa_fn" in inspect.signature(pin).parameters:
        pin(_mha, _sdpa)
    else:
        pin(_mha)


def test_worked_example_values():
    """The printed weights reproduced to their printed precision (the pin),
    and the causal row of "il" is the first five weights renormalised."""
    w = pins.pin_worked_example(_sdpa)
    np.testing.assert_allclose(100 * w, [3.99, 65.68, 4.67, 2.93, 13.86, 3.42, 5.45], atol=0.006)


@pytest.mark.parametrize("seed", range(6))
def test_brute_force_sdpa(seed):
    rs = np.random.default_rng(100 + seed)
    B, h = int(rs.integers(1, 3)), int(rs.integers(1, 3))
    n_q = int(rs.integers(1, 9))
    causal = bool(seed % 2)
    n_k = n_q if causal else int(rs.integers(1, 9))
    d_k, d_v = int(rs.integers(1, 5)), int(rs.integers(1, 5))
    Q = rs.standard_normal((B, h, n_q, d_k))
    K = rs.standard_normal((B, h, n_k, d_k))
    V = rs.standard_normal((B, h, n_k, d_v))
    lens = rs.integers(0, n_k + 1, size=B) if seed >= 2 else None
    scale = float(rs.uniform(0.1, 2.0))
    got = oracle.sdpa(Q, K, V, scale, oracle.MASK_CAUSAL if causal else oracle.MASK_NONE, lens)
    exp = np.asarray(brute.sdpa(Q, K, V, scale, causal, lens))
    np.testing.assert_allclose(got, exp, rtol=0, atol=ATOL)


@pytest.mark.parametrize("seed", range(4))
def test_brute_force_mha(seed):
    rs = np.random.default_rng(200 + seed)
    h = int(rs.choice([1, 2, 4]))
    d_model = h * int(rs.integers(1, 4))
    B = int(rs.integers(1, 3))
    n_q = int(rs.integers(1, 6))
    causal = seed == 1
    cross = seed >= 2
    n_k = int(rs.integers(1, 7)) if cross else n_q
    x_q = rs.standard_normal((B, n_q, d_model))
    x_kv = rs.standard_normal((B, n_k, d_model)) if cross else None
    W = [rs.standard_normal((d_model, d_model)) for _ in range(4)]
    lens = rs.integers(0, n_k + 1, size=B) if seed == 3 else None
    mk = oracle.MASK_CAUSAL if causal else oracle.MASK_NONE
    got = oracle.mha(x_q, x_kv, *W, h, mk, lens)
    exp = np.asarray(brute.mha(x_q, x_kv, *W, h, causal, lens))
    np.testing.assert_allclose(got, exp, rtol=0, atol=1e-10)


torch = pytest.importorskip("torch")


@pytest.mark.parametrize("case", ["none", "causal", "pad", "cross_pad", "causal_pad"])
def test_torch_sdpa_fp64(case):
    """torch.nn.functional.scaled_dot_product_attention on the CPU in float64
    (a library routine the oracle shares nothing with)."""
    import torch.nn.functional as F
    rs = np.random.default_rng(300)
    B, h, n_q, d = 3, 4, 33, 64
    n_k = 47 if case == "cross_pad" else n_q
    Q = rs.standard_normal((B, h, n_q, d))
    K = rs.standard_normal((B, h, n_k, d))
    V = rs.standard_normal((B, h, n_k, d))
    lens = rs.integers(1, n_k + 1, size=B) if "pad" in case else None
    causal = "causal" in case
    allow = np.ones((B, 1, n_q, n_k), dtype=bool)
    if causal:
        allow &= np.tril(np.ones((n_q, n_k), dtype=bool))[None, None]
    if lens is not None:
        allow &= (np.arange(n_k)[None, :] < lens[:, None])[:, None, None, :]
    ref = F.scaled_dot_product_attention(
        torch.from_numpy(Q), torch.from_numpy(K), torch.from_numpy(V),
        attn_mask=torch.from_numpy(allow), scale=0.125).numpy()
    got = oracle.sdpa(Q, K, V, 0.125, oracle.MASK_CAUSAL if causal else oracle.MASK_NONE, lens)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def check_against_torch_mha(mha_fn, case):
    """torch.nn.functional.multi_head_attention_forward, float64, no biases,
    separate projection weights.  torch multiplies by Wᵀ, so it is handed
    the transposes of the [d_model, h·d] right-multiplied weights."""
    import torch.nn.functional as F
    rs = np.random.default_rng(400)
    B, n_q, d_model, h = 2, 21, 64, 4
    cross = case == "cross_pad"
    n_k = 29 if cross else n_q
    x_q = rs.standard_normal((B, n_q, d_model))
    x_kv = rs.standard_normal((B, n_k, d_model)) if cross else None
    Wq, Wk, Wv, Wo = (rs.standard_normal((d_model, d_model)) / math.sqrt(d_model) for _ in range(4))
    lens = rs.integers(1, n_k + 1, size=B) if cross else None
    causal = case == "causal"
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))  # noqa: E731
    xq_t = t(x_q.transpose(1, 0, 2))
    xkv_t = xq_t if x_kv is None else t(x_kv.transpose(1, 0, 2))
    kpm = None
    if lens is not None:
        kpm = t(np.arange(n_k)[None, :] >= lens[:, None])
    am = None
    if causal:
        am = t(np.triu(np.ones((n_q, n_k), dtype=bool), k=1))
    ref, _ = F.multi_head_attention_forward(
        xq_t, xkv_t, xkv_t, d_model, h, None, None, None, None, False, 0.0,
        t(Wo.T), None, training=False, key_padding_mask=kpm, need_weights=False,
        attn_mask=am, use_separate_proj_weight=True, q_proj_weight=t(Wq.T),
        k_proj_weight=t(Wk.T), v_proj_weight=t(Wv.T))
    ref = ref.numpy().transpose(1, 0, 2)
    mk = oracle.MASK_CAUSAL if causal else oracle.MASK_NONE
    got = mha_fn(x_q, x_kv, Wq, Wk, Wv, Wo, h, mk, lens)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-11)


@pytest.mark.parametrize("case", ["self", "causal", "cross_pad"])
def test_torch_mha_fp64(case):
    check_against_torch_mha(oracle.mha, case)


def test_score_variance_matches_footnote():
    """nickwang.xyz §3.2.1 footnote (and ml-canon "Почему делим на √d_k"):
    for independent unit-variance components, q·k has mean 0 and variance
    d_k, so the scaled score has variance 1.  Checked on the synthetic
    generator's inputs at d_k = 64 and through the oracle's scores()."""
    from transformer_head_scaled_amd import synth
    ins = synth.sdpa_inputs(3, 1, 2, 512, 512, 64, dtype="bf16")
    q = ins["Q"][1][0, 0].astype(np.float64)
    k = ins["K"][1][0, 0].astype(np.float64)
    s_raw = oracle.scores(q, k, 1.0)
    s = oracle.scores(q, k, 1.0 / math.sqrt(64))
    assert abs(s_raw.var() / 64 - 1) < 0.05
    assert abs(s.var() - 1) < 0.05
    assert abs(s_raw.mean()) < 0.1


def test_fully_masked_and_empty():
    rs = np.random.default_rng(500)
    Q = rs.standard_normal((1, 1, 3, 4))
    K = rs.standard_normal((1, 1, 0, 4))
    V = rs.standard_normal((1, 1, 0, 4))
    out = oracle.sdpa(Q, K, V, 0.5)
    assert out.shape == (1, 1, 3, 4) and np.all(out == 0)
    K = rs.standard_normal((1, 1, 5, 4))
    V = rs.standard_normal((1, 1, 5, 4))
    out = oracle.sdpa(Q, K, V, 0.5, oracle.MASK_NONE, [0])
    assert np.all(out == 0)
    out = oracle.sdpa(Q, K, V, 0.5, oracle.MASK_NONE, [99])   # clamped to n_k
    np.testing.assert_allclose(out, oracle.sdpa(Q, K, V, 0.5), atol=0)


# ---- Add & Norm (oracle.layernorm)

@pytest.mark.parametrize("pin", pins.LN_PINS, ids=lambda p: p.__name__)
def test_add_norm_pin(pin):
    pin(oracle.add_norm)


@pytest.mark.parametrize("eps", [1e-6, 1e-5, 0.5])
def test_add_norm_torch_fp64(eps):
    """torch.nn.functional.layer_norm on the CPU in float64 (a library
    routine the oracle shares nothing with), applied to x + sub."""
    import torch.nn.functional as F
    rs = np.random.default_rng(500)
    x = rs.standard_normal((7, 96)) * 2 + 0.5
    sub = rs.standard_normal((7, 96))
    g, b = rs.standard_normal(96), rs.standard_normal(96)
    ref = F.layer_norm(torch.from_numpy(x + sub), (96,), torch.from_numpy(g), torch.from_numpy(b),
                       eps).numpy()
    np.testing.assert_allclose(oracle.add_norm(x, sub, g, b, eps), ref, rtol=0, atol=1e-12)


def test_mha_add_norm_torch_fp64():
    """The attention sub-layer with its Add & Norm against torch's own
    routines in float64: multi_head_attention_forward (no biases, separate
    projection weights) and layer_norm of x + its output, the post-norm
    order."""
    import torch.nn.functional as F
    rs = np.random.default_rng(501)
    B, n, d_model, h = 2, 13, 64, 4
    x = rs.standard_normal((B, n, d_model))
    Wq, Wk, Wv, Wo = (rs.standard_normal((d_model, d_model)) / math.sqrt(d_model) for _ in range(4))
    g, b = rs.standard_normal(d_model), rs.standard_normal(d_model)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))  # noqa: E731
    xt = t(x.transpose(1, 0, 2))
    attn, _ = F.multi_head_attention_forward(
        xt, xt, xt, d_model, h, None, None, None, None, False, 0.0, t(Wo.T), None,
        training=False, need_weights=False, use_separate_proj_weight=True,
        q_proj_weight=t(Wq.T), k_proj_weight=t(Wk.T), v_proj_weight=t(Wv.T))
    ref = F.layer_norm(xt + attn, (d_model,), t(g), t(b), 1e-5).numpy().transpose(1, 0, 2)
    got = oracle.mha_add_norm(x, None, Wq, Wk, Wv, Wo, g, b, 1e-5, h)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-11)


# ---- restricted attention (oracle.band)

def _window(Q, K, V, scale, left, right, lens):
    return oracle.sdpa(Q, K, V, scale, oracle.MASK_NONE, lens, window=(left, right))


@pytest.mark.parametrize("pin", pins.WINDOW_PINS, ids=lambda p: p.__name__)
def test_window_pin(pin):
    import inspect
    if "sdpa_fn" in inspect.signature(pin).parameters:
        pin(_window, _sdpa)
    else:
        pin(_window)


@pytest.mark.parametrize("seed", range(6))
def test_brute_force_window(seed):
    rs = np.random.default_rng(700 + seed)
    B, h = int(rs.integers(1, 3)), int(rs.integers(1, 3))
    n_q, n_k = int(rs.integers(1, 10)), int(rs.integers(1, 10))
    d = int(rs.integers(1, 5))
    Q, K, V = (rs.standard_normal((B, h, n, d)) for n in (n_q, n_k, n_k))
    left, right = int(rs.integers(0, 5)), int(rs.integers(0, 5))
    lens = rs.integers(0, n_k + 1, size=B) if seed % 2 else None
    got = oracle.sdpa(Q, K, V, 0.5, oracle.MASK_NONE, lens, window=(left, right))
    exp = np.asarray(brute.sdpa(Q, K, V, 0.5, False, lens, window=(left, right)))
    np.testing.assert_allclose(got, exp, rtol=0, atol=ATOL)


def test_window_torch_fp64():
    """torch's CPU float64 scaled_dot_product_attention with the band as a
    boolean mask (rows with at least one visible key)."""
    import torch.nn.functional as F
    rs = np.random.default_rng(701)
    B, h, n, d, left, right = 2, 3, 40, 16, 5, 2
    Q, K, V = (rs.standard_normal((B, h, n, d)) for _ in range(3))
    r = np.arange(n)[:, None]
    c = np.arange(n)[None, :]
    allow = (c >= r - left) & (c <= r + right)
    ref = F.scaled_dot_product_attention(torch.from_numpy(Q), torch.from_numpy(K),
                                         torch.from_numpy(V), attn_mask=torch.from_numpy(allow),
                                         scale=0.25).numpy()
    got = oracle.sdpa(Q, K, V, 0.25, oracle.MASK_NONE, None, window=(left, right))
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)
