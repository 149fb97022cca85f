"""Add & Norm on the GPU against the fp64 oracle: mha_add_norm (LayerNorm of
x + sub) and mha_forward_add_norm (the attention sub-layer with its residual
connection and layer normalisation).

Tolerance: max-abs 2e-2 for bf16/fp16 storage (1e-5 for fp32, mha_add_norm
only) on top of the output's own final rounding, REL·|expected| with REL =
2^-8 for bf16 and 2^-11 for fp16 (twice the unit roundoff).  Layer
normalisation outputs reach |y| ~ 5-8 (unit variance times the gain), where
one bf16 rounding alone is up to 0.016-0.03, more than the attention
outputs' 2e-2 was set for (|O| <= ~2); the absolute part still bounds what
the path computes before that rounding.  The pins of ``tests/pins.py``
re-run through the API with the plain max-abs bound; their inputs and most
of their outputs are exact or small in every storage dtype.
"""

import numpy as np
import pytest

import oracle
from gpu_util import TOL, from_dev, lens_dev, note, require_gpu, rounded, to_dev, torch
import pins
from transformer_head_scaled_amd import libmha, synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


REL = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11, "f32": 0.0}


def _check(got, exp, dtype, what):
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    excess = np.abs(got - exp) - REL[dtype] * np.abs(exp)
    err = float(np.max(excess)) if got.size else 0.0
    raw = float(np.max(np.abs(got - exp))) if got.size else 0.0
    print(f"[parity] {what}: max-abs {raw:.3e}, beyond the output rounding {err:.3e} "
          f"(tol {TOL[dtype]:.0e})", flush=True)
    assert err <= TOL[dtype], f"{what}: error beyond output rounding {err:.3e} > {TOL[dtype]}"


def _dev(a, dtype):
    return to_dev(rounded(np.asarray(a, dtype=np.float64), dtype)[0], dtype)


def gpu_add_norm(dtype, inplace=False):
    def fn(x, sub, gamma, beta, eps):
        tx, ts, tg, tb = (_dev(a, dtype) for a in (x, sub, gamma, beta))
        out = libmha.add_norm(tx, ts, tg, tb, eps, out=tx if inplace else None)
        torch.cuda.synchronize()
        return from_dev(out)
    return fn


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("pin", pins.LN_PINS, ids=lambda p: p.__name__)
def test_add_norm_pin_through_api(pin, dtype):
    note(f"add_norm {dtype} {pin.__name__}")
    pin(gpu_add_norm(dtype), atol=TOL[dtype])


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("rows,d", [(1, 64), (3, 100), (1001, 512), (37, 1024), (5, 4096), (2, 4),
                                    (3072, 1024)])  # the benchmark's launch
def test_add_norm_random(dtype, rows, d):
    rs = np.random.default_rng(rows * 7 + d)
    x = rounded(rs.standard_normal((rows, d)) * 2 + 0.3, dtype)[1]
    sub = rounded(rs.standard_normal((rows, d)), dtype)[1]
    g = rounded(1 + 0.2 * rs.standard_normal(d), dtype)[1]
    b = rounded(0.1 * rs.standard_normal(d), dtype)[1]
    note(f"add_norm {dtype} [{rows},{d}]")
    got = gpu_add_norm(dtype)(x, sub, g, b, 1e-5)
    _check(got, oracle.add_norm(x, sub, g, b, 1e-5), dtype, f"add_norm {dtype} [{rows},{d}]")


def test_add_norm_in_place():
    rs = np.random.default_rng(9)
    x = rounded(rs.standard_normal((300, 1024)), "bf16")[1]
    sub = rounded(rs.standard_normal((300, 1024)), "bf16")[1]
    g, b = np.ones(1024), np.zeros(1024)
    note("add_norm bf16 in place [300,1024]")
    got = gpu_add_norm("bf16", inplace=True)(x, sub, g, b, 1e-6)
    _check(got, oracle.add_norm(x, sub, g, b, 1e-6), "bf16", "add_norm in place")


def _ln_params(d_model, dtype, seed):
    rs = np.random.default_rng(seed)
    g = rounded(1 + 0.2 * rs.standard_normal(d_model), dtype)
    b = rounded(0.1 * rs.standard_normal(d_model), dtype)
    return g, b


def _run_fan(ins, g, b, dtype, h, mask="none", lens=None, workspace=True, eps=1e-5):
    dev = {k: to_dev(v[0], dtype) for k, v in ins.items()}
    tg, tb = to_dev(g[0], dtype), to_dev(b[0], dtype)
    ws = None
    if workspace:
        B, n_q, dm = dev["x_q"].shape
        n_k = dev["x_kv"].shape[1] if "x_kv" in dev else n_q
        code = {"bf16": libmha.MHA_BF16, "f16": libmha.MHA_F16}[dtype]
        ws = torch.empty(libmha.add_norm_workspace_size(B, n_q, n_k, dm, h, code),
                         dtype=torch.uint8, device="cuda")
    out = libmha.forward_add_norm(dev["x_q"], dev["Wq"], dev["Wk"], dev["Wv"], dev["Wo"], tg, tb,
                                  h, eps=eps, x_kv=dev.get("x_kv"), mask=mask,
                                  kv_lens=lens_dev(lens), workspace=ws)
    torch.cuda.synchronize()
    return from_dev(out)


def _oracle_fan(ins, g, b, h, mask="none", lens=None, eps=1e-5):
    mk = oracle.MASK_CAUSAL if mask == "causal" else oracle.MASK_NONE
    x_kv = ins["x_kv"][1] if "x_kv" in ins else None
    return oracle.mha_add_norm(ins["x_q"][1], x_kv, ins["Wq"][1], ins["Wk"][1], ins["Wv"][1],
                               ins["Wo"][1], g[1], b[1], eps, h, mk, lens)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("workspace", [True, False])
def test_forward_add_norm_base_encoder(dtype, workspace):
    """Base-model encoder self-attention with key padding (B 32, n 64,
    d_model 512, h 8) plus its Add & Norm."""
    ins, lens = synth.workload_inputs(2, dtype=dtype)
    g, b = _ln_params(512, dtype, 1)
    note(f"forward_add_norm {dtype} base encoder ws={workspace}")
    got = _run_fan(ins, g, b, dtype, 8, "none", lens, workspace)
    _check(got, _oracle_fan(ins, g, b, 8, "none", lens), dtype, f"base encoder add&norm {dtype}")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_forward_add_norm_big_cross(dtype):
    """Big-model encoder-decoder attention (B 8, n_q 384, n_k 512, d_model
    1024, h 16) plus Add & Norm; the residual is the decoder stream x_q."""
    ins, _ = synth.workload_inputs(4, dtype=dtype)
    g, b = _ln_params(1024, dtype, 2)
    note(f"forward_add_norm {dtype} big cross")
    got = _run_fan(ins, g, b, dtype, 16)
    _check(got, _oracle_fan(ins, g, b, 16), dtype, f"big cross add&norm {dtype}")


@pytest.mark.parametrize("case", [
    # (B, n_q, n_k, d_model, h, cross, mask, lens)
    (2, 100, 100, 512, 8, False, "causal", None),       # decoder self-attention
    (2, 300, 20, 512, 8, True, "none", [20, 3]),        # few keys: fp32 rows after the concat
    (3, 77, 77, 256, 4, False, "causal", [77, 5, 0]),   # a batch with no visible key
    (1, 1, 1, 64, 1, False, "none", None),
    (2, 130, 130, 512, 32, False, "none", None),        # d_k = 16
])
def test_forward_add_norm_ragged(case):
    B, n_q, n_k, dm, h, cross, mask, lens = case
    ins = synth.mha_inputs(600 + n_q, B, n_q, n_k, dm, h, cross, dtype="bf16")
    g, b = _ln_params(dm, "bf16", n_q)
    note(f"forward_add_norm ragged {case}")
    got = _run_fan(ins, g, b, "bf16", h, mask, lens)
    _check(got, _oracle_fan(ins, g, b, h, mask, lens), "bf16", f"add&norm {case}")


def test_forward_add_norm_matches_forward_then_add_norm():
    """The fused call against mha_forward followed by mha_add_norm: the same
    up to the one bf16 rounding of the sub-layer output that the unfused
    chain makes."""
    ins = synth.mha_inputs(650, 2, 64, 64, 512, 8, False, dtype="bf16")
    g, b = _ln_params(512, "bf16", 3)
    dev = {k: to_dev(v[0], "bf16") for k, v in ins.items()}
    tg, tb = to_dev(g[0], "bf16"), to_dev(b[0], "bf16")
    note("forward_add_norm vs forward + add_norm")
    fused = libmha.forward_add_norm(dev["x_q"], dev["Wq"], dev["Wk"], dev["Wv"], dev["Wo"], tg, tb, 8)
    sub = libmha.forward(dev["x_q"], dev["Wq"], dev["Wk"], dev["Wv"], dev["Wo"], 8)
    chain = libmha.add_norm(dev["x_q"], sub, tg, tb)
    torch.cuda.synchronize()
    _check(from_dev(fused), from_dev(chain), "bf16", "fused vs chained add&norm")
