"""mha_sdpa_strided / mha_sdpa_window_strided on the GPU against the fp64
oracle: the operands as views into larger tensors, without copies.

* Q, K and V as the three parts of one packed projection [B, n, 3, h, d]
  (x·[W^Q W^K W^V] in one product) and O written straight into the concat
  layout [B, n, h·d] -- the head split and concat of the ml-canon.vercel.app
  "32 Transformer" sketch (a view of the projected rows per head, and their
  concatenation), done by strides;
* one K/V head shared by every query head (head stride 0);
* padded rows (row stride above d) and a batch stride that is not the
  product of the others.

Tolerance (max-abs): 2e-2 for bf16/fp16, 1e-5 for fp32, as for mha_sdpa.
"""

import math

import numpy as np
import pytest

import oracle
from gpu_util import TOL, from_dev, note, require_gpu, torch
from transformer_head_scaled_amd import libmha, synth

pytestmark = pytest.mark.gpu

TORCH = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _dev(values, dtype):
    """float64 host values (already representable in dtype) -> device tensor."""
    return torch.from_numpy(np.asarray(values, dtype=np.float32)).cuda().to(TORCH[dtype])


def _rounded(shape, seed, dtype):
    st, v = synth.round_to(synth.rng(900, seed).standard_normal(shape, dtype=np.float32), dtype)
    return v.astype(np.float64)


def _check(got, exp, dtype, what):
    got = got.astype(np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = float(np.max(np.abs(got - exp)))
    print(f"[parity] {what}: max-abs {err:.3e} (tol {TOL[dtype]:.0e})", flush=True)
    assert err <= TOL[dtype], f"{what}: max-abs {err:.3e}"


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("d", [16, 64, 128, 256])
@pytest.mark.parametrize("mask", ["none", "causal"])
def test_packed_qkv_into_concat(dtype, d, mask):
    """Q/K/V from one packed [B, n, 3, h, d] tensor; O into [B, n, h·d]."""
    if dtype == "f32" and d > 128:
        pytest.skip("the fp32 path stops at d 128")
    B, n, h = 3, 200, 4
    lens = [200, 137, 1] if mask == "none" else None
    scale = 1 / math.sqrt(d)
    qkv = _rounded((B, n, 3, h, d), d, dtype)
    t = _dev(qkv, dtype)
    Q, K, V = (t[:, :, j].transpose(1, 2) for j in range(3))       # [B, h, n, d] views
    out = torch.full((B, n, h * d), float("nan"), dtype=TORCH[dtype], device="cuda")
    O = out.view(B, n, h, d).transpose(1, 2)
    note(f"sdpa_strided {dtype} d={d} {mask} packed qkv -> concat")
    libmha.sdpa_strided(Q, K, V, mask=mask, seq_lens=None if lens is None else
                        torch.tensor(lens, dtype=torch.int32, device="cuda"), out=O)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().reshape(B, n, h, d).transpose(0, 2, 1, 3)
    q64, k64, v64 = (qkv[:, :, j].transpose(0, 2, 1, 3) for j in range(3))
    exp = oracle.sdpa(q64, k64, v64, scale, oracle.MASK_CAUSAL if mask == "causal" else
                      oracle.MASK_NONE, lens)
    _check(got, exp, dtype, f"{dtype} d={d} {mask} packed qkv -> concat")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_shared_kv_head_and_padded_rows(dtype):
    """K and V of one head used by all 8 query heads (head stride 0), Q rows
    padded to 96 elements, a batch stride with a gap, O contiguous."""
    B, h, n_q, n_k, d = 2, 8, 150, 300, 64
    q = _rounded((B, h, n_q, d), 1, dtype)
    k = _rounded((B, 1, n_k, d), 2, dtype)
    v = _rounded((B, 1, n_k, d), 3, dtype)
    qbuf = torch.zeros((B, h * n_q + 5, 96), dtype=TORCH[dtype], device="cuda")
    qbuf[:, :h * n_q, :d] = _dev(q.reshape(B, h * n_q, d), dtype)
    Q = qbuf.as_strided((B, h, n_q, d), (qbuf.stride(0), n_q * 96, 96, 1))
    K = _dev(k, dtype).expand(B, h, n_k, d)
    V = _dev(v, dtype).expand(B, h, n_k, d)
    note(f"sdpa_strided {dtype} shared K/V head, padded Q rows")
    for mask in ("none",):
        out = libmha.sdpa_strided(Q, K, V, scale=0.125, mask=mask)
        torch.cuda.synchronize()
        exp = oracle.sdpa(q, np.broadcast_to(k, (B, h, n_k, d)), np.broadcast_to(v, (B, h, n_k, d)),
                          0.125)
        _check(from_dev(out), exp, dtype, f"{dtype} shared K/V {mask}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_window_strided(dtype):
    """mha_sdpa_window_strided on the packed layout, reach (40, 9)."""
    B, n, h, d = 2, 300, 2, 64
    qkv = _rounded((B, n, 3, h, d), 7, dtype)
    t = _dev(qkv, dtype)
    Q, K, V = (t[:, :, j].transpose(1, 2) for j in range(3))
    note(f"sdpa_window_strided {dtype}")
    out = libmha.sdpa_window_strided(Q, K, V, 40, 9, scale=0.125)
    torch.cuda.synchronize()
    q64, k64, v64 = (qkv[:, :, j].transpose(0, 2, 1, 3) for j in range(3))
    exp = oracle.sdpa(q64, k64, v64, 0.125, window=(40, 9))
    _check(from_dev(out), exp, dtype, f"{dtype} window strided")


def test_default_scale_is_one_over_sqrt_dk():
    """scale=None passes NaN; the library uses 1/sqrt(d_k): the same output
    as an explicit 1/sqrt(d_k), bit for bit."""
    ins = synth.sdpa_inputs(11, 2, 2, 130, 130, 128, dtype="bf16")
    tq, tk, tv = (torch.from_numpy(ins[n_][0].view(np.int16)).cuda().view(torch.bfloat16) for n_ in "QKV")
    note("default scale")
    a = libmha.sdpa(tq, tk, tv)
    b = libmha.sdpa(tq, tk, tv, scale=1 / math.sqrt(128))
    torch.cuda.synchronize()
    assert torch.equal(a, b)
