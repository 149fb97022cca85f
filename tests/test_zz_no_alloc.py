"""mha_forward_noalloc on the GPU: the multi-head attention sub-layer with
the library's own scratch array as its workspace, against mha_forward with
a caller-given workspace (the same kernels: bitwise equal) and the fp64
oracle (2e-2), on two calls in a row, the second smaller than the first, so
that the second reads a scratch array the first left full of its own data.
"""

import ctypes

import numpy as np
import pytest

import oracle
from gpu_util import TOL, from_dev, note, require_gpu, to_dev, torch
from transformer_head_scaled_amd import libmha, synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _mha_inputs(seed, B, n_q, n_k, d_model, h, cross, lens_range):
    r = lambda i: synth.rng(seed, i)  # noqa: E731
    x_q = r(0).standard_normal((B, n_q, d_model), dtype=np.float32)
    x_kv = r(1).standard_normal((B, n_k, d_model), dtype=np.float32) if cross else None
    Ws = [r(2 + i).standard_normal((d_model, d_model), dtype=np.float32) / np.sqrt(d_model)
          for i in range(4)]
    lens = None if lens_range is None else r(6).integers(lens_range[0], lens_range[1] + 1, size=B).astype(np.int32)
    st = {}
    for name, a in [("x_q", x_q), ("x_kv", x_kv), ("Wq", Ws[0]), ("Wk", Ws[1]), ("Wv", Ws[2]), ("Wo", Ws[3])]:
        if a is not None:
            st[name] = synth.round_to(a, "bf16")
    return st, lens


def _call_both(st, lens, h, mask):
    t = {k: to_dev(v[0], "bf16") for k, v in st.items()}
    x_kv = t.get("x_kv")
    lens_d = None if lens is None else torch.from_numpy(lens).cuda()
    B, n_q, d_model = t["x_q"].shape
    n_k = n_q if x_kv is None else x_kv.shape[1]
    out_ref = torch.empty((B, n_q, d_model), dtype=torch.bfloat16, device="cuda")
    out_na = torch.full((B, n_q, d_model), float("nan"), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(libmha.workspace_size(B, n_q, n_k, d_model, h, libmha.MHA_BF16),
                     dtype=torch.uint8, device="cuda")
    libmha.forward(t["x_q"], t["Wq"], t["Wk"], t["Wv"], t["Wo"], h, x_kv=x_kv, mask=mask,
                   kv_lens=lens_d, out=out_ref, workspace=ws)
    # through the C ABI directly
    L = libmha.lib()
    p = lambda x: None if x is None else ctypes.c_void_p(x.data_ptr())  # noqa: E731
    rc = L.mha_forward_noalloc(p(t["x_q"]), p(x_kv), p(t["Wq"]), p(t["Wk"]), p(t["Wv"]), p(t["Wo"]),
                               p(out_na), libmha.MHA_BF16, B, n_q, n_k, d_model, h,
                               libmha.MHA_MASK_CAUSAL if mask == "causal" else libmha.MHA_MASK_NONE,
                               p(lens_d), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == libmha.MHA_OK, libmha.last_error()
    torch.cuda.synchronize()
    return out_ref, out_na


CASES = [
    # (seed, B, n_q, n_k, d_model, h, cross, lens, mask): the big cross-attention
    # sub-layer (29.4 MB of scratch), then the base encoder with key padding,
    # then a small causal decoder -- each smaller than the one before
    (41, 8, 384, 512, 1024, 16, True, None, "none"),
    (42, 32, 64, 64, 512, 8, False, (16, 64), "none"),
    (43, 3, 50, 50, 256, 4, False, None, "causal"),
]


def test_noalloc_matches_forward_two_calls():
    for seed, B, n_q, n_k, dm, h, cross, lens_range, mask in CASES:
        st, lens = _mha_inputs(seed, B, n_q, n_k, dm, h, cross, lens_range)
        note(f"mha_forward_noalloc B={B} n_q={n_q} n_k={n_k} d_model={dm} h={h} {mask}")
        ref, got = _call_both(st, lens, h, mask)
        assert torch.equal(ref, got), "mha_forward_noalloc differs from mha_forward"
        if B * n_q <= 2048:   # oracle on the smaller ones
            exp = oracle.mha(st["x_q"][1], None if "x_kv" not in st else st["x_kv"][1], st["Wq"][1],
                             st["Wk"][1], st["Wv"][1], st["Wo"][1], h,
                             oracle.MASK_CAUSAL if mask == "causal" else oracle.MASK_NONE, lens)
            err = float(np.max(np.abs(from_dev(got) - exp)))
            print(f"[parity] noalloc B={B} n_q={n_q} d_model={dm}: max-abs {err:.3e}", flush=True)
            assert err <= TOL["bf16"]


def test_noalloc_refuses_oversized_without_touching_memory():
    B, n, dm, h = 16, 512, 1024, 16     # 67 MB of workspace
    L = libmha.lib()
    rc = L.mha_forward_noalloc(ctypes.c_void_p(0x1000), None, ctypes.c_void_p(0x100000),
                               ctypes.c_void_p(0x200000), ctypes.c_void_p(0x300000),
                               ctypes.c_void_p(0x400000), ctypes.c_void_p(0x500000),
                               libmha.MHA_BF16, B, n, n, dm, h, 0, None, None)
    assert rc == libmha.MHA_ERR_WORKSPACE and "scratch" in libmha.last_error()
