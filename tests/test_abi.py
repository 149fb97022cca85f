"""The C ABI on the CPU: the library loads, exports every symbol the header
declares, and rejects bad arguments on the host before touching a device.

No call here reaches a kernel launch: every call either fails validation or
is a zero-size no-op, both of which return before any HIP call.
"""

import ctypes
import os
import re

import pytest

from transformer_head_scaled_amd import libmha as M

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mha.h")

pytestmark = pytest.mark.skipif(not os.path.exists(M.LIB_PATH), reason="libmha.so not built")


def declared_functions():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mha_\w+)\s*\(", text)))


def test_header_declares_expected_api():
    assert declared_functions() == sorted(M.EXPORTS)


def test_every_declared_symbol_is_exported():
    L = ctypes.CDLL(M.LIB_PATH)
    for name in declared_functions():
        assert hasattr(L, name), f"libmha.so does not export {name}"


def test_status_strings_and_version():
    assert M.status_string(M.MHA_OK) == "MHA_OK"
    for code in range(-7, 0):
        s = M.status_string(code)
        assert s.startswith("MHA_ERR_"), s
    assert "unknown" in M.status_string(-99)
    assert M.version() == 300


def _sdpa(dtype=M.MHA_BF16, B=1, h=1, n_q=8, n_k=8, d_k=64, d_v=64, scale=0.125,
          mask=M.MHA_MASK_NONE, Q=0x1000, K=0x100000, V=0x200000, O=0x300000, lens=None):
    L = M.lib()
    return L.mha_sdpa(Q, K, V, O, dtype, B, h, n_q, n_k, d_k, d_v, scale, mask, lens, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=7), M.MHA_ERR_DTYPE),
    (dict(mask=3), M.MHA_ERR_INVALID_ARG),
    (dict(B=-1), M.MHA_ERR_SHAPE),
    (dict(d_k=0), M.MHA_ERR_SHAPE),
    (dict(n_k=9, mask=M.MHA_MASK_CAUSAL), M.MHA_ERR_SHAPE),
    (dict(scale=float("inf")), M.MHA_ERR_INVALID_ARG),
    (dict(scale=float("-inf")), M.MHA_ERR_INVALID_ARG),
    (dict(d_k=1024, d_v=1024), M.MHA_ERR_UNSUPPORTED),
    (dict(d_k=256, d_v=256, dtype=M.MHA_F32), M.MHA_ERR_UNSUPPORTED),
    (dict(d_k=48, d_v=48), M.MHA_ERR_UNSUPPORTED),
    (dict(d_k=64, d_v=32), M.MHA_ERR_UNSUPPORTED),
    (dict(dtype=M.MHA_F32, d_k=48, d_v=48), M.MHA_ERR_UNSUPPORTED),
    (dict(Q=None), M.MHA_ERR_INVALID_ARG),
    (dict(O=None), M.MHA_ERR_INVALID_ARG),
    (dict(V=None), M.MHA_ERR_INVALID_ARG),
    (dict(O=0x1000 + 64), M.MHA_ERR_ALIAS),        # O overlaps Q
    (dict(O=0x200000 - 16), M.MHA_ERR_ALIAS),      # O's tail runs into V
    (dict(n_q=1 << 31), M.MHA_ERR_SHAPE),
    (dict(K=0x100000 + 8), M.MHA_ERR_INVALID_ARG),  # not 16-byte aligned
    (dict(lens=0x900002), M.MHA_ERR_INVALID_ARG),
])
def test_sdpa_rejects(kw, code):
    assert _sdpa(**kw) == code
    assert M.last_error() != ""


def test_sdpa_alias_edges():
    # O (8 rows x 64 bf16 = 1024 bytes) starting 1008 bytes before K: its
    # last 16 bytes are K's first 16; ending exactly at K is no overlap
    assert _sdpa(O=0x100000 - 8 * 64 * 2 + 16) == M.MHA_ERR_ALIAS


def test_zero_sizes_are_noops():
    for kw in (dict(B=0), dict(h=0), dict(n_q=0), dict(B=0, Q=None, O=None)):
        assert _sdpa(**kw) == M.MHA_OK


def test_nan_scale_means_the_default():
    """scale NaN is the pages' 1/sqrt(d_k), resolved in the library: it passes
    validation (a zero-size call returns OK after it) where ±inf does not."""
    assert _sdpa(B=0, scale=float("nan")) == M.MHA_OK
    assert _sdpa(B=0, scale=float("inf")) == M.MHA_ERR_INVALID_ARG


def test_library_resolves_all_its_symbols():
    """Every libmha function the library calls is defined in it (a source
    left out of the link would show as an undefined mha symbol)."""
    import shutil
    import subprocess
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm not available")
    out = subprocess.run([nm, "-D", "--undefined-only", M.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    assert not [ln for ln in out.splitlines() if "mha" in ln.lower()], out


@pytest.mark.skipif(os.path.exists("/dev/kfd"), reason="a GPU driver is present")
def test_valid_call_without_a_device_is_a_hip_error():
    """On a host with no GPU a call that passes validation fails at its first
    HIP call with MHA_ERR_HIP (and a message), not a crash.  The tensors are
    host buffers here; with no device nothing is ever launched."""
    import numpy as np
    buf = np.zeros(1 << 20, dtype=np.uint8)
    a = (buf.ctypes.data + 255) & ~255
    L = M.lib()
    rc = L.mha_sdpa(a, a + 65536, a + 131072, a + 196608, M.MHA_BF16, 1, 1, 8, 8, 64, 64, 0.125,
                    M.MHA_MASK_NONE, None, None)
    assert rc == M.MHA_ERR_HIP and "mha_sdpa" in M.last_error()
    st = M.SdpaStrides()
    for f in "qkvo":
        getattr(st, f)[:] = (8 * 64, 8 * 64, 64)
    rc = L.mha_sdpa_strided(a, a + 65536, a + 131072, a + 196608, ctypes.byref(st), M.MHA_BF16,
                            1, 1, 8, 8, 64, 64, float("nan"), M.MHA_MASK_CAUSAL, None, None)
    assert rc == M.MHA_ERR_HIP


# ---- strided operands

def _strided(q=(512, 512, 64), k=(512, 512, 64), v=(512, 512, 64), o=(512, 512, 64),
             dtype=M.MHA_BF16, B=2, h=1, n_q=8, n_k=8, d=64, O=0x300000, K=0x100000, null=False):
    st = M.SdpaStrides()
    st.q[:], st.k[:], st.v[:], st.o[:] = q, k, v, o
    return M.lib().mha_sdpa_strided(0x1000, K, 0x200000, O, None if null else ctypes.byref(st),
                                    dtype, B, h, n_q, n_k, d, d, 0.125, M.MHA_MASK_NONE, None, None)


@pytest.mark.parametrize("kw,code", [
    (dict(null=True), M.MHA_ERR_INVALID_ARG),
    (dict(q=(512, 512, -64)), M.MHA_ERR_INVALID_ARG),      # negative stride
    (dict(k=(512, 512, 68)), M.MHA_ERR_INVALID_ARG),       # rows not on 16 bytes
    (dict(v=(516, 512, 64)), M.MHA_ERR_INVALID_ARG),
    (dict(o=(512, 512, 32)), M.MHA_ERR_INVALID_ARG),       # output rows overlap
    (dict(o=(256, 512, 64)), M.MHA_ERR_INVALID_ARG),       # batches overlap
    (dict(o=(0, 0, 64)), M.MHA_ERR_INVALID_ARG),           # batch stride 0 on the output
    (dict(dtype=M.MHA_F32, q=(512, 512, 66)), M.MHA_ERR_INVALID_ARG),
    (dict(k=(512, 512, 1 << 21), n_k=1024), M.MHA_ERR_UNSUPPORTED),   # K rows span > 2 GiB
    (dict(q=(1 << 62, 512, 64)), M.MHA_ERR_INVALID_ARG),   # a stride past 2^46 bytes
    (dict(o=(1 << 62, 512, 64)), M.MHA_ERR_INVALID_ARG),
    (dict(q=(1 << 40, 512, 64), B=64), M.MHA_ERR_SHAPE),   # allowed strides, span past 2^46 bytes
    (dict(O=0x1000 + 512 * 2 * 2 - 16), M.MHA_ERR_ALIAS),  # O starts inside Q's span
    (dict(q=(8192, 512, 64), O=0x1000 + 8192 * 2), M.MHA_ERR_ALIAS),  # O in the gap between Q's batches
])
def test_strided_rejects(kw, code):
    assert _strided(**kw) == code
    assert M.last_error() != ""


def test_strided_accepts_views_and_broadcast():
    """Layouts that pass the stride checks (n_q = 0 then returns OK before any
    pointer is used): a [B, n, h, d] view of one projected matrix as
    [B, h, n, d], and K/V shared by every head (head stride 0)."""
    view = (8 * 2 * 64, 64, 2 * 64)   # x·W^Q of [B, n=8, h=2, d=64] seen as [B, h, n, d]
    assert _strided(q=view, o=view, h=2, n_q=0) == M.MHA_OK
    assert _strided(k=(512, 0, 64), v=(512, 0, 64), o=(1024, 512, 64), h=2, n_q=0) == M.MHA_OK


# ---- routes: which kernel each workload and each GPU test's shape runs on

ROUTES = [
    # (dtype, B, h, n_q, n_k, d, mask, window) -> (kernel, waves, workgroups or None)
    ((M.MHA_F32, 1, 1, 16, 16, 64, "none", None), ("f32", 1, 1)),          # single head fp32
    ((M.MHA_F32, 1, 2, 70, 70, 64, "none", None), ("f32", 1, 10)),         # four lanes a row
    ((M.MHA_F32, 16, 64, 70, 70, 64, "causal", None), ("f32", 1, 2048)),   # one lane a row
    ((M.MHA_BF16, 32, 8, 64, 64, 64, "none", None), ("pairs", 2, 256)),    # base encoder sub-layer
    ((M.MHA_BF16, 16, 8, 512, 512, 64, "causal", None), ("pairs", 4, 512)),  # decoder causal
    ((M.MHA_BF16, 8, 16, 384, 512, 64, "none", None), ("pairs", 8, 256)),  # big cross-attention
    ((M.MHA_BF16, 4, 8, 4096, 4096, 64, "none", None), ("blocks", 8, 256)),  # long, unmasked
    ((M.MHA_BF16, 4, 8, 4096, 4096, 64, "causal", None), ("pairs", 8, 512)),  # long, causal
    ((M.MHA_BF16, 64, 8, 1, 2048, 64, "none", None), ("decode", 8, 512)),  # decoding step
    # shapes GPU tests rely on
    ((M.MHA_BF16, 1, 3, 2304, 2304, 64, "causal", None), ("pairs", 4, None)),
    ((M.MHA_BF16, 1, 4, 1536, 1536, 64, "none", None), ("pairs", 4, None)),
    ((M.MHA_BF16, 8, 8, 2560, 2560, 64, "none", None), ("blocks", 4, None)),
    ((M.MHA_BF16, 8, 16, 1000, 1000, 64, "none", None), ("blocks", 4, None)),
    ((M.MHA_BF16, 8, 8, 4000, 4000, 64, "none", None), ("blocks", 8, 512)),
    ((M.MHA_BF16, 64, 32, 50, 70, 64, "none", None), ("blocks", 1, None)),
    ((M.MHA_BF16, 64, 32, 50, 70, 128, "none", None), ("blocks", 1, None)),
    ((M.MHA_BF16, 8, 16, 1000, 1000, 16, "causal", None), ("blocks", 4, None)),
    ((M.MHA_BF16, 8, 16, 1000, 1000, 128, "causal", None), ("pairs", 4, None)),
    ((M.MHA_BF16, 8, 4, 1, 2048, 16, "none", None), ("split", 4, None)),
    ((M.MHA_BF16, 4, 2, 4, 1000, 128, "none", None), ("split", 2, None)),
    ((M.MHA_BF16, 1, 2, 200, 200, 32, "causal", None), ("blocks", 2, None)),
    ((M.MHA_BF16, 1, 2, 200, 200, 512, "causal", None), ("wide", 8, 14)),  # key tiles split in two
    ((M.MHA_BF16, 1, 2, 200, 200, 512, "none", None), ("wide", 8, 8)),   # two 32-row blocks a workgroup
    ((M.MHA_BF16, 1, 2, 200, 200, 256, "causal", None), ("wide", 4, 14)),
    ((M.MHA_BF16, 8, 16, 1000, 1000, 64, "none", (128, 128)), ("window", 2, None)),
    ((M.MHA_BF16, 8, 16, 2600, 2600, 64, "none", (1500, 600)), ("window", 4, None)),
    ((M.MHA_BF16, 8, 16, 1000, 1000, 64, "none", (2000, 2000)), ("blocks", 4, None)),  # reaches all
]


@pytest.mark.parametrize("args,expect", ROUTES, ids=lambda x: "x".join(map(str, x)) if isinstance(x, tuple) else None)
def test_route(args, expect):
    dtype, B, h, n_q, n_k, d, mask, window = args
    r = M.sdpa_route(dtype, B, h, n_q, n_k, d, mask=mask, window=window)
    assert (r["kernel"], r["waves"]) == expect[:2], r
    if expect[2] is not None:
        assert r["workgroups"] == expect[2], r
    assert r["rows_per_workgroup"] * r["workgroups"] >= n_q * B * h or r["kernel"] == "blocks"


def test_route_window_forms():
    """A window reaching every earlier key and no later one runs as the
    causal mask; the route reports it."""
    r = M.sdpa_route(M.MHA_BF16, 2, 2, 300, 300, 64, window=(299, 0))
    assert r["kernel"] == "pairs" and r["mask_kind"] == M.MHA_MASK_CAUSAL
    with pytest.raises(M.MhaError):
        M.sdpa_route(M.MHA_BF16, 2, 2, 300, 301, 64, mask="causal")


def _fwd(dtype=M.MHA_BF16, B=2, n_q=8, n_k=8, d_model=128, h=2, mask=M.MHA_MASK_NONE,
         x_q=0x1000, x_kv=None, W=(0x100000, 0x200000, 0x300000, 0x400000), out=0x500000,
         lens=None, ws=None, ws_bytes=0):
    L = M.lib()
    return L.mha_forward(x_q, x_kv, W[0], W[1], W[2], W[3], out, dtype, B, n_q, n_k, d_model, h,
                         mask, lens, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=5), M.MHA_ERR_DTYPE),
    (dict(dtype=M.MHA_F32), M.MHA_ERR_UNSUPPORTED),
    (dict(d_model=129, h=2), M.MHA_ERR_SHAPE),
    (dict(d_model=2048, h=2), M.MHA_ERR_UNSUPPORTED),    # head dim 1024
    (dict(d_model=96, h=2), M.MHA_ERR_UNSUPPORTED),      # head dim 48
    (dict(d_model=96, h=3), M.MHA_ERR_UNSUPPORTED),      # head dim 32, d_model not a multiple of 64
    (dict(h=0), M.MHA_ERR_SHAPE),
    (dict(n_k=9), M.MHA_ERR_SHAPE),                       # self-attention, n_k != n_q
    (dict(n_k=9, x_kv=0x600000, mask=M.MHA_MASK_CAUSAL), M.MHA_ERR_SHAPE),
    (dict(mask=9), M.MHA_ERR_INVALID_ARG),
    (dict(x_q=None), M.MHA_ERR_INVALID_ARG),
    (dict(W=(0x100000, None, 0x300000, 0x400000)), M.MHA_ERR_INVALID_ARG),
    (dict(ws=0x700000, ws_bytes=16), M.MHA_ERR_WORKSPACE),
    (dict(ws=0x700010, ws_bytes=1 << 20), M.MHA_ERR_INVALID_ARG),   # misaligned workspace
    (dict(out=0x1000), M.MHA_ERR_ALIAS),
    (dict(out=0x400000 + 16), M.MHA_ERR_ALIAS),
    (dict(ws=0x500000, ws_bytes=1 << 20), M.MHA_ERR_ALIAS),
    (dict(out=0x500008), M.MHA_ERR_INVALID_ARG),   # not 16-byte aligned
])
def test_forward_rejects(kw, code):
    assert _fwd(**kw) == code


def _fna(B=2, n_q=8, n_k=8, d_model=128, h=2, dtype=M.MHA_BF16, x_kv=None, mask=M.MHA_MASK_NONE,
         out=0x500000):
    return M.lib().mha_forward_noalloc(0x1000, x_kv, 0x100000, 0x200000, 0x300000, 0x400000, out,
                                       dtype, B, n_q, n_k, d_model, h, mask, None, None)


@pytest.mark.parametrize("kw,code", [
    (dict(B=8, n_q=4096, n_k=4096, d_model=1024, h=16), M.MHA_ERR_WORKSPACE),   # 268 MB > 32 MiB
    (dict(dtype=M.MHA_F32), M.MHA_ERR_UNSUPPORTED),
    (dict(d_model=129), M.MHA_ERR_SHAPE),
    (dict(n_k=9), M.MHA_ERR_SHAPE),
    (dict(mask=7), M.MHA_ERR_INVALID_ARG),
    (dict(dtype=9), M.MHA_ERR_DTYPE),
])
def test_forward_noalloc_rejects(kw, code):
    """Oversized problems are refused before anything touches a device; bad
    arguments give mha_forward's errors."""
    assert _fna(**kw) == code
    assert M.last_error().startswith("mha_forward_noalloc")


def test_forward_noalloc_limit():
    """The largest workspace the scratch takes: the big-model cross-attention
    sub-layer fits, twice its batch does not."""
    L = M.lib()
    assert L.mha_forward_workspace_size(8, 384, 512, 1024, 16, M.MHA_BF16) <= M.NOALLOC_SCRATCH_BYTES
    assert L.mha_forward_workspace_size(16, 384, 512, 1024, 16, M.MHA_BF16) > M.NOALLOC_SCRATCH_BYTES
    assert _fna(B=16, n_q=384, n_k=512, d_model=1024, h=16, x_kv=0x900000) == M.MHA_ERR_WORKSPACE
    assert _fna(B=0) == M.MHA_OK


def test_forward_zero_sizes_are_noops():
    assert _fwd(B=0) == M.MHA_OK
    assert _fwd(n_q=0, n_k=0) == M.MHA_OK


def test_workspace_size():
    L = M.lib()
    B, n_q, n_k, dm, h = 8, 384, 512, 1024, 16
    need = L.mha_forward_workspace_size(B, n_q, n_k, dm, h, M.MHA_BF16)
    assert need >= 2 * (2 * B * n_q * dm + 2 * B * n_k * dm)
    assert need % 256 == 0
    assert need < 2 * (2 * B * n_q * dm + 2 * B * n_k * dm) + 4 * 256
    assert L.mha_forward_workspace_size(B, n_q, n_k, dm, 0, M.MHA_BF16) == 0
    # sizes mha_forward rejects as beyond its range give 0 too (no overflowed
    # byte count): a huge batch, a huge batch x rows, a huge d_model
    for args in ((1 << 40, 64, 64, 512, 8), (65535, 1 << 20, 1 << 20, 512, 8),
                 (4, 64, 64, 1 << 40, 8)):
        assert L.mha_forward_workspace_size(*args, M.MHA_BF16) == 0, args
        assert L.mha_forward_add_norm_workspace_size(*args, M.MHA_BF16) == 0, args
    assert L.mha_forward_workspace_size(B, n_q, n_k, 1000, 16, M.MHA_BF16) == 0


def _an(dtype=M.MHA_BF16, rows=4, d=64, eps=1e-5, x=0x1000, sub=0x100000, g=0x200000,
        b=0x300000, out=0x400000):
    L = M.lib()
    return L.mha_add_norm(x, sub, g, b, eps, out, dtype, rows, d, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=9), M.MHA_ERR_DTYPE),
    (dict(rows=-1), M.MHA_ERR_SHAPE),
    (dict(d=0), M.MHA_ERR_SHAPE),
    (dict(d=66), M.MHA_ERR_UNSUPPORTED),          # not a multiple of 4
    (dict(d=8192), M.MHA_ERR_UNSUPPORTED),        # above 4096
    (dict(eps=-1.0), M.MHA_ERR_INVALID_ARG),
    (dict(eps=float("nan")), M.MHA_ERR_INVALID_ARG),
    (dict(eps=float("inf")), M.MHA_ERR_INVALID_ARG),
    (dict(g=None), M.MHA_ERR_INVALID_ARG),
    (dict(sub=None), M.MHA_ERR_INVALID_ARG),
    (dict(x=0x1008), M.MHA_ERR_INVALID_ARG),      # not 16-byte aligned
    (dict(out=0x1000 + 16), M.MHA_ERR_ALIAS),      # partial overlap with x
    (dict(out=0x200000), M.MHA_ERR_ALIAS),         # overlaps gamma
    (dict(out=0x300000 - 64), M.MHA_ERR_ALIAS),    # runs into beta
])
def test_add_norm_rejects(kw, code):
    assert _an(**kw) == code
    assert M.last_error() != ""


def test_add_norm_zero_rows_is_noop():
    assert _an(rows=0) == M.MHA_OK
    assert _an(rows=0, x=None, out=None) == M.MHA_OK


def _fan(dtype=M.MHA_BF16, B=2, n_q=8, n_k=8, d_model=128, h=2, eps=1e-5,
         g=0x700000, b=0x710000, out=0x500000, ws=None, ws_bytes=0, x_kv=None):
    L = M.lib()
    return L.mha_forward_add_norm(0x1000, x_kv, 0x100000, 0x200000, 0x300000, 0x400000, g, b, eps,
                                  out, dtype, B, n_q, n_k, d_model, h, 0, None, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(g=None), M.MHA_ERR_INVALID_ARG),
    (dict(b=None), M.MHA_ERR_INVALID_ARG),
    (dict(eps=-0.5), M.MHA_ERR_INVALID_ARG),
    (dict(d_model=8192, h=128), M.MHA_ERR_UNSUPPORTED),   # above 4096
    (dict(dtype=M.MHA_F32), M.MHA_ERR_UNSUPPORTED),
    (dict(out=0x700000 - 16), M.MHA_ERR_ALIAS),          # out runs into gamma
    (dict(g=0x700008), M.MHA_ERR_INVALID_ARG),            # misaligned gamma
    (dict(ws=0x800000, ws_bytes=16), M.MHA_ERR_WORKSPACE),
])
def test_forward_add_norm_rejects(kw, code):
    assert _fan(**kw) == code
    assert M.last_error().startswith("mha_forward_add_norm")


def test_forward_add_norm_workspace_size():
    L = M.lib()
    # z (fp32) fits below the concat: the same bytes as mha_forward
    args = (8, 384, 512, 1024, 16, M.MHA_BF16)
    assert L.mha_forward_add_norm_workspace_size(*args) == L.mha_forward_workspace_size(*args)
    # few keys: Q/K/V are smaller than the fp32 rows, which go after the concat
    B, n_q, n_k, dm = 2, 300, 20, 512
    base = L.mha_forward_workspace_size(B, n_q, n_k, dm, 8, M.MHA_BF16)
    need = L.mha_forward_add_norm_workspace_size(B, n_q, n_k, dm, 8, M.MHA_BF16)
    assert need == base + B * n_q * dm * 4
    assert L.mha_forward_add_norm_workspace_size(B, n_q, n_k, dm, 0, M.MHA_BF16) == 0


def _win(left=1, right=1, dtype=M.MHA_BF16, n_q=8, n_k=8, O=0x300000, d=64):
    L = M.lib()
    return L.mha_sdpa_window(0x1000, 0x100000, 0x200000, O, dtype, 1, 1, n_q, n_k, d, d, 0.125,
                             left, right, None, None)


@pytest.mark.parametrize("kw,code", [
    (dict(left=-1), M.MHA_ERR_INVALID_ARG),
    (dict(right=-5), M.MHA_ERR_INVALID_ARG),
    (dict(O=0x1000), M.MHA_ERR_ALIAS),
    (dict(dtype=4), M.MHA_ERR_DTYPE),
    (dict(d=256), M.MHA_ERR_UNSUPPORTED),          # the window needs d <= 128
])
def test_window_rejects(kw, code):
    assert _win(**kw) == code
    assert M.last_error().startswith("mha_sdpa_window")


def test_window_zero_rows_is_noop():
    assert _win(n_q=0) == M.MHA_OK
