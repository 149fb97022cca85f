"""ctypes binding of libmha.so -- argument marshalling only.

Same names as the C ABI in include/mha.h.  Tensors are torch tensors on the
current HIP device; the binding passes their data pointers, sizes and the
current torch stream to the library and raises ``MhaError`` on a non-zero
status.  Nothing here computes: every step runs in the library's kernels.
If the library is not built, ``lib()`` raises instead of falling back.
"""

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_lib", "libmha.so")

MHA_F32, MHA_BF16, MHA_F16 = 0, 1, 2
MHA_MASK_NONE, MHA_MASK_CAUSAL = 0, 1
MHA_OK = 0
MHA_ERR_INVALID_ARG = -1
MHA_ERR_SHAPE = -2
MHA_ERR_DTYPE = -3
MHA_ERR_UNSUPPORTED = -4
MHA_ERR_WORKSPACE = -5
MHA_ERR_ALIAS = -6
MHA_ERR_HIP = -7
NOALLOC_SCRATCH_BYTES = 32 << 20   # MHA_NOALLOC_SCRATCH_BYTES

# every symbol include/mha.h declares
EXPORTS = ("mha_sdpa", "mha_sdpa_strided", "mha_sdpa_window", "mha_sdpa_window_strided",
           "mha_sdpa_route", "mha_forward", "mha_forward_workspace_size", "mha_forward_noalloc",
           "mha_add_norm",
           "mha_forward_add_norm", "mha_forward_add_norm_workspace_size", "mha_status_string",
           "mha_last_error", "mha_version")

# mha_route.kernel values
KERNELS = {0: "f32", 1: "blocks", 2: "pairs", 3: "split", 4: "decode", 5: "window", 6: "wide"}


class SdpaStrides(ctypes.Structure):
    """mha_sdpa_strides: [batch, head, row] element strides of Q, K, V, O."""
    _fields_ = [("q", ctypes.c_int64 * 3), ("k", ctypes.c_int64 * 3), ("v", ctypes.c_int64 * 3),
                ("o", ctypes.c_int64 * 3)]


class Route(ctypes.Structure):
    """mha_route."""
    _fields_ = [("kernel", ctypes.c_int32), ("waves", ctypes.c_int32),
                ("rows_per_workgroup", ctypes.c_int32), ("mask_kind", ctypes.c_int32),
                ("workgroups", ctypes.c_int64)]

_lib = None


class MhaError(RuntimeError):
    def __init__(self, status, detail):
        self.status = status
        super().__init__(f"{status_string(status)} ({detail})" if detail else status_string(status))


def lib():
    """Load libmha.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"libmha.so is not built ({LIB_PATH}); run "
                           "python -m transformer_head_scaled_amd.build")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    L.mha_sdpa.argtypes = [vp, vp, vp, vp, i32, i64, i64, i64, i64, i64, i64, f32, i32, vp, vp]
    L.mha_sdpa.restype = ctypes.c_int
    L.mha_sdpa_window.argtypes = [vp, vp, vp, vp, i32, i64, i64, i64, i64, i64, i64, f32, i64, i64,
                                  vp, vp]
    L.mha_sdpa_window.restype = ctypes.c_int
    sp = ctypes.POINTER(SdpaStrides)
    L.mha_sdpa_strided.argtypes = [vp, vp, vp, vp, sp, i32, i64, i64, i64, i64, i64, i64, f32, i32,
                                   vp, vp]
    L.mha_sdpa_strided.restype = ctypes.c_int
    L.mha_sdpa_window_strided.argtypes = [vp, vp, vp, vp, sp, i32, i64, i64, i64, i64, i64, i64, f32,
                                          i64, i64, vp, vp]
    L.mha_sdpa_window_strided.restype = ctypes.c_int
    L.mha_sdpa_route.argtypes = [i32, i64, i64, i64, i64, i64, i64, i32, i32, i64, i64,
                                 ctypes.POINTER(Route)]
    L.mha_sdpa_route.restype = ctypes.c_int
    L.mha_forward.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i64, i64, i64, i64, i32, i32, vp,
                              vp, ctypes.c_size_t, vp]
    L.mha_forward.restype = ctypes.c_int
    L.mha_forward_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i64, i64, i64, i64, i32,
                                      i32, vp, vp]
    L.mha_forward_noalloc.restype = ctypes.c_int
    L.mha_forward_workspace_size.argtypes = [i64, i64, i64, i64, i32, i32]
    L.mha_forward_workspace_size.restype = ctypes.c_size_t
    L.mha_add_norm.argtypes = [vp, vp, vp, vp, f32, vp, i32, i64, i64, vp]
    L.mha_add_norm.restype = ctypes.c_int
    L.mha_forward_add_norm.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, f32, vp, i32, i64, i64,
                                       i64, i64, i32, i32, vp, vp, ctypes.c_size_t, vp]
    L.mha_forward_add_norm.restype = ctypes.c_int
    L.mha_forward_add_norm_workspace_size.argtypes = [i64, i64, i64, i64, i32, i32]
    L.mha_forward_add_norm_workspace_size.restype = ctypes.c_size_t
    L.mha_status_string.argtypes = [ctypes.c_int]
    L.mha_status_string.restype = ctypes.c_char_p
    L.mha_last_error.argtypes = []
    L.mha_last_error.restype = ctypes.c_char_p
    L.mha_version.argtypes = []
    L.mha_version.restype = ctypes.c_int
    _lib = L
    return L


def status_string(status):
    return lib().mha_status_string(int(status)).decode()


def last_error():
    return lib().mha_last_error().decode()


def version():
    return lib().mha_version()


def _check(status):
    if status != MHA_OK:
        raise MhaError(status, last_error())


def dtype_code(t):
    import torch
    codes = {torch.float32: MHA_F32, torch.bfloat16: MHA_BF16, torch.float16: MHA_F16}
    if t.dtype not in codes:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return codes[t.dtype]


def _mask_code(mask):
    if mask in (None, "none", MHA_MASK_NONE):
        return MHA_MASK_NONE
    if mask in ("causal", MHA_MASK_CAUSAL):
        return MHA_MASK_CAUSAL
    raise ValueError(f"unknown mask {mask!r}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _contig(t, name):
    if t is not None and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _scale(scale):
    """None -> NaN: the library then uses 1/sqrt(d_k)."""
    return float("nan") if scale is None else float(scale)


def _lens(t, B, name):
    if t is None:
        return None
    import torch
    if t.dtype != torch.int32 or t.numel() != B or not t.is_cuda:
        raise ValueError(f"{name} must be a device int32 tensor of {B} elements")
    return _contig(t, name)


def sdpa(Q, K, V, scale=None, mask="none", seq_lens=None, out=None, stream=None):
    """mha_sdpa: Q [B,h,n_q,d_k], K [B,h,n_k,d_k], V [B,h,n_k,d_v] -> O
    [B,h,n_q,d_v] (allocated if ``out`` is None)."""
    import torch
    for n, t in (("Q", Q), ("K", K), ("V", V)):
        _contig(t, n)
        if t.dim() != 4:
            raise ValueError(f"{n} must be 4-d [B, h, n, d]")
    B, h, n_q, d_k = Q.shape
    n_k, d_v = K.shape[2], V.shape[3]
    if out is None:
        out = torch.empty((B, h, n_q, d_v), dtype=Q.dtype, device=Q.device)
    _contig(out, "out")
    lens = _lens(seq_lens, B, "seq_lens")
    _check(lib().mha_sdpa(_ptr(Q), _ptr(K), _ptr(V), _ptr(out), dtype_code(Q), B, h, n_q, n_k,
                          d_k, d_v, _scale(scale), _mask_code(mask), _ptr(lens), _stream(stream)))
    return out


def sdpa_window(Q, K, V, left, right, scale=None, seq_lens=None, out=None, stream=None):
    """mha_sdpa_window: restricted attention, key c visible to query r iff
    r - left <= c <= r + right.  Shapes as sdpa()."""
    import torch
    for n, t in (("Q", Q), ("K", K), ("V", V)):
        _contig(t, n)
        if t.dim() != 4:
            raise ValueError(f"{n} must be 4-d [B, h, n, d]")
    B, h, n_q, d_k = Q.shape
    n_k, d_v = K.shape[2], V.shape[3]
    if out is None:
        out = torch.empty((B, h, n_q, d_v), dtype=Q.dtype, device=Q.device)
    _contig(out, "out")
    lens = _lens(seq_lens, B, "seq_lens")
    _check(lib().mha_sdpa_window(_ptr(Q), _ptr(K), _ptr(V), _ptr(out), dtype_code(Q), B, h, n_q,
                                 n_k, d_k, d_v, _scale(scale), int(left), int(right), _ptr(lens),
                                 _stream(stream)))
    return out


def _bhnd(t, name):
    """(shape, [batch, head, row] strides) of a [B, h, n, d] tensor view whose
    last axis is contiguous."""
    if t.dim() != 4:
        raise ValueError(f"{name} must be 4-d [B, h, n, d]")
    if t.shape[3] > 1 and t.stride(3) != 1:
        raise ValueError(f"{name}: the last axis must be contiguous")
    # (a dimension of size 1 is never stepped along: its stride is passed as 0)
    return tuple(t.shape), tuple(0 if t.shape[i] == 1 else t.stride(i) for i in range(3))


def _strides(Q, K, V, O):
    st = SdpaStrides()
    for f, t, n in (("q", Q, "Q"), ("k", K, "K"), ("v", V, "V"), ("o", O, "out")):
        getattr(st, f)[:] = _bhnd(t, n)[1]
    return st


def sdpa_strided(Q, K, V, scale=None, mask="none", seq_lens=None, out=None, stream=None):
    """mha_sdpa_strided: as sdpa(), for [B, h, n, d] views with any strides
    (last axis contiguous), e.g. ``x.view(B, n, h, d).transpose(1, 2)``.
    ``out`` may be a strided view too (allocated contiguous if None)."""
    import torch
    (B, h, n_q, d_k), _ = _bhnd(Q, "Q")
    (_, _, n_k, _), _ = _bhnd(K, "K")
    d_v = V.shape[3]
    if out is None:
        out = torch.empty((B, h, n_q, d_v), dtype=Q.dtype, device=Q.device)
    lens = _lens(seq_lens, B, "seq_lens")
    st = _strides(Q, K, V, out)
    _check(lib().mha_sdpa_strided(_ptr(Q), _ptr(K), _ptr(V), _ptr(out), ctypes.byref(st),
                                  dtype_code(Q), B, h, n_q, n_k, d_k, d_v, _scale(scale),
                                  _mask_code(mask), _ptr(lens), _stream(stream)))
    return out


def sdpa_window_strided(Q, K, V, left, right, scale=None, seq_lens=None, out=None, stream=None):
    """mha_sdpa_window_strided: sdpa_window() on strided views."""
    import torch
    (B, h, n_q, d_k), _ = _bhnd(Q, "Q")
    (_, _, n_k, _), _ = _bhnd(K, "K")
    d_v = V.shape[3]
    if out is None:
        out = torch.empty((B, h, n_q, d_v), dtype=Q.dtype, device=Q.device)
    lens = _lens(seq_lens, B, "seq_lens")
    st = _strides(Q, K, V, out)
    _check(lib().mha_sdpa_window_strided(_ptr(Q), _ptr(K), _ptr(V), _ptr(out), ctypes.byref(st),
                                         dtype_code(Q), B, h, n_q, n_k, d_k, d_v, _scale(scale),
                                         int(left), int(right), _ptr(lens), _stream(stream)))
    return out


def sdpa_route(dtype, B, h, n_q, n_k, d_k, mask="none", window=None, d_v=None):
    """mha_sdpa_route: the kernel mha_sdpa (or, with ``window`` = (left,
    right), mha_sdpa_window) runs for these sizes.  ``dtype`` is an MHA_*
    code.  Returns a dict; needs no device."""
    r = Route()
    left, right = (0, 0) if window is None else window
    _check(lib().mha_sdpa_route(int(dtype), B, h, n_q, n_k, d_k, d_k if d_v is None else d_v,
                                _mask_code(mask), 0 if window is None else 1, int(left), int(right),
                                ctypes.byref(r)))
    return {"kernel": KERNELS.get(r.kernel, r.kernel), "waves": r.waves,
            "rows_per_workgroup": r.rows_per_workgroup, "mask_kind": r.mask_kind,
            "workgroups": r.workgroups}


def workspace_size(B, n_q, n_k, d_model, h, dtype):
    return int(lib().mha_forward_workspace_size(B, n_q, n_k, d_model, h, dtype))


def forward(x_q, Wq, Wk, Wv, Wo, h, x_kv=None, mask="none", kv_lens=None, out=None,
            workspace=None, stream=None):
    """mha_forward: x_q [B,n_q,d_model], x_kv [B,n_k,d_model] or None (self),
    W* [d_model, d_model] -> out [B,n_q,d_model].  ``workspace`` is a uint8
    device tensor of at least workspace_size(...) bytes, or None (the
    library allocates stream-ordered)."""
    import torch
    for n, t in (("x_q", x_q), ("x_kv", x_kv), ("Wq", Wq), ("Wk", Wk), ("Wv", Wv), ("Wo", Wo)):
        _contig(t, n)
    B, n_q, d_model = x_q.shape
    n_k = n_q if x_kv is None else x_kv.shape[1]
    for n, t in (("Wq", Wq), ("Wk", Wk), ("Wv", Wv), ("Wo", Wo)):
        if tuple(t.shape) != (d_model, d_model):
            raise ValueError(f"{n} must be [{d_model}, {d_model}]")
    if out is None:
        out = torch.empty((B, n_q, d_model), dtype=x_q.dtype, device=x_q.device)
    _contig(out, "out")
    lens = _lens(kv_lens, B, "kv_lens")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().mha_forward(_ptr(x_q), _ptr(x_kv), _ptr(Wq), _ptr(Wk), _ptr(Wv), _ptr(Wo),
                             _ptr(out), dtype_code(x_q), B, n_q, n_k, d_model, int(h),
                             _mask_code(mask), _ptr(lens), _ptr(workspace), ws_bytes,
                             _stream(stream)))
    return out


def forward_noalloc(x_q, Wq, Wk, Wv, Wo, h, x_kv=None, mask="none", kv_lens=None, out=None,
                    stream=None):
    """mha_forward_noalloc: forward() with the library's own scratch array as
    the workspace (no allocation inside the call; calls overlapping on one
    GPU race).  ``out`` must be given by callers that cannot allocate."""
    import torch
    for n, t in (("x_q", x_q), ("x_kv", x_kv), ("Wq", Wq), ("Wk", Wk), ("Wv", Wv), ("Wo", Wo)):
        _contig(t, n)
    B, n_q, d_model = x_q.shape
    n_k = n_q if x_kv is None else x_kv.shape[1]
    for n, t in (("Wq", Wq), ("Wk", Wk), ("Wv", Wv), ("Wo", Wo)):
        if tuple(t.shape) != (d_model, d_model):
            raise ValueError(f"{n} must be [{d_model}, {d_model}]")
    if out is None:
        out = torch.empty((B, n_q, d_model), dtype=x_q.dtype, device=x_q.device)
    _contig(out, "out")
    lens = _lens(kv_lens, B, "kv_lens")
    _check(lib().mha_forward_noalloc(_ptr(x_q), _ptr(x_kv), _ptr(Wq), _ptr(Wk), _ptr(Wv), _ptr(Wo),
                                     _ptr(out), dtype_code(x_q), B, n_q, n_k, d_model, int(h),
                                     _mask_code(mask), _ptr(lens), _stream(stream)))
    return out


def add_norm_workspace_size(B, n_q, n_k, d_model, h, dtype):
    return int(lib().mha_forward_add_norm_workspace_size(B, n_q, n_k, d_model, h, dtype))


def add_norm(x, sub, gamma, beta, eps=1e-5, out=None, stream=None):
    """mha_add_norm: out = LayerNorm(x + sub) over the last axis.  x, sub
    [..., d_model]; gamma, beta [d_model]; all one dtype.  ``out`` may be x
    or sub (in place)."""
    import torch
    for n, t in (("x", x), ("sub", sub), ("gamma", gamma), ("beta", beta)):
        _contig(t, n)
    d_model = x.shape[-1]
    if tuple(sub.shape) != tuple(x.shape):
        raise ValueError("x and sub must have the same shape")
    for n, t in (("gamma", gamma), ("beta", beta)):
        if tuple(t.shape) != (d_model,):
            raise ValueError(f"{n} must be [{d_model}]")
    if out is None:
        out = torch.empty_like(x)
    _contig(out, "out")
    rows = x.numel() // d_model if d_model else 0
    _check(lib().mha_add_norm(_ptr(x), _ptr(sub), _ptr(gamma), _ptr(beta), float(eps), _ptr(out),
                              dtype_code(x), rows, d_model, _stream(stream)))
    return out


def forward_add_norm(x_q, Wq, Wk, Wv, Wo, gamma, beta, h, eps=1e-5, x_kv=None, mask="none",
                     kv_lens=None, out=None, workspace=None, stream=None):
    """mha_forward_add_norm: LayerNorm(x_q + MultiHead(x_q, x_kv, x_kv)).
    Arguments as forward(), plus gamma, beta [d_model] and eps."""
    import torch
    for n, t in (("x_q", x_q), ("x_kv", x_kv), ("Wq", Wq), ("Wk", Wk), ("Wv", Wv), ("Wo", Wo),
                 ("gamma", gamma), ("beta", beta)):
        _contig(t, n)
    B, n_q, d_model = x_q.shape
    n_k = n_q if x_kv is None else x_kv.shape[1]
    for n, t in (("Wq", Wq), ("Wk", Wk), ("Wv", Wv), ("Wo", Wo)):
        if tuple(t.shape) != (d_model, d_model):
            raise ValueError(f"{n} must be [{d_model}, {d_model}]")
    for n, t in (("gamma", gamma), ("beta", beta)):
        if tuple(t.shape) != (d_model,):
            raise ValueError(f"{n} must be [{d_model}]")
    if out is None:
        out = torch.empty((B, n_q, d_model), dtype=x_q.dtype, device=x_q.device)
    _contig(out, "out")
    lens = _lens(kv_lens, B, "kv_lens")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().mha_forward_add_norm(_ptr(x_q), _ptr(x_kv), _ptr(Wq), _ptr(Wk), _ptr(Wv),
                                      _ptr(Wo), _ptr(gamma), _ptr(beta), float(eps), _ptr(out),
                                      dtype_code(x_q), B, n_q, n_k, d_model, int(h),
                                      _mask_code(mask), _ptr(lens), _ptr(workspace), ws_bytes,
                                      _stream(stream)))
    return out
