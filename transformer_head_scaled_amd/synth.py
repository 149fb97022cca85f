"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds no attention arithmetic: it only draws random numbers,
rounds them to the storage dtype and describes the workload shapes.  Both the
HIP path and the fp64 oracle receive the very same values from here (the
oracle upcasts them exactly), and neither side depends on the other.

Recipe: ``numpy.random.default_rng(SeedSequence([cfg_id, tensor_idx]))``,
float32 ``standard_normal`` draws, weights scaled by 1/sqrt(d_model) (variance
1/d_model), key lengths drawn with ``integers(lo, hi + 1)``, then rounded to
the storage dtype: bfloat16 by round-to-nearest-even on the float32 bits,
float16 by numpy's own conversion, float32 unchanged.

The shapes follow the base (d_model=512, h=8) and big (d_model=1024, h=16)
models of nickwang.xyz "Lire « Attention Is All You Need »" (Table 3), with
d_k = d_v = 64, and the variable sequence lengths of its length-bucketed
batches (§5.1).
"""

import numpy as np

# tensor indices inside one workload's seed sequence
T_Q, T_K, T_V = 0, 1, 2
T_XQ, T_XKV, T_WQ, T_WK, T_WV, T_WO, T_LENS = 0, 1, 2, 3, 4, 5, 6

DTYPES = ("f32", "bf16", "f16")

# The workloads: sizes only.  "sdpa" workloads feed Q/K/V directly; "mha"
# workloads feed x_q, x_kv and the four weights.  1-5 are the sublayer's
# configurations; 6 is one decoding step of the base model (beam search with
# 4 beams over 16 sequences, [N] §6.1: each beam's new position attends to
# its cached keys and values; caches of similar length, as in
# length-bucketed batches).
WORKLOADS = {
    1: dict(name="sdpa_f32_b1_h1_n16_d64", kind="sdpa", dtype="f32", B=1, h=1,
            n_q=16, n_k=16, d=64, masks=("none",), lens=None),
    2: dict(name="mha_self_bf16_b32_n64_dm512_h8_keypad", kind="mha",
            dtype="bf16", B=32, n_q=64, n_k=64, d_model=512, h=8,
            cross=False, masks=("none",), lens=(16, 64)),
    3: dict(name="sdpa_causal_bf16_b16_h8_n512_d64", kind="sdpa",
            dtype="bf16", B=16, h=8, n_q=512, n_k=512, d=64,
            masks=("causal",), lens=None),
    4: dict(name="mha_cross_bf16_b8_nq384_nk512_dm1024_h16", kind="mha",
            dtype="bf16", B=8, n_q=384, n_k=512, d_model=1024, h=16,
            cross=True, masks=("none",), lens=None),
    5: dict(name="sdpa_bf16_b4_h8_n4096_d64", kind="sdpa", dtype="bf16", B=4,
            h=8, n_q=4096, n_k=4096, d=64, masks=("none", "causal"),
            lens=None),
    6: dict(name="sdpa_decode_bf16_b64_h8_nq1_nk2048_cache", kind="sdpa", dtype="bf16",
            B=64, h=8, n_q=1, n_k=2048, d=64, masks=("none",), lens=(1792, 2048)),
}


def rng(cfg_id, tensor_idx):
    return np.random.default_rng(np.random.SeedSequence([int(cfg_id), int(tensor_idx)]))


def bf16_bits(x):
    """float32 array -> uint16 bfloat16 bit patterns, round to nearest even.
    NaN stays a quiet NaN."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = ((u[nan] >> np.uint64(16)).astype(np.uint16) | np.uint16(0x0040))
    return r


def bf16_to_f32(bits):
    """uint16 bfloat16 bit patterns -> float32 values (exact)."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_to(x, dtype):
    """Round a float32 array to ``dtype`` storage.

    Returns (storage, values): ``storage`` is what is copied to the device
    (uint16 bits for bf16, float16 for f16, float32 for f32) and ``values``
    is the same numbers as float32, exactly.
    """
    x = np.asarray(x, dtype=np.float32)
    if dtype == "f32":
        return x.copy(), x.copy()
    if dtype == "bf16":
        b = bf16_bits(x)
        return b, bf16_to_f32(b)
    if dtype == "f16":
        h = x.astype(np.float16)
        return h, h.astype(np.float32)
    raise ValueError(f"unknown dtype {dtype}")


def normal(cfg_id, tensor_idx, shape, std=1.0):
    g = rng(cfg_id, tensor_idx)
    x = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def key_lengths(cfg_id, B, lo, hi):
    """B valid key lengths, uniform integers in [lo, hi] (inclusive)."""
    return rng(cfg_id, T_LENS).integers(lo, hi + 1, size=B).astype(np.int32)


def sdpa_inputs(cfg_id, B, h, n_q, n_k, d_k, d_v=None, dtype="bf16"):
    """Q [B,h,n_q,d_k], K [B,h,n_k,d_k], V [B,h,n_k,d_v] ~ N(0, 1).

    Returns dict name -> (storage, float32 values)."""
    d_v = d_k if d_v is None else d_v
    out = {}
    for name, idx, shape in (("Q", T_Q, (B, h, n_q, d_k)),
                             ("K", T_K, (B, h, n_k, d_k)),
                             ("V", T_V, (B, h, n_k, d_v))):
        out[name] = round_to(normal(cfg_id, idx, shape), dtype)
    return out


def mha_inputs(cfg_id, B, n_q, n_k, d_model, h, cross, dtype="bf16"):
    """x_q [B,n_q,d_model] ~ N(0,1); x_kv [B,n_k,d_model] ~ N(0,1) when
    ``cross`` (else absent: self-attention); Wq/Wk/Wv [d_model, d_model] and
    Wo [d_model, d_model] ~ N(0, 1/d_model).  Returns dict name ->
    (storage, float32 values)."""
    wstd = 1.0 / np.sqrt(d_model)
    out = {"x_q": round_to(normal(cfg_id, T_XQ, (B, n_q, d_model)), dtype)}
    if cross:
        out["x_kv"] = round_to(normal(cfg_id, T_XKV, (B, n_k, d_model)), dtype)
    for name, idx in (("Wq", T_WQ), ("Wk", T_WK), ("Wv", T_WV), ("Wo", T_WO)):
        out[name] = round_to(normal(cfg_id, idx, (d_model, d_model), wstd), dtype)
    return out


def workload_inputs(cfg_id, dtype=None):
    """All inputs of one of the five workloads, plus its key lengths."""
    w = WORKLOADS[cfg_id]
    dt = dtype or w["dtype"]
    if w["kind"] == "sdpa":
        ins = sdpa_inputs(cfg_id, w["B"], w["h"], w["n_q"], w["n_k"], w["d"], dtype=dt)
    else:
        ins = mha_inputs(cfg_id, w["B"], w["n_q"], w["n_k"], w["d_model"], w["h"],
                         w["cross"], dtype=dt)
    lens = None
    if w["lens"] is not None:
        lens = key_lengths(cfg_id, w["B"], *w["lens"])
    return ins, lens
