"""mha_sdpa on the GPU against the fp64 oracle, element by element.

Tolerance (max-abs): 2e-2 for bf16/fp16 inputs, 1e-5 for the fp32 path.
Sizes span several tiles with ragged tails; the full-size long-sequence
workload is checked on whole sampled heads plus sampled rows of every head
(each sampled causal row r against the unmasked attention of q_r over keys
0..r, the reduction the pins establish for the oracle).
"""

import math

import numpy as np
import pytest

import oracle
from gpu_util import (TOL, from_dev, gpu_sdpa, lens_dev, note, require_gpu, rounded, to_dev,
                      torch)
import pins
from transformer_head_scaled_amd import libmha, synth

pytestmark = pytest.mark.gpu

MASKS = {"none": oracle.MASK_NONE, "causal": oracle.MASK_CAUSAL}
_TORCH = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _run(ins, dtype, mask, lens=None, scale=0.125):
    tq, tk, tv = (to_dev(ins[n][0], dtype) for n in "QKV")
    out = libmha.sdpa(tq, tk, tv, scale=scale, mask=mask, seq_lens=lens_dev(lens))
    torch.cuda.synchronize()
    return from_dev(out)


def _check(got, exp, dtype, what):
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = float(np.max(np.abs(got - exp))) if got.size else 0.0
    print(f"[parity] {what}: max-abs {err:.3e} (tol {TOL[dtype]:.0e})", flush=True)
    assert err <= TOL[dtype], f"{what}: max-abs {err:.3e} > {TOL[dtype]}"


def test_workload_f32_single_head():
    """[1,1,16,64] fp32, no mask, scale 1/8: the 1e-5 parity case."""
    w = synth.WORKLOADS[1]
    ins = synth.sdpa_inputs(1, w["B"], w["h"], w["n_q"], w["n_k"], w["d"], dtype="f32")
    note("sdpa f32 [1,1,16,64]")
    got = _run(ins, "f32", "none")
    exp = oracle.sdpa(ins["Q"][1], ins["K"][1], ins["V"][1], 0.125)
    _check(got, exp, "f32", "f32 [1,1,16,64]")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_workload_causal_b16_n512(dtype):
    """[16,8,512,64] causal (decoder self-attention), all outputs."""
    ins = synth.sdpa_inputs(3, 16, 8, 512, 512, 64, dtype=dtype)
    note(f"sdpa {dtype} causal [16,8,512,64]")
    got = _run(ins, dtype, "causal")
    exp = oracle.sdpa(ins["Q"][1], ins["K"][1], ins["V"][1], 0.125, oracle.MASK_CAUSAL)
    _check(got, exp, dtype, f"{dtype} causal [16,8,512,64]")


def test_causal_resident_grid_second_round_order():
    """Causal [8,8,600,64]: 320 four-wave pair workgroups, all resident at
    once, whose second-round slots take the row groups shortest first.  Rows
    are ragged (600 = 4·128 + 88) and so are the key lengths; every output
    against the oracle, then bitwise against the opposite launch order."""
    B, h, n = 8, 8, 600
    r = libmha.sdpa_route(libmha.MHA_BF16, B, h, n, n, 64, mask="causal")
    assert (r["kernel"], r["waves"], r["workgroups"]) == ("pairs", 4, 320), r
    ins = synth.sdpa_inputs(14, B, h, n, n, 64, dtype="bf16")
    lens = np.random.default_rng(14).integers(250, n + 1, size=B).astype(np.int32)
    lens[0] = n
    note(f"sdpa bf16 causal [8,8,600,64] lens {lens.tolist()}")
    got = _run(ins, "bf16", "causal", lens=lens)
    exp = oracle.sdpa(ins["Q"][1], ins["K"][1], ins["V"][1], 0.125, oracle.MASK_CAUSAL, lens)
    _check(got, exp, "bf16", "causal [8,8,600,64] ragged lens")


@pytest.mark.parametrize("mask", ["none", "causal"])
def test_workload_long_b4_n4096_all_heads(mask):
    """[4,8,4096,64], the launch the bench times: every output of every one
    of the 32 heads against the oracle."""
    dtype = "bf16"
    ins = synth.sdpa_inputs(5, 4, 8, 4096, 4096, 64, dtype=dtype)
    note(f"sdpa bf16 {mask} [4,8,4096,64]")
    got = _run(ins, dtype, mask)
    Q, K, V = (ins[n][1] for n in "QKV")
    mk = MASKS[mask]
    err = 0.0
    for b in range(4):
        for i in range(8):
            exp, _ = oracle.attention_head(Q[b, i], K[b, i], V[b, i], 0.125, mk)
            assert np.all(np.isfinite(got[b, i])), f"head ({b},{i}): non-finite output"
            err = max(err, float(np.max(np.abs(got[b, i] - exp))))
    print(f"[parity] {mask} [4,8,4096,64] all 32 heads: max-abs {err:.3e}", flush=True)
    assert err <= TOL[dtype]


@pytest.mark.parametrize("shape,mask,route", [
    ((1, 3, 2304, 64), "causal", ("pairs", 4)),   # few heads: four-wave pair workgroups past 2048 rows
    ((1, 4, 1536, 64), "none", ("pairs", 4)),     # unmasked pair layout, four waves by the makespan rule
    ((8, 8, 2560, 64), "none", ("blocks", 4)),    # two-block layout, four waves (ragged eight-wave round)
])
def test_workgroup_size_rules_sampled(shape, mask, route):
    """Shapes whose workgroup size comes from the grid-size rules (few heads,
    ragged last rounds; the route is asserted): one whole head, plus sampled
    rows of every head."""
    B, H, n, d = shape
    r = libmha.sdpa_route(libmha.MHA_BF16, B, H, n, n, d, mask=mask)
    assert (r["kernel"], r["waves"]) == route, r
    ins = synth.sdpa_inputs(57, B, H, n, n, d, dtype="bf16")
    note(f"sdpa bf16 {mask} {list(shape)}")
    got = _run(ins, "bf16", mask)
    Q, K, V = (ins[x][1] for x in "QKV")
    mk = MASKS[mask]
    exp, _ = oracle.attention_head(Q[B - 1, H - 1], K[B - 1, H - 1], V[B - 1, H - 1], 0.125, mk)
    _check(got[B - 1, H - 1], exp, "bf16", f"{mask} {list(shape)} last head, all rows")
    rs = np.random.default_rng(58)
    rows = np.concatenate([[0, 255, 256, n - 1], rs.integers(0, n, size=4)])
    err = 0.0
    for b in range(B):
        for i in range(H):
            for r in rows:
                top = r + 1 if mask == "causal" else n
                e, _ = oracle.attention_head(Q[b, i, r:r + 1], K[b, i, :top], V[b, i, :top], 0.125)
                err = max(err, float(np.max(np.abs(got[b, i, r] - e[0]))))
    print(f"[parity] {mask} {list(shape)} sampled rows: max-abs {err:.3e}", flush=True)
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_four_wave_workgroups_ragged_lens(dtype):
    """[8,16,1000,1000] with per-batch key lengths (0, 1, 63, 64, 500, 999,
    1000, and one past n_k): enough row blocks for the 4-wave (256-row)
    workgroups, with a ragged last row block and key-length boundary tiles.
    One whole head per batch is compared."""
    lens = [1000, 999, 500, 64, 63, 1, 0, 1100]
    ins = synth.sdpa_inputs(31, 8, 16, 1000, 1000, 64, dtype=dtype)
    note(f"sdpa {dtype} [8,16,1000,1000] key lengths {lens}")
    got = _run(ins, dtype, "none", lens)
    Q, K, V = (ins[n][1] for n in "QKV")
    for b in range(8):
        i = (5 * b) % 16
        exp = oracle.sdpa(Q[b:b + 1, i:i + 1], K[b:b + 1, i:i + 1], V[b:b + 1, i:i + 1], 0.125,
                          oracle.MASK_NONE, [lens[b]])[0, 0]
        _check(got[b, i], exp, dtype, f"{dtype} 4-wave head ({b},{i}) len {lens[b]}")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_eight_wave_workgroups_ragged_lens(dtype):
    """[8,8,4000,4000] unmasked with key lengths (0, 1, 63, 64, 1000, 3999,
    4000, and one past n_k): the two-block layout with eight-wave (512-row)
    workgroups (the route is asserted), a ragged last one (4000 = 7·512 +
    416) and key-length boundary tiles.  One whole head per batch."""
    lens = [4000, 3999, 1000, 64, 63, 1, 0, 5000]
    r = libmha.sdpa_route(libmha.dtype_code(torch.empty(0, dtype=_TORCH[dtype])), 8, 8, 4000, 4000, 64)
    assert (r["kernel"], r["waves"]) == ("blocks", 8), r
    ins = synth.sdpa_inputs(37, 8, 8, 4000, 4000, 64, dtype=dtype)
    note(f"sdpa {dtype} [8,8,4000,4000] key lengths {lens}")
    got = _run(ins, dtype, "none", lens)
    Q, K, V = (ins[n][1] for n in "QKV")
    for b in range(8):
        i = (3 * b + 2) % 8
        exp = oracle.sdpa(Q[b:b + 1, i:i + 1], K[b:b + 1, i:i + 1], V[b:b + 1, i:i + 1], 0.125,
                          oracle.MASK_NONE, [lens[b]])[0, 0]
        _check(got[b, i], exp, dtype, f"{dtype} 8-wave head ({b},{i}) len {lens[b]}")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
def test_many_short_heads(dtype, d):
    """[64,32,50,70] unmasked with key lengths: 2048 heads of fewer than 64
    query rows, enough waves for the one-wave two-block workgroups (fewer
    heads take the pair layout).  Every head is compared."""
    lens = [70, 69, 64, 63, 1, 0, 33, 100] * 8
    scale = 1 / math.sqrt(d)
    ins = synth.sdpa_inputs(77 + d, 64, 32, 50, 70, d, dtype=dtype)
    note(f"sdpa {dtype} d={d} [64,32,50,70] key lengths")
    got = _run(ins, dtype, "none", lens, scale=scale)
    exp = oracle.sdpa(ins["Q"][1], ins["K"][1], ins["V"][1], scale, oracle.MASK_NONE, lens)
    _check(got, exp, dtype, f"{dtype} d={d} 2048 short heads")


# ragged shapes: tails of the 128-row query blocks and 64-key tiles, tiny
# sizes, cross-attention n_q != n_k, key padding including 0 and > n_k
RAGGED = [
    # (B, h, n_q, n_k, mask, lens)
    (1, 1, 1, 1, "none", None),
    (2, 3, 1, 77, "none", None),
    (1, 2, 33, 33, "causal", None),
    (2, 2, 129, 129, "causal", None),
    (3, 1, 200, 200, "causal", [0, 150, 999]),
    (2, 2, 100, 300, "none", [1, 300]),
    (1, 4, 257, 65, "none", None),
    (2, 1, 64, 64, "none", [64, 17]),
    (1, 1, 384, 512, "none", None),
]


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("case", RAGGED, ids=lambda c: "x".join(map(str, c[:4])) + f"_{c[4]}" + ("_lens" if c[5] else ""))
def test_ragged(dtype, case):
    B, h, n_q, n_k, mask, lens = case
    ins = synth.sdpa_inputs(100 + n_q, B, h, n_q, n_k, 64, dtype=dtype)
    note(f"sdpa {dtype} ragged {case}")
    got = _run(ins, dtype, mask, lens)
    exp = oracle.sdpa(ins["Q"][1], ins["K"][1], ins["V"][1], 0.125, MASKS[mask], lens)
    _check(got, exp, dtype, f"{dtype} {case}")


# Keys up to the 2 GiB range of one head's K (and V) buffer: the key and
# value rows are a random block of P rows (P prime) repeated R times, so
# attention over all R·P keys is attention over one copy (every weight of a
# copy appears R times and R cancels in the normalisation), which the oracle
# computes on the block.  A 32-bit offset that wrapped (2^32 bytes = 2^25
# rows, not a multiple of P) or a range that ended early would read other
# rows.
_P, _R = 65521, 255  # 255·65521 keys · 128 bytes = 99.6 % of 2^31 − 1


@pytest.mark.parametrize("n_q,kernel", [(1, "decode"), (64, "split")])
def test_keys_at_the_buffer_limit(n_q, kernel):
    d = 64
    n_k = _P * _R
    assert n_k * d * 2 <= 2**31 - 1 and n_k * d * 2 > 0.99 * 2**31
    r = libmha.sdpa_route(libmha.MHA_BF16, 1, 1, n_q, n_k, d)
    assert r["kernel"] == kernel, r
    ins = synth.sdpa_inputs(4242 + n_q, 1, 1, n_q, _P, d)
    q = to_dev(ins["Q"][0], "bf16")
    k = to_dev(np.tile(ins["K"][0], (1, 1, _R, 1)), "bf16")
    v = to_dev(np.tile(ins["V"][0], (1, 1, _R, 1)), "bf16")
    note(f"sdpa bf16 [1,1,{n_q},{n_k}] ({kernel} kernel), K and V {n_k * d * 2 / 2**30:.3f} GiB each")
    for lens, copies in ((None, _R), ([200 * _P], 200)):
        out = libmha.sdpa(q, k, v, scale=0.125, seq_lens=lens_dev(lens))
        torch.cuda.synchronize()
        got = from_dev(out)
        exp = oracle.sdpa(ins["Q"][1], ins["K"][1], ins["V"][1], 0.125, oracle.MASK_NONE)
        _check(got, exp, "bf16", f"[1,1,{n_q},{n_k}] {copies} copies of {_P} keys")
    del k, v
    torch.cuda.empty_cache()


@pytest.mark.parametrize("mask", ["none", "causal"])
def test_long_sequence_sampled_rows(mask):
    """[1,2,65536,64]: a thousand key tiles per row block; sampled rows
    (both ends, tile and block boundaries, random) against the oracle on
    exactly the keys each sees."""
    B, h, n, d = 1, 2, 65536, 64
    ins = synth.sdpa_inputs(65536, B, h, n, n, d)
    note(f"sdpa bf16 [1,2,65536,64] {mask}")
    got = _run(ins, "bf16", mask)
    rng = np.random.default_rng(7)
    rows = sorted(set([0, 1, 31, 32, 63, 64, 4095, 4096, 32767, 32768, n - 65, n - 64, n - 2, n - 1] +
                      list(rng.integers(0, n, 12))))
    Q, K, V = (ins[x][1] for x in "QKV")
    for hh in range(h):
        for r in rows:
            kend = r + 1 if mask == "causal" else n
            exp = oracle.sdpa(Q[:, hh:hh + 1, r:r + 1], K[:, hh:hh + 1, :kend], V[:, hh:hh + 1, :kend],
                              0.125, oracle.MASK_NONE)
            _check(got[:, hh:hh + 1, r:r + 1], exp, "bf16", f"[1,2,65536,64] {mask} head {hh} row {r}")


@pytest.mark.parametrize("d", [16, 32, 128])
def test_f32_head_dims(d):
    ins = synth.sdpa_inputs(7, 2, 2, 70, 45, d, dtype="f32")
    note(f"sdpa f32 d={d}")
    got = _run(ins, "f32", "none", [45, 12], scale=1 / math.sqrt(d))
    exp = oracle.sdpa(ins["Q"][1], ins["K"][1], ins["V"][1], 1 / math.sqrt(d), oracle.MASK_NONE, [45, 12])
    _check(got, exp, "f32", f"f32 d={d}")


@pytest.mark.parametrize("d,mask", [(16, "none"), (64, "causal"), (128, "none")])
def test_f32_lanes_per_row(d, mask):
    """Both forms of the fp32 kernel: [1,2,70,70] takes four lanes a row
    (16-row workgroups), [16,64,70,70] one lane a row (64-row workgroups,
    enough of them to fill the SIMDs); key lengths ragged per batch."""
    for B, h, rows in ((1, 2, 16), (16, 64, 64)):
        r = libmha.sdpa_route(libmha.MHA_F32, B, h, 70, 70, d, mask=mask)
        assert (r["kernel"], r["rows_per_workgroup"]) == ("f32", rows), r
        lens = [(70 - 9 * i) % 71 for i in range(B)]
        ins = synth.sdpa_inputs(1700 + d + B, B, h, 70, 70, d, dtype="f32")
        note(f"sdpa f32 d={d} {mask} [{B},{h},70,70] rows/workgroup {rows}")
        got = _run(ins, "f32", mask, lens, scale=1 / math.sqrt(d))
        exp = oracle.sdpa(ins["Q"][1], ins["K"][1], ins["V"][1], 1 / math.sqrt(d), MASKS[mask], lens)
        _check(got, exp, "f32", f"f32 d={d} {mask} [{B},{h},70,70]")


# Head dimensions of Table 3 rows (A) and (C) of the nickwang.xyz page
# (d_model fixed, h and d_k = d_v = d_model / h varied): the MFMA kernel for
# each, on one- and two-wave workgroups, with ragged query blocks and key
# tiles, key padding (0, 1, past n_k) and both masks.
HEAD_DIM_CASES = [
    # (B, h, n_q, n_k, mask, lens)
    (3, 2, 50, 90, "none", [90, 7, 0]),
    (2, 3, 200, 200, "causal", [150, 200]),
    (2, 2, 257, 130, "none", [130, 1]),
    (1, 3, 129, 129, "causal", None),
]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [16, 32, 128])
@pytest.mark.parametrize("case", HEAD_DIM_CASES,
                         ids=lambda c: "x".join(map(str, c[:4])) + f"_{c[4]}" + ("_lens" if c[5] else ""))
def test_head_dims(dtype, d, case):
    B, h, n_q, n_k, mask, lens = case
    scale = 1 / math.sqrt(d)
    ins = synth.sdpa_inputs(300 + d + n_q, B, h, n_q, n_k, d, dtype=dtype)
    note(f"sdpa {dtype} d={d} {case}")
    got = _run(ins, dtype, mask, lens, scale=scale)
    exp = oracle.sdpa(ins["Q"][1], ins["K"][1], ins["V"][1], scale, MASKS[mask], lens)
    _check(got, exp, dtype, f"{dtype} d={d} {case}")


# Wide heads (d_k = 256, 512: Table 3 row (A) of the nickwang.xyz page with
# h = 2 and h = 1 at d_model 512): the kernel that splits d across the waves
# of a workgroup; ragged query blocks and 32-key tiles, key padding, both
# masks.
WIDE_CASES = [
    # (B, h, n_q, n_k, mask, lens)
    (2, 1, 70, 70, "causal", None),
    (3, 2, 50, 97, "none", [97, 31, 0]),
    (1, 1, 257, 257, "causal", [200]),
    (2, 1, 33, 600, "none", None),
    (2, 2, 300, 300, "none", [300, 129]),   # unmasked: five 64-row workgroups, the last ragged
]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [256, 512])
@pytest.mark.parametrize("case", WIDE_CASES,
                         ids=lambda c: "x".join(map(str, c[:4])) + f"_{c[4]}" + ("_lens" if c[5] else ""))
def test_wide_heads(dtype, d, case):
    B, h, n_q, n_k, mask, lens = case
    scale = 1 / math.sqrt(d)
    ins = synth.sdpa_inputs(900 + d + n_q, B, h, n_q, n_k, d, dtype=dtype)
    note(f"sdpa {dtype} wide d={d} {case}")
    got = _run(ins, dtype, mask, lens, scale=scale)
    exp = oracle.sdpa(ins["Q"][1], ins["K"][1], ins["V"][1], scale, MASKS[mask], lens)
    _check(got, exp, dtype, f"{dtype} wide d={d} {case}")


# The head-dimension sweep's other launches, [4, h, 4096, d] with h·d = 512
# (and 1024 for h 8, d 128), and the route each runs on at that size.
SWEEP_ROUTES = {
    (32, 16, "none"): ("blocks", 4), (32, 16, "causal"): ("blocks", 4),
    (16, 32, "none"): ("blocks", 4), (16, 32, "causal"): ("blocks", 4),
    (4, 128, "none"): ("pairs", 4), (4, 128, "causal"): ("pairs", 4),
    (8, 128, "none"): ("blocks", 4), (8, 128, "causal"): ("pairs", 4),
}


@pytest.mark.parametrize("key", sorted(SWEEP_ROUTES), ids=lambda k: f"h{k[0]}_d{k[1]}_{k[2]}")
def test_head_dim_sweep_launches(key):
    """Each launch of the benchmark's head-dimension sweep at its full size
    and route: the first and the last head compared whole against the
    oracle (the other heads run the same code on other rows)."""
    h, d, mask = key
    B, n = 4, 4096
    r = libmha.sdpa_route(libmha.MHA_BF16, B, h, n, n, d, mask=mask)
    assert (r["kernel"], r["waves"]) == SWEEP_ROUTES[key], r
    ins = synth.sdpa_inputs(5, B, h, n, n, d, dtype="bf16")
    note(f"sdpa bf16 {mask} [{B},{h},{n},{d}] (the head-dimension sweep's launch)")
    scale = 1 / math.sqrt(d)
    got = _run(ins, "bf16", mask, scale=scale)
    assert np.all(np.isfinite(got)), "non-finite output"
    Q, K, V = (ins[k][1] for k in "QKV")
    err = 0.0
    for b, i in ((0, 0), (B - 1, h - 1)):
        exp, _ = oracle.attention_head(Q[b, i], K[b, i], V[b, i], scale, MASKS[mask])
        err = max(err, float(np.max(np.abs(got[b, i] - exp))))
    print(f"[parity] {mask} [{B},{h},{n},{d}] heads (0,0), ({B - 1},{h - 1}): max-abs {err:.3e}",
          flush=True)
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("h,d", [(2, 256), (1, 512)])
@pytest.mark.parametrize("mask", ["none", "causal"])
def test_wide_heads_bench_launch_all_heads(h, d, mask):
    """The wide-head launches the benchmark's head-dimension sweep times:
    [4,2,4096,256] and [4,1,4096,512] ([N] Table 3 (A), h·d = 512), scale
    1/sqrt(d), with the route each runs on asserted (unmasked: two 32-row
    blocks a workgroup; causal d 512: the key split); every output of every
    head against the oracle."""
    B, n = 4, 4096
    want = {"none": (8, 64), "causal": (8 if d == 512 else 4, 32)}[mask]
    r = libmha.sdpa_route(libmha.MHA_BF16, B, h, n, n, d, mask=mask)
    assert (r["kernel"], r["waves"], r["rows_per_workgroup"]) == ("wide",) + want, r
    ins = synth.sdpa_inputs(5, B, h, n, n, d, dtype="bf16")
    note(f"sdpa bf16 {mask} [{B},{h},{n},{d}] (the head-dimension sweep's launch)")
    scale = 1 / math.sqrt(d)
    got = _run(ins, "bf16", mask, scale=scale)
    Q, K, V = (ins[k][1] for k in "QKV")
    err = 0.0
    for b in range(B):
        for i in range(h):
            exp, _ = oracle.attention_head(Q[b, i], K[b, i], V[b, i], scale, MASKS[mask])
            assert np.all(np.isfinite(got[b, i])), f"head ({b},{i}): non-finite output"
            err = max(err, float(np.max(np.abs(got[b, i] - exp))))
    print(f"[parity] {mask} [{B},{h},{n},{d}] all heads: max-abs {err:.3e}", flush=True)
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [256, 512])
def test_wide_causal_long(dtype, d):
    """Causal wide heads over many key tiles: [2,2,1000,1000] with key lengths
    (1000, 777): at d 512 each row block's key tiles are split between two
    wave groups (odd tile counts, groups without a last tile, rows past the
    key length) and the two partial results merged.  Every output."""
    lens = [1000, 777]
    scale = 1 / math.sqrt(d)
    r = libmha.sdpa_route(libmha.MHA_BF16 if dtype == "bf16" else libmha.MHA_F16, 2, 2, 1000, 1000, d,
                          mask="causal")
    assert (r["kernel"], r["waves"]) == ("wide", 8 if d == 512 else 4), r
    ins = synth.sdpa_inputs(960 + d, 2, 2, 1000, 1000, d, dtype=dtype)
    note(f"sdpa {dtype} wide causal d={d} [2,2,1000,1000] lens {lens}")
    got = _run(ins, dtype, "causal", lens, scale=scale)
    exp = oracle.sdpa(ins["Q"][1], ins["K"][1], ins["V"][1], scale, oracle.MASK_CAUSAL, lens)
    _check(got, exp, dtype, f"{dtype} wide causal d={d} long")


@pytest.mark.parametrize("d", [16, 32, 128])
@pytest.mark.parametrize("mask", ["none", "causal"])
def test_head_dims_four_wave(d, mask):
    """[8,16,1000,1000] bf16 with per-batch key lengths: four-wave
    workgroups for each head dimension; one whole head per batch."""
    lens = [1000, 999, 500, 64, 63, 1, 0, 1100]
    scale = 1 / math.sqrt(d)
    ins = synth.sdpa_inputs(330 + d, 8, 16, 1000, 1000, d, dtype="bf16")
    note(f"sdpa bf16 d={d} {mask} [8,16,1000,1000] key lengths {lens}")
    got = _run(ins, "bf16", mask, lens, scale=scale)
    Q, K, V = (ins[n][1] for n in "QKV")
    for b in range(8):
        i = (3 * b + 1) % 16
        exp = oracle.sdpa(Q[b:b + 1, i:i + 1], K[b:b + 1, i:i + 1], V[b:b + 1, i:i + 1], scale,
                          MASKS[mask], [lens[b]])[0, 0]
        _check(got[b, i], exp, "bf16", f"d={d} {mask} head ({b},{i}) len {lens[b]}")


# Decoding steps (a few new query positions against the cached keys and
# values of a sequence, as in beam-search inference): the four waves of a
# workgroup split the key range and merge their partial results.  Key
# lengths leave some waves without any tile (0, 1, 64, 65), give ragged
# last tiles, and run past n_k; one and two 32-row query blocks.
DECODE_CASES = [
    # (B, h, n_q, n_k, lens)
    (8, 4, 1, 2048, [2048, 1, 0, 64, 65, 300, 1999, 5000]),
    (4, 2, 4, 1000, [1000, 513, 256, 3]),
    (3, 2, 33, 512, None),
    (2, 3, 64, 777, [777, 700]),
]


# Non-finite value rows inside masked tiles.  A masked key's weight is
# exactly 0, so its value row must have no effect even when it holds NaN or
# ±inf, while a row that does see the key takes its NaN or infinity.  The
# special keys sit inside 32-row blocks (not on block or tile boundaries), so
# that rows of the same block on either side of the key load it with their
# diagonal (or window-edge) tile; they fall in the tiles where both blocks
# of a wave are masked (key 40), where one block is (170, 183), and in the
# middle of a window edge (101).  Each key holds a different mix of NaN, +inf
# and -inf columns, so rows that see several keys get NaN from inf - inf.
NONFINITE_KEYS = {40: {5: "nan", 6: "inf"}, 101: {1: "-inf"}, 170: {0: "nan", 2: "inf", 3: "inf"},
                  183: {2: "-inf", 3: "inf", 7: "nan"}}


def _plant_nonfinite(ins, dtype, d):
    """Write the special values into the stored V (and its float64 copy)."""
    bits = {"bf16": {"nan": 0x7fc0, "inf": 0x7f80, "-inf": 0xff80},
            "f16": {"nan": 0x7e00, "inf": 0x7c00, "-inf": 0xfc00}}
    val = {"nan": np.nan, "inf": np.inf, "-inf": -np.inf}
    st, v64 = ins["V"][0], ins["V"][1]
    for key, cols in NONFINITE_KEYS.items():
        for col, kind in cols.items():
            j = col % d
            if dtype == "f32":
                st[:, :, key, j] = np.float32(val[kind])
            else:
                st.view(np.uint16)[:, :, key, j] = bits[dtype][kind]
            v64[:, :, key, j] = val[kind]


def _check_nonfinite(got, exp, dtype, what):
    """NaN exactly where the oracle has NaN, the same infinities, and the
    finite outputs within the tolerance."""
    assert np.array_equal(np.isnan(got), np.isnan(exp)), f"{what}: NaN positions differ"
    inf = np.isinf(exp)
    assert np.array_equal(np.isinf(got), inf) and np.array_equal(got[inf], exp[inf]), \
        f"{what}: infinities differ"
    fin = np.isfinite(exp)
    err = float(np.max(np.abs(got[fin] - exp[fin])))
    n_bad = int((~fin).sum())
    print(f"[parity] {what}: {n_bad} non-finite outputs match, finite max-abs {err:.3e}", flush=True)
    assert n_bad > 0 and err <= TOL[dtype], f"{what}: max-abs {err:.3e}"


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("d", [16, 32, 64, 128, 256, 512])
def test_nonfinite_values_inside_masked_tiles(dtype, d):
    """Causal [1,2,200,200] (and key lengths 200, 190) with NaN/±inf value
    elements at keys 40, 101, 170, 183: every output row against the oracle,
    NaN and infinities included.  Covers the two-block layout (d 16, 32),
    the pair layout (d 64, 128), the wide-head kernel (d 256, 512) and the
    fp32 kernel."""
    if dtype == "f32" and d > 128:
        pytest.skip("the fp32 path stops at d 128")
    scale = 1 / math.sqrt(d)
    for lens in (None, [200, 190]):
        B = 1 if lens is None else 2
        ins = synth.sdpa_inputs(47 + d, B, 2, 200, 200, d, dtype=dtype)
        _plant_nonfinite(ins, dtype, d)
        note(f"sdpa {dtype} d={d} causal [{B},2,200,200] non-finite values, lens {lens}")
        got = _run(ins, dtype, "causal", lens, scale=scale)
        exp = oracle.sdpa(ins["Q"][1], ins["K"][1], ins["V"][1], scale, oracle.MASK_CAUSAL, lens)
        _check_nonfinite(got, exp, dtype, f"{dtype} d={d} causal non-finite values lens {lens}")


@pytest.mark.parametrize("mask", ["none", "causal"])
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("d", [16, 64, 128])
def test_nonfinite_queries_and_keys(mask, dtype, d):
    """[1,2,200,200] with a NaN query element (head 0, row 77), an infinite
    element in the first key (head 0, key 0: a score of +∞ or −∞ by the sign
    of the query element it meets, so some rows start from a −∞ score) and a
    NaN key element (head 1, key 150): NaN exactly where the oracle has it
    (the rows that see the NaN key or meet +∞, row 77, and causal row 0,
    whose only score is −∞), every other output within the tolerance."""
    scale = 1 / math.sqrt(d)
    ins = synth.sdpa_inputs(61 + d, 1, 2, 200, 200, d, dtype=dtype)
    # row 0 of head 0 meets −∞ at key 0: under the causal mask its only key,
    # so its softmax is 0/0 (NaN); unmasked, the other keys keep it finite
    st, v64 = ins["Q"]
    if v64[0, 0, 0, 3 % d] > 0:
        v64[0, 0, 0, 3 % d] = -v64[0, 0, 0, 3 % d]
        if dtype == "f32":
            st[0, 0, 0, 3 % d] = -st[0, 0, 0, 3 % d]
        else:
            st.view(np.uint16)[0, 0, 0, 3 % d] ^= 0x8000
    bits = {"bf16": {"nan": 0x7fc0, "inf": 0x7f80}, "f16": {"nan": 0x7e00, "inf": 0x7c00}}
    for name, hh, row, col, kind in (("Q", 0, 77, 5 % d, "nan"), ("K", 0, 0, 3 % d, "inf"),
                                     ("K", 1, 150, 7 % d, "nan")):
        st, v64 = ins[name]
        if dtype == "f32":
            st[0, hh, row, col] = np.float32(np.nan if kind == "nan" else np.inf)
        else:
            st.view(np.uint16)[0, hh, row, col] = bits[dtype][kind]
        v64[0, hh, row, col] = np.nan if kind == "nan" else np.inf
    note(f"sdpa {dtype} d={d} {mask} [1,2,200,200] non-finite Q and K")
    got = _run(ins, dtype, mask, scale=scale)
    exp = oracle.sdpa(ins["Q"][1], ins["K"][1], ins["V"][1], scale, MASKS[mask])
    # some rows meet −∞ at key 0 and stay finite
    assert np.isfinite(exp[0, 0, 1:, 0]).any()
    _check_nonfinite(got, exp, dtype, f"{dtype} d={d} {mask} non-finite Q and K")


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("d", [16, 64, 128])
def test_nonfinite_values_window_edges(dtype, d):
    """Restricted attention over [1,2,200,200] (reach 37 back, 5 forward)
    with the same non-finite value elements: each special key lies inside
    the windows of some rows of its block and outside those of others."""
    scale = 1 / math.sqrt(d)
    ins = synth.sdpa_inputs(53 + d, 1, 2, 200, 200, d, dtype=dtype)
    _plant_nonfinite(ins, dtype, d)
    tq, tk, tv = (to_dev(ins[n][0], dtype) for n in "QKV")
    note(f"sdpa_window {dtype} d={d} [1,2,200,200] (37, 5) non-finite values")
    out = libmha.sdpa_window(tq, tk, tv, 37, 5, scale=scale)
    torch.cuda.synchronize()
    exp = oracle.sdpa(ins["Q"][1], ins["K"][1], ins["V"][1], scale, window=(37, 5))
    _check_nonfinite(from_dev(out), exp, dtype, f"{dtype} d={d} window non-finite values")


def test_workload_decode_step():
    """The decoding-step workload (64 beams, h 8, one query row against a
    2048-entry cache with lengths in [1792, 2048]), all outputs."""
    w = synth.WORKLOADS[6]
    ins, lens = synth.workload_inputs(6)
    note("sdpa bf16 decode workload [64,8,1,2048]")
    got = _run(ins, "bf16", "none", lens)
    exp = oracle.sdpa(ins["Q"][1], ins["K"][1], ins["V"][1], 0.125, oracle.MASK_NONE, lens)
    _check(got, exp, "bf16", w["name"])


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [16, 32, 64, 128])
@pytest.mark.parametrize("case", DECODE_CASES,
                         ids=lambda c: "x".join(map(str, c[:4])) + ("_lens" if c[4] else ""))
def test_decode_key_split(dtype, d, case):
    B, h, n_q, n_k, lens = case
    scale = 1 / math.sqrt(d)
    ins = synth.sdpa_inputs(400 + d + n_q, B, h, n_q, n_k, d, dtype=dtype)
    note(f"sdpa {dtype} decode d={d} {case}")
    got = _run(ins, dtype, "none", lens, scale=scale)
    exp = oracle.sdpa(ins["Q"][1], ins["K"][1], ins["V"][1], scale, oracle.MASK_NONE, lens)
    _check(got, exp, dtype, f"{dtype} decode d={d} {case}")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
def test_decode_padding_nan_inf(dtype, d):
    """One query row against 777 cached keys (the decoding-step kernel) with
    key lengths 777, 700, 513, 8, 0: the K and V rows past each length hold
    NaN and +/-inf, which must have no effect (a masked key's weight is
    exactly 0 and its value never enters).  Lengths that are not a multiple
    of a wave's run leave its last step partly past the length."""
    B, h, n_k = 5, 3, 777
    lens = [777, 700, 513, 8, 0]
    ins = synth.sdpa_inputs(450 + d, B, h, 1, n_k, d, dtype=dtype)
    bad = {"bf16": (0x7fc0, 0x7f80, 0xff80), "f16": (0x7e00, 0x7c00, 0xfc00)}[dtype]
    for name in "KV":
        st = ins[name][0].view(np.uint16)
        for b, n in enumerate(lens):
            st[b, :, n:, 0::3] = bad[0]
            st[b, :, n:, 1::3] = bad[1]
            st[b, :, n:, 2::3] = bad[2]
    scale = 1 / math.sqrt(d)
    note(f"sdpa {dtype} decode d={d} NaN/inf past the key lengths")
    got = _run(ins, dtype, "none", lens, scale=scale)
    Q, K, V = (ins[n][1] for n in "QKV")
    exp = np.zeros_like(got)
    for b, n in enumerate(lens):   # the oracle sees the valid keys only
        if n:
            exp[b] = oracle.sdpa(Q[b:b + 1], K[b:b + 1, :, :n], V[b:b + 1, :, :n], scale)[0]
    _check(got, exp, dtype, f"{dtype} decode d={d} with NaN/inf padding")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("scale", [-0.3, 0.0, 1.0])
def test_unusual_scales(dtype, scale):
    """A negative scale (the kernel negates Q exactly), scale 0 (uniform
    weights) and an unscaled softmax."""
    ins = synth.sdpa_inputs(8, 2, 2, 130, 130, 64, dtype=dtype)
    note(f"sdpa {dtype} scale={scale}")
    for mask in ("none", "causal"):
        got = _run(ins, dtype, mask, [130, 61], scale=scale)
        exp = oracle.sdpa(ins["Q"][1], ins["K"][1], ins["V"][1], scale, MASKS[mask], [130, 61])
        _check(got, exp, dtype, f"{dtype} scale={scale} {mask}")


@pytest.mark.parametrize("case", [
    # (B, h, n_q, n_k, d, mask, window, lens): layouts whose first tile takes its reference
    # value from the scores in registers, and the d 64 pre-pass
    (2, 2, 300, 300, 64, "none", (0, 0), None),       # window: a row sees one key
    (2, 2, 300, 300, 64, "none", (3, 5), [300, 151]),
    (2, 2, 300, 300, 64, "none", (40, 20), None),
    (4, 2, 4, 1000, 64, "none", None, [1000, 700, 65, 1]),  # key split
    (2, 4, 300, 300, 32, "causal", None, [300, 77]),   # two-block causal, d 32
    (2, 4, 300, 300, 16, "none", None, None),
    (2, 4, 300, 300, 128, "causal", None, [300, 180]),  # pair layout, d 128
])
def test_large_logits(case):
    """Scale 1 on unit-variance inputs (logits of standard deviation 8): the
    accept test fails on many tiles after the first, so the exact path and
    its rescale run again and again on top of the first tile's reference
    value."""
    B, h, n_q, n_k, d, mask, window, lens = case
    ins = synth.sdpa_inputs(15, B, h, n_q, n_k, d, dtype="bf16")
    tq, tk, tv = (to_dev(ins[n][0], "bf16") for n in "QKV")
    note(f"sdpa bf16 scale 1 {case}")
    if window is None:
        out = libmha.sdpa(tq, tk, tv, scale=1.0, mask=mask, seq_lens=lens_dev(lens))
    else:
        out = libmha.sdpa_window(tq, tk, tv, window[0], window[1], scale=1.0, seq_lens=lens_dev(lens))
    torch.cuda.synchronize()
    got = from_dev(out)
    exp = oracle.sdpa(ins["Q"][1], ins["K"][1], ins["V"][1], 1.0, MASKS[mask], lens, window=window)
    _check(got, exp, "bf16", f"scale 1 {case}")


# ---- the oracle's pins, re-run through the library

GPU_PINS = [pins.pin_rows_sum_to_one, pins.pin_zero_query_is_mean, pins.pin_causal_row0,
            pins.pin_permutation, pins.pin_one_hot, pins.pin_mask_reduces,
            pins.pin_masked_contents_ignored]


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("pin", GPU_PINS, ids=lambda p: p.__name__)
def test_pin_through_api(pin, dtype):
    fn, rnd = gpu_sdpa(dtype)
    note(f"pin {pin.__name__} {dtype}")
    kw = {"rnd": rnd}
    if pin in (pins.pin_causal_row0, pins.pin_masked_contents_ignored):
        kw["atol"] = 0.0          # exact: row 0 sees one key; masked rows never read
    else:
        kw["atol"] = TOL[dtype]
    pin(fn, **kw)


def test_pin_rows_sum_long():
    fn, rnd = gpu_sdpa("bf16")
    note("pin rows-sum-to-one long")
    pins.pin_rows_sum_to_one(fn, atol=TOL["bf16"], rnd=rnd,
                             shapes=((1, 2, 1000, 1000, 64), (2, 1, 300, 700, 64)))


def test_empty_rows():
    for dtype in ("bf16", "f32"):
        fn, _ = gpu_sdpa(dtype)
        note(f"pin empty rows {dtype}")
        pins.pin_empty_rows(fn)


def test_worked_example_fp32():
    """The printed worked example (query "il", seven 2-d keys, scale 1/√2)
    reproduced at its printed precision through the fp32 path, with and
    without the causal toggle."""
    fn, _ = gpu_sdpa("f32")
    note("worked example f32")
    pins.pin_worked_example(fn, sum_atol=1e-6)
    pins.pin_worked_example_causal(fn, sum_atol=1e-6)


def test_worked_example_bf16_vs_oracle():
    """The same example through the bf16 MFMA path (q, k zero-padded to 64):
    equal to the oracle on the bf16-rounded inputs within 2e-2."""
    g = pins.worked_example()
    n = len(g["keys"])
    Q = np.zeros((1, 1, n, 64))
    K = np.zeros((1, 1, n, 64))
    Q[0, 0, :, :2] = g["query"]
    K[0, 0, :, :2] = g["keys"]
    V = np.zeros((1, 1, n, 64))
    V[0, 0, :, :n] = np.eye(n)
    fn, rnd = gpu_sdpa("bf16")
    note("worked example bf16")
    for mask in (oracle.MASK_NONE, oracle.MASK_CAUSAL):
        got = fn(Q, K, V, g["scale"], mask, None)
        exp = oracle.sdpa(rnd(Q), rnd(K), rnd(V), g["scale"], mask)
        _check(got, exp, "bf16", f"worked example mask={mask}")


def test_saturation_fp32():
    """σ(8) and σ(1) of the saturation example, through the fp32 path."""
    fn, _ = gpu_sdpa("f32")
    d = 64
    Q = np.zeros((1, 1, 1, d)); Q[0, 0, 0, 0] = 8.0
    K = np.zeros((1, 1, 2, d)); K[0, 0, 0, 0] = 1.0; K[0, 0, 1, 1] = 1.0
    V = np.zeros((1, 1, 2, d)); V[0, 0, 0, 0] = 1.0; V[0, 0, 1, 1] = 1.0
    sig = lambda x: 1 / (1 + math.exp(-x))  # noqa: E731
    note("saturation f32")
    p = fn(Q, K, V, 1.0, oracle.MASK_NONE, None)[0, 0, 0, :2]
    np.testing.assert_allclose(p, [sig(8), sig(-8)], atol=1e-6)
    p = fn(Q, K, V, 0.125, oracle.MASK_NONE, None)[0, 0, 0, :2]
    np.testing.assert_allclose(p, [sig(1), sig(-1)], atol=1e-6)


def test_shift_and_linearity_exact_grid():
    """Softmax shift invariance and linearity in V through the bf16 path,
    on inputs whose shifted / combined values are exactly representable in
    bf16 (multiples of 1/8 and 1/16 of small magnitude).  Both sides of the
    linearity check carry their own final bf16 rounding, so the
    coefficients are kept small (|α| + |β| < 1) to keep the sum of those
    roundings well inside the tolerance."""
    rs = np.random.default_rng(77)
    B, h, n, d = 2, 2, 150, 64
    Q = rs.integers(-8, 9, size=(B, h, n, d)) / 32.0
    K = rs.integers(-16, 17, size=(B, h, n, d)) / 8.0
    V1 = rs.integers(-8, 9, size=(B, h, n, d)) / 4.0
    V2 = rs.integers(-8, 9, size=(B, h, n, d)) / 4.0
    u = np.full(d, 4.0)
    fn, rnd = gpu_sdpa("bf16")
    for arr in (Q, K, K + u, V1, V2, 0.5 * V1 - 0.25 * V2):
        assert np.array_equal(rnd(arr), arr)
    note("shift/linearity bf16")
    for mask in (oracle.MASK_NONE, oracle.MASK_CAUSAL):
        O = fn(Q, K, V1, 0.125, mask, None)
        Os = fn(Q, K + u, V1, 0.125, mask, None)
        _check(Os, O, "bf16", f"shift invariance mask={mask}")
        O2 = fn(Q, K, V2, 0.125, mask, None)
        O12 = fn(Q, K, 0.5 * V1 - 0.25 * V2, 0.125, mask, None)
        _check(O12, 0.5 * O - 0.25 * O2, "bf16", f"linearity mask={mask}")


def test_causal_row0_bit_exact_full_size():
    """Causal row 0 is V[0] exactly, at the long-sequence size."""
    ins = synth.sdpa_inputs(5, 4, 8, 4096, 4096, 64, dtype="bf16")
    note("causal row0 [4,8,4096,64]")
    tq, tk, tv = (to_dev(ins[n][0], "bf16") for n in "QKV")
    out = libmha.sdpa(tq, tk, tv, scale=0.125, mask="causal")
    torch.cuda.synchronize()
    assert torch.equal(out[:, :, 0, :], tv[:, :, 0, :])


def test_repeatable_bitwise():
    """Fixed reduction order, no atomics: two runs are bitwise equal."""
    ins = synth.sdpa_inputs(9, 2, 8, 1000, 1000, 64, dtype="bf16")
    tq, tk, tv = (to_dev(ins[n][0], "bf16") for n in "QKV")
    note("repeatability bf16 [2,8,1000,64]")
    for mask in ("none", "causal"):
        a = libmha.sdpa(tq, tk, tv, mask=mask)
        b = libmha.sdpa(tq, tk, tv, mask=mask)
        torch.cuda.synchronize()
        assert torch.equal(a, b)


@pytest.mark.parametrize("shape,mask", [
    ((8, 8, 2048, 64), "none"),      # two-block layout, eight waves
    ((2, 8, 2048, 64), "causal"),    # pair layout
    ((8, 8, 600, 64), "causal"),     # pair layout, second round shortest first
    ((4, 4, 640, 64), "none"),       # unmasked pair layout
    ((3, 2, 1000, 32), "causal"),    # two-block causal layout (blocks u, nb - 1 - u)
    ((8, 4, 3, 1500, 64), "none"),   # key split (n_q 3 against 1500 keys)
])
def test_bitwise_same_in_reversed_workgroup_order(shape, mask, monkeypatch):
    """Each output row is produced by one workgroup in a fixed order of
    operations, so launching the workgroups in the opposite order
    (MHA_GRID_ORDER=reverse) gives bitwise the same result."""
    if len(shape) == 5:
        B, h, n_q, n_k, d = shape
    else:
        B, h, n_q, d = shape
        n_k = n_q
    ins = synth.sdpa_inputs(13, B, h, n_q, n_k, d, dtype="bf16")
    tq, tk, tv = (to_dev(ins[n][0], "bf16") for n in "QKV")
    note(f"grid order {shape} {mask}")
    a = libmha.sdpa(tq, tk, tv, mask=mask)
    monkeypatch.setenv("MHA_GRID_ORDER", "reverse")
    b = libmha.sdpa(tq, tk, tv, mask=mask)
    monkeypatch.delenv("MHA_GRID_ORDER")
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_output_guard_band():
    """The kernel writes exactly O: canary regions before and after it in
    the same allocation stay untouched."""
    B, h, n, d = 2, 3, 77, 64
    ins = synth.sdpa_inputs(10, B, h, n, n, d, dtype="bf16")
    tq, tk, tv = (to_dev(ins[n_][0], "bf16") for n_ in "QKV")
    pad = 4096
    buf = torch.full((pad + B * h * n * d + pad,), 7.0, dtype=torch.bfloat16, device="cuda")
    out = buf[pad:pad + B * h * n * d].view(B, h, n, d)
    note("guard band")
    libmha.sdpa(tq, tk, tv, mask="causal", out=out)
    torch.cuda.synchronize()
    assert torch.all(buf[:pad] == 7.0) and torch.all(buf[-pad:] == 7.0)
    exp = oracle.sdpa(ins["Q"][1], ins["K"][1], ins["V"][1], 0.125, oracle.MASK_CAUSAL)
    _check(from_dev(out), exp, "bf16", "guard band output")
