"""Benchmark: fused SDPA forward TFLOP/s on MI355X, h=8, d_k=64, causal and
non-causal.

One step = one pass of the attention hot path over the long-sequence batch
[B=4, h=8, n_q=n_k=4096, d=64] bf16 in both modes: mha_sdpa without a mask,
then mha_sdpa with the causal mask (Q/K/V already resident in HBM).  The
metric counts algorithmic flops only: 4·d per visible (query, key) pair, so
the causal half that is skipped is not counted.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--settle-seconds S]
                    [--no-cpu-baseline]
    python bench.py --head-dims     # the head-dimension variants instead

Prints one JSON line.  Only one GPU is used: there is no multi-GPU path.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # dense bf16 MFMA, 256 CU x 2.4 GHz x 4096 flop/clk/CU
PEAK_HBM_GBS = 8000.0
WORKLOAD = dict(B=4, h=8, n=4096, d=64)
COPY_BYTES = 512 << 20   # plain device copy used to calibrate the HBM byte counters
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "sdpa_fwd_traffic.json")
# the sources the attention kernel is compiled from (the traffic record is
# tied to their hash)
KERNEL_SRCS = [os.path.join(ROOT, "transformer_head_scaled_amd", "csrc", f)
               for f in ("sdpa_fwd_kernel.h", "sdpa_fwd.hip", "device_common.h")] + [
    os.path.join(ROOT, "transformer_head_scaled_amd", "build.py")]  # (its compiler flags)


def sdpa_flops(B, h, n_q, n_k, d, causal):
    pairs = n_q * (n_q + 1) // 2 if causal else n_q * n_k
    return 4.0 * d * pairs * B * h


def kernel_hash():
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256_16") != kernel_hash():
        return None
    return t.get("noncausal_bytes_per_launch")


def mha_flops(B, n_q, n_k, d_model, h, causal=False, lens=None):
    """Algorithmic flops of mha_forward: four projections (2·M·N·K each) plus
    4·d per visible (query, key) pair."""
    d = d_model // h
    proj = 2.0 * d_model * d_model * (2 * B * n_q + 2 * B * n_k)
    if lens is not None:
        pairs = float(n_q) * float(sum(int(x) for x in lens))
    elif causal:
        pairs = B * n_q * (n_q + 1) / 2.0
    else:
        pairs = float(B) * n_q * n_k
    return proj + 4.0 * d * pairs * h


def time_calls(fn, stream, iters, flush=None):
    """Per-call device time (µs) of fn() with HIP events on ``stream``.  With
    ``flush`` (a callable that overwrites a large buffer) every call starts
    with cold caches.  Returns (median, min)."""
    import numpy as np
    import torch
    ts = []
    for _ in range(iters):
        if flush is not None:
            flush()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        ts.append((e0, e1))
    torch.cuda.synchronize()
    us = np.array([a.elapsed_time(b) * 1e3 for a, b in ts])
    return float(np.median(us)), float(us.min())


def time_batches(fn, stream, calls=10, reps=7):
    """Device time per call (µs) of ``calls`` back-to-back calls of fn()
    inside one event pair (the clock of the bench line's per-mode figures),
    over ``reps`` batches.  Returns (median, min) of the batch means."""
    import numpy as np
    import torch
    res = []
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(calls):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        res.append(e0.elapsed_time(e1) * 1e3 / calls)
    return float(np.median(res)), float(min(res))


def other_configs(dev, stream, iters=100):
    """The other workloads of the hot path, timed warm (and cold where the
    working set fits the 256 MB last-level cache): mha_forward self
    attention with key padding (B 32, n 64, d_model 512, h 8), causal SDPA
    (B 16, h 8, n 512), mha_forward cross attention (B 8, n_q 384, n_k 512,
    d_model 1024, h 16) also with its Add & Norm, the Add & Norm alone on
    those rows, restricted attention on the long-sequence batch (a window
    of 513 keys), and one decoding step (B 64, h 8, one query row against a
    2048-entry key/value cache, HBM-bound).  Rates use algorithmic
    flops and bytes.  Cold calls follow a read of a 512 MB buffer (a read
    leaves clean lines; an overwrite would leave dirty ones that the timed
    call then writes back)."""
    import numpy as np
    import torch
    from transformer_head_scaled_amd import libmha, synth

    def dev_t(st):
        return torch.from_numpy(np.ascontiguousarray(st).view(np.int16)).to(dev).view(torch.bfloat16)

    scratch = torch.ones(128 << 20, dtype=torch.float32, device=dev)  # 512 MB

    def flush():
        scratch.sum()

    res = {}
    # the single-head fp32 case: launch latency, neither roofline applies
    w = synth.WORKLOADS[1]
    ins1 = synth.sdpa_inputs(1, w["B"], w["h"], w["n_q"], w["n_k"], w["d"], dtype="f32")
    Q1, K1, V1 = (torch.from_numpy(ins1[k][0]).to(dev) for k in "QKV")
    O1 = torch.empty_like(Q1)

    def call1():
        libmha.sdpa(Q1, K1, V1, scale=0.125, out=O1, stream=stream)
    for _ in range(20):
        call1()
    med, mn = time_calls(call1, stream, iters)
    res[w["name"]] = {"call": "mha_sdpa f32", "us_median": round(med, 2), "us_min": round(mn, 2),
                      "flops": sdpa_flops(1, 1, 16, 16, 64, False), "bytes": 4 * 16 * 64 * 4}
    for cfg in (2, 4):
        w = synth.WORKLOADS[cfg]
        ins, lens = synth.workload_inputs(cfg)
        t = {k: dev_t(v[0]) for k, v in ins.items()}
        lens_d = None if lens is None else torch.from_numpy(lens).to(dev)
        B, n_q, n_k, dm, h = w["B"], w["n_q"], w["n_k"], w["d_model"], w["h"]
        ws = torch.empty(libmha.workspace_size(B, n_q, n_k, dm, h, 1), dtype=torch.uint8, device=dev)
        out = torch.empty((B, n_q, dm), dtype=torch.bfloat16, device=dev)

        def call():
            libmha.forward(t["x_q"], t["Wq"], t["Wk"], t["Wv"], t["Wo"], h, x_kv=t.get("x_kv"),
                           kv_lens=lens_d, out=out, workspace=ws, stream=stream)
        for _ in range(20):
            call()
        med, mn = time_calls(call, stream, iters)
        fl = mha_flops(B, n_q, n_k, dm, h, lens=lens)
        nbytes = 2 * (B * n_q * dm * 2 + (B * n_k * dm if w["cross"] else 0) + 4 * dm * dm)
        entry = {"call": "mha_forward", "us_median": round(med, 2), "us_min": round(mn, 2),
                 "tflops": round(fl / (med * 1e-6) / 1e12, 2), "flops": fl, "bytes": nbytes}
        if cfg == 2:
            cmed, cmn = time_calls(call, stream, max(iters // 4, 10), flush)
            entry["us_median_cold"] = round(cmed, 2)
        res[w["name"]] = entry
    # Add & Norm on the big cross-attention workload: the sub-layer with its
    # residual and layer normalisation in one call, and the normalisation
    # alone (HBM-bound: x and sub read, out written once)
    w = synth.WORKLOADS[4]
    ins, _ = synth.workload_inputs(4)
    t = {k: dev_t(v[0]) for k, v in ins.items()}
    B, n_q, n_k, dm, h = w["B"], w["n_q"], w["n_k"], w["d_model"], w["h"]
    gamma = torch.ones(dm, dtype=torch.bfloat16, device=dev)
    beta = torch.zeros(dm, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(libmha.add_norm_workspace_size(B, n_q, n_k, dm, h, 1), dtype=torch.uint8,
                     device=dev)
    out = torch.empty((B, n_q, dm), dtype=torch.bfloat16, device=dev)

    def call_fan():
        libmha.forward_add_norm(t["x_q"], t["Wq"], t["Wk"], t["Wv"], t["Wo"], gamma, beta, h,
                                x_kv=t["x_kv"], out=out, workspace=ws, stream=stream)
    for _ in range(20):
        call_fan()
    med, mn = time_calls(call_fan, stream, iters)
    res[w["name"] + "_add_norm"] = {"call": "mha_forward_add_norm", "us_median": round(med, 2),
                                    "us_min": round(mn, 2)}
    sub = torch.empty_like(out).normal_()

    def call_an():
        libmha.add_norm(t["x_q"], sub, gamma, beta, out=out, stream=stream)
    for _ in range(20):
        call_an()
    med, mn = time_calls(call_an, stream, iters)
    cmed, _ = time_calls(call_an, stream, max(iters // 4, 10), flush)
    nbytes = 3 * B * n_q * dm * 2 + 2 * dm * 2
    res["add_norm_bf16_rows3072_d1024"] = {
        "call": "mha_add_norm", "us_median": round(med, 2), "us_min": round(mn, 2),
        "us_median_cold": round(cmed, 2), "gbs": round(nbytes / (med * 1e-6) / 1e9, 1),
        "gbs_cold": round(nbytes / (cmed * 1e-6) / 1e9, 1),
        "hbm_frac_cold": round(nbytes / (cmed * 1e-6) / 1e9 / PEAK_HBM_GBS, 4), "bytes": nbytes}
    del t, ws, out, sub

    w = synth.WORKLOADS[3]
    ins, _ = synth.workload_inputs(3)
    Q, K, V = (dev_t(ins[k][0]) for k in "QKV")
    O = torch.empty_like(Q)

    def call3():
        libmha.sdpa(Q, K, V, scale=0.125, mask="causal", out=O, stream=stream)
    for _ in range(20):
        call3()
    med, mn = time_calls(call3, stream, iters)
    cmed, _ = time_calls(call3, stream, max(iters // 4, 10), flush)
    fl = sdpa_flops(w["B"], w["h"], w["n_q"], w["n_k"], w["d"], True)
    nbytes = 4 * w["B"] * w["h"] * w["n_q"] * w["d"] * 2
    res[w["name"]] = {"call": "mha_sdpa causal", "us_median": round(med, 2), "us_min": round(mn, 2),
                      "us_median_cold": round(cmed, 2),
                      "tflops": round(fl / (med * 1e-6) / 1e12, 2),
                      "gbs": round(nbytes / (med * 1e-6) / 1e9, 1),
                      "gbs_cold": round(nbytes / (cmed * 1e-6) / 1e9, 1),
                      "hbm_frac_cold": round(nbytes / (cmed * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                      "flops": fl, "bytes": nbytes}
    # restricted self-attention on the long-sequence workload: a centred
    # neighbourhood of 513 keys (reach 256 on each side); flops on the
    # visible pairs only
    w5 = synth.WORKLOADS[5]
    ins5 = synth.sdpa_inputs(5, w5["B"], w5["h"], w5["n_q"], w5["n_k"], w5["d"], dtype="bf16")
    Q5, K5, V5 = (dev_t(ins5[k][0]) for k in "QKV")
    O5 = torch.empty_like(Q5)
    reach = 256

    def call_w():
        libmha.sdpa_window(Q5, K5, V5, reach, reach, scale=0.125, out=O5, stream=stream)
    for _ in range(20):
        call_w()
    med, mn = time_calls(call_w, stream, iters)
    n5 = w5["n_q"]
    r = np.arange(n5)
    pairs = float(np.sum(np.minimum(n5 - 1, r + reach) - np.maximum(0, r - reach) + 1))
    fl = 4.0 * w5["d"] * pairs * w5["B"] * w5["h"]
    res["sdpa_window_bf16_b4_h8_n4096_d64_reach256"] = {
        "call": "mha_sdpa_window", "us_median": round(med, 2), "us_min": round(mn, 2),
        "tflops": round(fl / (med * 1e-6) / 1e12, 2),
        "pct_peak": round(100 * fl / (med * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 2), "flops": fl}
    del Q5, K5, V5, O5

    # decoding step: bytes = the visible K and V rows + Q + O
    w = synth.WORKLOADS[6]
    ins, lens = synth.workload_inputs(6)
    Qd, Kd, Vd = (dev_t(ins[k][0]) for k in "QKV")
    Od = torch.empty_like(Qd)
    lens_d = torch.from_numpy(lens).to(dev)

    def call6():
        libmha.sdpa(Qd, Kd, Vd, scale=0.125, mask="none", seq_lens=lens_d, out=Od, stream=stream)
    for _ in range(20):
        call6()
    med, mn = time_calls(call6, stream, iters)
    cmed, _ = time_calls(call6, stream, max(iters // 4, 10), flush)
    nbytes = w["h"] * int(lens.sum()) * w["d"] * 2 * 2 + 2 * w["B"] * w["h"] * w["n_q"] * w["d"] * 2
    res[w["name"]] = {"call": "mha_sdpa (one-row decoding kernel)", "us_median": round(med, 2), "us_min": round(mn, 2),
                      "us_median_cold": round(cmed, 2),
                      "gbs": round(nbytes / (med * 1e-6) / 1e9, 1),
                      "gbs_cold": round(nbytes / (cmed * 1e-6) / 1e9, 1),
                      "hbm_frac_cold": round(nbytes / (cmed * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                      "bytes": nbytes}
    del scratch
    return res


# Table 3 row (A) of the nickwang.xyz page: d_model fixed at 512, h and
# d_k = d_v = d_model / h varied from 32 heads of 16 to one head of 512 (the
# FLOPs stay the same); plus d_k 128 at d_model 1024 (row (C)).
HEAD_DIM_VARIANTS = ((8, 64), (32, 16), (16, 32), (4, 128), (2, 256), (1, 512), (8, 128))


def head_dim_sweep(dev, stream, B=4, n=4096, settle_s=1.0):
    """mha_sdpa TFLOP/s for each head-dimension variant at [B, h, n, d],
    both masks, scale 1/sqrt(d), timed in batches of back-to-back calls (as
    the bench line's per-mode figures).  Rates use algorithmic flops."""
    import numpy as np
    import torch
    from transformer_head_scaled_amd import libmha, synth

    res = {}
    for vi, (h, d) in enumerate(HEAD_DIM_VARIANTS):
        ins = synth.sdpa_inputs(5, B, h, n, n, d, dtype="bf16")
        Q, K, V = (torch.from_numpy(ins[k][0].view(np.int16)).to(dev).view(torch.bfloat16)
                   for k in "QKV")
        O = torch.empty_like(Q)
        entry = {"B": B, "h": h, "n": n, "d": d}
        t0 = time.perf_counter()
        # both masks, as the timed calls run them; the first variant longer: a
        # fresh process's calls take several seconds to reach their steady time
        while time.perf_counter() - t0 < (settle_s if vi else 5 * settle_s):
            for i in range(20):
                libmha.sdpa(Q, K, V, scale=d ** -0.5, mask="causal" if i % 2 else "none", out=O,
                            stream=stream)
            torch.cuda.synchronize()
        for mk in ("none", "causal"):
            def call():
                libmha.sdpa(Q, K, V, scale=d ** -0.5, mask=mk, out=O, stream=stream)
            for _ in range(5):
                call()
            med, mn = time_batches(call, stream)
            fl = sdpa_flops(B, h, n, n, d, mk == "causal")
            entry[mk] = {"us_median": round(med, 2), "us_min": round(mn, 2),
                         "tflops": round(fl / (med * 1e-6) / 1e12, 1),
                         "pct_peak": round(100 * fl / (med * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 2)}
        res[f"h{h}_d{d}"] = entry
        del Q, K, V, O
    return res


def profile_workloads(dev, names, steps):
    """Run each named workload ``steps`` times, warm, back to back (for the
    rocprofv3 counter passes, whose per-dispatch readings then belong to one
    workload each).  Names: nc, c (the long-sequence batch unmasked and
    causal), cfg1, cfg2, cfg3, cfg4."""
    import numpy as np
    import torch
    from transformer_head_scaled_amd import libmha, synth

    def dev_t(st):
        return torch.from_numpy(np.ascontiguousarray(st).view(np.int16)).to(dev).view(torch.bfloat16)
    stream = torch.cuda.current_stream()
    done = []
    for name in names:
        if name in ("nc", "c", "cfg3", "cfg1"):
            cfg = {"nc": 5, "c": 5, "cfg3": 3, "cfg1": 1}[name]
            w = synth.WORKLOADS[cfg]
            ins = synth.sdpa_inputs(cfg, w["B"], w["h"], w["n_q"], w["n_k"], w["d"], dtype=w["dtype"])
            if w["dtype"] == "f32":
                Q, K, V = (torch.from_numpy(ins[k][0]).to(dev) for k in "QKV")
            else:
                Q, K, V = (dev_t(ins[k][0]) for k in "QKV")
            O = torch.empty_like(Q)
            mask = "none" if name in ("nc", "cfg1") else "causal"

            def call():
                libmha.sdpa(Q, K, V, scale=0.125, mask=mask, out=O, stream=stream)
        elif name in ("cfg2", "cfg4"):
            cfg = int(name[3])
            w = synth.WORKLOADS[cfg]
            ins, lens = synth.workload_inputs(cfg)
            t = {k: dev_t(v[0]) for k, v in ins.items()}
            lens_d = None if lens is None else torch.from_numpy(lens).to(dev)
            B, n_q, n_k, dm, h = w["B"], w["n_q"], w["n_k"], w["d_model"], w["h"]
            ws = torch.empty(libmha.workspace_size(B, n_q, n_k, dm, h, 1), dtype=torch.uint8, device=dev)
            out = torch.empty((B, n_q, dm), dtype=torch.bfloat16, device=dev)

            def call():
                libmha.forward(t["x_q"], t["Wq"], t["Wk"], t["Wv"], t["Wo"], h, x_kv=t.get("x_kv"),
                               kv_lens=lens_d, out=out, workspace=ws, stream=stream)
        else:
            raise SystemExit(f"unknown workload {name}")
        for _ in range(3 + steps):
            call()
        torch.cuda.synchronize()
        done.append(name)
    print(json.dumps({"profiled": done, "calls_each": 3 + steps}), flush=True)
    return 0


def cpu_baseline(ins, budget_s=12.0):
    """The fp64 oracle, untuned, on a bounded sample of the same workload:
    whole (batch, head) pairs, alternating unmasked and causal, until the
    time budget is used.  Returns the bench's cpu_baseline object."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - threadpoolctl missing
        blas = 1
    host_cores = len(os.sched_getaffinity(0))
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    Q, K, V = (ins[n][1].astype(np.float64) for n in "QKV")
    B, h, n, d = Q.shape
    done, flops, t_total = [], 0.0, 0.0
    k = 0
    while t_total < budget_s and k < 2 * B * h:
        b, i = (k // 2) // h % B, (k // 2) % h
        causal = k % 2 == 1
        t0 = time.perf_counter()
        oracle.attention_head(Q[b, i], K[b, i], V[b, i], 0.125,
                              oracle.MASK_CAUSAL if causal else oracle.MASK_NONE)
        t_total += time.perf_counter() - t0
        flops += sdpa_flops(1, 1, n, n, d, causal)
        done.append(f"({b},{i},{'causal' if causal else 'none'})")
        k += 1
    # cores: the threads the oracle actually ran on -- numpy's BLAS threads
    # (the matrix products), at most the host cores this process may use
    return {"value": flops / t_total / 1e12, "unit": "TFLOP/s", "cores": min(blas, host_cores),
            "kind": "oracle", "blas_threads": blas, "host_cores_available": host_cores,
            "cpu_model": cpu_model,
            "sample": f"{len(done)} whole heads of [4,8,4096,64] (alternating unmasked/causal, "
                      f"first {done[0]} .. last {done[-1]}), {t_total:.1f} s fp64 numpy"}


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--settle-seconds", type=float, default=2.0,
                    help="untimed steps before the warmup until this much time has passed, so that "
                         "the GPU clocks have ramped up when timing starts")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="skip the timings of the smaller workloads (reported under other_configs)")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--head-dims", action="store_true",
                    help="only time the head-dimension variants (d_k 16/32/64/128) of mha_sdpa")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 512 MiB device copy (for scaling HBM counters)")
    ap.add_argument("--profile-workload", default=None,
                    help="only run these workloads --steps times each, warm (comma-separated: nc, c, "
                         "cfg1, cfg2, cfg3, cfg4), for the counter passes")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: libmha runs on one GPU only (no multi-GPU path is built); "
              "run with --gpus 1", file=sys.stderr)
        return 2

    import numpy as np
    import torch
    from transformer_head_scaled_amd import libmha, synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": COPY_BYTES, "launches": 3}), flush=True)
        return 0
    if args.profile_workload:
        return profile_workloads(dev, args.profile_workload.split(","), args.steps)
    if args.head_dims:
        out = {"head_dim_variants": head_dim_sweep(dev, torch.cuda.current_stream()),
               "dtype": "bf16", "data": "synthetic", "unit": "TFLOP/s"}
        print(json.dumps(out), flush=True)
        return 0
    w = WORKLOAD
    B, h, n, d = w["B"], w["h"], w["n"], w["d"]
    ins = synth.sdpa_inputs(5, B, h, n, n, d, dtype="bf16")

    def dev_t(st):
        return torch.from_numpy(st.view(np.int16)).to(dev).view(torch.bfloat16)

    Q, K, V = (dev_t(ins[k][0]) for k in "QKV")
    O_nc = torch.empty_like(Q)
    O_c = torch.empty_like(Q)
    stream = torch.cuda.current_stream()

    def step():
        libmha.sdpa(Q, K, V, scale=0.125, mask="none", out=O_nc, stream=stream)
        libmha.sdpa(Q, K, V, scale=0.125, mask="causal", out=O_c, stream=stream)

    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < args.settle_seconds:
        for _ in range(20):
            step()
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: exactly K steps, synchronised on both sides
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # average launch duration of each mode's kernel: K launches back to back
    # on the launch stream between one pair of HIP events (events around
    # every launch would add their own ~2 µs to each)
    def mode_ms(mask, out):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            libmha.sdpa(Q, K, V, scale=0.125, mask=mask, out=out, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps
    nc_ms = mode_ms("none", O_nc)
    c_ms = mode_ms("causal", O_c)

    f_nc = sdpa_flops(B, h, n, n, d, False)
    f_c = sdpa_flops(B, h, n, n, d, True)
    ms_per_step = wall * 1e3 / args.steps
    value = (f_nc + f_c) / (ms_per_step * 1e-3) / 1e12

    # spot parity of what was timed (one head per mode) against the oracle
    import oracle
    errs = {}
    for name, out, mk in (("none", O_nc, oracle.MASK_NONE), ("causal", O_c, oracle.MASK_CAUSAL)):
        b, i = 1, 5
        got = out[b, i].float().cpu().numpy()
        exp, _ = oracle.attention_head(ins["Q"][1][b, i], ins["K"][1][b, i], ins["V"][1][b, i],
                                       0.125, mk)
        errs[name] = float(np.abs(got - exp).max())

    ach_nc = f_nc / (nc_ms * 1e-3) / 1e12
    ach_c = f_c / (c_ms * 1e-3) / 1e12
    res = {
        "metric": "SDPA fwd TFLOP/s + % bf16 MFMA peak (h=8,d_k=64; causal & non-causal)",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_seconds": args.settle_seconds,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "sdpa_fwd_bf16_b4_h8_n4096_d64_causal+noncausal", "B": B, "h": h,
                   "n_q": n, "n_k": n, "d_k": d, "d_v": d, "global_batch": B, "seq_len": n,
                   "parallelism": "none (1 GPU)"},
        "pct_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "modes": {
            "noncausal": {"tflops": round(ach_nc, 2), "pct_peak": round(100 * ach_nc / PEAK_BF16_TFLOPS, 2),
                          "kernel_ms": round(nc_ms, 5), "flops": f_nc, "max_abs_err_sampled": errs["none"]},
            "causal": {"tflops": round(ach_c, 2), "pct_peak": round(100 * ach_c / PEAK_BF16_TFLOPS, 2),
                       "kernel_ms": round(c_ms, 5), "flops": f_c, "max_abs_err_sampled": errs["causal"]},
        },
        "roofline": {"bound": "mfma", "achieved": round(ach_nc, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(ach_nc / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(),
                     "kernel": "sdpa_fwd_kernel<bf16, d 64, non-causal, 8 waves>"},
        "roofline_causal": {"bound": "mfma", "achieved": round(ach_c, 2), "peak": PEAK_BF16_TFLOPS,
                            "unit": "TFLOP/s", "frac": round(ach_c / PEAK_BF16_TFLOPS, 4),
                            "kernel": "sdpa_fwd_kernel<bf16, d 64, causal pair layout, 8 waves>"},
    }
    if not args.no_other_configs:
        res["other_configs"] = other_configs(dev, stream)
    if not args.no_cpu_baseline:
        cb = cpu_baseline(ins, args.cpu_budget)
        cb["gpu_over_cpu"] = round(value / cb["value"], 1)   # information only
        res["cpu_baseline"] = cb
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
