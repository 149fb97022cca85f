"""Summarise rocprofv3 CSV output into the short text/JSON kept under profiles/.

    python -m transformer_head_scaled_amd.profsum stats  <kernel_stats.csv> <out.md> "<command>"
    python -m transformer_head_scaled_amd.profsum traffic <copy_fetch_dir> <copy_write_dir> \
        <out.json> "<commands>" bench=<fetch_dir>,<write_dir> [label=<fetch_dir>,<write_dir> ...]

    python -m transformer_head_scaled_amd.profsum counters <pmc_dir> <out.md> "<command>"
    python -m transformer_head_scaled_amd.profsum traffic_md <traffic.json> <kernel_stats.csv> <out.md>

``stats`` turns a ``--kernel-trace --stats`` kernel_stats.csv into a markdown
table.  ``counters`` turns one ``--pmc`` run of the SQ/GRBM counters below
into per-kernel utilisation figures.  ``traffic`` reads pairs of ``--pmc``
runs (FETCH_SIZE, then WRITE_SIZE), one pair for a plain device copy of
known size and one per workload group (the bench's two attention launches;
the smaller workloads), scales each counter by known-bytes /
counter-reading of the copy, and records the HBM bytes per launch of every
libmha kernel together with a hash of the attention kernel's source the
counters were taken on (the bench only reports the figure while the source
is unchanged).
"""

import csv
import collections
import hashlib
import json
import os
import re
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KERNEL_SRCS = [os.path.join(ROOT, "transformer_head_scaled_amd", "csrc", f)
               for f in ("sdpa_fwd_kernel.h", "sdpa_fwd.hip", "device_common.h")] + [
    os.path.join(ROOT, "transformer_head_scaled_amd", "build.py")]  # (its compiler flags)
COPY_BYTES = 512 << 20


def kernel_hash():
    """Hash of the attention kernel's sources (the same as bench.py's)."""
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_stats(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def stats_md(csv_path, out_md, command):
    rows = read_stats(csv_path)
    lines = ["# rocprofv3 kernel statistics", "", "Command:", "", "```", command, "```", "",
             "| kernel | calls | average µs | min µs | max µs | share % |",
             "|---|---|---|---|---|---|"]
    for r in rows:
        lines.append("| `{}` | {} | {:.2f} | {:.2f} | {:.2f} | {:.2f} |".format(
            r["Name"], r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
            float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")


def counter_means(run_dir, counter):
    path = None
    for dp, _, files in os.walk(run_dir):
        for fn in files:
            if fn.endswith("counter_collection.csv"):
                path = os.path.join(dp, fn)
    if path is None:
        raise FileNotFoundError(f"no counter_collection.csv under {run_dir}")
    agg = collections.defaultdict(list)
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter:
                agg[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in agg.items()}


SIMDS = 256 * 4  # MI355X: 256 compute units of 4 SIMDs
CUS = 256
XCDS = 8  # rocprofv3 reports GRBM_GUI_ACTIVE summed over the 8 XCDs
COUNTERS = ["SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE", "SQ_INSTS_VALU", "SQ_INSTS_MFMA",
            "SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT", "SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES"]


def counters_md(run_dir, out_md, command, top=10):
    """Per kernel (mean over its dispatches): the MFMA busy fraction
    (sum over SIMDs of SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE times
    the SIMD count, rocprofv3's MfmaUtil), the clock (GRBM_GUI_ACTIVE over
    the dispatch time), VALU instructions per MFMA instruction, LDS bank
    conflict cycles per LDS instruction and resident waves per CU, for the
    kernels with the longest dispatches
    (SQ_WAVE_CYCLES counts in units of 4 cycles).  GRBM_GUI_ACTIVE comes
    summed over the XCDs: one XCD's count is the device's busy cycles."""
    path = None
    for dp, _, files in os.walk(run_dir):
        for fn in files:
            if fn.endswith("counter_collection.csv"):
                path = os.path.join(dp, fn)
    if path is None:
        raise FileNotFoundError(f"no counter_collection.csv under {run_dir}")
    vals = collections.defaultdict(lambda: collections.defaultdict(list))
    durs = collections.defaultdict(dict)
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            k = r["Kernel_Name"]
            vals[k][r["Counter_Name"]].append(float(r["Counter_Value"]))
            durs[k][r["Dispatch_Id"]] = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
    rows = []
    for k, cs in vals.items():
        if "mha::" not in k:  # the library's kernels only
            continue
        m = {c: sum(v) / len(v) for c, v in cs.items()}
        ns = sum(durs[k].values()) / len(durs[k])
        g = m.get("GRBM_GUI_ACTIVE", 0.0) / XCDS
        if g <= 0:
            continue
        rows.append((ns, k, len(durs[k]), ns / 1e3, g / ns,
                     100.0 * m.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (g * SIMDS),
                     (m.get("SQ_INSTS_VALU", 0.0) / m["SQ_INSTS_MFMA"]) if m.get("SQ_INSTS_MFMA") else None,
                     m.get("SQ_LDS_BANK_CONFLICT", 0.0) / max(m.get("SQ_INSTS_LDS", 0.0), 1.0),
                     4.0 * m.get("SQ_WAVE_CYCLES", 0.0) / (g * CUS)))
    rows.sort(reverse=True)
    lines = ["# rocprofv3 counters per kernel", "", "Command:", "", "```", command, "```", "",
             "G = GRBM_GUI_ACTIVE / 8 (rocprofv3 sums it over the 8 XCDs): the device's busy "
             "cycles. MFMA busy % = 100 · Σ SQ_VALU_MFMA_BUSY_CYCLES / (G · 1024 SIMDs), "
             "rocprofv3's MfmaUtil; clock = G / dispatch time; waves/CU = 4 · SQ_WAVE_CYCLES / "
             "(G · 256); SQ_INSTS_VALU counts the MFMAs too. Dispatch times are under counter "
             "collection (kernels serialised): take durations from the kernel-trace summary; the "
             "clock column means something only for dispatches much longer than that overhead "
             "(the attention kernels of the first rows), and the shorter ones read above the "
             "2.4 GHz maximum.", "",
             "| kernel | dispatches | µs (under counters) | clock GHz | MFMA busy % | VALU insts / MFMA inst "
             "| LDS bank-conflict cycles / LDS inst | waves / CU |",
             "|---|---|---|---|---|---|---|---|"]
    for _, k, n, us, ghz, busy, vpm, conf, wpc in rows[:top]:
        vs = "n/a" if vpm is None else f"{vpm:.1f}"
        lines.append(f"| `{k}` | {n} | {us:.1f} | {ghz:.2f} | {busy:.1f} | {vs} | {conf:.3f} | {wpc:.1f} |")
    with open(out_md, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    return rows


def traffic(cfetch_dir, cwrite_dir, out_json, commands, runs):
    """runs: {label: (fetch_dir, write_dir)}, one pair of --pmc runs per
    workload group.  Every libmha kernel's FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch, mean over its dispatches in that run), scaled by the bytes per
    counter unit of a plain device copy of known size."""
    cf = counter_means(cfetch_dir, "FETCH_SIZE")
    cw = counter_means(cwrite_dir, "WRITE_SIZE")
    copy_name = max(cf, key=lambda k: cf[k])  # the 512 MiB copy dominates
    fetch_factor = COPY_BYTES / (cf[copy_name] * 1024.0)
    write_factor = COPY_BYTES / (cw[copy_name] * 1024.0)
    res = {"kernel_source_sha256_16": kernel_hash(), "copy_kernel": copy_name,
           "copy_bytes": COPY_BYTES, "fetch_size_kib_per_copy": cf[copy_name],
           "write_size_kib_per_copy": cw[copy_name], "fetch_factor": fetch_factor,
           "write_factor": write_factor, "runs": {}, "commands": commands}
    for label, (fetch_dir, write_dir) in runs.items():
        f = counter_means(fetch_dir, "FETCH_SIZE")
        w = counter_means(write_dir, "WRITE_SIZE")
        ks = {}
        for name in f:
            if "mha::" not in name:
                continue
            fb = f[name] * 1024.0 * fetch_factor
            wb = w.get(name, 0.0) * 1024.0 * write_factor
            ks[name] = {"fetch_kib": f[name], "write_kib": w.get(name), "fetch_bytes": fb,
                        "write_bytes": wb, "bytes_per_launch": fb + wb}
        res["runs"][label] = ks
    # the bench workload's kernels (template arguments: dtype, d, causal,
    # waves, key split, window, pair layout), for bench.py's roofline
    targs = re.compile(r"sdpa_fwd_kernel<(\d+), (\d+), (true|false), (\d+), (true|false), "
                       r"(true|false)(?:, (?:true|false))?>")
    for mode, causal in (("noncausal", "false"), ("causal", "true")):
        cands = []
        for k, v in res["runs"].get("bench", {}).items():
            m = targs.search(k)
            if m and m.group(2) == "64" and m.group(3) == causal and m.group(5) == "false" \
                    and m.group(6) == "false":
                cands.append(v["bytes_per_launch"])
        if cands:
            res[mode + "_bytes_per_launch"] = max(cands)
    with open(out_json, "w") as fh:
        json.dump(res, fh, indent=1)
        fh.write("\n")
    return res


# Algorithmic HBM bytes per launch of the kernels the counter runs cover:
# inputs read once plus outputs written once (bf16).  (run label, kernel
# name fragment, what it is, bytes)
ALGORITHMIC = [
    ("bench", "sdpa_fwd_kernel<1, 64, false, 8, false, false, false>", "[4,8,4096,64] unmasked", 67108864),
    ("bench", "sdpa_fwd_kernel<1, 64, true, 8, false, false, true>", "[4,8,4096,64] causal", 67108864),
    ("cfg3", "sdpa_fwd_kernel<1, 64, true, 4, false, false, true>", "[16,8,512,64] causal", 33554432),
    ("cfg2", "mha_short_kernel<1, true, 4>",
     "base encoder Q/K/V projections + attention, one launch (x 2 MB, W^Q/K/V 3·0.5 MB, concat 2 MB)",
     2097152 + 3 * 524288 + 2097152),
    ("cfg2", "gemm_kernel<1, 64, 64, 32, 32, 2, 128>", "base encoder W^O (concat 2 MB, W 0.5 MB, out 2 MB)",
     2 * 2097152 + 524288),
    ("cfg4", "sdpa_fwd_kernel<1, 64, false, 8, false, false, true>", "[8,16,384→512,64]",
     2 * (2 * 8 * 16 * 384 * 64 + 2 * 8 * 16 * 512 * 64)),
    ("cfg4", "gemm_kernel<1, 128, 128, 64, 64, 2, 32>",
     "big cross-attention Q/K/V projections (x_q, x_kv, 3 W, Q/K/V out)",
     2 * (3072 * 1024 + 4096 * 1024 + 3 * 1024 * 1024 + 3072 * 1024 + 2 * 4096 * 1024)),
    ("cfg4", "gemm_kernel<1, 64, 64, 32, 32, 2, 64>", "big cross-attention W^O (concat, W, out)",
     2 * (3072 * 1024 + 1024 * 1024 + 3072 * 1024)),
]


def traffic_md(traffic_json, kernel_stats_csv, out_md):
    """Counter bytes next to the algorithmic bytes, and both as GB/s over
    the kernels' mean duration in the kernel trace."""
    t = json.load(open(traffic_json))
    durs = {r["Name"]: (float(r["AverageNs"]), float(r["MinNs"])) for r in read_stats(kernel_stats_csv)}
    lines = ["# HBM traffic per launch: counters against algorithmic bytes", "",
             "Counter bytes = FETCH_SIZE and WRITE_SIZE (KiB per dispatch) scaled by what the same "
             "counters read for a 512 MiB device copy (fetch x{:.3f}, write x{:.3f}); each workload "
             "run alone, warm, so the reads include hits in the 256 MB last-level cache. Durations: "
             "mean (min) of the kernel-trace summary, whose runs include cold-cache calls of the small "
             "workloads. Commands: see sdpa_fwd_traffic.json and the kernel-statistics summary.".format(
                 t["fetch_factor"], t["write_factor"]), "",
             "| workload | kernel | counter MB | algorithmic MB | ratio | µs mean (min) | GB/s counters | GB/s algorithmic |",
             "|---|---|---|---|---|---|---|---|"]
    for label, frag, what, alg in ALGORITHMIC:
        for name, v in t["runs"].get(label, {}).items():
            if frag not in name:
                continue
            full = next((k for k in durs if frag in k), None)
            mean_ns, min_ns = durs.get(full, (float("nan"), float("nan")))
            b = v["bytes_per_launch"]
            lines.append("| {} | `{}` | {:.2f} | {:.2f} | {:.2f} | {:.2f} ({:.2f}) | {:.0f} | {:.0f} |".format(
                what, frag, b / 1e6, alg / 1e6, b / alg, mean_ns / 1e3, min_ns / 1e3, b / mean_ns,
                alg / mean_ns))
    with open(out_md, "w") as fh:
        fh.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    if sys.argv[1] == "stats":
        stats_md(sys.argv[2], sys.argv[3], sys.argv[4])
    elif sys.argv[1] == "traffic_md":
        traffic_md(sys.argv[2], sys.argv[3], sys.argv[4])
    elif sys.argv[1] == "counters":
        counters_md(sys.argv[2], sys.argv[3], sys.argv[4])
    elif sys.argv[1] == "traffic":
        # traffic <copy_fetch_dir> <copy_write_dir> <out.json> "<commands>" label=fetch_dir,write_dir ...
        runs = {}
        for spec in sys.argv[6:]:
            label, dirs = spec.split("=", 1)
            runs[label] = tuple(dirs.split(","))
        print(json.dumps(traffic(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5], runs), indent=1))
    else:
        raise SystemExit(__doc__)
