"""The rocprofv3 summary tool on hand-made counter files (CPU only): the
derived figures it writes under profiles/ follow from the raw counters by
the formulas it states."""

import csv
import json
import os

from transformer_head_scaled_amd import profsum

FIELDS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id",
          "Grid_Size", "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size",
          "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "Counter_Name",
          "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def write_run(dirpath, dispatches):
    """dispatches: list of (kernel name, start ns, end ns, {counter: value})."""
    os.makedirs(dirpath, exist_ok=True)
    with open(os.path.join(dirpath, "p_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for i, (name, t0, t1, counters) in enumerate(dispatches):
            for cname, value in counters.items():
                w.writerow({"Correlation_Id": i + 1, "Dispatch_Id": i + 1, "Agent_Id": "Agent 1",
                            "Queue_Id": 1, "Process_Id": 1, "Thread_Id": 1, "Grid_Size": 1,
                            "Kernel_Id": 1, "Kernel_Name": name, "Workgroup_Size": 256,
                            "LDS_Block_Size": 0, "Scratch_Size": 0, "VGPR_Count": 0,
                            "Accum_VGPR_Count": 0, "SGPR_Count": 0, "Counter_Name": cname,
                            "Counter_Value": value, "Start_Timestamp": t0, "End_Timestamp": t1})


def table_rows(md_path):
    rows = []
    for line in open(md_path, encoding="utf-8"):
        if line.startswith("| `"):
            rows.append([c.strip() for c in line.strip().strip("|").split("|")])
    return rows


def test_counters_derived_figures(tmp_path):
    # a 100 µs dispatch at 2 GHz: 200000 busy cycles per XCD, reported summed over 8
    g = 200_000.0
    k = "void mha::(anonymous namespace)::sdpa_fwd_kernel<1, 64, false, 8, false, false, false>(mha::SdpaArgs)"
    counters = {
        "GRBM_GUI_ACTIVE": 8 * g,
        "SQ_VALU_MFMA_BUSY_CYCLES": 0.25 * g * 1024,  # a quarter of every SIMD's cycles
        "SQ_INSTS_VALU": 900.0, "SQ_INSTS_MFMA": 100.0,
        "SQ_INSTS_LDS": 50.0, "SQ_LDS_BANK_CONFLICT": 5.0,
        "SQ_WAVE_CYCLES": 6.0 * g * 256 / 4,  # six resident waves per CU on average
        "SQ_BUSY_CYCLES": g,
    }
    other = dict(counters, SQ_INSTS_MFMA=0.0)
    write_run(str(tmp_path / "run"), [
        (k, 0, 100_000, counters),
        (k, 200_000, 300_000, counters),
        ("void mha::(anonymous namespace)::sdpa_decode_kernel<1, 64>(mha::SdpaArgs)", 0, 50_000, other),
        ("void at::native::reduce_kernel<512>(x)", 0, 900_000, counters),  # not the library's
    ])
    out = tmp_path / "c.md"
    profsum.counters_md(str(tmp_path / "run"), str(out), "the command")
    rows = table_rows(out)
    assert [r[0] for r in rows] == [f"`{k}`", "`void mha::(anonymous namespace)::sdpa_decode_kernel<1, 64>(mha::SdpaArgs)`"]
    first = rows[0]
    assert first[1] == "2"                     # dispatches
    assert float(first[2]) == 100.0            # µs
    assert float(first[3]) == 2.0              # GHz
    assert float(first[4]) == 25.0             # MFMA busy %
    assert float(first[5]) == 9.0              # VALU per MFMA
    assert float(first[6]) == 0.1              # conflict cycles per LDS instruction
    assert float(first[7]) == 6.0              # waves per CU
    assert rows[1][5] == "n/a"                 # no MFMAs
    assert "the command" in out.read_text(encoding="utf-8")


def test_traffic_scales_by_the_copy(tmp_path):
    k = "void mha::(anonymous namespace)::sdpa_fwd_kernel<1, 64, false, 8, false, false, false>(mha::SdpaArgs)"
    kc = "void mha::(anonymous namespace)::sdpa_fwd_kernel<1, 64, true, 8, false, false, true>(mha::SdpaArgs)"
    copy = "__amd_rocclr_copyBuffer"
    cb = profsum.COPY_BYTES
    # the copy reads twice its bytes and writes them once by the counters
    write_run(str(tmp_path / "f"), [(k, 0, 1, {"FETCH_SIZE": 1000.0}), (kc, 0, 1, {"FETCH_SIZE": 3000.0})])
    write_run(str(tmp_path / "w"), [(k, 0, 1, {"WRITE_SIZE": 500.0}), (kc, 0, 1, {"WRITE_SIZE": 500.0})])
    write_run(str(tmp_path / "cf"), [(copy, 0, 1, {"FETCH_SIZE": 2.0 * cb / 1024.0})])
    write_run(str(tmp_path / "cw"), [(copy, 0, 1, {"WRITE_SIZE": cb / 1024.0})])
    # a second workload group, its own pair of runs
    k3 = "void mha::(anonymous namespace)::sdpa_fwd_kernel<1, 64, true, 4, false, false, true>(mha::SdpaArgs)"
    write_run(str(tmp_path / "f3"), [(k3, 0, 1, {"FETCH_SIZE": 64.0})])
    write_run(str(tmp_path / "w3"), [(k3, 0, 1, {"WRITE_SIZE": 32.0})])
    res = profsum.traffic(str(tmp_path / "cf"), str(tmp_path / "cw"), str(tmp_path / "t.json"), "cmds",
                          {"bench": (str(tmp_path / "f"), str(tmp_path / "w")),
                           "cfg3": (str(tmp_path / "f3"), str(tmp_path / "w3"))})
    assert res["fetch_factor"] == 0.5 and res["write_factor"] == 1.0
    assert res["runs"]["cfg3"][k3]["bytes_per_launch"] == 64.0 * 1024 * 0.5 + 32.0 * 1024
    assert k3 not in res["runs"]["bench"]
    assert res["noncausal_bytes_per_launch"] == 1000.0 * 1024 * 0.5 + 500.0 * 1024
    assert res["causal_bytes_per_launch"] == 3000.0 * 1024 * 0.5 + 500.0 * 1024
    assert res["kernel_source_sha256_16"] == profsum.kernel_hash()
    assert json.load(open(tmp_path / "t.json"))["commands"] == "cmds"
