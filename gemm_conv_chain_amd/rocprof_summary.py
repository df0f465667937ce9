"""Summaries of rocprofv3 output for this library's kernels.

    python -m gemm_conv_chain_amd.rocprof_summary trace  DIR        # --kernel-trace --stats -f csv
    python -m gemm_conv_chain_amd.rocprof_summary pmc    DIR WORKLOAD [--json profiles/traffic.json]
    python -m gemm_conv_chain_amd.rocprof_summary mfma   DIR [WORKLOAD --json profiles/traffic.json]
        (DIR from --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_F16 GRBM_GUI_ACTIVE; run after pmc)
    python -m gemm_conv_chain_amd.rocprof_summary lds    DIR
        (DIR from --pmc SQ_LDS_IDX_ACTIVE SQ_LDS_BANK_CONFLICT SQ_LDS_ADDR_CONFLICT SQ_INSTS_LDS
         SQ_ACTIVE_INST_LDS GRBM_GUI_ACTIVE)

``trace``: the kernel_stats.csv rows (calls, average/min/max duration).
``mfma``: matrix-core activity per dispatch of this library's kernels.  On
MI355X one fp16 MFMA "MOP" is 512 FLOP (SQ_INSTS_VALU_MFMA_MOPS_F16 x 512 is
the executed FLOP count) and SQ_VALU_MFMA_BUSY_CYCLES is the sum over all
SIMDs of their busy clocks (it equals executed FLOP / 1024, the fp16 rate of
one SIMD per clock); GRBM_GUI_ACTIVE is summed over the 8 XCDs, so the
busy fraction of the 1024 SIMDs is BUSY / (GRBM_GUI_ACTIVE / 8 * 1024).
``pmc``: FETCH_SIZE / WRITE_SIZE per dispatch (KiB, mean over the dispatches of
each kernel) from two ``--pmc`` runs (DIR/fetch, DIR/write) of
``bench.py --calib-copy``; WORKLOAD is the bench workload, or WORKLOAD@VARIANT
for a run with ``--variant`` other than the workload's own.  Each counter is scaled by what it reads for the
256 MiB device-to-device copy that ``--calib-copy`` issues (known bytes; the largest copy dispatch):
scale = 262144 KiB / counter value of that dispatch.  With --json the scaled
HBM bytes of the fused kernel (and the sum over the unfused kernels) are
recorded for bench.py, keyed by the hash of the kernel sources they were taken
on (bench.py reports them only while that hash still matches).
"""
from __future__ import annotations

import csv
import glob
import json
import os
import sys


def _rows(path_glob):
    out = []
    for f in sorted(glob.glob(path_glob, recursive=True)):
        with open(f) as fh:
            out.extend(csv.DictReader(fh))
    return out


def trace(d):
    rows = _rows(os.path.join(d, "**", "*kernel_stats.csv"))
    print("| kernel | calls | avg (us) | min (us) | max (us) | % of time |")
    print("|---|---|---|---|---|---|")
    for r in rows:
        print("| `%s` | %s | %.3f | %.3f | %.3f | %.1f |" % (
            r["Name"][:90], r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
            float(r["MaxNs"]) / 1e3, float(r["Percentage"])))


def _ours(name):
    """This library's kernels: templates appear demangled (fc::...), plain
    functions keep their mangled name (_ZN2fc...)."""
    return "fc::" in name or name.startswith("_ZN2fc")


def _pmc(d, counter):
    rows = [r for r in _rows(os.path.join(d, "**", "*counter_collection.csv")) if r["Counter_Name"] == counter]
    copies = [r for r in rows if "copyBuffer" in r["Kernel_Name"]]
    if not copies:
        raise SystemExit("no calibration copy dispatch in %s" % d)
    # the 256 MiB calibration copy is by far the largest copy dispatch of the run
    calib = max(copies, key=lambda r: float(r["Counter_Value"]))
    scale = 262144.0 / float(calib["Counter_Value"])
    per = {}
    for r in rows:
        # padding is input preparation and the matrix-core probe is not part of any chain
        if _ours(r["Kernel_Name"]) and "k_pad_mid" not in r["Kernel_Name"] and "k_mfma_probe" not in r["Kernel_Name"]:
            per.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return scale, float(calib["Counter_Value"]), {k: sum(v) / len(v) for k, v in per.items()}


def mfma(d, workload=None, json_path=None):
    rows = _rows(os.path.join(d, "**", "*counter_collection.csv"))
    per = {}
    for r in rows:
        if "fc::" in r["Kernel_Name"]:
            per.setdefault(r["Kernel_Name"], {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    print("| kernel | executed GFLOP (MOPS x 512) | MFMA busy (SIMD-clk) | GRBM_GUI_ACTIVE / 8 (clk) | MFMA busy fraction |")
    print("|---|---|---|---|---|")
    for k in sorted(per):
        v = {c: sum(x) / len(x) for c, x in per[k].items()}
        mops, busy, act = (v.get(c, 0.0) for c in ("SQ_INSTS_VALU_MFMA_MOPS_F16", "SQ_VALU_MFMA_BUSY_CYCLES",
                                                  "GRBM_GUI_ACTIVE"))
        frac = busy / (act / 8 * 1024) if act else 0.0
        print("| `%s` | %.3f | %.0f | %.0f | %.3f |" % (k[:90], mops * 512 / 1e9, busy, act / 8, frac))
        if json_path and workload:
            with open(json_path) as f:
                db = json.load(f)
            e = db.get("workloads", {}).get(workload)
            if e and e.get("kernel") == k:
                e.update({"mfma_busy_frac": round(frac, 4), "mfma_executed_flops": int(mops * 512)})
                with open(json_path, "w") as f:
                    json.dump(db, f, indent=1, sort_keys=True)


def pmc(d, workload, json_path=None):
    fs, fcal, fetch = _pmc(os.path.join(d, "fetch"), "FETCH_SIZE")
    ws, wcal, write = _pmc(os.path.join(d, "write"), "WRITE_SIZE")
    print("calibration (256 MiB copy): FETCH_SIZE %.0f KiB -> scale %.4f; WRITE_SIZE %.0f KiB -> scale %.4f"
          % (fcal, fs, wcal, ws))
    print()
    print("| kernel | FETCH_SIZE (KiB) | WRITE_SIZE (KiB) | scaled HBM bytes (MB) |")
    print("|---|---|---|---|")
    tot = {}
    for k in sorted(fetch):
        b = fetch[k] * fs * 1024 + write.get(k, 0.0) * ws * 1024
        tot[k] = b
        print("| `%s` | %.1f | %.1f | %.2f |" % (k[:90], fetch[k], write.get(k, 0.0), b / 1e6))
    if json_path:
        sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
        import bench
        fused = {"b2b_gemm_tiny": "k_chain_rf", "b2b_gemm_rf": "k_chain_rf", "b2b_gemm_lds": "k_gemm_lds<4, true",
                 "b2b_gemm_lds@stream": "k_chain_stream", "gemm3_rf": "k_chain_rf",
                 "conv3x3_conv1x1": "k_conv2_pipe<1, 0>", "conv3x3_conv1x1@rf": "k_chain_rf",
                 "conv3x3_conv1x1x2": "k_conv2_pipe<1, 1>", "conv3x3_conv1x1x2@rf": "k_chain_rf",
                 # pooled convs: the register-weights kernel is the automatic choice at these shapes
                 "conv3x3_relu_maxpool": "k_conv_pool_wr", "conv3x3_bn_relu_maxpool": "k_conv_pool_wr",
                 "conv3x3_relu_avgpool": "k_conv_pool_wr",
                 "conv3x3_relu_maxpool@reg_weights": "k_conv_pool_wr",
                 "conv3x3_relu_maxpool@lds_weights": "k_conv_w<4, 1",
                 "conv3x3_bn_relu_maxpool@lds_weights": "k_conv_w<4, 1",
                 "conv3x3_relu_avgpool@lds_weights": "k_conv_w<4, 2",
                 "conv3x3_relu_maxpool@winograd": "k_conv_pool_wino"}[workload]
        fk = [k for k in fetch if fused in k]
        if len(fk) != 1:
            raise SystemExit("cannot identify the fused kernel among %s" % list(fetch))
        fk = fk[0]
        unf = sum(v for k, v in tot.items() if k != fk)
        db = {"workloads": {}}
        if os.path.exists(json_path):
            with open(json_path) as f:
                db = json.load(f)
        db.setdefault("workloads", {})[workload] = {
            "kernel": fk, "src_hash": bench.kernel_src_hash(), "fetch_kib": fetch[fk], "write_kib": write.get(fk, 0.0),
            "fetch_scale": fs, "write_scale": ws, "unfused_bytes": int(unf)}
        with open(json_path, "w") as f:
            json.dump(db, f, indent=1, sort_keys=True)


LDS_COUNTERS = ("SQ_LDS_IDX_ACTIVE", "SQ_LDS_BANK_CONFLICT", "SQ_LDS_ADDR_CONFLICT", "SQ_INSTS_LDS",
                "SQ_ACTIVE_INST_LDS", "GRBM_GUI_ACTIVE")


def lds(d):
    """LDS activity per dispatch of this library's kernels (DIR from --pmc of
    LDS_COUNTERS).  bank-conflict ratio = SQ_LDS_BANK_CONFLICT /
    (SQ_LDS_IDX_ACTIVE - SQ_LDS_BANK_CONFLICT): stalled cycles per useful LDS
    cycle; LDS busy = SQ_LDS_IDX_ACTIVE over the 256 CUs' active clocks
    (GRBM_GUI_ACTIVE is summed over the 8 XCDs)."""
    rows = _rows(os.path.join(d, "**", "*counter_collection.csv"))
    per = {}
    for r in rows:
        if _ours(r["Kernel_Name"]) and "k_mfma_probe" not in r["Kernel_Name"]:
            per.setdefault(r["Kernel_Name"], {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    print("| kernel | LDS instructions | LDS active (clk) | bank-conflict stall (clk) | address-conflict stall (clk) "
          "| conflicts / useful cycle | LDS busy fraction |")
    print("|---|---|---|---|---|---|---|")
    for k in sorted(per):
        v = {c: sum(x) / len(x) for c, x in per[k].items()}
        idx, bank, addr, insts, act = (v.get(c, 0.0) for c in ("SQ_LDS_IDX_ACTIVE", "SQ_LDS_BANK_CONFLICT",
                                                                "SQ_LDS_ADDR_CONFLICT", "SQ_INSTS_LDS",
                                                                "GRBM_GUI_ACTIVE"))
        ratio = bank / (idx - bank) if idx > bank else 0.0
        busy = idx / (act / 8 * 256) if act else 0.0
        print("| `%s` | %.0f | %.0f | %.0f | %.0f | %.4f | %.3f |" % (k[:90], insts, idx, bank, addr, ratio, busy))


if __name__ == "__main__":
    if sys.argv[1] == "trace":
        trace(sys.argv[2])
    elif sys.argv[1] == "lds":
        lds(sys.argv[2])
    elif sys.argv[1] == "mfma":
        jp = sys.argv[sys.argv.index("--json") + 1] if "--json" in sys.argv else None
        mfma(sys.argv[2], sys.argv[3] if len(sys.argv) > 3 and sys.argv[3] != "--json" else None, jp)
    else:
        jp = sys.argv[sys.argv.index("--json") + 1] if "--json" in sys.argv else None
        pmc(sys.argv[2], sys.argv[3], jp)
