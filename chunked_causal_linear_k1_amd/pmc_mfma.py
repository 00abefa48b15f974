"""MFMA utilisation per prefill kernel launch from one rocprofv3 counter run.

Reads the counter_collection CSV of a run with
  --pmc MfmaUtil SQ_INSTS_VALU_MFMA_MOPS_BF16
(MfmaUtil is rocprofv3's derived metric: MFMA-busy cycles summed over the SIMDs, divided by
the GPU-active cycles times the SIMD count, in percent; SQ_INSTS_VALU_MFMA_MOPS_BF16 counts
bf16 MFMA multiply-add work in units of 512 flops) and the kernel-trace statistics CSV of a
separate timing run, and writes per kernel: the busy percentage, the bf16 MFMA flops one launch
executes, and those flops over the launch's average duration.

Usage:
  python -m chunked_causal_linear_k1_amd.pmc_mfma PMC_DIR KERNEL_STATS_CSV [OUT_JSON]
(OUT_JSON defaults to profiles/mfma.json)
"""
from __future__ import annotations

import csv
import glob
import json
import os
import sys
from collections import defaultdict

from .pmc_traffic import source_hash

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA

# kernel-name substring -> key
KERNELS = {
    "k_output_sh<64, 128, true, false, false, false>": "k_output_retnet_128k",
    "k_summary<64, 128, true, false, false, false>": "k_summary_retnet_128k",
    "k_output_w8<64, 128, false, true, true, false>": "k_output_elu1_8k",
    "k_summary<64, 128, false, true, true, true>": "k_summary_elu1_8k",  # single-rounded (no final state)
    "k_output_prf<64, 128, 256, false, true, false, false>": "k_output_prf256_4k",
    "k_output_prf<64, 128, 256, false, true, false, true>": "k_output_prf256_4k_qshift",
    "k_summary_prf<64, 128, 256, false, true>": "k_summary_prf256_4k",
    "k_output_gla_m<128, false>": "k_output_gated_8k",
    "k_summary_gla_m<128>": "k_summary_gated_8k",
    "k_bwd_query<false, true, false, false>": "k_bwd_query_retnet_128k",
    "k_bwd_key<false, true, false, false>": "k_bwd_key_retnet_128k",
    "k_bwd_query<true, false, true, false>": "k_bwd_query_elu1_8k",
    "k_bwd_key<true, false, true, false>": "k_bwd_key_elu1_8k",
}


def read_counters(run_dir: str) -> dict:
    """kernel name -> counter name -> list of per-dispatch values."""
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {run_dir}")
    per = defaultdict(lambda: defaultdict(lambda: defaultdict(float)))
    for f in files:
        with open(f, newline="") as fh:
            for r in csv.DictReader(fh):
                per[r["Kernel_Name"]][r["Counter_Name"]][r["Dispatch_Id"]] += float(r["Counter_Value"])
    return {k: {c: list(d.values()) for c, d in v.items()} for k, v in per.items()}


def read_durations(stats_csv: str) -> dict:
    """kernel name -> average duration in ns (rocprofv3 --stats kernel_stats.csv)."""
    with open(stats_csv, newline="") as fh:
        return {r["Name"]: float(r["AverageNs"]) for r in csv.DictReader(fh)}


def pick(table: dict, sub: str):
    hits = [v for name, v in table.items() if sub in name]
    return hits[0] if hits else None


def main(pmc_dir: str, stats_csv: str, path: str = "") -> dict:
    counters = read_counters(pmc_dir)
    durations = read_durations(stats_csv)
    out = {"source_hash": source_hash(), "peak_bf16_tflops": PEAK_BF16_TFLOPS}
    for sub, key in KERNELS.items():
        c, ns = pick(counters, sub), pick(durations, sub)
        if c is None or "MfmaUtil" not in c or "SQ_INSTS_VALU_MFMA_MOPS_BF16" not in c:
            continue
        util = sum(c["MfmaUtil"]) / len(c["MfmaUtil"])
        flops = 512.0 * sum(c["SQ_INSTS_VALU_MFMA_MOPS_BF16"]) / len(c["SQ_INSTS_VALU_MFMA_MOPS_BF16"])
        row = {"mfma_busy_pct": round(util, 2), "mfma_bf16_flops": flops}
        if ns:
            row["avg_ns"] = ns
            row["mfma_tflops"] = round(flops / ns / 1e3, 2)
            row["frac_of_peak"] = round(flops / ns / 1e3 / PEAK_BF16_TFLOPS, 4)
        out[key] = row
    path = path or os.path.join(ROOT, "profiles", "mfma.json")
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as fh:
        json.dump(out, fh, indent=1)
    return out


if __name__ == "__main__":
    if len(sys.argv) not in (3, 4):
        print(__doc__)
        sys.exit(2)
    print(json.dumps(main(sys.argv[1], sys.argv[2], sys.argv[3] if len(sys.argv) == 4 else ""), indent=1))
