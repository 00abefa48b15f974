"""HBM traffic per kernel launch from two rocprofv3 counter runs.

Reads the counter_collection CSV of a FETCH_SIZE run and of a WRITE_SIZE run (both in KiB
per dispatch), scales each counter by what it reads for a plain copy kernel of known
size in the same run (the --copy-probe of bench.py: the negation of an fp32 vector into
another, reading and writing MIB MiB each, then MIB/4 MiB; the two sizes must agree on the
scale within 1%), and writes bytes per launch for the prefill
and decode kernels to profiles/traffic.json, stamped with a hash of the kernel sources
so that bench.py can tell when the figures no longer describe the current kernels.

Usage:
  python -m chunked_causal_linear_k1_amd.pmc_traffic FETCH_DIR WRITE_DIR COPY_MIB [OUT_JSON]
(OUT_JSON defaults to profiles/traffic.json)
"""
from __future__ import annotations

import csv
import glob
import hashlib
import json
import os
import sys
from collections import defaultdict

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)

# kernel-name substring -> key in traffic.json
KERNELS = {
    "k_output_sh<64, 128, true, false, false, false>": "k_output_retnet_128k",
    "k_summary<64, 128, true, false, false, false>": "k_summary_retnet_128k",  # 128k summaries fold 64-token steps
    "k_segment_scan": "k_segment_scan",
    "k_decode": "k_decode_32x64",
}
COPY_KERNEL = "neg"  # the --copy-probe kernel of bench.py (torch.neg of an fp32 vector)


def source_hash() -> str:
    """Hash of every kernel and dispatch source (csrc/), in name order."""
    h = hashlib.sha1()
    src = os.path.join(HERE, "csrc")
    for f in sorted(os.listdir(src)):
        if f.endswith((".hip", ".hpp", ".cpp", ".h")):
            h.update(f.encode())
            with open(os.path.join(src, f), "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()[:16]


def read_counter(run_dir: str, counter: str) -> dict:
    """kernel name -> list of per-dispatch counter values (KiB)."""
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {run_dir}")
    per = defaultdict(lambda: defaultdict(float))
    for f in files:
        with open(f, newline="") as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] != counter:
                    continue
                per[r["Kernel_Name"]][r["Dispatch_Id"]] += float(r["Counter_Value"])
    return {k: [v[d] for d in sorted(v, key=int)] for k, v in per.items()}  # in dispatch order


def pick(per: dict, sub: str):
    vals = [x for name, xs in per.items() if sub in name for x in xs]
    return sum(vals) / len(vals) if vals else None


def main(fetch_dir: str, write_dir: str, copy_mib: int, path: str = "") -> dict:
    fetch = read_counter(fetch_dir, "FETCH_SIZE")
    write = read_counter(write_dir, "WRITE_SIZE")
    # the probe runs the copy twice, copy_mib MiB and then a quarter of it: both sizes must give
    # the same scale for the counters to be read as bytes
    fl = [x for name, xs in fetch.items() if COPY_KERNEL in name for x in xs]
    wl = [x for name, xs in write.items() if COPY_KERNEL in name for x in xs]
    if len(fl) < 2 or len(wl) < 2:
        raise RuntimeError("the two copy probe dispatches were not found in the counter runs")
    sizes_kib = (copy_mib * 1024.0, copy_mib * 256.0)
    fsc = [sizes_kib[i] / fl[i] for i in range(2)]
    wsc = [sizes_kib[i] / wl[i] for i in range(2)]
    for a, b in (fsc, wsc):
        if abs(a - b) > 0.01 * a:
            raise RuntimeError(f"copy probe scales disagree between sizes: {a:.4f} vs {b:.4f}")
    fs, ws = fsc[0], wsc[0]
    out = {"source_hash": source_hash(),
           "calibration": {"copy_MiB": [copy_mib, copy_mib // 4], "fetch_KiB_read": fl[:2], "write_KiB_read": wl[:2],
                           "fetch_scale": fs, "write_scale": ws, "fetch_scale_small": fsc[1],
                           "write_scale_small": wsc[1]}}
    for sub, key in KERNELS.items():
        f, w = pick(fetch, sub), pick(write, sub)
        if f is None or w is None:
            continue
        out[key] = {"bytes": round((f * fs + w * ws) * 1024.0), "fetch_bytes": round(f * fs * 1024.0),
                    "write_bytes": round(w * ws * 1024.0)}
    path = path or os.path.join(ROOT, "profiles", "traffic.json")
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as fh:
        json.dump(out, fh, indent=1)
    return out


if __name__ == "__main__":
    if len(sys.argv) not in (4, 5):
        print(__doc__)
        sys.exit(2)
    print(json.dumps(main(sys.argv[1], sys.argv[2], int(sys.argv[3]), sys.argv[4] if len(sys.argv) == 5 else ""),
                     indent=1))
