"""Summaries of rocprofv3 CSV output for the library's kernels.

    python -m block_sparse_attention_candidates_amd.profsum stats <kernel_stats.csv>
    python -m block_sparse_attention_candidates_amd.profsum traffic <fetch_dir> <write_dir> <workload> <mode>

`stats` prints a markdown table of a `--kernel-trace --stats` summary.
`traffic` reads two `--pmc FETCH_SIZE` / `--pmc WRITE_SIZE` runs of
`bench.py --calib-copy`, takes the per-dispatch average of the sparse
attention kernel, scales it by what the same counter reads for the 1 GiB
elementwise copy in the same run (1 GiB read, 1 GiB written), and records
the result in profiles/sparse_attn_traffic.json under "<workload>/<mode>",
together with the SHA-256 of the attention kernel's sources it was taken on.
"""
from __future__ import annotations

import csv
import glob
import hashlib
import json
import os
import sys
from collections import defaultdict

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
GIB = float(1 << 30)


def _short(name: str) -> str:
    for key in ("attn_kernel", "score_kernel", "select_kernel", "pool_kernel", "cand_count_kernel",
                "cand_fill_kernel", "scan_kernel"):
        if key in name:
            i = name.index(key)
            j = name.find("(", i)
            return name[i:j if j > 0 else None]
    return name[:70]


def stats(path: str) -> str:
    rows = list(csv.DictReader(open(path)))
    out = ["| kernel | calls | avg (us) | min (us) | max (us) | share |", "|---|---|---|---|---|---|"]
    for r in rows:
        out.append(f"| `{_short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                   f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.1f}% |")
    return "\n".join(out)


def _counter(run_dir: str, counter: str):
    f = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not f:
        raise SystemExit(f"no counter_collection.csv under {run_dir}")
    per = defaultdict(list)
    for r in csv.DictReader(open(f[0])):
        if r["Counter_Name"] == counter:
            per[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    attn = [v for k, vs in per.items() if "attn_kernel" in k and "true" in k.split("attn_kernel", 1)[1][:40]
            for v in vs]
    copy = [v for k, vs in per.items() if "MulFunctor" in k or "mul_kernel" in k.lower() for v in vs]
    if not attn or not copy:
        raise SystemExit(f"{counter}: attention or copy dispatch missing in {run_dir}")
    return sum(attn) / len(attn), max(copy)


# the sources the sparse-attention kernel is compiled from
ATTENTION_SOURCES = ("attention.hip", "groups.hip", "lds_dma.h", "dr_internal.h")


def attention_source_digest() -> str:
    """SHA-256 over the attention kernel's source files, in a fixed order."""
    h = hashlib.sha256()
    for name in ATTENTION_SOURCES:
        with open(os.path.join(PKG, "csrc", name), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def traffic(fetch_dir: str, write_dir: str, workload: str, mode: str) -> dict:
    fa, fc = _counter(fetch_dir, "FETCH_SIZE")
    wa, wc = _counter(write_dir, "WRITE_SIZE")
    f_scale, w_scale = GIB / (fc * 1024.0), GIB / (wc * 1024.0)
    rec = {
        "fetch_kib_per_launch": fa, "write_kib_per_launch": wa,
        "copy_fetch_kib": fc, "copy_write_kib": wc,
        "fetch_scale": f_scale, "write_scale": w_scale,
        "hbm_bytes_per_launch": fa * 1024.0 * f_scale + wa * 1024.0 * w_scale,
        "attention_src_sha256": attention_source_digest(),
    }
    path = os.path.join(ROOT, "profiles", "sparse_attn_traffic.json")
    db = json.load(open(path)) if os.path.exists(path) else {}
    db[f"{workload}/{mode}"] = rec
    with open(path, "w") as fh:
        json.dump(db, fh, indent=1, sort_keys=True)
    return rec


if __name__ == "__main__":
    if len(sys.argv) >= 3 and sys.argv[1] == "stats":
        print(stats(sys.argv[2]))
    elif len(sys.argv) == 6 and sys.argv[1] == "traffic":
        print(json.dumps(traffic(*sys.argv[2:6]), indent=1))
    else:
        print(__doc__)
        sys.exit(2)
