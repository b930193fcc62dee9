"""Summaries of rocprofv3 CSV output for the library's kernels.

    python -m block_sparse_attention_candidates_amd.profsum stats <kernel_stats.csv | results.db>
    python -m block_sparse_attention_candidates_amd.profsum traffic <fetch_dir> <write_dir> <workload> <mode>
    python -m block_sparse_attention_candidates_amd.profsum sq <pass_a_dir> <pass_b_dir>
    python -m block_sparse_attention_candidates_amd.profsum benchtable <bench.jsonl>

`stats` prints a markdown table of a `--kernel-trace --stats` summary (the
csv one, or the per-kernel totals of the rocpd database).
`traffic` reads two `--pmc FETCH_SIZE` / `--pmc WRITE_SIZE` runs of
`bench.py --calib-copy`, takes the per-dispatch average of the sparse
attention kernel, scales it by what the same counter reads for the 1 GiB
elementwise copy in the same run (1 GiB read, 1 GiB written), and records
the result in profiles/sparse_attn_traffic.json under "<workload>/<mode>",
together with the SHA-256 of the attention kernel's sources it was taken on;
the pooling kernel's scaled FETCH_SIZE per dispatch is recorded beside it.
`sq` prints the SQ counters of two `--pmc` passes (the counters of SQ_PASS_A
and SQ_PASS_B) for the sparse and the dense attention kernel, with the derived
MFMA and VALU occupancy. `benchtable` prints a markdown table of bench.py
JSON lines.
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


def _stats_rows(path: str):
    """(name, calls, avg ns, min ns, max ns, share %) per kernel, from a
    `--stats -f csv` kernel_stats.csv or from the dispatches of a rocpd
    results database (the default output format)."""
    if path.endswith(".db"):
        import sqlite3
        con = sqlite3.connect(path)
        rows = con.execute("SELECT name, COUNT(*), AVG(duration), MIN(duration), MAX(duration), SUM(duration) "
                           "FROM kernels GROUP BY name ORDER BY SUM(duration) DESC").fetchall()
        con.close()
        total = sum(r[5] for r in rows) or 1.0
        return [(r[0], r[1], r[2], r[3], r[4], 100.0 * r[5] / total) for r in rows]
    return [(r["Name"], int(r["Calls"]), float(r["AverageNs"]), float(r["MinNs"]), float(r["MaxNs"]),
             float(r["Percentage"])) for r in csv.DictReader(open(path))]


def stats(path: str) -> str:
    out = ["| kernel | calls | avg (us) | min (us) | max (us) | share |", "|---|---|---|---|---|---|"]
    for name, calls, avg, mn, mx, share in _stats_rows(path):
        out.append(f"| `{_short(name)}` | {calls} | {avg / 1e3:.1f} | {mn / 1e3:.1f} | {mx / 1e3:.1f} | {share:.1f}% |")
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
    """SHA-256 over the attention kernel's source files, in a fixed order, and
    the compiler flags its file is built with."""
    from block_sparse_attention_candidates_amd import build
    h = hashlib.sha256()
    for name in ATTENTION_SOURCES:
        with open(os.path.join(PKG, "csrc", name), "rb") as fh:
            h.update(fh.read())
    h.update(" ".join(build.COMMON[:-2] + build.EXTRA.get("attention.hip", [])).encode())
    return h.hexdigest()


def _kernel_mean(run_dir: str, counter: str, key: str) -> float:
    f = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    vals = defaultdict(float)
    for r in csv.DictReader(open(f[0])):
        if r["Counter_Name"] == counter and key in r["Kernel_Name"]:
            vals[r["Dispatch_Id"]] += float(r["Counter_Value"])
    if not vals:
        raise SystemExit(f"{counter}: no {key} dispatch in {run_dir}")
    return sum(vals.values()) / len(vals)


def traffic(fetch_dir: str, write_dir: str, workload: str, mode: str) -> dict:
    fa, fc = _counter(fetch_dir, "FETCH_SIZE")
    wa, wc = _counter(write_dir, "WRITE_SIZE")
    f_scale, w_scale = GIB / (fc * 1024.0), GIB / (wc * 1024.0)
    rec = {
        "fetch_kib_per_launch": fa, "write_kib_per_launch": wa,
        "copy_fetch_kib": fc, "copy_write_kib": wc,
        "fetch_scale": f_scale, "write_scale": w_scale,
        "hbm_bytes_per_launch": fa * 1024.0 * f_scale + wa * 1024.0 * w_scale,
        "pool_fetch_bytes_per_launch": _kernel_mean(fetch_dir, "FETCH_SIZE", "pool_kernel") * 1024.0 * f_scale,
        "attention_src_sha256": attention_source_digest(),
    }
    path = os.path.join(ROOT, "profiles", "sparse_attn_traffic.json")
    db = json.load(open(path)) if os.path.exists(path) else {}
    db[f"{workload}/{mode}"] = rec
    with open(path, "w") as fh:
        json.dump(db, fh, indent=1, sort_keys=True)
    return rec


SQ_PASS_A = ("SQ_WAVES SQ_BUSY_CYCLES SQ_WAVE_CYCLES SQ_VALU_MFMA_BUSY_CYCLES SQ_VALU_MFMA_COEXEC_CYCLES "
             "SQ_ACTIVE_INST_VALU SQ_INSTS_VALU SQ_INSTS_MFMA GRBM_GUI_ACTIVE")
SQ_PASS_B = ("SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_WAIT_INST_LDS SQ_ACTIVE_INST_LDS SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT "
             "SQ_LDS_IDX_ACTIVE SQ_INSTS_VALU_TRANS_F32")


def sq(dir_a: str, dir_b: str) -> str:
    """SQ counters (summed over the shader engines and XCDs) of the last
    dispatch of the sparse and of the dense attention kernel in two passes.
    SIMD-cycles = GRBM_GUI_ACTIVE (summed over the 8 XCDs) x 128 SIMDs per XCD;
    SQ_ACTIVE_INST_VALU counts quad-cycles."""
    def last(run_dir, sparse):
        f = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)[0]
        per = defaultdict(lambda: defaultdict(float))
        for r in csv.DictReader(open(f)):
            k = r["Kernel_Name"]
            if "attn_kernel" not in k:
                continue
            is_sparse = "true" in k.split("attn_kernel", 1)[1][:40]
            if is_sparse != sparse:
                continue
            per[int(r["Dispatch_Id"])][r["Counter_Name"]] += float(r["Counter_Value"])
        return per[max(per)] if per else None
    out = ["| kernel | MFMA busy | VALU busy | VALU during MFMA | VALU instr / MFMA | exp / MFMA | "
           "wait (any) / wave-cycles | wait for issue / wave-cycles | LDS bank conflicts / LDS active |",
           "|---|---|---|---|---|---|---|---|---|"]
    for sparse in (True, False):
        a, b = last(dir_a, sparse), last(dir_b, sparse)
        if not a or not b:
            continue
        c = dict(a)
        c.update(b)
        simd = c["GRBM_GUI_ACTIVE"] * 128.0
        out.append(f"| {'sparse' if sparse else 'dense'} | {c['SQ_VALU_MFMA_BUSY_CYCLES'] / simd:.1%} | "
                   f"{4 * c['SQ_ACTIVE_INST_VALU'] / simd:.1%} | {c['SQ_VALU_MFMA_COEXEC_CYCLES'] / simd:.1%} | "
                   f"{c['SQ_INSTS_VALU'] / c['SQ_INSTS_MFMA']:.2f} | {c['SQ_INSTS_VALU_TRANS_F32'] / c['SQ_INSTS_MFMA']:.2f} | "
                   f"{c['SQ_WAIT_ANY'] / c['SQ_WAVE_CYCLES']:.1%} | {c['SQ_WAIT_INST_ANY'] / c['SQ_WAVE_CYCLES']:.1%} | "
                   f"{c['SQ_LDS_BANK_CONFLICT'] / max(c['SQ_LDS_IDX_ACTIVE'], 1):.2%} |")
    return "\n".join(out)


def benchtable(path: str) -> str:
    out = ["| workload | mode | sparsity | ms / step | TFLOP/s (step) | sparse attn ms | roofline frac | "
           "select ms | dense ms | speedup (step) | speedup (attention) | oracle TFLOP/s (cores) |",
           "|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for line in open(path):
        line = line.strip()
        if not line.startswith("{"):
            continue
        r = json.loads(line)
        st = r["stage_ms"]
        sel = st.get("score_select", st.get("token_select", st.get("mask_build")))
        cpu = r.get("cpu_baseline")
        cpu_s = f"{cpu['value']:.4f} ({cpu['cores']})" if cpu else "n/a"
        out.append(f"| {r['config']['workload']} | {r['config']['mode']} | {r['sparsity']:.3f} | {r['ms_per_step']:.2f} | "
                   f"{r['value']:.0f} | {st['sparse_attn']:.2f} | {r['roofline']['frac']:.3f} | {sel:.2f} | "
                   f"{st['dense_attn']:.1f} | {r['speedup_vs_dense']:.2f} | {r['speedup_vs_dense_attention_only']:.2f} | "
                   f"{cpu_s} |")
    return "\n".join(out)


if __name__ == "__main__":
    if len(sys.argv) >= 3 and sys.argv[1] == "stats":
        print(stats(sys.argv[2]))
    elif len(sys.argv) == 6 and sys.argv[1] == "traffic":
        print(json.dumps(traffic(*sys.argv[2:6]), indent=1))
    elif len(sys.argv) == 4 and sys.argv[1] == "sq":
        print(sq(sys.argv[2], sys.argv[3]))
    elif len(sys.argv) == 3 and sys.argv[1] == "benchtable":
        print(benchtable(sys.argv[2]))
    else:
        print(__doc__)
        sys.exit(2)
