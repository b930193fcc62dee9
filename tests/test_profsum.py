"""Host logic of the profile summaries (block_sparse_attention_candidates_amd/profsum.py)
on small synthetic rocprofv3 outputs: the kernel table from a results database and
from a stats csv, the FETCH/WRITE scaling of the traffic record, the SQ summary and
the bench table. CPU only."""
import csv
import json
import os
import sqlite3

import pytest

from block_sparse_attention_candidates_amd import profsum as P

SPARSE = "void dr::(anonymous namespace)::attn_kernel<128, 32, true, 9>(dr::AttnParams)"
DENSE = "void dr::(anonymous namespace)::attn_kernel<128, 32, false, 9>(dr::AttnParams)"
COPY = "void at::native::vectorized_elementwise_kernel<4, at::native::MulFunctor<float>>(int)"
POOL = "void dr::(anonymous namespace)::pool_kernel<128>(dr::PoolParams)"


def test_stats_from_results_database(tmp_path):
    db = tmp_path / "run_results.db"
    con = sqlite3.connect(db)
    con.execute("CREATE TABLE kernels (name TEXT, duration INTEGER)")
    con.executemany("INSERT INTO kernels VALUES (?, ?)",
                    [(SPARSE, 10_000_000), (SPARSE, 12_000_000), (DENSE, 100_000_000), (POOL, 300_000)])
    con.commit()
    con.close()
    rows = P._stats_rows(str(db))
    assert [r[0] for r in rows] == [DENSE, SPARSE, POOL]          # by total time
    name, calls, avg, mn, mx, share = rows[1]
    assert (calls, avg, mn, mx) == (2, 11_000_000, 10_000_000, 12_000_000)
    assert share == pytest.approx(100.0 * 22_000_000 / 122_300_000)
    table = P.stats(str(db))
    assert "| `attn_kernel<128, 32, true, 9>` | 2 | 11000.0 | 10000.0 | 12000.0 |" in table


def test_stats_from_csv(tmp_path):
    f = tmp_path / "run_kernel_stats.csv"
    with open(f, "w", newline="") as fh:
        wr = csv.writer(fh)
        wr.writerow(["Name", "Calls", "AverageNs", "MinNs", "MaxNs", "Percentage"])
        wr.writerow([SPARSE, 3, 1500.0, 1000.0, 2000.0, 75.0])
    assert "| `attn_kernel<128, 32, true, 9>` | 3 | 1.5 | 1.0 | 2.0 | 75.0% |" in P.stats(str(f))


def _counter_csv(path, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as fh:
        wr = csv.writer(fh)
        wr.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for r in rows:
            wr.writerow(r)


def test_traffic_scaling(tmp_path, monkeypatch):
    """FETCH_SIZE (KiB, one row per dispatch) scaled by the 1 GiB copy's reading
    (half the bytes: scale 2), WRITE_SIZE by its own (all the bytes: scale 1),
    averaged over the sparse kernel's dispatches; the pooling kernel's fetch
    beside it."""
    fetch, write = tmp_path / "f", tmp_path / "w"
    _counter_csv(fetch, [(1, SPARSE, "FETCH_SIZE", 900.0), (2, SPARSE, "FETCH_SIZE", 1100.0),
                         (3, DENSE, "FETCH_SIZE", 7.0), (4, COPY, "FETCH_SIZE", 524288.0),
                         (5, POOL, "FETCH_SIZE", 50.0)])
    _counter_csv(write, [(1, SPARSE, "WRITE_SIZE", 20.0), (2, SPARSE, "WRITE_SIZE", 40.0),
                         (4, COPY, "WRITE_SIZE", 1048576.0)])
    monkeypatch.setattr(P, "ROOT", str(tmp_path))
    os.makedirs(tmp_path / "profiles")
    rec = P.traffic(str(fetch), str(write), "w", "static")
    assert rec["fetch_scale"] == 2.0 and rec["write_scale"] == 1.0
    assert rec["fetch_kib_per_launch"] == 1000.0 and rec["write_kib_per_launch"] == 30.0
    assert rec["hbm_bytes_per_launch"] == 1000.0 * 1024 * 2 + 30.0 * 1024
    assert rec["pool_fetch_bytes_per_launch"] == 50.0 * 1024 * 2
    saved = json.load(open(tmp_path / "profiles" / "sparse_attn_traffic.json"))
    assert saved["w/static"]["attention_src_sha256"] == P.attention_source_digest()


def test_attention_digest_follows_sources_and_flags(monkeypatch):
    """The traffic record is tied to the attention kernel as built: its digest
    changes with attention.hip's compiler flags and with the include path
    left out (so it is the same on every machine)."""
    from block_sparse_attention_candidates_amd import build
    d0 = P.attention_source_digest()
    monkeypatch.setitem(build.EXTRA, "attention.hip", build.EXTRA["attention.hip"][:1])
    assert P.attention_source_digest() != d0
    monkeypatch.undo()
    assert P.attention_source_digest() == d0
    monkeypatch.setattr(build, "COMMON", build.COMMON[:-1] + ["/elsewhere/include"])
    assert P.attention_source_digest() == d0


def test_sq_summary(tmp_path):
    """MFMA busy = MFMA busy cycles / SIMD-cycles; VALU busy = 4 x active VALU
    quad-cycles / SIMD-cycles; waits per wave-cycle; the last dispatch of the
    sparse kernel of each pass."""
    a, b = tmp_path / "a", tmp_path / "b"
    simd = 1000.0 / 128      # GRBM_GUI_ACTIVE x 128 SIMDs = 1000 SIMD-cycles
    _counter_csv(b, [(5, SPARSE, "SQ_INSTS_VALU_TRANS_F32", 100.0), (5, SPARSE, "SQ_WAIT_ANY", 40.0),
                     (5, SPARSE, "SQ_WAIT_INST_ANY", 10.0), (5, SPARSE, "SQ_LDS_BANK_CONFLICT", 1.0),
                     (5, SPARSE, "SQ_LDS_IDX_ACTIVE", 100.0)])
    _counter_csv(a, [(5, SPARSE, "GRBM_GUI_ACTIVE", simd), (5, SPARSE, "SQ_VALU_MFMA_BUSY_CYCLES", 250.0),
                     (5, SPARSE, "SQ_ACTIVE_INST_VALU", 100.0), (5, SPARSE, "SQ_VALU_MFMA_COEXEC_CYCLES", 50.0),
                     (5, SPARSE, "SQ_INSTS_VALU", 800.0), (5, SPARSE, "SQ_INSTS_MFMA", 100.0),
                     (5, SPARSE, "SQ_WAVE_CYCLES", 100.0)])
    row = [l for l in P.sq(str(a), str(b)).splitlines() if l.startswith("| sparse")][0]
    cells = [c.strip() for c in row.strip("|").split("|")]
    assert cells == ["sparse", "25.0%", "40.0%", "5.0%", "8.00", "1.00", "40.0%", "10.0%", "1.00%"]


def test_bench_table(tmp_path):
    line = {"config": {"workload": "w", "mode": "static"}, "sparsity": 0.9, "ms_per_step": 2.0, "value": 100.0,
            "stage_ms": {"score_select": 0.5, "sparse_attn": 1.0, "dense_attn": 20.0},
            "roofline": {"frac": 0.25}, "speedup_vs_dense": 10.0, "speedup_vs_dense_attention_only": 20.0,
            "cpu_baseline": {"value": 0.001, "cores": 8}}
    f = tmp_path / "b.jsonl"
    f.write_text("# a comment line\n" + json.dumps(line) + "\n")
    rows = [l for l in P.benchtable(str(f)).splitlines() if l.startswith("| w ")]
    assert rows == ["| w | static | 0.900 | 2.00 | 100 | 1.00 | 0.250 | 0.50 | 20.0 | 10.00 | 20.00 | 0.0010 (8) |"]
