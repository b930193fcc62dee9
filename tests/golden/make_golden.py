"""Writes tests/golden/candidates.json from the CPU oracle only.

For each workload: the number of blocks, the candidate count, the row-length
range and SHA-256 digests of the oracle's candidate CSR (row_ptr and cols as
little-endian int32). GPU tests compare the library's CSR against these
digests at full size without re-running the (slow) oracle.

Run from the repository root:  python tests/golden/make_golden.py
"""
import hashlib
import json
import os
import sys
from concurrent.futures import ProcessPoolExecutor

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402
from oracle import dynrad_oracle as O  # noqa: E402


def digest(a):
    return hashlib.sha256(np.ascontiguousarray(a, dtype="<i4").tobytes()).hexdigest()


def one(name):
    w = workloads.get_workload(name)
    row_ptr, cols = O.candidate_csr(**w.radial_kwargs())
    lens = np.diff(row_ptr)
    return name, {
        "radial": w.radial_kwargs(),
        "num_blocks": int(w.num_blocks),
        "nnz": int(row_ptr[-1]),
        "row_len_min": int(lens.min()), "row_len_max": int(lens.max()),
        "row_ptr_sha256": digest(row_ptr), "cols_sha256": digest(cols),
    }


if __name__ == "__main__":
    names = list(workloads.WORKLOADS)
    with ProcessPoolExecutor(max_workers=len(names)) as ex:
        res = dict(ex.map(one, names))
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "candidates.json")
    with open(out, "w") as f:
        json.dump({"source": "oracle/dynrad_oracle.py candidate_csr (DynamicRad §3.1, Eqs. 1-7)",
                   "workloads": res}, f, indent=1, sort_keys=True)
    print("wrote", out)
