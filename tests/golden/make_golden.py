"""Writes oracle_c1.json: the oracle's answer on the seeded smoke workload.

Calls only the oracle and the seeded generators.  The stored answer guards
against silent drift of either (a numpy RNG change, an oracle edit); it is
not an independent pin -- the pins live in test_oracle.py.

Run from the repository root:  python tests/golden/make_golden.py
"""

import hashlib
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
from workloads import make_workload  # noqa: E402


def main():
    w = make_workload("C1")
    st, idx, val = oracle.topk(w.raw, w.dtype, w.n, w.k, w.sorted_index, True)
    assert st == 0
    doc = {
        "what": "top-64 of each row of the seeded bf16 smoke workload (4 x 8192 N(0,1), seed 1), "
                "indices ascending, values as bf16 bit patterns",
        "written_by": "tests/golden/make_golden.py (oracle + workloads only)",
        "input_sha256": hashlib.sha256(w.raw.tobytes()).hexdigest(),
        "batch": w.batch, "n": w.n, "k": w.k,
        "indices": idx.tolist(),
        "values_bits": val.astype("uint16").tolist(),
    }
    with open(os.path.join(HERE, "oracle_c1.json"), "w") as f:
        json.dump(doc, f, indent=0)
        f.write("\n")


if __name__ == "__main__":
    main()
