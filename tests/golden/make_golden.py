"""Writes tests/golden/c1_oracle.json from the CPU oracle (and nothing else).

Run from the repository root:  python tests/golden/make_golden.py
The fixture freezes the oracle's answer on the tiny integer-grid workload
(B=1 S=256 H=4 D=32 m=4 W=64 top_k=16, seed 1): every index, and the scores
of a few rows as exact hex floats.
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from synth import make_config  # noqa: E402

SCORE_ROWS = [3, 4, 63, 64, 100, 171, 254, 255]


def main():
    P = make_config("c1")
    s, idx = oracle.select(P)
    out = {
        "what": "CPU-oracle output on the tiny integer-grid workload; regression fixture",
        "written_by": "tests/golden/make_golden.py (calls only oracle/ and synth/)",
        "workload": "c1: B=1 S=256 H=4 D=32 m=4 W=64 top_k=16, integer grid, seed 1",
        "idx": idx.tolist(),
        "score_rows": SCORE_ROWS,
        "scores_hex": [[float(x).hex() for x in s[r]] for r in SCORE_ROWS],
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c1_oracle.json")
    with open(path, "w") as f:
        json.dump(out, f, separators=(",", ":"))
        f.write("\n")
    print("wrote", path)


if __name__ == "__main__":
    main()
