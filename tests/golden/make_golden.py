"""Writes tests/golden/tiny_oracle_rows.json: oracle outputs for a few rows of the tiny workload
(E=8, K=256, N=128, top-2, M=16, weight seed 1, activation seed 101, routing seed 201).
Calls only oracle/ and the seeded input generators; it is a regression guard of the oracle, not a
pin against the pages (the pages print no output values)."""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import moe_forward  # noqa: E402
from synth import CONFIGS, ExpertStore, gen_hidden, gen_routing_softmax  # noqa: E402

ROWS = [0, 7, 15]
COLS = [0, 1, 127, 128, 255]


def main():
    d = CONFIGS["tiny"]
    x = gen_hidden(16, d.K, 101)
    ids, w = gen_routing_softmax(16, d.E, d.topk, 201)
    out = moe_forward(d, x, ids, w, ExpertStore(d, 1))
    rec = {"rows": ROWS, "cols": COLS, "ids": ids[ROWS].tolist(),
           "values": [[float(out[r, c]).hex() for c in COLS] for r in ROWS]}
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_oracle_rows.json"), "w") as f:
        json.dump(rec, f, indent=1)


if __name__ == "__main__":
    main()
