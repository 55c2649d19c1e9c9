"""Writes the stored expected values under tests/golden/ from the CPU oracle only.

Run from the repository root:  python tests/golden/make_golden.py

Fixture c1_expected.json: the oracle's answer on the first benchmark workload
(batch 1, seq 16384, k 512, N(0,1) scores seeded 1000, page_size 64, identity
table) -- the selected positions (sorted), the threshold key and the counts
that make the answer unique.  The pages print no worked example with values,
so every stored value here comes from the oracle on seeded inputs.
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import workloads  # noqa: E402
from oracle import topk_transform  # noqa: E402


def c1_fixture():
    w = workloads.c1()
    out, raw, infos = topk_transform(w.scores, w.seq_lens, w.page_table, w.k, w.page_size)
    info = infos[0]
    return {
        "workload": w.name,
        "seed": w.seed,
        "k": w.k,
        "page_size": w.page_size,
        "n": info.n,
        "threshold_key": info.threshold,
        "n_greater": info.n_greater,
        "n_equal": info.n_equal,
        "selected_positions_sorted": sorted(int(x) for x in raw[0][: info.n]),
        "transformed_sorted": sorted(int(x) for x in out[0][: info.n]),
    }


if __name__ == "__main__":
    with open(os.path.join(HERE, "c1_expected.json"), "w") as f:
        json.dump(c1_fixture(), f)
        f.write("\n")
    print("wrote", os.path.join(HERE, "c1_expected.json"))
