"""Writes workload_fixtures.json: pinned facts of the seeded synthetic inputs.

Calls only the ``workloads`` generators (no oracle value and nothing from the GPU path is
stored here).  Run from the repository root: python tests/golden/make_workload_fixtures.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402
import workloads as wl  # noqa: E402


def main():
    c1 = wl.config1()
    rng = np.random.default_rng(3)
    counts_rank = rng.multinomial(16384, wl.zipf_rank_weights(64, 1.1))
    rng = np.random.default_rng(3)
    w = rng.zipf(1.1, 64).astype(np.float64)
    counts_sampled = rng.multinomial(16384, w / w.sum())
    rng = np.random.default_rng(4)
    cu = rng.integers(256, 2049, 64)
    rng = np.random.default_rng(5)
    shapes = []
    for _ in range(1024):
        m = int(rng.integers(64, 1025))
        n = int(rng.choice((128, 256, 512)))
        k = int(rng.choice((128, 256, 512)))
        shapes.append([m, n, k])
    rng = np.random.default_rng(7)
    cu_attn = rng.integers(256, 2049, 64)
    wg = wl.wgrad(30, 5, 300, 16, 24, counts=np.array([100, 0, 7, 150, 43]))
    att = wl.attention(70, 3, 2, 128, 64, counts=np.array([5, 0, 9]))
    small = wl.dense(100, 33, 40, 24, dist="normal", b_layout=wl.B_NK, scale=0.5)
    fx = {
        "_about": "Seeded synthetic workloads standing in for the production cases of the pages "
                  "(How We Built TLX: 'TLX in Production' table, Case Studies 2 and 3). "
                  "Written by make_workload_fixtures.py from the workloads generators only.",
        "config1_digest": wl.digest(c1.A, c1.B),
        "dense_small_digest": wl.digest(small.A, small.B),
        "config3_counts_rank_zipf": [int(x) for x in counts_rank],
        "config3_counts_sampled_zipf": [int(x) for x in counts_sampled],
        "config4_candidates_per_user": [int(x) for x in cu],
        "config5_shapes": shapes,
        "attention_candidates_per_user": [int(x) for x in cu_attn],
        "wgrad_small_digest": wl.digest(wg.X, wg.dY),
        "attention_small_digest": wl.digest(att.Q, att.K, att.V),
    }
    with open(os.path.join(HERE, "workload_fixtures.json"), "w") as f:
        json.dump(fx, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
