"""Write sweep_alpha.json: the Zipf exponent that reaches each maxvio level.

For the sweep shape (R=8, E=64, S=4096, K=8) and seeds 0..2, bisect alpha in
[0, 3] (at most 40 halvings) until the maxvio of the drawn routing, counted by
the CPU oracle, is within 0.02 of the level.  Level 0 is not reachable by a
Zipf law on this shape and uses the balanced routing instead (no entry here).

Run from the repository root after building:  python tests/golden/make_sweep_alpha.py
"""
import json
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))

import oracle  # noqa: E402
import synth  # noqa: E402

LEVELS = (0.5, 1.0, 2.0, 4.0)
SEEDS = (0, 1, 2)
TOL = 0.02


def maxvio_at(w, seed, alpha):
    topk = synth.zipf_topk(seed, w.N, w.E, w.K, alpha)
    return oracle.route_stats(w.R, w.E, w.S, w.K, topk)[1]


def solve(w, seed, level):
    lo, hi = 0.0, 3.0
    best = None
    for it in range(40):
        mid = 0.5 * (lo + hi)
        mv = maxvio_at(w, seed, mid)
        if best is None or abs(mv - level) < abs(best[1] - level):
            best = (mid, mv, it + 1)
        if abs(mv - level) <= TOL:
            break
        if mv < level:
            lo = mid
        else:
            hi = mid
    return {"alpha": best[0], "maxvio": best[1], "iterations": best[2],
            "within_tol": abs(best[1] - level) <= TOL}


def main():
    w = synth.WORKLOADS["sweep"]
    table = {}
    for seed in SEEDS:
        table[str(seed)] = {f"{lv:g}": solve(w, seed, lv) for lv in LEVELS}
        print(seed, table[str(seed)])
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "sweep_alpha.json")
    with open(out, "w") as f:
        json.dump({"_about": "Zipf alpha per seed and maxvio level for the sweep shape "
                             "R8 E64 S4096 K8; written by make_sweep_alpha.py", **table},
                  f, indent=1, sort_keys=True)
        f.write("\n")


if __name__ == "__main__":
    main()
