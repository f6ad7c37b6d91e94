"""Replica counts of both planners on the benchmark workloads (CPU, oracle
only): every plan is within the bounds any plan obeys, and the largest-first
policy never needs more replicas than the lowest-id one there.

  lower bound: max(#overfull ranks, #underfull ranks) -- each overfull rank
               gives to at least one replica, each underfull rank hosts one;
  walk bound:  (#spilling experts + #underfull ranks - 1) -- the two-pointer
               walk makes one replica per boundary of the union of the two
               lists' running totals.

The table printed with -s is the one quoted in the design notes."""
import numpy as np
import pytest

import oracle
import synth

CASES = ([("tiny", synth.WORKLOADS["tiny"], 0), ("dsv3", synth.WORKLOADS["dsv3"], 0),
          ("adversarial", synth.WORKLOADS["adversarial"], 0)] +
         [(f"sweep mv{lv:g} seed {sd}", synth.sweep_workload(lv, sd), sd)
          for sd in (0, 1, 2) for lv in synth.SWEEP_LEVELS])


@pytest.mark.parametrize("name,w,seed", CASES, ids=[c[0] for c in CASES])
def test_replica_counts_within_bounds(name, w, seed):
    topk, _ = synth.routing(w, seed)
    T, mv = oracle.route_stats(w.R, w.E, w.S, w.K, topk)
    L, C = w.E // w.R, w.C
    load = T.reshape(w.R, L).sum(1)
    over, under = int((load > C).sum()), int((load < C).sum())
    row = [name, f"{mv:.3f}", max(over, under)]
    reps = {}
    for policy in (oracle.PLAN_LOWEST_ID, oracle.PLAN_LARGEST_FIRST):
        pl = oracle.plan(w.R, w.E, w.S, w.K, T, policy)
        walk = pl.n_spill + pl.n_deficit - 1 if pl.n_rep else 0
        assert max(over, under) <= pl.n_rep <= max(walk, 0)
        assert pl.n_deficit == under
        reps[policy] = pl.n_rep
        row += [pl.n_rep, walk, pl.max_rep_rank]
    assert reps[oracle.PLAN_LARGEST_FIRST] <= reps[oracle.PLAN_LOWEST_ID]
    print("| " + " | ".join(str(v) for v in row) + " |")
