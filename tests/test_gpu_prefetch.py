"""GPU parity of the replica weight slots and the weight prefetch.

Through the C-ABI, against the CPU oracle: the slot table bit-exact at several
B (none, inference-sized, training B = E/R, more than any rank needs), the
prefetched pool byte-exact, rows without a replica untouched.  Weight rows of
several 4 KiB chunks with a ragged tail at small sizes; at the benchmark's
sweep shape the whole pool is compared; at the DeepSeek-V3-like shape every
slotted row is compared on the GPU with its expert's row.
"""
import numpy as np
import pytest
import torch

import load_balancing_amd as mx
import oracle
import synth
from gpu_harness import oracle_plan, shape_of, to_dev

pytestmark = pytest.mark.gpu

SENTINEL = 0xA5


def run_prefetch(w, seed, Bs, wbytes, topk=None):
    print(f"[case] {w} seed={seed} B={Bs} wbytes={wbytes}", flush=True)
    if topk is None:
        topk, _ = synth.routing(w, seed)
    T, mv, pl, slot_of, src_of_slot = oracle_plan(w, topk)
    s = shape_of(w)
    b = mx.allocate(s)
    mx.plan_step(b, to_dev(topk))
    w_home = synth.expert_weights(w.E, wbytes, seed)
    d_home = to_dev(w_home)
    for B in Bs:
        ws = torch.full((w.E + w.R,), 12345, dtype=torch.int32, device="cuda")
        mx.moonep_weight_slots(s, b.plan, B, ws)
        pool = torch.full((w.R * B, wbytes), SENTINEL, dtype=torch.uint8, device="cuda")
        mx.moonep_prefetch_weights(s, b.plan, ws, B, wbytes, d_home, pool)
        torch.cuda.synchronize()
        o_ws = oracle.weight_slots(w.R, w.E, B, pl)
        np.testing.assert_array_equal(ws.cpu().numpy(), o_ws)
        o_pool = oracle.prefetch_weights(pl, o_ws, w_home,
                                         np.full((w.R * B, wbytes), SENTINEL, np.uint8))
        np.testing.assert_array_equal(pool.cpu().numpy(), o_pool)
    return pl


SMALL = [
    synth.WORKLOADS["tiny"],
    synth.Workload("max_R_max_E", 512, 1024, 8, 2, 16, "zipf", alpha=1.2),
    synth.Workload("skew", 4, 16, 100, 4, 64, "zipf", alpha=2.5),
    synth.Workload("many_ranks", 16, 32, 64, 2, 64, "zipf", alpha=1.3),
    synth.Workload("one_rank", 1, 4, 50, 2, 64, "zipf", alpha=1.0),
    synth.Workload("adversarial_small", 8, 32, 64, 4, 64, "fixed", gates="uniform"),
]


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_prefetch_small(w):
    L = w.E // w.R
    # 16 * (2 * 1024 + 37) bytes: two whole 16 KiB chunks and a ragged tail
    pl = run_prefetch(w, 0, sorted({0, 1, 2, L, L + 3}), 16 * (2 * 1024 + 37))
    if w.name != "one_rank":
        assert pl.n_rep > 0


def test_prefetch_balanced_has_nothing_to_copy():
    w = synth.sweep_workload(0.0)
    w = synth.Workload("balanced_small", w.R, w.E, 256, w.K, 64, "balanced")
    pl = run_prefetch(w, 0, [1, w.E // w.R], 4096)
    assert pl.n_rep == 0


@pytest.mark.parametrize("level", [2.0, 4.0])
def test_prefetch_sweep_full(level):
    """The benchmark shape: rows of gate+up+down = 3 * 2048 * 1408 bf16;
    training B = E/R and an inference B = 4; whole pool compared."""
    w = synth.sweep_workload(level, seed=0)
    run_prefetch(w, 0, [4, w.E // w.R], 3 * w.H * synth.SWEEP_FFN * 2)


def test_prefetch_dsv3_slotted_rows():
    """DeepSeek-V3-like shape, rows of 3 * 7168 * 2048 bf16 (88 MB).  The
    weights are a seeded 88 MB row plus the expert id (int16 add), so every
    row differs everywhere; the GPU compares each slotted pool row with its
    expert's row and checks that every other row kept the sentinel."""
    w = synth.WORKLOADS["dsv3"]
    print(f"[case] {w.name}", flush=True)
    topk, _ = synth.routing(w, 0)
    T, mv, pl, slot_of, src_of_slot = oracle_plan(w, topk)
    s = shape_of(w)
    b = mx.allocate(s)
    mx.plan_step(b, to_dev(topk))
    del b.buf
    wbytes = 3 * 7168 * 2048 * 2
    row = to_dev(synth.expert_weights(1, wbytes, 0).view(np.int16))
    w_home = torch.empty((w.E, wbytes // 2), dtype=torch.int16, device="cuda")
    for e in range(w.E):
        torch.add(row[0], e, out=w_home[e])
    for B in (4, w.E // w.R):
        ws = torch.empty(w.E + w.R, dtype=torch.int32, device="cuda")
        mx.moonep_weight_slots(s, b.plan, B, ws)
        pool = torch.full((w.R * B, wbytes // 2), -23131, dtype=torch.int16, device="cuda")
        mx.moonep_prefetch_weights(s, b.plan, ws, B, wbytes, w_home, pool)
        torch.cuda.synchronize()
        o_ws = oracle.weight_slots(w.R, w.E, B, pl)
        np.testing.assert_array_equal(ws.cpu().numpy(), o_ws)
        slotted = np.nonzero(o_ws[:pl.n_rep] >= 0)[0]
        for j in slotted:
            assert torch.equal(pool[int(o_ws[j])], w_home[int(pl.rep_expert[j])]), f"replica {j}"
        free = np.setdiff1d(np.arange(w.R * B), o_ws[slotted])
        for r in free:
            assert bool((pool[int(r)] == -23131).all()), f"pool row {r} written"
        n_over = int((o_ws[:pl.n_rep] < 0).sum())
        print(f"[dsv3] B={B} n_rep={pl.n_rep} prefetched={slotted.size} overflow={n_over}")
        del pool
