"""moonep_plan_noalloc -- route statistics and the plan with the library's
static per-device scratch in place of a caller's workspace, for callers that
cannot allocate -- against moonep_route_stats + moonep_plan with a workspace
of their own: two calls in a row, the second on a smaller shape (the scratch
keeps the first call's contents), every output bit for bit."""
import numpy as np
import pytest
import torch

import load_balancing_amd as mx
import synth
from gpu_harness import shape_of, to_dev

pytestmark = pytest.mark.gpu


def outputs_noalloc(w, d_topk):
    s = shape_of(w)
    cnt = torch.full((w.E,), -1, dtype=torch.int32, device="cuda")
    mv = torch.full((1,), float("nan"), dtype=torch.float32, device="cuda")
    plan = torch.full((mx.moonep_plan_bytes(s) // 4,), -7, dtype=torch.int32, device="cuda")
    slot_of = torch.full((w.NK,), -9, dtype=torch.int32, device="cuda")
    src = torch.full((w.NK,), -9, dtype=torch.int32, device="cuda")
    mx.moonep_plan_noalloc(s, d_topk, cnt, mv, plan, slot_of, src)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in (cnt, mv, plan, slot_of, src)]


def outputs_workspace(w, d_topk):
    b = mx.allocate(shape_of(w))
    mx.plan_step(b, d_topk)
    torch.cuda.synchronize()
    assert mx.moonep_read_error(b.workspace) == mx.DEV_OK
    return [t.cpu().numpy() for t in (b.expert_counts, b.maxvio, b.plan, b.slot_of, b.src_of_slot)]


CASES = [
    # 1,048,576 entries over 1024 experts: 2048 wave segments, so the
    # counts fill the whole scratch
    (synth.Workload("noalloc_full_scratch", 2, 1024, 65536, 8, 8, "zipf", alpha=1.0), 0),
    # the benchmark's routing shape at maxvio 4
    (synth.sweep_workload(4.0, 0), 0),
    # a smaller shape after the larger ones
    (synth.Workload("noalloc_small", 4, 16, 100, 2, 8, "zipf", alpha=1.5), 1),
]


def test_noalloc_equals_workspace_calls_in_a_row():
    for w, seed in CASES:
        print(f"[case] {w.name} R={w.R} E={w.E} S={w.S} K={w.K}", flush=True)
        topk, _ = synth.routing(w, seed)
        d_topk = to_dev(topk)
        want = outputs_workspace(w, d_topk)
        got = outputs_noalloc(w, d_topk)
        for name, g, r in zip(("expert_counts", "maxvio", "plan", "slot_of", "src_of_slot"),
                              got, want):
            np.testing.assert_array_equal(g.view(np.int32), r.view(np.int32), err_msg=name)
