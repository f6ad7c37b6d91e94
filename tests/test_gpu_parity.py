"""GPU parity at sizes the oracle covers element by element.

Every case runs the whole path through the C-ABI (route_stats, plan,
dispatch, stand-in expert, combine, combine_bwd, the stand-in expert's
backward, dispatch_bwd, replica_grad_reduce) and compares every output with
the CPU oracle:
  counts, maxvio, plan, slot maps, dispatch buffer, d_out, dx, replica grads:
  bit-exact;
  combine output: bit-exact (both sum the exact products in fp64 in ascending k
  and round once), also on signed expert rows and signed, cancelling gates;
  gate gradients: |gpu - oracle| <= 1e-5 * sum_h |dy_h * out_h|.
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

import load_balancing_amd as mx
import oracle
import synth
from gpu_harness import (bf16_dev, bits, compare_plan, oracle_plan, shape_of,
                         signed_combine_inputs, stand_in_expert, to_dev)

pytestmark = pytest.mark.gpu


def bf16_f64(b):
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def run_and_compare(w, seed, topk=None, gates=None, G=None, largest_first=False):
    print(f"[case] {w} seed={seed} largest_first={largest_first}", flush=True)
    if topk is None:
        topk, gates = synth.routing(w, seed)
    x = synth.activations(w, seed)
    dy = synth.activations(w, seed, synth.TAG_DY)
    scale = synth.expert_scale(w.E)
    G = w.G if G is None else G
    cap = w.E + w.R
    home = synth.normal_f32(seed, synth.TAG_GRAD_HOME, w.E * G, 0.01).reshape(w.E, G)
    rep = synth.normal_f32(seed, synth.TAG_GRAD_REP, cap * G, 0.01).reshape(cap, G)

    # ---- oracle ----------------------------------------------------------
    policy = oracle.PLAN_LARGEST_FIRST if largest_first else oracle.PLAN_LOWEST_ID
    T, mv, pl, slot_of, src_of_slot = oracle_plan(w, topk, policy)
    o_buf = oracle.dispatch(w.K, w.H, x, slot_of)
    o_out = oracle.expert(w.H, o_buf, oracle.row_expert(topk, src_of_slot), scale)
    o_y = oracle.combine(w.K, w.H, o_out, gates, slot_of)
    o_dout, o_dg = oracle.combine_bwd(w.K, w.H, dy, o_out, gates, slot_of)
    o_dbuf = oracle.expert(w.H, o_dout, oracle.row_expert(topk, src_of_slot), scale)
    o_dx = oracle.dispatch_bwd(w.K, w.H, o_dbuf, slot_of)
    o_home, o_rep = oracle.replica_grad_reduce(w.E, pl, G, home, rep)

    # ---- GPU through the C-ABI ------------------------------------------
    s = shape_of(w)
    b = mx.allocate(s)
    d_topk = to_dev(topk)
    d_gates = to_dev(gates)
    d_x = bf16_dev(x)
    d_dy = bf16_dev(dy)
    b.buf.view(torch.int16).fill_(-1)                      # sentinel
    mx.plan_step(b, d_topk, largest_first=largest_first)
    mx.moonep_dispatch(s, d_x, b.slot_of, b.buf)
    out = stand_in_expert(d_topk, b.src_of_slot, to_dev(scale), b.buf)
    y = torch.empty((w.N, w.H), dtype=torch.bfloat16, device="cuda")
    mx.moonep_combine(s, out, d_gates, b.slot_of, y)
    d_out = torch.empty_like(out)
    d_out.view(torch.int16).fill_(-1)
    d_g = torch.full((w.NK,), float("nan"), dtype=torch.float32, device="cuda")
    mx.moonep_combine_bwd(s, d_dy, out, d_gates, b.slot_of, d_out, d_g)
    d_buf = stand_in_expert(d_topk, b.src_of_slot, to_dev(scale), d_out)
    dx = torch.empty((w.N, w.H), dtype=torch.bfloat16, device="cuda")
    dx.view(torch.int16).fill_(-1)
    mx.moonep_dispatch_bwd(s, d_buf, b.slot_of, dx)
    d_home = to_dev(home)
    d_rep = to_dev(rep)
    mx.moonep_replica_grad_reduce(s, b.plan, G, d_home, d_rep)
    # combine again on signed expert rows, and on rows whose leading terms cancel
    eo, eo_c, sg_c = signed_combine_inputs(w, seed, slot_of)
    y_s = torch.empty_like(y)
    mx.moonep_combine(s, bf16_dev(eo), d_gates, b.slot_of, y_s)
    y_c = torch.empty_like(y)
    mx.moonep_combine(s, bf16_dev(eo_c), to_dev(sg_c), b.slot_of, y_c)
    torch.cuda.synchronize()
    assert mx.moonep_read_error(b.workspace) == mx.DEV_OK

    # ---- compare -----------------------------------------------------------
    np.testing.assert_array_equal(b.expert_counts.cpu().numpy(), T)
    assert b.maxvio.item() == mv
    compare_plan(b.plan_fields(), pl, w.E, w.R)
    np.testing.assert_array_equal(b.slot_of.cpu().numpy(), slot_of)
    np.testing.assert_array_equal(b.src_of_slot.cpu().numpy(), src_of_slot)
    np.testing.assert_array_equal(bits(b.buf), o_buf)
    np.testing.assert_array_equal(bits(out), o_out)
    np.testing.assert_array_equal(bits(y), o_y)
    np.testing.assert_array_equal(bits(y_s), oracle.combine(w.K, w.H, eo, gates, slot_of))
    np.testing.assert_array_equal(bits(y_c), oracle.combine(w.K, w.H, eo_c, sg_c, slot_of))
    np.testing.assert_array_equal(bits(d_out), o_dout)
    g_gpu = d_g.cpu().numpy().astype(np.float64)
    if w.NK:
        l1 = np.abs(bf16_f64(dy)[np.arange(w.NK) // w.K] * bf16_f64(o_out)[slot_of]).sum(1)
        err = np.abs(g_gpu - o_dg.astype(np.float64))
        assert (err <= 1e-5 * l1 + 1e-30).all(), f"gate grad err {err.max()}"
    np.testing.assert_array_equal(bits(d_buf), o_dbuf)
    np.testing.assert_array_equal(bits(dx), o_dx)
    np.testing.assert_array_equal(d_home.cpu().numpy(), o_home)
    np.testing.assert_array_equal(d_rep.cpu().numpy(), o_rep)
    return {"n_rep": pl.n_rep}


def test_tiny_config_full_chain():
    w = synth.WORKLOADS["tiny"]
    r = run_and_compare(w, 0)
    assert r["n_rep"] > 0


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_tiny_other_seeds(seed):
    run_and_compare(synth.WORKLOADS["tiny"], seed)


EDGE = [
    # ragged entry count (NK = 222) and 3 vectors per row
    synth.Workload("ragged", 3, 6, 37, 2, 24, "zipf", alpha=1.5, G=40),
    # one rank: nothing to balance
    synth.Workload("one_rank", 1, 4, 50, 3, 16, "zipf", alpha=1.0, G=16),
    # one expert per rank, every expert chosen by every token
    synth.Workload("k_eq_e", 4, 4, 33, 4, 8, "zipf", alpha=0.5, G=12),
    # a row of 65 vectors crosses a wave
    synth.Workload("wide_row", 5, 20, 300, 3, 520, "zipf", alpha=1.3, G=1000),
    # all tokens to experts 0..7 of rank 0, uniform gates
    synth.Workload("adversarial_small", 16, 128, 64, 8, 64, "fixed", gates="uniform", G=64),
    # heavy skew over many segments
    synth.Workload("heavy_skew", 8, 64, 700, 8, 136, "zipf", alpha=2.0, G=2048 + 3),
    # balanced routing: no replica
    synth.Workload("balanced", 8, 64, 512, 8, 64, "balanced", G=64),
    # G not a multiple of 4 (scalar reduce path)
    synth.Workload("odd_G", 4, 16, 128, 2, 64, "zipf", alpha=1.0, G=1001),
    # top-1 routing
    synth.Workload("k1", 2, 4, 100, 1, 64, "zipf", alpha=1.0, G=32),
    # top-6, rows of 17 vectors
    synth.Workload("k6", 4, 12, 50, 6, 136, "zipf", alpha=0.8, G=48),
    # K above one pass of eight: two passes, the second partial
    synth.Workload("k9", 4, 16, 40, 9, 64, "zipf", alpha=0.7, G=24),
]


@pytest.mark.parametrize("w", EDGE, ids=lambda w: w.name)
def test_edge_shapes(w):
    run_and_compare(w, 0)


def test_empty_input():
    """S = 0: every entry point accepts the empty step and writes nothing it
    should not (the replica reduction and the prefetch have no replica)."""
    w = synth.Workload("empty", 2, 8, 0, 2, 64, "zipf", G=16)
    s = shape_of(w)
    b = mx.allocate(s)
    e = torch.empty(0, dtype=torch.int32, device="cuda")
    b.expert_counts.fill_(-7)
    b.maxvio.fill_(3.0)
    mx.plan_step(b, e)
    x = torch.empty((0, w.H), dtype=torch.bfloat16, device="cuda")
    g0 = torch.empty(0, device="cuda")
    mx.moonep_dispatch(s, x, b.slot_of, b.buf)
    mx.moonep_combine(s, b.buf, g0, b.slot_of, x)
    mx.moonep_combine_bwd(s, x, b.buf, g0, b.slot_of, b.buf.clone(), g0.clone())
    mx.moonep_dispatch_bwd(s, b.buf, b.slot_of, x.clone())
    home = torch.full((w.E, w.G), 1.5, device="cuda")
    rep = torch.full((w.E + w.R, w.G), 2.5, device="cuda")
    mx.moonep_replica_grad_reduce(s, b.plan, w.G, home, rep)
    ws = torch.full((w.E + w.R,), 9, dtype=torch.int32, device="cuda")
    mx.moonep_weight_slots(s, b.plan, 2, ws)
    wh = torch.ones((w.E, 128 * 64), dtype=torch.bfloat16, device="cuda")
    pool = torch.full((w.R * 2, 128 * 64), 3.0, dtype=torch.bfloat16, device="cuda")
    mx.moonep_prefetch_weights(s, b.plan, ws, 2, 128 * 64 * 2, wh, pool)
    mx.moonep_expert_gemm(s, b.plan, ws, 2, 64, 128, x, wh, pool, 128 * 64, 0,
                          torch.empty((0, 128), dtype=torch.bfloat16, device="cuda"))
    torch.cuda.synchronize()
    assert mx.moonep_read_error(b.workspace) == mx.DEV_OK
    assert (b.expert_counts.cpu() == 0).all() and b.maxvio.item() == 0.0
    f = b.plan_fields()
    assert f["n_rep"] == 0 and (f["keep"] == 0).all()
    assert (home.cpu() == 1.5).all() and (rep.cpu() == 2.5).all()
    assert (ws.cpu() == -1).all() and (pool.float().cpu() == 3.0).all()


LIMITS = [
    # the largest E and R the plan tables hold (E = 1024, R = 512)
    synth.Workload("max_R_max_E", 512, 1024, 8, 2, 16, "zipf", alpha=1.2, G=16),
    synth.Workload("max_E_two_ranks", 2, 1024, 512, 8, 64, "zipf", alpha=1.0, G=24),
    synth.Workload("max_R_one_hot", 512, 512, 16, 4, 8, "fixed", gates="uniform", G=8),
]


@pytest.mark.parametrize("w", LIMITS, ids=lambda w: w.name)
def test_shape_limits(w):
    r = run_and_compare(w, 0)
    assert r["n_rep"] > 0


# More than 2^22 tokens: the movers' grids are capped at 2^22 workgroups, so
# dispatch, combine and dispatch_bwd loop over their grid and combine_bwd runs
# in two launches.  Rows of 8 elements keep every array small.
MANY_TOKENS = [
    synth.Workload("many_tokens_k1", 8, 16, 540000, 1, 8, "zipf", alpha=1.0, G=8),
    synth.Workload("many_tokens_k2", 4, 16, 1050000, 2, 8, "zipf", alpha=1.0, G=8),
]


@pytest.mark.parametrize("w", MANY_TOKENS, ids=lambda w: w.name)
def test_more_tokens_than_one_grid(w):
    assert w.N > 1 << 22
    r = run_and_compare(w, 0)
    assert r["n_rep"] > 0


def test_bad_expert_id_sets_error_word_and_stays_in_bounds():
    w = synth.WORKLOADS["tiny"]
    topk, gates = synth.routing(w, 0)
    topk = topk.copy()
    topk[5] = w.E + 3
    topk[77] = -1
    s = shape_of(w)
    b = mx.allocate(s)
    d_topk = to_dev(topk)
    mx.plan_step(b, d_topk)
    torch.cuda.synchronize()
    assert mx.moonep_read_error(b.workspace) == mx.DEV_BAD_EXPERT_ID
    assert mx.moonep_read_error(b.workspace) == mx.DEV_OK        # read clears it
    so = b.slot_of.cpu().numpy()
    assert so[5] == -1 and so[77] == -1
    # the other entries still form valid distinct slots
    rest = np.delete(so, [5, 77])
    assert (rest >= 0).all() and (rest < w.NK).all() and len(set(rest.tolist())) == rest.size
    # dispatch_bwd skips the two unplaced entries: their tokens sum the other
    # K-1 rows (the oracle sees them as a row of zeros appended to d_buf)
    d_buf = synth.normal_bf16(3, synth.TAG_DY, w.NK * w.H).reshape(w.NK, w.H)
    dx = torch.empty((w.N, w.H), dtype=torch.bfloat16, device="cuda")
    mx.moonep_dispatch_bwd(s, bf16_dev(d_buf), b.slot_of, dx)
    torch.cuda.synchronize()
    padded = np.concatenate([d_buf, np.zeros((1, w.H), np.uint16)])
    want = oracle.dispatch_bwd(w.K, w.H, padded, np.where(so < 0, w.NK, so).astype(np.int32))
    np.testing.assert_array_equal(bits(dx), want)


def test_repeat_is_bitwise_deterministic():
    w = replace(synth.WORKLOADS["tiny"], S=1000)
    topk, gates = synth.routing(w, 4)
    s = shape_of(w)
    d_topk, d_gates = to_dev(topk), to_dev(gates)
    d_x = bf16_dev(synth.activations(w, 4))
    results = []
    for _ in range(2):
        b = mx.allocate(s)
        mx.plan_step(b, d_topk)
        mx.moonep_dispatch(s, d_x, b.slot_of, b.buf)
        y = torch.empty((w.N, w.H), dtype=torch.bfloat16, device="cuda")
        mx.moonep_combine(s, b.buf, d_gates, b.slot_of, y)   # expert_out may be buf itself
        torch.cuda.synchronize()
        results.append((b.plan.cpu(), b.slot_of.cpu(), b.src_of_slot.cpu(), bits(b.buf), bits(y)))
    for a, c in zip(*results):
        assert np.array_equal(np.asarray(a), np.asarray(c))


def test_plan_with_several_chunk_batches_per_wave():
    # 4.2M entries: 2048 segments of 2048 entries, so each wave walks two
    # batches of 16 chunks
    w = synth.Workload("long_segments", 16, 64, 32768, 8, 8, "zipf", alpha=1.1)
    topk, _ = synth.routing(w, 0)
    T, mv, pl, slot_of, src_of_slot = oracle_plan(w, topk)
    s = shape_of(w)
    b = mx.allocate(s)
    mx.plan_step(b, to_dev(topk))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(b.expert_counts.cpu().numpy(), T)
    assert b.maxvio.item() == mv
    compare_plan(b.plan_fields(), pl, w.E, w.R)
    np.testing.assert_array_equal(b.slot_of.cpu().numpy(), slot_of)
    np.testing.assert_array_equal(b.src_of_slot.cpu().numpy(), src_of_slot)


@pytest.mark.parametrize("S,nseg", [(1000, 1000), (9500, 1900)])
def test_plan_partial_scan_groups(S, nseg):
    """Segment counts that are a multiple of 4 but leave the last threads of
    the column scan past the end (4 and 8 counts per thread): the 16-byte
    scan path with a partial last group."""
    w = synth.Workload(f"scan_groups_{nseg}", 8 if S == 1000 else 16, 64, S, 8, 8, "zipf", alpha=1.1)
    s = shape_of(w)
    assert (mx.moonep_workspace_bytes(s) - 256) // (4 * w.E) == nseg
    topk, _ = synth.routing(w, 0)
    T, mv, pl, slot_of, src_of_slot = oracle_plan(w, topk)
    b = mx.allocate(s)
    mx.plan_step(b, to_dev(topk))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(b.expert_counts.cpu().numpy(), T)
    assert b.maxvio.item() == mv
    compare_plan(b.plan_fields(), pl, w.E, w.R)
    np.testing.assert_array_equal(b.slot_of.cpu().numpy(), slot_of)
    np.testing.assert_array_equal(b.src_of_slot.cpu().numpy(), src_of_slot)


def test_two_streams_with_own_workspaces():
    """Two layers' route_stats, plan, dispatch and combine on two streams at
    once, each with its own buffers and workspace, interleaved call by call:
    each equals the same layer run alone, bit for bit."""
    w = synth.Workload("streams", 8, 64, 512, 8, 64, "zipf", alpha=1.2)
    s = shape_of(w)
    ins = []
    for seed in (3, 4):
        topk, gates = synth.routing(w, seed)
        ins.append((to_dev(topk), to_dev(gates), bf16_dev(synth.activations(w, seed))))

    def layer_calls(b, tk, gt, x, y, st):
        return [lambda: mx.moonep_route_stats(s, tk, b.expert_counts, b.maxvio, b.workspace, st),
                lambda: mx.moonep_plan(s, tk, b.expert_counts, b.workspace, b.plan, b.slot_of,
                                       b.src_of_slot, st),
                lambda: mx.moonep_dispatch(s, x, b.slot_of, b.buf, st),
                lambda: mx.moonep_combine(s, b.buf, gt, b.slot_of, y, st)]

    def snap(b, y):
        return [t.cpu().numpy().copy() for t in (b.plan, b.slot_of, b.src_of_slot,
                                                 b.buf.view(torch.int16), y.view(torch.int16))]

    alone = []
    for tk, gt, x in ins:
        b = mx.allocate(s)
        y = torch.empty((w.N, w.H), dtype=torch.bfloat16, device="cuda")
        for c in layer_calls(b, tk, gt, x, y, None):
            c()
        torch.cuda.synchronize()
        alone.append(snap(b, y))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]   # default priority
    bufs = [mx.allocate(s) for _ in ins]
    ys = [torch.empty((w.N, w.H), dtype=torch.bfloat16, device="cuda") for _ in ins]
    torch.cuda.synchronize()
    for rep in range(3):
        calls = [layer_calls(bufs[i], *ins[i], ys[i], streams[i]) for i in range(2)]
        for c0, c1 in zip(*calls):
            c0()
            c1()
        torch.cuda.synchronize()
        for i in range(2):
            assert mx.moonep_read_error(bufs[i].workspace) == 0
            for got, want in zip(snap(bufs[i], ys[i]), alone[i]):
                np.testing.assert_array_equal(got, want, err_msg=f"rep {rep} layer {i}")


@pytest.mark.parametrize("largest_first", [False, True], ids=["lowest_id", "largest_first"])
def test_plan_random_shapes(largest_first):
    """Plan, counts, maxvio and slot maps on 300 random small shapes (skews
    from uniform to one hot expert), bit-exact against the oracle, for both
    planners."""
    policy = oracle.PLAN_LARGEST_FIRST if largest_first else oracle.PLAN_LOWEST_ID
    rng = np.random.default_rng(11)
    for case in range(300):
        R = int(rng.integers(1, 17))
        L = int(rng.integers(1, 9))
        E = R * L
        K = int(rng.integers(1, min(E, 8) + 1))
        S = int(rng.integers(0, 60))
        N = R * S
        skew = rng.uniform(0, 3)
        p = (np.arange(E) + 1.0) ** -skew
        p = p[rng.permutation(E)]
        p /= p.sum()
        topk = np.concatenate([rng.choice(E, size=K, replace=False, p=p) for _ in range(N)]
                              ).astype(np.int32) if N else np.zeros(0, dtype=np.int32)
        w = synth.Workload(f"rand{case}", R, E, S, K, 8, "zipf")
        T, mv, pl, slot_of, src_of_slot = oracle_plan(w, topk, policy)
        s = shape_of(w)
        b = mx.allocate(s)
        mx.plan_step(b, to_dev(topk) if N else torch.empty(0, dtype=torch.int32, device="cuda"),
                     largest_first=largest_first)
        torch.cuda.synchronize()
        msg = f"case {case}: R={R} E={E} S={S} K={K}"
        np.testing.assert_array_equal(b.expert_counts.cpu().numpy(), T, err_msg=msg)
        assert b.maxvio.item() == mv, msg
        compare_plan(b.plan_fields(), pl, E, R)
        if N:
            np.testing.assert_array_equal(b.slot_of.cpu().numpy(), slot_of, err_msg=msg)
            np.testing.assert_array_equal(b.src_of_slot.cpu().numpy(), src_of_slot, err_msg=msg)


# Many experts per lane of the planning wave (E = 512 and 1024: 8 and 16 per
# lane) with 1M routed entries, so each wave's segment is 512 entries and the
# slot loop takes its chunks 8 at a time.
WIDE_LONG = [
    synth.Workload("wide8_long", 32, 512, 4096, 8, 8, "zipf", alpha=1.2),
    synth.Workload("wide16_long", 16, 1024, 8192, 8, 8, "zipf", alpha=1.0),
]


@pytest.mark.parametrize("largest_first", [False, True], ids=["lowest_id", "largest_first"])
@pytest.mark.parametrize("w", WIDE_LONG, ids=lambda w: w.name)
def test_plan_many_experts_per_lane_long_segments(w, largest_first):
    """Counts, maxvio, every plan field and both slot maps, bit-exact against
    the oracle, for both planners."""
    assert w.NK >= 1 << 20 and w.E > 256
    policy = oracle.PLAN_LARGEST_FIRST if largest_first else oracle.PLAN_LOWEST_ID
    topk, _ = synth.routing(w, 0)
    T, mv, pl, slot_of, src_of_slot = oracle_plan(w, topk, policy)
    assert pl.n_rep > 0
    b = mx.allocate(shape_of(w))
    mx.plan_step(b, to_dev(topk), largest_first=largest_first)
    torch.cuda.synchronize()
    assert mx.moonep_read_error(b.workspace) == mx.DEV_OK
    np.testing.assert_array_equal(b.expert_counts.cpu().numpy(), T)
    assert b.maxvio.item() == mv
    compare_plan(b.plan_fields(), pl, w.E, w.R)
    np.testing.assert_array_equal(b.slot_of.cpu().numpy(), slot_of)
    np.testing.assert_array_equal(b.src_of_slot.cpu().numpy(), src_of_slot)


@pytest.mark.parametrize("w", [synth.WORKLOADS["tiny"]] + [e for e in EDGE if e.name in (
    "ragged", "heavy_skew", "k9", "adversarial_small")] + LIMITS[:2], ids=lambda w: w.name)
def test_whole_chain_largest_first(w):
    """The element-by-element chain with the largest-first planner: its plan
    feeds the same slot assignment, movers and reduction."""
    run_and_compare(w, 0, largest_first=True)


def test_whole_chain_random_shapes():
    """The element-by-element chain (plan, dispatch, combine, both backwards,
    the reduction) on 40 random shapes: ranks, experts per rank, K up to 9
    (a second pass of the K loop), ragged token counts, rows of 1 to 257
    16-byte vectors, and skews from uniform to a few hot experts."""
    rng = np.random.default_rng(23)
    for case in range(40):
        R = int(rng.integers(1, 13))
        L = int(rng.integers(1, 7))
        E = R * L
        K = int(rng.integers(1, min(E, 9) + 1))
        S = int(rng.integers(1, 70))
        H = 8 * int(rng.choice([1, 2, 3, 8, 17, 64, 257]))
        G = int(rng.integers(1, 300))
        w = synth.Workload(f"rand{case}", R, E, S, K, H, "zipf",
                           alpha=float(rng.uniform(0.0, 2.5)), G=G)
        run_and_compare(w, case)
