"""Helpers for the GPU parity tests: upload synthetic inputs, run the path
through the C-ABI binding, build the stand-in expert, compare with the oracle.

The stand-in expert (not part of the path) multiplies the rows of expert e by
fp32(1 + e/E) and rounds to bf16; here it runs as plain torch ops on the GPU,
in the oracle as plain C.
"""
import numpy as np
import torch

import load_balancing_amd as mx
import oracle
import synth


def shape_of(w) -> mx.Shape:
    return mx.Shape(w.R, w.E, w.S, w.K, w.H)


def to_dev(a: np.ndarray, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.to("cuda", non_blocking=False)


def bf16_dev(a_u16: np.ndarray):
    return to_dev(a_u16.view(np.int16), torch.int16).view(torch.bfloat16)


def bits(t) -> np.ndarray:
    """bf16 tensor -> uint16 bit patterns on the host."""
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def ordinal(b: np.ndarray) -> np.ndarray:
    """bf16 bits -> integers ordered like the values (+0 and -0 coincide)."""
    b = b.astype(np.int32)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def ulp_diff(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    return np.abs(ordinal(a) - ordinal(b))


def stand_in_expert(topk_dev, src_of_slot_dev, scale_dev, buf, rows_per_chunk=1 << 16):
    """out[r] = bf16(fp32(buf[r]) * scale[expert of the entry at row r])."""
    out = torch.empty_like(buf)
    n = buf.shape[0]
    for r0 in range(0, n, rows_per_chunk):
        r1 = min(n, r0 + rows_per_chunk)
        e = topk_dev[src_of_slot_dev[r0:r1].long()].long()
        out[r0:r1] = (buf[r0:r1].float() * scale_dev[e][:, None]).to(torch.bfloat16)
    return out


def bf16_f64(b: np.ndarray) -> np.ndarray:
    """bf16 bits -> float64 values."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def assert_gate_grads(g_gpu, o_dg, dy, out, slot_of, K, chunk=8192):
    """Gate gradients within the componentwise bound, for every entry n:
    |gpu - oracle| <= 1e-5 * sum_h |dy[n div K, h] * out[slot_of[n], h]|
    (dy [N, H] and out [R*S*K, H] as bf16 bits; out indexed by buffer row)."""
    g = np.asarray(g_gpu, dtype=np.float64)
    o = np.asarray(o_dg, dtype=np.float64)
    for n0 in range(0, slot_of.size, chunk):
        n1 = min(slot_of.size, n0 + chunk)
        l1 = np.abs(bf16_f64(dy[np.arange(n0, n1) // K]) * bf16_f64(out[slot_of[n0:n1]])).sum(1)
        err = np.abs(g[n0:n1] - o[n0:n1])
        bad = np.nonzero(err > 1e-5 * l1 + 1e-30)[0]
        assert bad.size == 0, f"gate grad of entry {n0 + bad[0]}: err {err[bad[0]]}, l1 {l1[bad[0]]}"


def signed_combine_inputs(w, seed, slot_of):
    """Combine inputs with terms of both signs, as a real expert's outputs have.
    Returns (rows, rows_cancel, gates_cancel): `rows` are N(0,1) bf16 expert
    rows (to go with the workload's own softmax gates); `rows_cancel` repeat
    them except that, for every token with K >= 2, the row of its second entry
    repeats its first, and `gates_cancel` are signed N(0,1) gates with the
    second gate -(1 + 2^-20) times the first, so the two leading terms cancel to
    about a millionth of either."""
    eo = synth.normal_bf16(seed, synth.TAG_EXPERT_OUT, w.NK * w.H).reshape(w.NK, w.H)
    g_c = synth.normal_f32(seed, synth.TAG_SIGNED_GATE, w.NK)
    eo_c = eo.copy()
    if w.K >= 2 and w.NK:
        n0 = np.arange(0, w.NK, w.K)
        n1 = n0 + 1
        eo_c[slot_of[n1]] = eo_c[slot_of[n0]]
        g_c[n1] = (-g_c[n0].astype(np.float64) * (1.0 + 2.0 ** -20)).astype(np.float32)
    return eo, eo_c, g_c


def oracle_plan(w, topk, policy=oracle.PLAN_LOWEST_ID):
    T, mv = oracle.route_stats(w.R, w.E, w.S, w.K, topk)
    pl = oracle.plan(w.R, w.E, w.S, w.K, T, policy)
    slot_of, src_of_slot = oracle.slots(w.R, w.E, w.S, w.K, topk, pl)
    return T, mv, pl, slot_of, src_of_slot


def compare_plan(gpu: dict, pl: oracle.Plan, E: int, R: int):
    """Every plan field, bit for bit."""
    assert gpu["n_rep"] == pl.n_rep
    assert gpu["n_spill"] == pl.n_spill
    assert gpu["n_deficit"] == pl.n_deficit
    assert gpu["max_rep_rank"] == pl.max_rep_rank
    for f in ("rep_expert", "rep_host", "rep_count", "rep_spill_off", "rep_row_off", "spill",
              "keep", "home_row_off", "rep_first", "rep_cnt", "load", "rank_rep_first",
              "rank_rep_cnt"):
        np.testing.assert_array_equal(gpu[f], getattr(pl, f), err_msg=f)
    spill_experts = np.nonzero(pl.spill)[0]
    np.testing.assert_array_equal(gpu["exp_rep_list"][:len(spill_experts)], spill_experts)
    assert (gpu["exp_rep_list"][len(spill_experts):] == 0).all()
