"""CPU oracle for the balanced expert-parallel hot path -- TEST INFRASTRUCTURE.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the GPU library and
its binding) never touches it.

The arithmetic lives in ``oracle.c`` (plain single-threaded C, fp64 where the
pages fix no precision); this module builds it with gcc and marshals numpy
arrays.  Functions without an independent pin: none -- every step is checked
in ``tests/test_oracle_pins.py`` against closed forms, invariants, brute
force or exact rational arithmetic.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
# A planted-mistake copy may be loaded instead, by the mutation test only.
_BUILT = os.path.join(_HERE, "liboracle.so")
_LIB = os.environ.get("MOONEP_ORACLE_LIB") or _BUILT

OK, ERR_SHAPE, ERR_EXPERT_ID, ERR_INTERNAL = 0, -1, -2, -3


def build(verbose: bool = False, src: str = _SRC, out: str = _BUILT) -> str:
    # -O1 and no fast-math: plain IEEE double arithmetic in source order.
    cmd = ["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-fno-fast-math",
           "-ffp-contract=off", src, "-o", out, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    return out


class _CPlan(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("n_rep", "n_spill", "n_deficit", "max_rep_rank")] + [
        (n, ctypes.c_void_p) for n in (
            "rep_expert", "rep_host", "rep_count", "rep_spill_off", "rep_row_off",
            "spill", "keep", "home_row_off", "rep_first", "rep_cnt",
            "load", "rank_rep_first", "rank_rep_cnt")]


_REP_FIELDS = ("rep_expert", "rep_host", "rep_count", "rep_spill_off", "rep_row_off")
_EXP_FIELDS = ("spill", "keep", "home_row_off", "rep_first", "rep_cnt")
_RANK_FIELDS = ("load", "rank_rep_first", "rank_rep_cnt")


@dataclass
class Plan:
    n_rep: int
    n_spill: int
    n_deficit: int
    max_rep_rank: int
    arrays: dict  # name -> np.int32 array (replica arrays have capacity E + R)

    def __getattr__(self, name):
        arrays = self.__dict__.get("arrays", {})
        if name in arrays:
            return arrays[name]
        raise AttributeError(name)


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            raise RuntimeError(f"{_LIB} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(_LIB)
        i32, i64, p = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
        L.orc_bf16_to_double.restype = ctypes.c_double
        L.orc_bf16_to_double.argtypes = [ctypes.c_uint16]
        L.orc_bf16_from_double.restype = ctypes.c_uint16
        L.orc_bf16_from_double.argtypes = [ctypes.c_double]
        L.orc_route_stats.restype = ctypes.c_int
        L.orc_route_stats.argtypes = [i32, i32, i32, i32, p, p, p]
        L.orc_plan.restype = ctypes.c_int
        L.orc_plan.argtypes = [i32, i32, i32, i32, p, ctypes.POINTER(_CPlan)]
        L.orc_plan_policy.restype = ctypes.c_int
        L.orc_plan_policy.argtypes = [i32, i32, i32, i32, p, i32, ctypes.POINTER(_CPlan)]
        L.orc_slots.restype = ctypes.c_int
        L.orc_slots.argtypes = [i32, i32, i32, i32, p, ctypes.POINTER(_CPlan), p, p]
        L.orc_dispatch.restype = None
        L.orc_dispatch.argtypes = [i64, i32, i32, p, p, p]
        L.orc_dispatch_rows.restype = None
        L.orc_dispatch_rows.argtypes = [i32, i32, p, p, i64, p, p]
        L.orc_expert.restype = None
        L.orc_expert.argtypes = [i64, i32, p, p, p, p]
        L.orc_combine.restype = None
        L.orc_combine.argtypes = [i64, i32, i32, p, p, p, p]
        L.orc_forward_tokens.restype = None
        L.orc_forward_tokens.argtypes = [i32, i32, p, p, p, p, p, p, i64, p, p]
        L.orc_combine_bwd.restype = None
        L.orc_combine_bwd.argtypes = [i64, i32, i32, p, p, p, p, p, p]
        L.orc_dispatch_bwd.restype = None
        L.orc_dispatch_bwd.argtypes = [i64, i32, i32, p, p, p]
        L.orc_replica_grad_reduce.restype = None
        L.orc_replica_grad_reduce.argtypes = [i32, ctypes.POINTER(_CPlan), i64, p, p]
        L.orc_replica_grad_reduce_at.restype = None
        L.orc_replica_grad_reduce_at.argtypes = [i32, ctypes.POINTER(_CPlan), i64, p, p, i64, p]
        L.orc_expert_gemm_rows.restype = None
        L.orc_expert_gemm_rows.argtypes = [i32, i32, i32, i32, ctypes.POINTER(_CPlan), p, i32, i32,
                                           p, p, p, i64, i64, i64, p, i32, p]
        L.orc_weight_slots.restype = None
        L.orc_weight_slots.argtypes = [i32, i32, i32, ctypes.POINTER(_CPlan), p]
        L.orc_prefetch_weights.restype = None
        L.orc_prefetch_weights.argtypes = [i64, ctypes.POINTER(_CPlan), p, p, p]
        _lib = L
    return _lib


def _c(a: np.ndarray, dtype) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def _p(a: np.ndarray) -> int:
    return a.ctypes.data


class OracleError(RuntimeError):
    pass


def _check(rc: int, what: str):
    if rc != OK:
        raise OracleError(f"{what}: oracle error {rc}")


def bf16_to_double(b: int) -> float:
    return lib().orc_bf16_to_double(int(b))


def bf16_from_double(d: float) -> int:
    return int(lib().orc_bf16_from_double(float(d)))


def route_stats(R, E, S, K, topk):
    topk = _c(topk, np.int32)
    T = np.empty(E, dtype=np.int32)
    mv = np.empty(1, dtype=np.float32)
    _check(lib().orc_route_stats(R, E, S, K, _p(topk), _p(T), _p(mv)), "route_stats")
    return T, float(mv[0])


def _alloc_plan(E, R):
    cap = E + R
    arrays = {n: np.zeros(cap, dtype=np.int32) for n in _REP_FIELDS}
    arrays.update({n: np.zeros(E, dtype=np.int32) for n in _EXP_FIELDS})
    arrays.update({n: np.zeros(R, dtype=np.int32) for n in _RANK_FIELDS})
    c = _CPlan()
    for n, a in arrays.items():
        setattr(c, n, _p(a))
    return c, arrays


def _cplan_from(plan: Plan) -> _CPlan:
    c = _CPlan()
    c.n_rep, c.n_spill, c.n_deficit, c.max_rep_rank = (
        plan.n_rep, plan.n_spill, plan.n_deficit, plan.max_rep_rank)
    for n, a in plan.arrays.items():
        assert a.dtype == np.int32 and a.flags["C_CONTIGUOUS"]
        setattr(c, n, _p(a))
    return c


PLAN_LOWEST_ID, PLAN_LARGEST_FIRST = 0, 1


def plan(R, E, S, K, T, policy=PLAN_LOWEST_ID) -> Plan:
    """The replica plan; policy PLAN_LOWEST_ID spills an overfull rank's
    experts from the lowest id, PLAN_LARGEST_FIRST from the largest count."""
    T = _c(T, np.int32)
    c, arrays = _alloc_plan(E, R)
    _check(lib().orc_plan_policy(R, E, S, K, _p(T), int(policy), ctypes.byref(c)), "plan")
    return Plan(c.n_rep, c.n_spill, c.n_deficit, c.max_rep_rank, arrays)


def slots(R, E, S, K, topk, pl: Plan):
    topk = _c(topk, np.int32)
    NK = R * S * K
    slot_of = np.full(NK, -1, dtype=np.int32)
    src_of_slot = np.full(NK, -1, dtype=np.int32)
    c = _cplan_from(pl)
    _check(lib().orc_slots(R, E, S, K, _p(topk), ctypes.byref(c), _p(slot_of), _p(src_of_slot)),
           "slots")
    return slot_of, src_of_slot


def dispatch(K, H, x, slot_of):
    x = _c(x, np.uint16)
    slot_of = _c(slot_of, np.int32)
    NK = slot_of.size
    buf = np.zeros((NK, H), dtype=np.uint16)
    lib().orc_dispatch(NK, K, H, _p(x), _p(slot_of), _p(buf))
    return buf


def dispatch_rows(K, H, x, src_of_slot, rows):
    x = _c(x, np.uint16)
    src_of_slot = _c(src_of_slot, np.int32)
    rows = _c(rows, np.int64)
    out = np.empty((rows.size, H), dtype=np.uint16)
    lib().orc_dispatch_rows(K, H, _p(x), _p(src_of_slot), rows.size, _p(rows), _p(out))
    return out


def expert(H, buf, row_expert, scale):
    buf = _c(buf, np.uint16)
    row_expert = _c(row_expert, np.int32)
    scale = _c(scale, np.float32)
    rows = row_expert.size
    out = np.empty((rows, H), dtype=np.uint16)
    lib().orc_expert(rows, H, _p(buf), _p(row_expert), _p(scale), _p(out))
    return out


def combine(K, H, out, gates, slot_of):
    out = _c(out, np.uint16)
    gates = _c(gates, np.float32)
    slot_of = _c(slot_of, np.int32)
    N = slot_of.size // K
    y = np.empty((N, H), dtype=np.uint16)
    lib().orc_combine(N, K, H, _p(out), _p(gates), _p(slot_of), _p(y))
    return y


def forward_tokens(K, H, x, topk, gates, slot_of, src_of_slot, scale, toks):
    x = _c(x, np.uint16)
    topk = _c(topk, np.int32)
    gates = _c(gates, np.float32)
    slot_of = _c(slot_of, np.int32)
    src_of_slot = _c(src_of_slot, np.int32)
    scale = _c(scale, np.float32)
    toks = _c(toks, np.int64)
    y = np.empty((toks.size, H), dtype=np.uint16)
    lib().orc_forward_tokens(K, H, _p(x), _p(topk), _p(gates), _p(slot_of), _p(src_of_slot),
                             _p(scale), toks.size, _p(toks), _p(y))
    return y


def combine_bwd(K, H, dy, out, gates, slot_of):
    dy = _c(dy, np.uint16)
    out = _c(out, np.uint16)
    gates = _c(gates, np.float32)
    slot_of = _c(slot_of, np.int32)
    NK = slot_of.size
    N = NK // K
    d_out = np.zeros((NK, H), dtype=np.uint16)
    d_gates = np.empty(NK, dtype=np.float32)
    lib().orc_combine_bwd(N, K, H, _p(dy), _p(out), _p(gates), _p(slot_of), _p(d_out),
                          _p(d_gates))
    return d_out, d_gates


def dispatch_bwd(K, H, d_buf, slot_of):
    """dx [N, H] bf16 from the buffer gradient d_buf [N*K, H] bf16."""
    d_buf = _c(d_buf, np.uint16)
    slot_of = _c(slot_of, np.int32)
    N = slot_of.size // K
    dx = np.empty((N, H), dtype=np.uint16)
    lib().orc_dispatch_bwd(N, K, H, _p(d_buf), _p(slot_of), _p(dx))
    return dx


def replica_grad_reduce(E, pl: Plan, G, home, rep):
    """In place on copies; returns (home', rep')."""
    home = np.array(home, dtype=np.float32, copy=True, order="C")
    rep = np.array(rep, dtype=np.float32, copy=True, order="C")
    c = _cplan_from(pl)
    lib().orc_replica_grad_reduce(E, ctypes.byref(c), G, _p(home), _p(rep))
    return home, rep


def replica_grad_reduce_at(E, pl: Plan, G, home_at, rep_at):
    """home_at [E, m] and rep_at [n_rep, m] hold values at m chosen positions."""
    home_at = _c(home_at, np.float32)
    rep_at = _c(rep_at, np.float32)
    m = home_at.shape[1]
    out = np.empty_like(home_at)
    c = _cplan_from(pl)
    lib().orc_replica_grad_reduce_at(E, ctypes.byref(c), G, _p(home_at), _p(rep_at), m, _p(out))
    return out


def weight_slots(R, E, B, pl: Plan):
    """wslot [E+R] int32: prefetch slot d*B+b of each replica, -1 for overflow and j >= n_rep."""
    wslot = np.empty(E + R, dtype=np.int32)
    c = _cplan_from(pl)
    lib().orc_weight_slots(R, E, B, ctypes.byref(c), _p(wslot))
    return wslot


def prefetch_weights(pl: Plan, wslot, w_home, pool):
    """Copy of pool [R*B, wbytes] uint8 with every slotted replica's expert row of w_home [E, wbytes]."""
    w_home = _c(w_home, np.uint8)
    wslot = _c(wslot, np.int32)
    pool = np.array(pool, dtype=np.uint8, copy=True, order="C")
    wbytes = w_home.shape[1]
    assert pool.ndim == 2 and pool.shape[1] == wbytes
    c = _cplan_from(pl)
    lib().orc_prefetch_weights(wbytes, ctypes.byref(c), _p(wslot), _p(w_home), _p(pool))
    return pool


def expert_gemm(R, E, S, K, pl: Plan, wslot, in_dim, out_dim, x, w_home, pool, w_stride,
                w_offset=0, rows=None, x_compact=False):
    """y [len(rows), out_dim] bf16 bits: one projection of the listed buffer rows
    (all R*S*K rows if rows is None) by their segment's weight matrix.  With
    x_compact, x holds only the listed rows, in order."""
    x = _c(x, np.uint16)
    w_home = _c(w_home, np.uint16)
    pool = _c(pool, np.uint16) if pool is not None and np.size(pool) else np.zeros(1, np.uint16)
    wslot = _c(wslot, np.int32)
    rows = np.arange(R * S * K, dtype=np.int64) if rows is None else _c(rows, np.int64)
    y = np.empty((rows.size, out_dim), dtype=np.uint16)
    c = _cplan_from(pl)
    lib().orc_expert_gemm_rows(R, E, S, K, ctypes.byref(c), _p(wslot), in_dim, out_dim, _p(x),
                               _p(w_home), _p(pool), w_stride, w_offset, rows.size, _p(rows),
                               int(bool(x_compact)), _p(y))
    return y


def row_expert(topk, src_of_slot):
    """Expert served by each dispatch-buffer row (the expert of the entry placed there)."""
    return np.asarray(topk, dtype=np.int32)[np.asarray(src_of_slot, dtype=np.int64)]
