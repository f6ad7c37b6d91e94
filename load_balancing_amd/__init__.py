"""Python binding of libmoonep, the gfx950 balanced expert-parallel hot path.

Thin ctypes marshalling over the C-ABI in include/moonep.h: every function
here has the name of the C entry point it calls, checks that the tensors it
is given match the shape (device, dtype, size, contiguity) and passes their
device pointers and the stream on.  All work runs in the HIP kernels of
libmoonep.so; there is no other implementation.  PyTorch supplies device
memory and streams only.

If libmoonep.so is not built, importing works but the first call raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoonep.so")

MOONEP_OK = 0
ERRORS = {
    -1: "MOONEP_ERR_INVALID_SHAPE", -2: "MOONEP_ERR_NULL_PTR", -3: "MOONEP_ERR_MISALIGNED",
    -4: "MOONEP_ERR_WORKSPACE", -5: "MOONEP_ERR_HIP", -6: "MOONEP_ERR_ALIAS", -7: "MOONEP_ERR_ARG",
}
DEV_OK, DEV_BAD_EXPERT_ID = 0, 1
PLAN_HEADER = {"n_rep": 0, "n_spill": 1, "n_deficit": 2, "max_rep_rank": 3, "tmax": 4,
               "C": 5, "L": 6, "cap": 7}

EXPORTS = ("moonep_check_shape", "moonep_workspace_bytes", "moonep_plan_layout_of",
           "moonep_plan_bytes", "moonep_route_stats", "moonep_plan", "moonep_dispatch",
           "moonep_combine", "moonep_combine_bwd", "moonep_dispatch_bwd",
           "moonep_replica_grad_reduce", "moonep_weight_slots", "moonep_prefetch_weights",
           "moonep_expert_gemm", "moonep_read_error", "moonep_plan_largest_first",
           "moonep_plan_noalloc")


class MoonepError(RuntimeError):
    def __init__(self, what: str, code: int):
        super().__init__(f"{what}: {ERRORS.get(code, code)}")
        self.code = code


class Shape(ctypes.Structure):
    _fields_ = [("R", ctypes.c_int32), ("E", ctypes.c_int32), ("S", ctypes.c_int32),
                ("K", ctypes.c_int32), ("H", ctypes.c_int32)]

    @property
    def N(self):
        return self.R * self.S

    @property
    def NK(self):
        return self.R * self.S * self.K

    @property
    def C(self):
        return self.S * self.K

    def __repr__(self):
        return f"Shape(R={self.R}, E={self.E}, S={self.S}, K={self.K}, H={self.H})"


class PlanLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "words", "cap", "header", "rep_expert", "rep_host", "rep_count", "rep_spill_off",
        "rep_row_off", "spill", "keep", "home_row_off", "rep_first", "rep_cnt", "exp_rep_list",
        "load", "rank_rep_first", "rank_rep_cnt")]


_lib = None


def lib():
    """The loaded libmoonep.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m load_balancing_amd.build` (there is no fallback)")
        L = ctypes.CDLL(LIB_PATH)
        P, VP, SZ, I64 = ctypes.POINTER(Shape), ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int64
        sig = {
            "moonep_check_shape": (ctypes.c_int, [P]),
            "moonep_workspace_bytes": (SZ, [P]),
            "moonep_plan_layout_of": (ctypes.c_int, [P, ctypes.POINTER(PlanLayout)]),
            "moonep_plan_bytes": (SZ, [P]),
            "moonep_route_stats": (ctypes.c_int, [P, VP, VP, VP, VP, SZ, VP]),
            "moonep_plan": (ctypes.c_int, [P, VP, VP, VP, SZ, VP, VP, VP, VP]),
            "moonep_plan_largest_first": (ctypes.c_int, [P, VP, VP, VP, SZ, VP, VP, VP, VP]),
            "moonep_dispatch": (ctypes.c_int, [P, VP, VP, VP, VP]),
            "moonep_combine": (ctypes.c_int, [P, VP, VP, VP, VP, VP]),
            "moonep_combine_bwd": (ctypes.c_int, [P, VP, VP, VP, VP, VP, VP, VP]),
            "moonep_dispatch_bwd": (ctypes.c_int, [P, VP, VP, VP, VP]),
            "moonep_replica_grad_reduce": (ctypes.c_int, [P, VP, I64, VP, VP, VP]),
            "moonep_weight_slots": (ctypes.c_int, [P, VP, ctypes.c_int32, VP, VP]),
            "moonep_prefetch_weights": (ctypes.c_int, [P, VP, VP, ctypes.c_int32, I64, VP, VP, VP]),
            "moonep_expert_gemm": (ctypes.c_int, [P, VP, VP, ctypes.c_int32, ctypes.c_int32,
                                                  ctypes.c_int32, VP, VP, VP, I64, I64, VP, VP]),
            "moonep_read_error": (ctypes.c_int, [VP, SZ, ctypes.POINTER(ctypes.c_int32), VP]),
            "moonep_plan_noalloc": (ctypes.c_int, [P, VP, VP, VP, VP, VP, VP, VP]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(rc: int, what: str):
    if rc != MOONEP_OK:
        raise MoonepError(what, rc)


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


_BF16_OK = ("bfloat16", "int16", "uint16")


def _dev(t, what, numel, kinds):
    """Device pointer of tensor t after checking device, dtype, size, layout."""
    if t is None:
        if numel == 0:
            return None
        raise MoonepError(what, -2)
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError(f"{what}: tensor must be on a GPU")
    if str(t.dtype).replace("torch.", "") not in kinds:
        raise ValueError(f"{what}: dtype {t.dtype} not in {kinds}")
    if not t.is_contiguous():
        raise ValueError(f"{what}: tensor must be contiguous")
    if t.numel() != numel:
        raise ValueError(f"{what}: has {t.numel()} elements, needs {numel}")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return _torch().cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _nbytes(t):
    return t.numel() * t.element_size()


# ---------------------------------------------------------------------------
# the C-ABI, one Python function per entry point
# ---------------------------------------------------------------------------

def moonep_check_shape(shape: Shape) -> int:
    return lib().moonep_check_shape(ctypes.byref(shape))


def moonep_workspace_bytes(shape: Shape) -> int:
    return lib().moonep_workspace_bytes(ctypes.byref(shape))


def moonep_plan_bytes(shape: Shape) -> int:
    return lib().moonep_plan_bytes(ctypes.byref(shape))


def moonep_plan_layout_of(shape: Shape) -> PlanLayout:
    lay = PlanLayout()
    _check(lib().moonep_plan_layout_of(ctypes.byref(shape), ctypes.byref(lay)),
           "moonep_plan_layout_of")
    return lay


def moonep_route_stats(shape, topk_idx, expert_counts, maxvio, workspace, stream=None):
    _check(lib().moonep_route_stats(
        ctypes.byref(shape), _dev(topk_idx, "topk_idx", shape.NK, ("int32",)),
        _dev(expert_counts, "expert_counts", shape.E, ("int32",)),
        _dev(maxvio, "maxvio", 1, ("float32",)),
        _dev(workspace, "workspace", workspace.numel(), ("uint8",)), _nbytes(workspace),
        _stream(stream)), "moonep_route_stats")


def moonep_plan(shape, topk_idx, expert_counts, workspace, plan, slot_of, src_of_slot, stream=None):
    _check(lib().moonep_plan(
        ctypes.byref(shape), _dev(topk_idx, "topk_idx", shape.NK, ("int32",)),
        _dev(expert_counts, "expert_counts", shape.E, ("int32",)),
        _dev(workspace, "workspace", workspace.numel(), ("uint8",)), _nbytes(workspace),
        _dev(plan, "plan", moonep_plan_bytes(shape) // 4, ("int32",)),
        _dev(slot_of, "slot_of", shape.NK, ("int32",)),
        _dev(src_of_slot, "src_of_slot", shape.NK, ("int32",)), _stream(stream)), "moonep_plan")


def moonep_plan_largest_first(shape, topk_idx, expert_counts, workspace, plan, slot_of,
                              src_of_slot, stream=None):
    _check(lib().moonep_plan_largest_first(
        ctypes.byref(shape), _dev(topk_idx, "topk_idx", shape.NK, ("int32",)),
        _dev(expert_counts, "expert_counts", shape.E, ("int32",)),
        _dev(workspace, "workspace", workspace.numel(), ("uint8",)), _nbytes(workspace),
        _dev(plan, "plan", moonep_plan_bytes(shape) // 4, ("int32",)),
        _dev(slot_of, "slot_of", shape.NK, ("int32",)),
        _dev(src_of_slot, "src_of_slot", shape.NK, ("int32",)), _stream(stream)),
        "moonep_plan_largest_first")


def moonep_plan_noalloc(shape, topk_idx, expert_counts, maxvio, plan, slot_of, src_of_slot,
                        stream=None):
    _check(lib().moonep_plan_noalloc(
        ctypes.byref(shape), _dev(topk_idx, "topk_idx", shape.NK, ("int32",)),
        _dev(expert_counts, "expert_counts", shape.E, ("int32",)),
        _dev(maxvio, "maxvio", 1, ("float32",)),
        _dev(plan, "plan", moonep_plan_bytes(shape) // 4, ("int32",)),
        _dev(slot_of, "slot_of", shape.NK, ("int32",)),
        _dev(src_of_slot, "src_of_slot", shape.NK, ("int32",)), _stream(stream)),
        "moonep_plan_noalloc")


def moonep_dispatch(shape, x, slot_of, buf, stream=None):
    _check(lib().moonep_dispatch(
        ctypes.byref(shape), _dev(x, "x", shape.N * shape.H, _BF16_OK),
        _dev(slot_of, "slot_of", shape.NK, ("int32",)),
        _dev(buf, "buf", shape.NK * shape.H, _BF16_OK), _stream(stream)), "moonep_dispatch")


def moonep_combine(shape, expert_out, gates, slot_of, y, stream=None):
    _check(lib().moonep_combine(
        ctypes.byref(shape), _dev(expert_out, "expert_out", shape.NK * shape.H, _BF16_OK),
        _dev(gates, "gates", shape.NK, ("float32",)),
        _dev(slot_of, "slot_of", shape.NK, ("int32",)),
        _dev(y, "y", shape.N * shape.H, _BF16_OK), _stream(stream)), "moonep_combine")


def moonep_combine_bwd(shape, dy, expert_out, gates, slot_of, d_out, d_gates, stream=None):
    _check(lib().moonep_combine_bwd(
        ctypes.byref(shape), _dev(dy, "dy", shape.N * shape.H, _BF16_OK),
        _dev(expert_out, "expert_out", shape.NK * shape.H, _BF16_OK),
        _dev(gates, "gates", shape.NK, ("float32",)),
        _dev(slot_of, "slot_of", shape.NK, ("int32",)),
        _dev(d_out, "d_out", shape.NK * shape.H, _BF16_OK),
        _dev(d_gates, "d_gates", shape.NK, ("float32",)), _stream(stream)), "moonep_combine_bwd")


def moonep_dispatch_bwd(shape, d_buf, slot_of, dx, stream=None):
    _check(lib().moonep_dispatch_bwd(
        ctypes.byref(shape), _dev(d_buf, "d_buf", shape.NK * shape.H, _BF16_OK),
        _dev(slot_of, "slot_of", shape.NK, ("int32",)),
        _dev(dx, "dx", shape.N * shape.H, _BF16_OK), _stream(stream)), "moonep_dispatch_bwd")


def moonep_replica_grad_reduce(shape, plan, G, home_grads, replica_grads, stream=None):
    _check(lib().moonep_replica_grad_reduce(
        ctypes.byref(shape), _dev(plan, "plan", moonep_plan_bytes(shape) // 4, ("int32",)),
        int(G), _dev(home_grads, "home_grads", shape.E * G, ("float32",)),
        _dev(replica_grads, "replica_grads", (shape.E + shape.R) * G, ("float32",)),
        _stream(stream)), "moonep_replica_grad_reduce")


def moonep_weight_slots(shape, plan, B, wslot, stream=None):
    _check(lib().moonep_weight_slots(
        ctypes.byref(shape), _dev(plan, "plan", moonep_plan_bytes(shape) // 4, ("int32",)),
        int(B), _dev(wslot, "wslot", shape.E + shape.R, ("int32",)), _stream(stream)),
        "moonep_weight_slots")


def _dev_bytes(t, what, nbytes):
    """Device pointer of a contiguous tensor of any dtype holding exactly nbytes."""
    if t is None:
        if nbytes == 0:
            return None
        raise MoonepError(what, -2)
    if not t.is_cuda:
        raise ValueError(f"{what}: tensor must be on a GPU")
    if not t.is_contiguous():
        raise ValueError(f"{what}: tensor must be contiguous")
    if _nbytes(t) != nbytes:
        raise ValueError(f"{what}: has {_nbytes(t)} bytes, needs {nbytes}")
    return t.data_ptr()


def moonep_prefetch_weights(shape, plan, wslot, B, wbytes, w_home, pool, stream=None):
    """pool [R*B, wbytes] gets each slotted replica's row of w_home [E, wbytes]."""
    _check(lib().moonep_prefetch_weights(
        ctypes.byref(shape), _dev(plan, "plan", moonep_plan_bytes(shape) // 4, ("int32",)),
        _dev(wslot, "wslot", shape.E + shape.R, ("int32",)), int(B), int(wbytes),
        _dev_bytes(w_home, "w_home", shape.E * wbytes),
        _dev_bytes(pool, "pool", shape.R * B * wbytes), _stream(stream)),
        "moonep_prefetch_weights")


def moonep_expert_gemm(shape, plan, wslot, B, in_dim, out_dim, x, w_home, pool, w_stride,
                       w_offset, y, stream=None):
    """y [R*S*K, out_dim] = each buffer row of x [R*S*K, in_dim] times its
    segment's weights; w_home [E, w_stride] and pool [R*B, w_stride] bf16."""
    _check(lib().moonep_expert_gemm(
        ctypes.byref(shape), _dev(plan, "plan", moonep_plan_bytes(shape) // 4, ("int32",)),
        _dev(wslot, "wslot", shape.E + shape.R, ("int32",)), int(B), int(in_dim), int(out_dim),
        _dev(x, "x", shape.NK * in_dim, _BF16_OK),
        _dev_bytes(w_home, "w_home", shape.E * w_stride * 2),
        _dev_bytes(pool, "pool", shape.R * B * w_stride * 2), int(w_stride), int(w_offset),
        _dev(y, "y", shape.NK * out_dim, _BF16_OK), _stream(stream)), "moonep_expert_gemm")


def moonep_read_error(workspace, stream=None) -> int:
    code = ctypes.c_int32(0)
    _check(lib().moonep_read_error(_dev(workspace, "workspace", workspace.numel(), ("uint8",)),
                                   _nbytes(workspace), ctypes.byref(code), _stream(stream)),
           "moonep_read_error")
    return code.value


# ---------------------------------------------------------------------------
# static buffers of one MoE layer (allocated once; sizes depend on the shape only)
# ---------------------------------------------------------------------------

@dataclass
class Buffers:
    shape: Shape
    workspace: object      # uint8 [moonep_workspace_bytes], zeroed once
    expert_counts: object  # int32 [E]
    maxvio: object         # fp32 [1]
    plan: object           # int32 [moonep_plan_bytes / 4]
    slot_of: object        # int32 [R*S*K]
    src_of_slot: object    # int32 [R*S*K]
    buf: object            # bf16 [R*S*K, H]: the R per-rank [S*K, H] buffers

    def plan_fields(self) -> dict:
        """Plan table as named host int arrays (reads the device)."""
        lay = moonep_plan_layout_of(self.shape)
        p = self.plan.cpu().numpy()
        E, R, cap = self.shape.E, self.shape.R, lay.cap
        sizes = {"rep_expert": cap, "rep_host": cap, "rep_count": cap, "rep_spill_off": cap,
                 "rep_row_off": cap, "spill": E, "keep": E, "home_row_off": E, "rep_first": E,
                 "rep_cnt": E, "exp_rep_list": E, "load": R, "rank_rep_first": R,
                 "rank_rep_cnt": R}
        out = {k: p[getattr(lay, k):getattr(lay, k) + n] for k, n in sizes.items()}
        out.update({k: int(p[lay.header + i]) for k, i in PLAN_HEADER.items()})
        return out


def allocate(shape: Shape, device="cuda") -> Buffers:
    torch = _torch()
    _check(moonep_check_shape(shape), "allocate")
    ws = torch.zeros(moonep_workspace_bytes(shape), dtype=torch.uint8, device=device)
    return Buffers(
        shape=shape, workspace=ws,
        expert_counts=torch.empty(shape.E, dtype=torch.int32, device=device),
        maxvio=torch.empty(1, dtype=torch.float32, device=device),
        plan=torch.empty(moonep_plan_bytes(shape) // 4, dtype=torch.int32, device=device),
        slot_of=torch.empty(shape.NK, dtype=torch.int32, device=device),
        src_of_slot=torch.empty(shape.NK, dtype=torch.int32, device=device),
        buf=torch.empty((shape.NK, shape.H), dtype=torch.bfloat16, device=device),
    )


def plan_step(b: Buffers, topk_idx, stream=None, largest_first=False):
    """route_stats then plan (moonep_plan, or moonep_plan_largest_first):
    counts, maxvio, the plan and both slot maps."""
    moonep_route_stats(b.shape, topk_idx, b.expert_counts, b.maxvio, b.workspace, stream)
    planner = moonep_plan_largest_first if largest_first else moonep_plan
    planner(b.shape, topk_idx, b.expert_counts, b.workspace, b.plan, b.slot_of, b.src_of_slot,
            stream)
