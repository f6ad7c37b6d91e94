"""Seeded synthetic inputs for the balanced expert-parallel path.

This package draws the inputs that the CPU oracle and the GPU library both
consume: router top-K expert ids, gate weights, bf16 activations, fp32
gradients and the per-expert scale of the stand-in expert.  It holds none of
the method's arithmetic.  The heavy lifting is in ``synth.c`` (counter-based
SplitMix64 streams), built here with gcc into ``libsynth.so``.

Workload presets follow the five synthetic configurations of the benchmark
plan: a tiny forward, a maxvio sweep, a DeepSeek-V3-like shape, an
adversarial all-to-one-rank routing and the backward at the DeepSeek-V3-like
shape.  No public dataset is involved; every array is synthetic.
"""
from __future__ import annotations

import ctypes
import json
import os
import subprocess
from dataclasses import dataclass, replace

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_BUILT = os.path.join(_HERE, "libsynth.so")
# A sanitizer build may be loaded instead, by the sanitizer test only.
_LIB = os.environ.get("MOONEP_SYNTH_LIB") or _BUILT

# Stream tags (xor-ed into the per-seed key).
TAG_PERM, TAG_ROUTE, TAG_LOGIT, TAG_X, TAG_DY, TAG_GRAD_REP, TAG_GRAD_HOME = 1, 2, 3, 4, 5, 6, 7
TAG_WEIGHT = 8  # expert weights (bf16 N(0,1)), for the prefetch
TAG_EXPERT_OUT = 9  # signed expert-output rows (bf16 N(0,1)), for combine
TAG_SIGNED_GATE = 10  # signed fp32 N(0,1) gates, for combine under cancellation


def build(verbose: bool = False) -> str:
    """Compile libsynth.so with gcc (OpenMP; results do not depend on threads)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", _SRC, "-o", _BUILT, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    return _BUILT


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            raise RuntimeError(f"{_LIB} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(_LIB)
        u64, i64, i32, f64, p = (ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32,
                                 ctypes.c_double, ctypes.c_void_p)
        L.synth_key.restype = u64
        L.synth_key.argtypes = [u64, u64]
        for name in ("synth_u64", "synth_uniform", "synth_normal_f64", "synth_normal_bf16"):
            getattr(L, name).restype = None
            getattr(L, name).argtypes = [u64, u64, i64, p]
        L.synth_normal_f32.restype = None
        L.synth_normal_f32.argtypes = [u64, u64, i64, f64, p]
        L.synth_permutation.restype = None
        L.synth_permutation.argtypes = [u64, i32, p]
        L.synth_zipf_topk.restype = ctypes.c_int
        L.synth_zipf_topk.argtypes = [u64, i64, i32, i32, f64, p]
        L.synth_balanced_topk.restype = ctypes.c_int
        L.synth_balanced_topk.argtypes = [i64, i32, i32, p]
        L.synth_fixed_topk.restype = None
        L.synth_fixed_topk.argtypes = [i64, i32, p]
        L.synth_softmax_gates.restype = None
        L.synth_softmax_gates.argtypes = [u64, i64, i32, p]
        L.synth_fill_f32.restype = None
        L.synth_fill_f32.argtypes = [i64, ctypes.c_float, p]
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def key(seed: int, tag: int) -> int:
    return int(lib().synth_key(seed, tag))


def u64(seed: int, tag: int, n: int, start: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.uint64)
    lib().synth_u64(key(seed, tag), start, n, _ptr(out))
    return out


def uniform(seed: int, tag: int, n: int, start: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.float64)
    lib().synth_uniform(key(seed, tag), start, n, _ptr(out))
    return out


def normal_f64(seed: int, tag: int, n: int, start: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.float64)
    lib().synth_normal_f64(key(seed, tag), start, n, _ptr(out))
    return out


def normal_bf16_into(out: np.ndarray, seed: int, tag: int, start: int = 0) -> np.ndarray:
    """Fill a C-contiguous uint16 array with bf16 bits of N(0,1)."""
    assert out.dtype == np.uint16
    lib().synth_normal_bf16(key(seed, tag), start, out.size, _ptr(out))
    return out


def normal_bf16(seed: int, tag: int, n: int, start: int = 0) -> np.ndarray:
    return normal_bf16_into(np.empty(n, dtype=np.uint16), seed, tag, start)


def normal_f32_into(out: np.ndarray, seed: int, tag: int, std: float, start: int = 0) -> np.ndarray:
    assert out.dtype == np.float32
    lib().synth_normal_f32(key(seed, tag), start, out.size, float(std), _ptr(out))
    return out


def normal_f32(seed: int, tag: int, n: int, std: float = 1.0, start: int = 0) -> np.ndarray:
    return normal_f32_into(np.empty(n, dtype=np.float32), seed, tag, std, start)


def permutation(seed: int, E: int) -> np.ndarray:
    out = np.empty(E, dtype=np.int32)
    lib().synth_permutation(key(seed, TAG_PERM), E, _ptr(out))
    return out


def zipf_topk(seed: int, N: int, E: int, K: int, alpha: float) -> np.ndarray:
    out = np.empty(N * K, dtype=np.int32)
    rc = lib().synth_zipf_topk(seed, N, E, K, float(alpha), _ptr(out))
    if rc != 0:
        raise ValueError("zipf_topk: need 1 <= K <= E <= 65536")
    return out


def balanced_topk(N: int, E: int, K: int) -> np.ndarray:
    out = np.empty(N * K, dtype=np.int32)
    if lib().synth_balanced_topk(N, E, K, _ptr(out)) != 0:
        raise ValueError("balanced_topk: need E % K == 0")
    return out


def fixed_topk(N: int, K: int) -> np.ndarray:
    out = np.empty(N * K, dtype=np.int32)
    lib().synth_fixed_topk(N, K, _ptr(out))
    return out


def softmax_gates(seed: int, N: int, K: int) -> np.ndarray:
    out = np.empty(N * K, dtype=np.float32)
    lib().synth_softmax_gates(seed, N, K, _ptr(out))
    return out


def fill_f32(n: int, v: float) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    lib().synth_fill_f32(n, float(v), _ptr(out))
    return out


def expert_scale(E: int) -> np.ndarray:
    """Stand-in expert: expert e multiplies its rows by fp32(1 + e/E)."""
    return np.array([np.float32(1.0 + e / E) for e in range(E)], dtype=np.float32)


# ---------------------------------------------------------------------------
# Workload presets
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class Workload:
    name: str
    R: int          # logical ranks
    E: int          # experts (home rank of e is e div (E/R))
    S: int          # tokens per rank
    K: int          # top-k
    H: int          # hidden size (bf16 row = 2H bytes)
    routing: str    # "zipf" | "balanced" | "fixed"
    alpha: float = 1.0
    gates: str = "softmax"   # "softmax" | "uniform"
    G: int = 0      # elements per expert weight-gradient (backward reduce)
    maxvio_target: float | None = None

    @property
    def N(self) -> int:
        return self.R * self.S

    @property
    def NK(self) -> int:
        return self.R * self.S * self.K

    @property
    def C(self) -> int:
        return self.S * self.K


# Expert FFN width for the 64-expert, 2048-hidden sweep shape is not stated by
# the workload; 1408 is the published width of a 64-expert MoE with hidden 2048
# and serves only to size the expert weights (gate, up and down: 3 x 2048 x
# 1408 bf16, for the prefetch) and their gradients (the backward reduce).
SWEEP_FFN = 1408
# The DeepSeek-V3-like expert weight-gradient: 7168 x 2048.
DSV3_G = 7168 * 2048

WORKLOADS = {
    "tiny": Workload("tiny", 4, 16, 128, 2, 64, "zipf", alpha=1.0, G=64 * 32),
    "sweep": Workload("sweep", 8, 64, 4096, 8, 2048, "zipf", G=2048 * SWEEP_FFN),
    "dsv3": Workload("dsv3", 32, 256, 4096, 8, 7168, "zipf", alpha=1.2, G=DSV3_G),
    "adversarial": Workload("adversarial", 16, 128, 8192, 8, 4096, "fixed", gates="uniform",
                            G=4096 * 2048),
    "dsv3_bwd": Workload("dsv3_bwd", 32, 256, 4096, 8, 7168, "zipf", alpha=1.2, G=DSV3_G),
}

SWEEP_LEVELS = (0.0, 0.5, 1.0, 2.0, 4.0)
_ALPHA_TABLE = os.path.join(os.path.dirname(_HERE), "tests", "golden", "sweep_alpha.json")


def sweep_alpha(seed: int, level: float) -> float:
    """Zipf exponent that reaches the given maxvio on the sweep shape.

    The table is written by tests/golden/make_sweep_alpha.py (bisection on
    alpha, counting with the CPU oracle).  Level 0 uses the balanced routing.
    """
    with open(_ALPHA_TABLE) as f:
        table = json.load(f)
    return float(table[str(seed)][f"{level:g}"]["alpha"])


def sweep_workload(level: float, seed: int = 0) -> Workload:
    w = WORKLOADS["sweep"]
    if level == 0.0:
        return replace(w, name=f"sweep_mv{level:g}", routing="balanced", maxvio_target=0.0)
    return replace(w, name=f"sweep_mv{level:g}", alpha=sweep_alpha(seed, level), maxvio_target=level)


def routing(w: Workload, seed: int) -> tuple[np.ndarray, np.ndarray]:
    """(topk int32 [N*K], gates f32 [N*K]) for a workload."""
    if w.routing == "zipf":
        topk = zipf_topk(seed, w.N, w.E, w.K, w.alpha)
    elif w.routing == "balanced":
        topk = balanced_topk(w.N, w.E, w.K)
    elif w.routing == "fixed":
        topk = fixed_topk(w.N, w.K)
    else:
        raise ValueError(w.routing)
    if w.gates == "softmax":
        gates = softmax_gates(seed, w.N, w.K)
    else:
        gates = fill_f32(w.N * w.K, 1.0 / w.K)
    return topk, gates


def expert_weights(E: int, wbytes: int, seed: int) -> np.ndarray:
    """[E, wbytes] uint8: every expert's weights as bf16 bits of N(0,1), one
    stream over all experts (a row is one expert's gate, up and down)."""
    assert wbytes % 2 == 0
    return normal_bf16(seed, TAG_WEIGHT, E * (wbytes // 2)).view(np.uint8).reshape(E, wbytes)


def activations(w: Workload, seed: int, tag: int = TAG_X) -> np.ndarray:
    """bf16 bits [N, H] of N(0,1) (tag TAG_X for x, TAG_DY for dy)."""
    return normal_bf16(seed, tag, w.N * w.H).reshape(w.N, w.H)
