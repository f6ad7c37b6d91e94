"""Host-side parts of the benchmark: its byte accounting and its refusals.

Every GB/s figure the benchmark prints is a call's algorithmic bytes (each
input read once, each output written once) over its measured time, so the
accounting is pinned here against totals worked out by hand from the shapes:
a change to a formula shows up as a wrong total.
"""
import json
import os
import subprocess
import sys

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def fwd_bytes(w):
    b = bench.algorithmic_bytes(w.R, w.S, w.K, w.H)
    return b["dispatch"] + b["combine"]


def test_forward_bytes_per_workload():
    # tiny: N = 512, NK = 1024, H = 64 -> 65,536 + 131,072 + 4,096 and
    # 131,072 + 65,536 + 8,192
    assert fwd_bytes(synth.WORKLOADS["tiny"]) == 405_504
    # sweep: N = 32,768, NK = 262,144, H = 2048
    b = bench.algorithmic_bytes(8, 4096, 8, 2048)
    assert b["dispatch"] == 134_217_728 + 1_073_741_824 + 1_048_576 == 1_209_008_128
    assert b["combine"] == 1_073_741_824 + 134_217_728 + 2_097_152 == 1_210_056_704
    assert b["dispatch_bwd"] == b["dispatch"]
    assert fwd_bytes(synth.WORKLOADS["sweep"]) == 2_419_064_832
    # DeepSeek-V3-like: N = 131,072, NK = 1,048,576, H = 7168
    assert fwd_bytes(synth.WORKLOADS["dsv3"]) == 33_835_450_368
    # adversarial: N = 131,072, NK = 1,048,576, H = 4096
    assert fwd_bytes(synth.WORKLOADS["adversarial"]) == 19_339_935_744


def test_combine_bwd_bytes():
    # dy once, expert outputs read, d_out written, slot_of + gates + d_gates
    w = synth.WORKLOADS["dsv3_bwd"]
    b = bench.algorithmic_bytes(w.R, w.S, w.K, w.H)
    assert b["combine_bwd"] == 1_879_048_192 + 2 * 15_032_385_536 + 12_582_912 == 31_956_402_176


def test_reduce_bytes_hand_example():
    # experts with 2, 1 and 0 replicas, G = 10 fp32 per row:
    #   expert 0: read 2 replica rows + read and write home = 4 rows, zero 2 rows
    #   expert 1: read 1 replica row + read and write home = 3 rows, zero 1 row
    #   expert 2: untouched
    b = bench.algorithmic_bytes(2, 4, 2, 8, G=10, reps=[2, 1, 0])
    assert b["replica_grad_reduce"] == (4 + 2 + 3 + 1) * 40
    assert bench.algorithmic_bytes(2, 4, 2, 8, G=10, reps=[0, 0])["replica_grad_reduce"] == 0


def test_every_workload_has_a_name():
    for wl in ("sweep", "dsv3", "adversarial", "tiny"):
        assert wl in bench.WORKLOAD_NAME and wl in synth.WORKLOADS


def run_bench(args, env=None):
    e = dict(os.environ)
    e.update(env or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, env=e, timeout=60)


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    r = run_bench(["--gpus", "2"])
    assert r.returncode == 2
    assert "one GPU" in json.loads(r.stdout.strip().splitlines()[-1])["error"]
    r = run_bench([], env={"WORLD_SIZE": "4"})
    assert r.returncode == 2
