"""The seeded input generator: determinism and the stated distributions (CPU)."""
import os
import subprocess
import sys

import numpy as np

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_counter_streams_are_random_access():
    a = synth.normal_bf16(7, synth.TAG_X, 1000)
    b = synth.normal_bf16(7, synth.TAG_X, 500, start=500)
    np.testing.assert_array_equal(a[500:], b)
    u = synth.u64(7, synth.TAG_X, 8)
    assert len(set(u.tolist())) == 8


def test_thread_count_does_not_change_results():
    code = ("import sys; sys.path.insert(0, %r); import synth, hashlib;"
            "w = synth.WORKLOADS['tiny']; t, g = synth.routing(w, 5);"
            "x = synth.normal_bf16(5, 4, 100000);"
            "print(hashlib.sha256(t.tobytes() + g.tobytes() + x.tobytes()).hexdigest())" % ROOT)
    outs = []
    for nt in ("1", "4"):
        env = dict(os.environ, OMP_NUM_THREADS=nt)
        outs.append(subprocess.run([sys.executable, "-c", code], env=env, check=True,
                                   capture_output=True, text=True).stdout)
    assert outs[0] == outs[1]


def test_normal_moments():
    z = synth.normal_f64(1, synth.TAG_X, 400000)
    assert abs(z.mean()) < 0.01 and abs(z.std() - 1) < 0.01
    g = synth.normal_f32(1, synth.TAG_GRAD_REP, 400000, 0.01)
    assert abs(g.std() - 0.01) < 1e-4


def test_zipf_routing_distinct_and_skewed():
    w = synth.WORKLOADS["dsv3"]
    topk = synth.zipf_topk(0, 4096, w.E, w.K, 1.2).reshape(4096, w.K)
    assert all(len(set(r)) == w.K for r in topk.tolist())
    assert topk.min() >= 0 and topk.max() < w.E
    counts = np.bincount(topk.ravel(), minlength=w.E)
    rank_of = synth.permutation(0, w.E)
    # more popular ranks receive more tokens (rank 0 vs rank 50)
    assert counts[np.argmin(rank_of)] > counts[np.where(rank_of == 50)[0][0]]


def test_gates_are_a_softmax():
    g = synth.softmax_gates(3, 1000, 8).reshape(1000, 8)
    assert (g > 0).all()
    np.testing.assert_allclose(g.sum(1), 1.0, atol=1e-6)


def test_fixed_and_balanced_routings():
    t = synth.fixed_topk(5, 8).reshape(5, 8)
    assert (t == np.arange(8)).all()
    b = synth.balanced_topk(128, 16, 4).reshape(128, 4)
    assert all(len(set(r)) == 4 for r in b.tolist())
    assert (np.bincount(b.ravel(), minlength=16) == 32).all()
