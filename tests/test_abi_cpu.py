"""The C-ABI library loads, exports what include/moonep.h declares, and
validates arguments on the host (CPU only: no call here reaches the GPU)."""
import ctypes
import os
import re

import pytest

import load_balancing_amd as mx

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(mx.LIB_PATH):
        from load_balancing_amd import build
        build.build()
    return mx.lib()


def header_functions():
    src = open(os.path.join(ROOT, "include", "moonep.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moonep_[a-z_0-9]+)\s*\(", src)))


def test_exports_every_declared_function(L):
    names = header_functions()
    assert set(names) == set(mx.EXPORTS)
    for n in names:
        assert hasattr(L, n), n


def test_shape_rules(L):
    ok = mx.Shape(4, 16, 128, 2, 64)
    assert mx.moonep_check_shape(ok) == 0
    bad = [mx.Shape(3, 16, 128, 2, 64),     # E % R
           mx.Shape(4, 16, 128, 17, 64),    # K > E
           mx.Shape(4, 16, 128, 0, 64),     # K < 1
           mx.Shape(4, 16, 128, 2, 60),     # H % 8
           mx.Shape(4, 16, -1, 2, 64),      # S < 0
           mx.Shape(0, 16, 128, 2, 64),     # R < 1
           mx.Shape(2, 2048, 128, 2, 64),   # E above the on-chip plan limit
           mx.Shape(1024, 1024, 1 << 20, 2, 64)]  # R*S*K >= 2^31, R above limit
    for s in bad:
        assert mx.moonep_check_shape(s) == -1, s
        assert mx.moonep_workspace_bytes(s) == 0
        assert mx.moonep_plan_bytes(s) == 0
    assert mx.moonep_check_shape(mx.Shape(8, 64, (1 << 31) // 64, 8, 64)) == -1
    assert mx.moonep_check_shape(mx.Shape(4, 16, 0, 2, 64)) == 0     # empty is valid


def test_sizes_depend_on_shape_only(L):
    s = mx.Shape(32, 256, 4096, 8, 7168)
    lay = mx.moonep_plan_layout_of(s)
    assert lay.cap == 256 + 32
    assert lay.words == 16 + 5 * lay.cap + 6 * 256 + 3 * 32
    assert mx.moonep_plan_bytes(s) == lay.words * 4
    offs = sorted(getattr(lay, f) for f, _ in mx.PlanLayout._fields_ if f not in ("words", "cap"))
    assert offs[0] == 0 and len(set(offs)) == len(offs)
    ws = mx.moonep_workspace_bytes(s)
    assert ws % 256 == 0 and ws >= 256 + 256 * 4


def test_workspace_holds_the_wave_segments(L):
    """The workspace is a 256-byte control block plus E * nseg int32 counts,
    rounded up to 256 bytes.  Entries are cut into segments whose width is a
    multiple of 64 entries; the count aims at NK/512 within [1024, 2048], so
    the sweep's 262,144 entries take 1024 segments of 256 and the
    1M-entry shapes 2048 of 512."""
    cases = [
        # (R, E, S, K, expected nseg)
        (8, 64, 4096, 8, 1024),      # 262,144 entries: 256 each
        (32, 256, 4096, 8, 2048),    # 1,048,576: 512 each
        (16, 128, 8192, 8, 2048),    # 1,048,576
        (4, 16, 128, 2, 16),         # 1,024 entries: the 64-entry floor
        (8, 64, 1000, 8, 1000),      # 64,000: 64 each
        (16, 64, 9500, 8, 1900),     # 1,216,000: 640 each
        (4, 16, 0, 2, 0),            # empty
    ]
    for R, E, S, K, nseg in cases:
        s = mx.Shape(R, E, S, K, 64)
        want = 256 + (E * nseg * 4 + 255) // 256 * 256
        assert mx.moonep_workspace_bytes(s) == want, (R, E, S, K)


def test_host_errors_before_any_launch(L):
    s = mx.Shape(4, 16, 128, 2, 64)
    vp = ctypes.c_void_p
    B = ctypes.byref
    wsb = mx.moonep_workspace_bytes(s)
    fake = 0x100000  # never dereferenced: every call below fails validation first
    # null pointers
    assert L.moonep_route_stats(B(s), None, vp(fake), vp(fake), vp(fake), wsb, None) == -2
    assert L.moonep_dispatch(B(s), vp(fake), None, vp(fake), None) == -2
    # misalignment of a bf16 buffer
    assert L.moonep_dispatch(B(s), vp(fake + 2), vp(fake), vp(fake * 4), None) == -3
    # short workspace
    assert L.moonep_route_stats(B(s), vp(fake), vp(fake), vp(fake), vp(fake), wsb - 1, None) == -4
    assert L.moonep_plan(B(s), vp(fake), vp(fake), vp(fake), 16, vp(fake), vp(fake * 2),
                         vp(fake * 3), None) == -4
    # overlapping dispatch source and destination
    assert L.moonep_dispatch(B(s), vp(fake), vp(fake * 8), vp(fake + 4096), None) == -6
    # overlapping combine output and input
    assert L.moonep_combine(B(s), vp(fake), vp(fake * 8), vp(fake * 9), vp(fake + 1024), None) == -6
    # negative G, overlapping gradient arrays
    assert L.moonep_replica_grad_reduce(B(s), vp(fake), ctypes.c_int64(-1), vp(fake), vp(fake * 2),
                                        None) == -7
    assert L.moonep_replica_grad_reduce(B(s), vp(fake), ctypes.c_int64(64), vp(fake),
                                        vp(fake + 64), None) == -6
    # dispatch backward: null, misaligned, overlapping dx and d_buf
    assert L.moonep_dispatch_bwd(B(s), None, vp(fake), vp(fake * 8), None) == -2
    assert L.moonep_dispatch_bwd(B(s), vp(fake), vp(fake * 8), vp(fake * 16 + 8), None) == -3
    assert L.moonep_dispatch_bwd(B(s), vp(fake), vp(fake * 8), vp(fake + 4096), None) == -6
    # weight slots: negative B, null output
    assert L.moonep_weight_slots(B(s), vp(fake), -1, vp(fake * 2), None) == -7
    assert L.moonep_weight_slots(B(s), vp(fake), 2, None, None) == -2
    # prefetch: wbytes not whole 16-byte vectors, misaligned pool, overlap
    i64 = ctypes.c_int64
    assert L.moonep_prefetch_weights(B(s), vp(fake), vp(fake * 2), 2, i64(24), vp(fake * 4),
                                     vp(fake * 8), None) == -7
    assert L.moonep_prefetch_weights(B(s), vp(fake), vp(fake * 2), 2, i64(32), vp(fake * 4),
                                     vp(fake * 8 + 4), None) == -3
    assert L.moonep_prefetch_weights(B(s), vp(fake), vp(fake * 2), 2, i64(32), vp(fake * 4),
                                     vp(fake * 4 + 256), None) == -6
    assert L.moonep_prefetch_weights(B(s), vp(fake), vp(fake * 2), 2, i64(32), None,
                                     vp(fake * 8), None) == -2
    # expert GEMM: dimension rules, weight window past the row, null, misaligned, overlap
    g = lambda kin, kout, x, y, w_stride=i64(128 * 64), w_off=i64(0), wh=vp(fake * 4): \
        L.moonep_expert_gemm(B(s), vp(fake), vp(fake * 2), 2, kin, kout, x, wh, vp(fake * 8),
                             w_stride, w_off, y, None)
    assert g(96, 128, vp(fake * 16), vp(fake * 32)) == -7          # in_dim % 64
    assert g(64, 192, vp(fake * 16), vp(fake * 32)) == -7          # out_dim % 128
    assert g((1 << 22) + 64, 128, vp(fake * 16), vp(fake * 32),
             w_stride=i64(((1 << 22) + 64) * 128)) == -7           # in_dim above 2^22
    assert g(64, 128, vp(fake * 16), vp(fake * 32), w_off=i64(8)) == -7  # window past the row
    assert g(64, 128, None, vp(fake * 32)) == -2
    assert g(64, 128, vp(fake * 16 + 8), vp(fake * 32)) == -3
    assert g(64, 128, vp(fake * 16), vp(fake * 16 + 64)) == -6     # y overlaps x
    # invalid shape is reported first
    bad = mx.Shape(3, 16, 128, 2, 64)
    assert L.moonep_dispatch(B(bad), vp(fake), vp(fake), vp(fake * 4), None) == -1
    assert L.moonep_read_error(None, 256, None, None) == -2


def test_binding_raises_without_library(tmp_path, monkeypatch):
    monkeypatch.setattr(mx, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(mx, "_lib", None)
    with pytest.raises(RuntimeError, match="no fallback"):
        mx.moonep_check_shape(mx.Shape(4, 16, 128, 2, 64))


def test_ceilings_library_loads_outside_the_c_abi():
    """bench.py --ceilings loads its own library; none of its symbols is part
    of libmoonep's C-ABI (CPU only: nothing is launched)."""
    from load_balancing_amd import build
    if not os.path.exists(build.CEIL_LIB):
        build.build()
    C = ctypes.CDLL(build.CEIL_LIB)
    for n in ("ceil_stream", "ceil_rows", "ceil_mfma", "ceil_mfma_chains", "ceil_lds_dma", "ceil_lds_dma_loads",
              "ceil_lds_dma_waves"):
        assert hasattr(C, n), n
    assert C.ceil_mfma_chains() > 0 and C.ceil_lds_dma_loads() > 0 and C.ceil_lds_dma_waves() > 0
    assert not any(n.startswith("ceil_") for n in mx.EXPORTS)
    # the stream entry checks its arguments before any launch
    VP, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    C.ceil_stream.argtypes = [VP, VP, I64, I, I, I, I, I, I, VP, VP]
    for mode, unroll, grid, block in ((3, 4, 1, 64), (0, 3, 1, 64), (0, 4, 0, 64), (0, 8, 1, 96)):
        assert C.ceil_stream(None, None, 16, mode, unroll, 1, 0, grid, block, None, None) == -1
    C.ceil_rows.argtypes = [VP, VP, VP, VP, I64, I, I, I, VP, VP]
    fake = ctypes.c_void_p(16)  # never dereferenced: every call below is refused first
    for s_, d_, row_vecs, block, sink in ((None, None, 256, 256, None), (fake, None, 256, 256, None),
                                          (fake, fake, 256, 128, None), (fake, fake, 192, 64, None),
                                          (fake, fake, 512, 256, None)):
        assert C.ceil_rows(s_, d_, None, None, 8, row_vecs, 1, block, sink, None) == -1
