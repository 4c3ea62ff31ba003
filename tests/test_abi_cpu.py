"""The C ABI on a machine without a GPU: the library loads, exports every function that
include/gc.h declares, and every argument check returns its status before any HIP call.
Device pointers passed here are never dereferenced: each call fails validation first."""
import ctypes
import os
import re

import pytest

import two_point_angular_amd as gc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
                 if f.endswith(".h"))

OK, INVALID, UNSUPPORTED, WORKSPACE, DEVICE = 0, 1, 2, 3, 4
A = 4096  # a 256-aligned fake device address; never dereferenced
NO_GPU = not os.path.exists("/dev/kfd")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(gc.library_path()):
        from two_point_angular_amd import build
        build.build()
    return gc.load()


def header_functions(path):
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gc_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_function(lib):
    assert [os.path.basename(h) for h in HEADERS] == ["gc.h", "gc_diag.h", "gc_io.h", "gc_ladder.h"]
    names = [n for h in HEADERS for n in header_functions(h)]
    assert len(names) >= 16
    for name in names:
        assert hasattr(lib, name), name


def test_sizes(lib):
    assert lib.gc_prepared_bytes(-1) == 0
    assert lib.gc_prepared_bytes(0) == 64 * 36
    assert lib.gc_prepared_bytes(100) == (128 + 64) * 36
    assert lib.gc_prepared_bytes(gc.MAX_GALAXIES + 1) == 0
    assert lib.gc_prepared_bytes(10**5) % gc.ALIGNMENT == 0
    assert lib.gc_workspace_bytes(0) == 0
    assert lib.gc_workspace_bytes(gc.MAX_BINS + 1) == 0
    # the edge cosines and the bin table (up to 14337 8-byte entries), each 256-byte aligned
    assert lib.gc_workspace_bytes(720) == (721 * 8 + 255) // 256 * 256 + (14337 * 8 + 255) // 256 * 256
    assert lib.gc_workspace_bytes(gc.MAX_BINS) <= 256 * 1024  # fits the allocation-free call's scratch


def test_status_strings(lib):
    assert lib.gc_status_string(0) == b"ok"
    assert lib.gc_status_string(3) == b"workspace too small"
    assert lib.gc_status_string(5) == b"file input/output error"
    assert lib.gc_status_string(99) == b"unknown status"
    assert lib.gc_version().startswith(b"gc ")
    assert lib.gc_last_device_error() == 0


def test_prepare_validation(lib):
    P = ctypes.c_void_p
    assert lib.gc_prepare(None, None, -1, P(A), None) == INVALID
    assert lib.gc_prepare(P(A), P(A), gc.MAX_GALAXIES + 1, P(A), None) == UNSUPPORTED
    assert lib.gc_prepare(None, P(A), 5, P(A), None) == INVALID
    assert lib.gc_prepare(P(A), P(A), 5, None, None) == INVALID
    assert lib.gc_prepare(P(A), P(A), 5, P(A + 8), None) == INVALID      # misaligned blob
    assert lib.gc_prepare(None, None, 0, None, None) == OK               # empty, nothing enqueued


def _hist(lib, **kw):
    P = ctypes.c_void_p
    a = dict(pd=P(A), nd=10, pr=P(A), nr=10, nbins=720, w=0.25, dd=P(A), dr=P(A + 8192), rr=P(A + 16384),
             ws=P(A), wsb=gc.workspace_bytes(720) if kw.get("nbins", 720) in (720,) else 1 << 40, tuning=None)
    a.update(kw)
    if a["tuning"] is None:
        return lib.gc_histogram_dd_dr_rr(a["pd"], a["nd"], a["pr"], a["nr"], a["nbins"], a["w"], a["dd"],
                                         a["dr"], a["rr"], a["ws"], a["wsb"], None)
    return lib.gc_histogram_dd_dr_rr_tuned(a["pd"], a["nd"], a["pr"], a["nr"], a["nbins"], a["w"], a["dd"],
                                           a["dr"], a["rr"], a["ws"], a["wsb"], ctypes.byref(a["tuning"]),
                                           None)


def test_histogram_validation(lib):
    P = ctypes.c_void_p
    assert _hist(lib, nbins=0) == INVALID
    assert _hist(lib, nbins=-5) == INVALID
    assert _hist(lib, nbins=gc.MAX_BINS + 1) == UNSUPPORTED
    for w in (0.0, -0.25, float("inf"), float("nan")):
        assert _hist(lib, w=w) == INVALID
    assert _hist(lib, nd=-1) == INVALID
    assert _hist(lib, nr=gc.MAX_GALAXIES + 1) == UNSUPPORTED
    assert _hist(lib, pd=None) == INVALID
    assert _hist(lib, pr=P(A + 4)) == INVALID
    assert _hist(lib, dd=None) == INVALID
    assert _hist(lib, rr=P(A + 4)) == INVALID
    assert _hist(lib, ws=None) == INVALID
    assert _hist(lib, ws=P(A + 128)) == INVALID
    assert _hist(lib, wsb=gc.workspace_bytes(720) - 1) == WORKSPACE
    # dot, K, blocks/CU, shared histogram, span kernel, fast core, flush interval, histogram columns,
    # waves per workgroup, L1 share, reserved
    T = gc._Tuning
    for bad in (T(33, 0, 0, 0, 0, 0, 0), T(0, 5, 0, 0, 0, 0, 0), T(0, 0, 9, 0, 0, 0, 0),
                T(0, 0, -1, 0, 0, 0, 0), T(0, 0, 0, 3, 0, 0, 0), T(0, 0, 0, -1, 0, 0, 0),
                T(0, 0, 0, 0, 3, 0, 0), T(0, 0, 0, 0, 0, 4, 0), T(0, 0, 0, 0, 0, -1, 0), T(0, 0, 0, 0, 0, 0, -3),
                T(0, 0, 0, 0, 0, 0, 0, 2), T(0, 0, 0, 0, 0, 0, 0, 8), T(0, 0, 0, 0, 0, 0, 0, 0, 3),
                T(0, 0, 0, 0, 0, 0, 0, 0, 17), T(0, 0, 0, 0, 0, 0, 0, 0, 0, 5), T(0, 0, 0, 0, 0, 0, 0, 0, 0, -1),
                T(0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 1),
                T(0, 0, 0, 0, 0, 0, 0, 4),
                T(64, 0, 0, 0, 2, 0, 0)):                      # fp64 narrow core: 180 deg > 90 deg
        assert _hist(lib, tuning=bad) == INVALID
    # sixteen histogram columns of 3600 bins (230 KiB) do not fit in LDS
    assert _hist(lib, nbins=3600, w=0.05, tuning=T(0, 0, 0, 0, 0, 0, 0, 16)) == INVALID
    assert _hist(lib, nbins=720, tuning=T(0, 0, 0, 0, 0, 3, 0)) == INVALID         # no fast core 3
    assert _hist(lib, nbins=1500, w=0.001, tuning=T(32, 2, 0, 0, 0, 0, 0)) == INVALID  # K = 2: bin table only
    assert _hist(lib, nbins=700, tuning=T(0, 0, 0, 0, 2, 0, 0)) == INVALID  # 700 x 0.25 < 180 deg
    assert _hist(lib, nbins=361, tuning=T(64, 0, 0, 0, 2, 0, 0)) == INVALID  # 361 x 0.25 > 90 deg
    assert _hist(lib, nbins=1500, w=0.001, tuning=T(32, 0, 0, 0, 2, 0, 0)) == INVALID  # 1.5 < 180 deg
    # fast cores: the bin table (fp32 dot, full span, a table of at most 14337 entries: widths of
    # >= ~0.032 deg, a shared histogram) or the series (fp64 dot, bins ending by ~9 deg)
    assert _hist(lib, tuning=T(64, 0, 0, 0, 0, 2, 0)) == INVALID                      # 180 deg, fp64
    assert _hist(lib, nbins=100, w=0.1, tuning=T(64, 0, 0, 0, 0, 2, 0)) == INVALID     # 10 deg: series too short
    assert _hist(lib, nbins=8192, w=0.022, tuning=T(0, 0, 0, 0, 0, 2, 0)) == INVALID  # both tables too big
    assert _hist(lib, nbins=700, tuning=T(0, 0, 0, 0, 0, 2, 0)) == INVALID            # not full span
    assert _hist(lib, tuning=T(0, 0, 0, 1, 0, 2, 0)) == INVALID                       # private histograms
    assert _hist(lib, tuning=T(0, 0, 0, 0, 1, 2, 0)) == INVALID                       # generic core


@pytest.mark.skipif(not NO_GPU, reason="exercises the no-device error path; only without a GPU")
def test_histogram_reports_device_error_without_gpu(lib):
    # valid arguments: planning needs the device, which is absent -> GC_ERR_DEVICE
    assert _hist(lib) == DEVICE
    assert lib.gc_last_device_error() != 0


def test_totals_omega_core_validation(lib):
    P = ctypes.c_void_p
    assert lib.gc_histogram_totals(P(A), P(A), P(A), 0, P(A), None) == INVALID
    assert lib.gc_histogram_totals(P(A), P(A), P(A), gc.MAX_BINS + 1, P(A), None) == UNSUPPORTED
    assert lib.gc_histogram_totals(None, P(A), P(A), 10, P(A), None) == INVALID
    assert lib.gc_omega(P(A), P(A), P(A), 0, 1, 1, P(A), None) == INVALID
    assert lib.gc_omega(P(A), P(A), P(A), 10, -1, 1, P(A), None) == INVALID
    assert lib.gc_omega(P(A), P(A), None, 10, 1, 1, P(A), None) == INVALID
    assert lib.gc_omega(P(A), P(A), P(A), 10, 1, 1, P(A + 4), None) == INVALID
    ev = lambda *a: lib.gc_eval_angle_core(*a)  # noqa: E731
    assert ev(P(A), None, 10, 720, 0.25, 16, P(A), P(A), None, None, None, 0, None) == INVALID
    assert ev(None, None, 10, 720, 0.25, 32, P(A), P(A), None, None, None, 0, None) == INVALID
    assert ev(P(A), None, 0, 720, 0.25, 32, P(A), P(A), None, None, None, 0, None) == OK
    assert ev(P(A), None, 10, 0, 0.25, 32, P(A), P(A), None, None, None, 0, None) == INVALID
    assert ev(P(A), None, 10, 720, 0.25, 32, P(A), P(A), P(A), None, None, 0, None) == INVALID  # exact, no ws
    assert ev(P(A), None, 10, 720, 0.25, 32, P(A), P(A), P(A), None, P(A), 100, None) == WORKSPACE
    assert ev(P(A), None, 10, 720, 0.25, 32, P(A), P(A), None, None, None, 0, None) == INVALID  # table, no ws
    dm = lambda *a: lib.gc_eval_dot_mfma(*a)  # noqa: E731
    assert dm(P(A), P(A), P(A), P(A), P(A), P(A), -1, P(A), None) == INVALID
    assert dm(P(A), P(A), None, P(A), P(A), P(A), 4, P(A), None) == INVALID
    assert dm(P(A), P(A), P(A), P(A), P(A), P(A), 4, None, None) == INVALID
    assert dm(None, None, None, None, None, None, 0, None, None) == OK
    assert dm(P(A), P(A), P(A), P(A), P(A), P(A), 1 << 31, P(A), None) == UNSUPPORTED
    n = ctypes.c_uint64(0)
    sink = lib.gc_ceiling_sink_bytes()
    assert sink == 2048 * 1024 * 4
    assert lib.gc_ceiling_valu(3, 10, P(A), sink, ctypes.byref(n), None) == INVALID
    assert lib.gc_ceiling_valu(0, 0, P(A), sink, ctypes.byref(n), None) == INVALID
    assert lib.gc_ceiling_valu(0, 10, P(A), sink - 1, ctypes.byref(n), None) == WORKSPACE
    assert lib.gc_ceiling_lds_atomic(0, 0, 10, P(A), sink, ctypes.byref(n), None) == INVALID
    assert lib.gc_ceiling_lds_atomic(gc.MAX_BINS + 1, 0, 10, P(A), sink, ctypes.byref(n), None) == INVALID
    assert lib.gc_ceiling_lds_atomic(720, 0, 10, None, sink, ctypes.byref(n), None) == INVALID
    # LDS probes: kind, words, threads, sparse, cols, iters
    lds = lambda *a: lib.gc_ceiling_lds(*a, P(A), sink, ctypes.byref(n), None)  # noqa: E731
    assert lds(8, 1024, 256, 1, 0, 10) == INVALID          # no such kind
    assert lds(0, 1000, 256, 1, 0, 10) == INVALID          # words not a multiple of 128
    assert lds(0, 1024, 128, 1, 0, 10) == INVALID          # threads
    assert lds(7, 1024, 256, 0, 0, 10) == INVALID          # sparse < 1
    assert lds(0, 1024, 256, 1, 3, 10) == INVALID          # columns not a power of two
    assert lds(0, 1024, 256, 1, 128, 10) == INVALID        # more columns than lanes
    assert lds(0, 1024, 256, 1, 0, 0) == INVALID           # iters
    assert lds(6, 40960, 256, 1, 0, 10) == UNSUPPORTED     # 160 KiB + the 4 KiB histogram
    assert lib.gc_ceiling_lds(0, 1024, 256, 1, 0, 10, P(A), sink - 1, ctypes.byref(n), None) == WORKSPACE
    assert lib.gc_ceiling_l1(1000, 256, 10, P(A), sink, ctypes.byref(n), None) == INVALID
    assert lib.gc_ceiling_l1(1024, 256, 0, P(A), sink, ctypes.byref(n), None) == INVALID
    assert lib.gc_ceiling_l1(1024, 256, 10, P(A), sink, ctypes.byref(n), None) == WORKSPACE  # table + sink


def test_ladder_validation(lib):
    P = ctypes.c_void_p
    assert lib.gc_ladder_workspace_bytes(-1, 0) == 0
    assert lib.gc_ladder_workspace_bytes(0, gc_ladder_max() + 1) == 0
    assert lib.gc_ladder_workspace_bytes(10, 100) == 3 * (256 + 512)

    def lad(rung=3, acos=-1, tile=0, stride=0, nd=10, nr=10, nbins=720, w=0.25, ws=P(A), wsb=1 << 30, **kw):
        p = dict(rad=P(A), decd=P(A), rar=P(A), decr=P(A), dd=P(A), dr=P(A + 8192), rr=P(A + 16384))
        p.update(kw)
        return lib.gc_ladder_histogram(rung, acos, tile, stride, p["rad"], p["decd"], nd, p["rar"], p["decr"], nr,
                                       nbins, w, p["dd"], p["dr"], p["rr"], ws, wsb, None)

    for bad in (dict(rung=-1), dict(rung=6), dict(acos=-2), dict(acos=3), dict(rung=0, tile=64),
                dict(tile=32), dict(tile=100), dict(tile=2048), dict(stride=719), dict(nbins=0), dict(w=0.0),
                dict(w=float("nan")), dict(nd=-1), dict(rad=None), dict(decr=P(A + 2)), dict(dd=None),
                dict(rr=P(A + 4)), dict(ws=None), dict(ws=P(A + 8))):
        assert lad(**bad) == INVALID, bad
    assert lad(nbins=gc.MAX_BINS + 1) == UNSUPPORTED
    assert lad(nd=gc_ladder_max() + 1) == UNSUPPORTED
    assert lad(stride=40000) == UNSUPPORTED                       # LDS footprint above 160 KiB
    assert lad(rung=2, wsb=lib.gc_ladder_workspace_bytes(10, 10) - 1) == WORKSPACE
    if NO_GPU:  # valid arguments (rungs 0-1 need no workspace); the launch then fails without a device
        assert lad(rung=1, ws=None, wsb=0) == DEVICE


def gc_ladder_max():
    for line in open(os.path.join(ROOT, "include", "gc_ladder.h")):
        if line.startswith("#define GC_LADDER_MAX_GALAXIES"):
            return int(line.split()[2].rstrip("LL"))
    raise KeyError


def test_part_validation(lib):
    P = ctypes.c_void_p

    def part(p, n, **kw):
        a = dict(pd=P(A), nd=10, pr=P(A), nr=10, nbins=720, w=0.25)
        a.update(kw)
        return lib.gc_histogram_part(a["pd"], a["nd"], a["pr"], a["nr"], a["nbins"], a["w"], p, n, P(A),
                                     P(A + 8192), P(A + 16384), P(A), gc.workspace_bytes(720), None, None)

    for p, n in ((0, 0), (-1, 4), (4, 4), (5, 4), (0, gc.MAX_PARTS + 1)):
        assert part(p, n) == INVALID, (p, n)
    assert part(0, 2, nbins=0) == INVALID
    assert part(0, 2, pd=P(A + 4)) == INVALID
    if NO_GPU:
        assert part(1, 2) == DEVICE


def test_checkpoint_files(tmp_path):
    from two_point_angular_amd import parts
    import numpy as np
    meta = parts._meta(10, 12, 720, 0.25, 7, "k", None, 2)
    path = str(tmp_path / "ck.npz")
    assert parts.load_checkpoint(path, meta) is None
    h = np.arange(3 * 720, dtype=np.uint64).reshape(3, 720) * np.uint64(1 << 40)
    parts.save_checkpoint(path, meta, 3, h)
    nxt, back = parts.load_checkpoint(path, meta)
    assert nxt == 3 and np.array_equal(back, h)
    # another part count, another planned i-block height (the parts then cover other pairs), or
    # another tuning field is another job
    for other in (parts._meta(10, 12, 720, 0.25, 8, "k", None, 2), parts._meta(10, 12, 720, 0.25, 7, "k", None, 4),
                  parts._meta(10, 12, 720, 0.25, 7, "k", gc.Tuning(hist_columns=1), 2)):
        with pytest.raises(ValueError, match="another job"):
            parts.load_checkpoint(path, other)
    assert sorted(os.listdir(tmp_path)) == ["ck.npz"]          # the temporary file was renamed


@pytest.mark.skipif(not NO_GPU, reason="checks the no-device status; only without a GPU")
def test_bench_ceiling_probe_arguments_are_valid(lib):
    """The probe arguments bench.py uses pass every host check (no GPU here: GC_ERR_DEVICE)."""
    import sys
    sys.path.insert(0, ROOT)
    import bench
    out = ctypes.c_uint64(0)
    sink = ctypes.c_void_p(A)
    big = 1 << 30
    for _, kind, words, threads, cols in bench.LDS_CEILINGS:
        assert lib.gc_ceiling_lds(gc.LDS_PROBES[kind], words, threads, 1, cols, 512, sink, big,
                                  ctypes.byref(out), None) == DEVICE, (kind, words, cols)
    _, words, threads = bench.L1_CEILING
    assert lib.gc_ceiling_l1(words, threads, 256, sink, big, ctypes.byref(out), None) == DEVICE
