"""gc_histogram_dd_dr_rr_noalloc: the histogram call with the library's own per-GPU scratch.

CPU: every argument check returns before any HIP call.  GPU: two calls in a row, the second on a
smaller job (fewer galaxies, fewer bins, another core) than the first, each bit-identical to
gc_histogram_dd_dr_rr on the same inputs; the first call fills the scratch with the largest edge
table (8192 bins), over which the second call's smaller tables are built.
"""
import ctypes
import os

import numpy as np
import pytest

import two_point_angular_amd as gc
from two_point_angular_amd import catalogs

OK, INVALID, UNSUPPORTED, WORKSPACE, DEVICE = 0, 1, 2, 3, 4
A = 4096  # a 256-aligned fake device address; never dereferenced
NO_GPU = not os.path.exists("/dev/kfd")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(gc.library_path()):
        from two_point_angular_amd import build
        build.build()
    return gc.load()


def _call(lib, **kw):
    P = ctypes.c_void_p
    a = dict(pd=P(A), nd=10, pr=P(A), nr=10, nbins=720, w=0.25, dd=P(A), dr=P(A + 8192), rr=P(A + 16384))
    a.update(kw)
    return lib.gc_histogram_dd_dr_rr_noalloc(a["pd"], a["nd"], a["pr"], a["nr"], a["nbins"], a["w"], a["dd"],
                                             a["dr"], a["rr"], None)


def test_noalloc_validation(lib):
    P = ctypes.c_void_p
    assert _call(lib, nbins=0) == INVALID
    assert _call(lib, nbins=gc.MAX_BINS + 1) == UNSUPPORTED
    for w in (0.0, -1.0, float("inf"), float("nan")):
        assert _call(lib, w=w) == INVALID
    assert _call(lib, nd=-1) == INVALID
    assert _call(lib, nr=gc.MAX_GALAXIES + 1) == UNSUPPORTED
    assert _call(lib, pd=None) == INVALID
    assert _call(lib, pr=P(A + 4)) == INVALID
    assert _call(lib, dd=None) == INVALID
    assert _call(lib, rr=P(A + 4)) == INVALID


@pytest.mark.skipif(not NO_GPU, reason="exercises the no-device error path; only without a GPU")
def test_noalloc_reports_device_error_without_gpu(lib):
    assert _call(lib) == DEVICE
    assert lib.gc_last_device_error() != 0


def _dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


@pytest.mark.gpu
def test_noalloc_matches_workspace_call_twice():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gc.load()
    jobs = [
        # (D, R, nbins, width): the first fills the scratch with an 8192-bin edge table; the
        # second is smaller and runs the bin-table core over the stale contents
        (catalogs.clustered(20000, 41), catalogs.uniform_sphere(18000, 42), 8192, 180.0 / 8192),
        (catalogs.clustered(3000, 43), catalogs.uniform_sphere(2500, 44), 720, 0.25),
    ]
    for D, R, nbins, w in jobs:
        print(f"[gpu] noalloc vs workspace call: n_d={len(D)} n_r={len(R)} nbins={nbins}", flush=True)
        pd = gc.prepare(_dev(D.ra), _dev(D.dec))
        pr = gc.prepare(_dev(R.ra), _dev(R.dec))
        out = torch.full((3, nbins), -1, dtype=torch.int64, device="cuda")
        gc.histogram_dd_dr_rr_noalloc(pd, len(D), pr, len(R), nbins, w, out)
        ref = torch.empty_like(out)
        gc.histogram_dd_dr_rr(pd, len(D), pr, len(R), nbins, w, out=ref)
        torch.cuda.synchronize()
        got, want = out.cpu().numpy(), ref.cpu().numpy()
        assert got.sum(axis=1).tolist() == [len(D) ** 2, len(D) * len(R), len(R) ** 2]
        assert np.array_equal(got, want), f"nbins={nbins}: {int((got != want).sum())} bins differ"
