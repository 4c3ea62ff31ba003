"""ctypes front end of the CPU fp64 oracle (``gc_oracle.c``).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The GPU library neither imports nor links
anything here, and nothing here imports the GPU library.

The arithmetic lives in ``gc_oracle.c``; this file only builds it with gcc,
marshals numpy arrays, and checks a GPU histogram against the oracle with the
edge-flow rule stated in ``flow_check``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gc_oracle.c")
_LIB = os.path.join(_HERE, "libgc_oracle.so")

EDGE_TOL_DEG = 1e-5
FAMILIES = ("DD", "DR", "RR")

_lib = None


def build(force: bool = True) -> str:
    """Compile gc_oracle.c with gcc (-O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall",
                        "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB)
        f32p = np.ctypeslib.ndpointer(np.float32, flags="C_CONTIGUOUS")
        u64p = np.ctypeslib.ndpointer(np.uint64, flags="C_CONTIGUOUS")
        i64p = np.ctypeslib.ndpointer(np.int64, flags="C_CONTIGUOUS")
        f64p = np.ctypeslib.ndpointer(np.float64, flags="C_CONTIGUOUS")
        i64 = ctypes.c_int64
        lib.gco_pair_angle_deg.argtypes = [ctypes.c_float] * 4
        lib.gco_pair_angle_deg.restype = ctypes.c_double
        lib.gco_bin_index.argtypes = [ctypes.c_double, ctypes.c_double, i64]
        lib.gco_bin_index.restype = i64
        lib.gco_family_rows.argtypes = [f32p, f32p, i64, f32p, f32p, i64, i64, i64, ctypes.c_int,
                                        i64, ctypes.c_double, ctypes.c_int, u64p, u64p, u64p]
        lib.gco_family_rows.restype = ctypes.c_int
        lib.gco_histograms.argtypes = [f32p, f32p, i64, f32p, f32p, i64, i64, ctypes.c_double,
                                       ctypes.c_int, ctypes.c_int, u64p, u64p, u64p, u64p, u64p]
        lib.gco_histograms.restype = ctypes.c_int
        lib.gco_pair_bins.argtypes = [f32p, f32p, i64, f32p, f32p, i64, i64, ctypes.c_double,
                                      i64p, ctypes.c_void_p]
        lib.gco_pair_bins.restype = ctypes.c_int
        lib.gco_omega.argtypes = [u64p, u64p, u64p, i64, i64, i64, f64p]
        lib.gco_omega.restype = ctypes.c_int
        lib.gco_max_threads.argtypes = []
        lib.gco_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32)


def max_threads() -> int:
    return int(_load().gco_max_threads())


def pair_angle_deg(ra1, dec1, ra2, dec2) -> float:
    return float(_load().gco_pair_angle_deg(float(np.float32(ra1)), float(np.float32(dec1)),
                                            float(np.float32(ra2)), float(np.float32(dec2))))


def bin_index(theta_deg: float, w_deg: float, nbins: int) -> int:
    return int(_load().gco_bin_index(float(theta_deg), float(w_deg), int(nbins)))


def pair_bins(ra_a, dec_a, ra_b, dec_b, nbins: int, w_deg: float, with_theta: bool = False):
    ra_a, dec_a, ra_b, dec_b = map(_f32, (ra_a, dec_a, ra_b, dec_b))
    na, nb = len(ra_a), len(ra_b)
    bins = np.zeros(na * nb, dtype=np.int64)
    theta = np.zeros(na * nb, dtype=np.float64) if with_theta else None
    rc = _load().gco_pair_bins(ra_a, dec_a, na, ra_b, dec_b, nb, int(nbins), float(w_deg), bins,
                               theta.ctypes.data if with_theta else None)
    if rc:
        raise ValueError("gco_pair_bins rejected its arguments")
    bins = bins.reshape(na, nb)
    return (bins, theta.reshape(na, nb)) if with_theta else bins


@dataclass
class FamilyResult:
    hist: np.ndarray  # uint64 [nbins]
    lo: np.ndarray    # uint64 [nbins]: pairs within EDGE_TOL_DEG below edge e
    hi: np.ndarray    # uint64 [nbins]: pairs within EDGE_TOL_DEG at/above edge e


def family_rows(ra_a, dec_a, ra_b, dec_b, nbins: int, w_deg: float, row0: int = 0,
                row1: int | None = None, symmetric: bool = False, nthreads: int = 0) -> FamilyResult:
    ra_a, dec_a, ra_b, dec_b = map(_f32, (ra_a, dec_a, ra_b, dec_b))
    row1 = len(ra_a) if row1 is None else row1
    h, lo, hi = (np.zeros(nbins, dtype=np.uint64) for _ in range(3))
    rc = _load().gco_family_rows(ra_a, dec_a, len(ra_a), ra_b, dec_b, len(ra_b), int(row0), int(row1),
                                 int(bool(symmetric)), int(nbins), float(w_deg), int(nthreads), h, lo, hi)
    if rc:
        raise ValueError("gco_family_rows rejected its arguments")
    return FamilyResult(h, lo, hi)


@dataclass
class OracleResult:
    dd: FamilyResult
    dr: FamilyResult
    rr: FamilyResult

    def family(self, name: str) -> FamilyResult:
        return {"DD": self.dd, "DR": self.dr, "RR": self.rr}[name]


def histograms(d_ra, d_dec, r_ra, r_dec, nbins: int, w_deg: float, symmetric: bool = True,
               nthreads: int = 0) -> OracleResult:
    d_ra, d_dec, r_ra, r_dec = map(_f32, (d_ra, d_dec, r_ra, r_dec))
    out = [np.zeros(nbins, dtype=np.uint64) for _ in range(3)]
    lo = np.zeros(3 * nbins, dtype=np.uint64)
    hi = np.zeros(3 * nbins, dtype=np.uint64)
    rc = _load().gco_histograms(d_ra, d_dec, len(d_ra), r_ra, r_dec, len(r_ra), int(nbins), float(w_deg),
                                int(bool(symmetric)), int(nthreads), out[0], out[1], out[2], lo, hi)
    if rc:
        raise ValueError("gco_histograms rejected its arguments")
    fam = [FamilyResult(out[k], lo[k * nbins:(k + 1) * nbins].copy(), hi[k * nbins:(k + 1) * nbins].copy())
           for k in range(3)]
    return OracleResult(*fam)


def omega(dd, dr, rr, n_d: int, n_r: int) -> np.ndarray:
    dd, dr, rr = (np.ascontiguousarray(x, dtype=np.uint64) for x in (dd, dr, rr))
    out = np.zeros(len(dd), dtype=np.float64)
    rc = _load().gco_omega(dd, dr, rr, len(dd), int(n_d), int(n_r), out)
    if rc:
        raise ValueError("gco_omega rejected its arguments")
    return out


@dataclass
class FlowReport:
    ok: bool
    total_ok: bool
    max_abs_flow: int
    sum_abs_flow: int
    bad_edges: list
    message: str


def flow_check(gpu_hist, fam: FamilyResult, total_expected: int, moved_budget: float = 1e-6) -> FlowReport:
    """Compare a histogram with the oracle's by edge flow.

    Delta_b = gpu[b] - oracle[b]; f_e = -sum_{b<e} Delta_b is the net number of ordered
    pairs the GPU placed above edge e that the oracle placed below it.  The check passes
    iff the GPU total equals total_expected exactly, every f_e lies in
    [-hi[e], lo[e]] (each net crossing is explained by pairs whose fp64 angle is within
    1e-5 degrees of that edge), and sum_e |f_e| <= moved_budget * total_expected.
    """
    g = np.asarray(gpu_hist).astype(np.uint64).astype(object)
    o = fam.hist.astype(object)
    total = int(sum(g))
    delta = np.array([int(a) - int(b) for a, b in zip(g, o)], dtype=object)
    flows = [0] * len(g)
    run = 0
    for e in range(1, len(g)):
        run += int(delta[e - 1])
        flows[e] = -run
    bad = []
    for e in range(1, len(g)):
        f = flows[e]
        if f > int(fam.lo[e]) or -f > int(fam.hi[e]):
            bad.append((e, f, int(fam.lo[e]), int(fam.hi[e])))
    max_abs = max((abs(f) for f in flows), default=0)
    sum_abs = sum(abs(f) for f in flows)
    total_ok = total == int(total_expected)
    ok = total_ok and not bad and sum_abs <= moved_budget * int(total_expected)
    msg = (f"total {total} (expected {total_expected}), max|f| {max_abs}, sum|f| {sum_abs}, "
           f"unexplained edges {bad[:5]}")
    return FlowReport(ok, total_ok, max_abs, sum_abs, bad, msg)
