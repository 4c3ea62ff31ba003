"""GPU parity: the HIP path (through the C ABI) against the CPU fp64 oracle.

The rules (from the problem statement of "CUDA Deep Dive: 10B Galaxy Pairs on an RTX
5080", section "The problem", made operational):
  * every histogram sums to exactly N_a * N_b;
  * per bin, the GPU may differ from the oracle only by pairs whose fp64 angle lies
    within 1e-5 deg of a bin edge (edge-flow check against the oracle's near-edge
    counts), with at most 1e-6 * N_a * N_b moved pairs;
  * omega agrees within 1e-4 in every bin where the oracle's RR >= 1000.
"""
import math
import os
import sys

import numpy as np
import pytest

from oracle import oracle
from two_point_angular_amd import catalogs

sys.path.insert(0, os.path.dirname(__file__))
from test_golden_and_catalogs import read_fixture  # noqa: E402

pytestmark = pytest.mark.gpu

OMEGA_TOL = 1e-4
OMEGA_MIN_RR = 1000
MOVED_BUDGET = 1e-6


@pytest.fixture(scope="module")
def gc():
    import torch
    import two_point_angular_amd as gcm
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gcm.load()
    return gcm


def _dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def run_gpu(gc, D, R, nbins, w, tuning=None, same=False, prefill=None):
    import torch
    pd = gc.prepare(_dev(D.ra), _dev(D.dec))
    pr = pd if same else gc.prepare(_dev(R.ra), _dev(R.dec))
    n_r = len(D) if same else len(R)
    out = torch.empty((3, nbins), dtype=torch.int64, device="cuda")
    if prefill is not None:
        out.fill_(prefill)
    dd, dr, rr = gc.histogram_dd_dr_rr(pd, len(D), pr, n_r, nbins, w, out=out, tuning=tuning)
    tot = gc.histogram_totals(dd, dr, rr)
    om = gc.omega(dd, dr, rr, len(D), n_r)
    torch.cuda.synchronize()
    h = out.cpu().numpy().view(np.uint64)
    return h[0].copy(), h[1].copy(), h[2].copy(), tot.cpu().numpy().view(np.uint64), om.cpu().numpy()


def check_against(name, gpu, fams, n_d, n_r, gpu_omega=None, budget=MOVED_BUDGET, ties=None):
    """Edge-flow check of every family; ties (optional, per family): ordered pairs whose bin the
    definition leaves to fp64 rounding (see tie_pairs), allowed to move on top of the budget."""
    expected = {"DD": n_d * n_d, "DR": n_d * n_r, "RR": n_r * n_r}
    for k, fam in enumerate(oracle.FAMILIES):
        m = expected[fam]
        b = budget + (ties[fam] / m if ties and m else 0.0)
        rep = oracle.flow_check(gpu[k], fams[fam], m, moved_budget=b)
        assert rep.ok, f"{name} {fam}: {rep.message}"
    if gpu_omega is not None:
        ora = oracle.omega(fams["DD"].hist, fams["DR"].hist, fams["RR"].hist, n_d, n_r)
        rr = fams["RR"].hist
        sel = rr >= OMEGA_MIN_RR
        if sel.any():
            err = np.abs(gpu_omega[sel] - ora[sel])
            assert float(err.max()) <= OMEGA_TOL, f"{name}: max |d omega| {err.max()}"
        zero = rr == 0
        assert np.all(np.isnan(gpu_omega[zero]) == np.isnan(ora[zero]))


TIE_DEG = 1e-9


def tie_pairs(A, B, nbins, w):
    """Ordered pairs of A x B whose oracle angle lies within TIE_DEG of an inner bin edge: pairs
    that sit on an edge in exact arithmetic (constructed catalogs can hold them), whose bin fp64
    rounding decides, differently for the law of cosines and for a dot product; several results are
    then correct.  The GPU's exact recheck agrees with the oracle outside ~1e-11 deg of an edge."""
    _, th = oracle.pair_bins(A.ra, A.dec, B.ra, B.dec, nbins, w, with_theta=True)
    t = th / w
    e = np.round(t)
    return int((((e >= 1) & (e <= nbins - 1)) & (np.abs(t - e) * w < TIE_DEG)).sum())


def oracle_fams(D, R, nbins, w):
    res = oracle.histograms(D.ra, D.dec, R.ra, R.dec, nbins, w)
    return {f: res.family(f) for f in oracle.FAMILIES}


@pytest.mark.parametrize("n_d,n_r", [(1, 1), (2, 3), (3, 2), (63, 64), (64, 65), (65, 63), (511, 513),
                                     (512, 512), (1023, 1025), (1025, 700), (2500, 2100)])
def test_small_and_ragged(gc, n_d, n_r):
    print(f"[gpu] small/ragged n_d={n_d} n_r={n_r}", flush=True)
    D = catalogs.clustered(max(n_d, 1), 5).subset(0, n_d)
    R = catalogs.uniform_sphere(max(n_r, 1), 6).subset(0, n_r)
    for nbins, w in ((720, 0.25), (3600, 0.05)):
        dd, dr, rr, tot, om = run_gpu(gc, D, R, nbins, w)
        assert list(tot) == [n_d * n_d, n_d * n_r, n_r * n_r]
        check_against(f"n={n_d},{n_r} bins={nbins}", (dd, dr, rr), oracle_fams(D, R, nbins, w), n_d, n_r)


@pytest.mark.parametrize("nbins,w,tuning", [
    (8192, 180.0 / 8192, {}),                        # the largest histogram, full span
    (8192, 180.0 / 8192, dict(shared_histogram=1)),  # 8192-bin private histograms: 1 workgroup per CU
    (8192, 180.0 / 8192, dict(shared_histogram=2)),
    (8192, 0.0005, {}),                              # fp64 narrow core, 4.1 deg of bins
    (1, 1.0, {}),                                    # a single bin takes every pair
    (1, 1.0, dict(dot_precision=64)),
    (2, 90.0, {}),                                   # two bins: one per hemisphere of separations
    (2, 90.0, dict(dot_precision=64)),
])
def test_bin_count_extremes(gc, nbins, w, tuning):
    print(f"[gpu] bin extremes nbins={nbins} w={w} tuning={tuning}", flush=True)
    D = catalogs.clustered(1500, 21)
    R = catalogs.uniform_sphere(1300, 22)
    dd, dr, rr, tot, om = run_gpu(gc, D, R, nbins, w, tuning=gc.Tuning(**tuning))
    assert list(tot) == [1500 * 1500, 1500 * 1300, 1300 * 1300]
    check_against(f"bins={nbins} w={w} {tuning}", (dd, dr, rr), oracle_fams(D, R, nbins, w), 1500, 1300)


def test_empty_catalogs(gc):
    print("[gpu] empty catalogs", flush=True)
    D = catalogs.clustered(300, 8)
    E = D.subset(0, 0)
    dd, dr, rr, tot, om = run_gpu(gc, E, D, 720, 0.25, prefill=-1)
    assert dd.sum() == 0 and dr.sum() == 0 and int(rr.sum()) == 300 * 300 and np.all(np.isnan(om))
    dd, dr, rr, tot, om = run_gpu(gc, D, E, 720, 0.25, prefill=-1)
    assert int(dd.sum()) == 300 * 300 and dr.sum() == 0 and rr.sum() == 0
    dd, dr, rr, tot, om = run_gpu(gc, E, E, 720, 0.25, prefill=-1)
    assert dd.sum() == 0 and dr.sum() == 0 and rr.sum() == 0 and np.all(np.isnan(om))


@pytest.mark.parametrize("name,nbins,w", [("clustered100k_720", 720, 0.25), ("clustered100k_3600", 3600, 0.05),
                                          ("patch100k_1500", 1500, 0.001)])
def test_non_finite_coordinates(gc, name, nbins, w):
    """A galaxy with a NaN or infinite coordinate is placed at (0, 0): the histograms equal those
    of the same catalogs with that galaxy at (0, 0), and the totals hold."""
    print(f"[gpu] non-finite coordinates {name}", flush=True)
    D, R = catalogs.WORKLOADS[name].catalogs(n=2000)
    D, R = D.subset(0, 2000), R.subset(0, 1700)
    bad_d, bad_r = np.array([3, 700, 1999]), np.array([0, 5, 1000])
    Dn, Rn = catalogs.Catalog(D.ra.copy(), D.dec.copy()), catalogs.Catalog(R.ra.copy(), R.dec.copy())
    Dn.ra[bad_d] = [np.nan, np.inf, 1.0]
    Dn.dec[bad_d] = [2.0, 3.0, -np.inf]
    Rn.ra[bad_r] = [np.nan, -np.inf, np.nan]
    Rn.dec[bad_r] = [np.nan, 0.5, 7.0]
    Dz, Rz = catalogs.Catalog(D.ra.copy(), D.dec.copy()), catalogs.Catalog(R.ra.copy(), R.dec.copy())
    Dz.ra[bad_d] = 0.0
    Dz.dec[bad_d] = 0.0
    Rz.ra[bad_r] = 0.0
    Rz.dec[bad_r] = 0.0
    got = run_gpu(gc, Dn, Rn, nbins, w)
    want = run_gpu(gc, Dz, Rz, nbins, w)
    for k in range(3):
        assert np.array_equal(got[k], want[k])
    assert [int(t) for t in got[3]] == [2000 * 2000, 2000 * 1700, 1700 * 1700]


@pytest.mark.parametrize("nbins,w", [(720, 0.25), (3600, 0.05), (1500, 0.001)])
def test_poles_and_the_alpha_seam(gc, nbins, w):
    """Galaxies exactly at the poles (every alpha names the same point), within 1.5 degrees of the
    north pole (where alpha spreads fast), and on the seam alpha = 0 / 21600 (the same meridian):
    edge-flow check against the oracle for the bin-table (coarse and fine) and series cores."""
    print(f"[gpu] poles and seam {nbins} x {w}", flush=True)
    rng = np.random.default_rng(2024)
    ra = rng.uniform(0.0, 21600.0, 1500)
    dec = np.empty(1500)
    dec[:200] = 5400.0
    dec[200:300] = -5400.0
    dec[300:1100] = 5400.0 - rng.uniform(0.0, 90.0, 800)
    dec[1100:] = rng.uniform(-5400.0, 5400.0, 400)
    ra[1100:1200] = 0.0
    ra[1200:1300] = 21600.0
    D = catalogs.Catalog(ra.astype(np.float32), dec.astype(np.float32))
    R2 = catalogs.uniform_sphere(1200, 77)
    rdec = R2.dec.copy()
    rdec[:600] = (5400.0 - rng.uniform(0.0, 90.0, 600)).astype(np.float32)  # near the pole too
    R = catalogs.Catalog(R2.ra.copy(), rdec)
    dd, dr, rr, tot, om = run_gpu(gc, D, R, nbins, w)
    assert list(tot) == [1500 * 1500, 1500 * 1200, 1200 * 1200]
    # galaxies on the seam meridian whose declinations differ by a whole number of bins lie exactly
    # on an edge (two such DD pairs at 3600 x 0.05 deg): their moves are allowed beyond the budget
    ties = {"DD": tie_pairs(D, D, nbins, w), "DR": tie_pairs(D, R, nbins, w), "RR": tie_pairs(R, R, nbins, w)}
    check_against(f"poles {nbins} x {w}", (dd, dr, rr), oracle_fams(D, R, nbins, w), 1500, 1200, om, ties=ties)


def test_alpha_outside_one_turn(gc):
    """Right ascension is periodic: alpha anywhere in [-2, 3) turns (and negative zero) gives the
    oracle's histograms up to the edge-flow tolerance."""
    print("[gpu] alpha outside one turn", flush=True)
    rng = np.random.default_rng(99)
    D = catalogs.clustered(2000, 31)
    R = catalogs.uniform_sphere(1700, 32)
    Dk = catalogs.Catalog((D.ra + 21600.0 * rng.integers(-2, 3, 2000)).astype(np.float32), D.dec.copy())
    Rk = catalogs.Catalog((R.ra - 21600.0 * rng.integers(0, 2, 1700)).astype(np.float32), R.dec.copy())
    Dk.ra[:5] = np.float32(-0.0)
    for nbins, w in ((720, 0.25), (3600, 0.05)):
        dd, dr, rr, tot, om = run_gpu(gc, Dk, Rk, nbins, w)
        check_against(f"alpha turns {nbins}", (dd, dr, rr), oracle_fams(Dk, Rk, nbins, w), 2000, 1700, om)


@pytest.mark.parametrize("nbins,w,modulus", [(720, 0.25, 960), (3600, 0.05, 192)])
def test_equator_exact_bins(gc, nbins, w, modulus):
    """Galaxies on the equator: exact integer bins (no oracle involved)."""
    print(f"[gpu] equator exact bins={nbins}", flush=True)
    rng = np.random.default_rng(11)
    n = min(modulus // 2, 400)
    res = rng.permutation(modulus)[: 2 * n]
    k = lambda r: rng.integers(0, (21600 * 64) // modulus, len(r)) * modulus + r  # noqa: E731
    kd, kr = k(res[:n]), k(res[n:])
    D = catalogs.Catalog((kd / 64.0).astype(np.float32), np.zeros(n, np.float32))
    R = catalogs.Catalog((kr / 64.0).astype(np.float32), np.zeros(n, np.float32))
    edge = 960 if nbins == 720 else 192

    def expect(ka, kb):
        d = np.abs(ka[:, None] - kb[None, :])
        t = np.minimum(d, 21600 * 64 - d)
        return np.bincount(np.minimum(t // edge, nbins - 1).ravel(), minlength=nbins)

    dd, dr, rr, tot, om = run_gpu(gc, D, R, nbins, w)
    np.testing.assert_array_equal(dd, expect(kd, kd))
    np.testing.assert_array_equal(dr, expect(kd, kr))
    np.testing.assert_array_equal(rr, expect(kr, kr))


def test_uniform10k_full(gc):
    print("[gpu] uniform10k_720 full vs fixture", flush=True)
    wl = catalogs.WORKLOADS["uniform10k_720"]
    D, R = wl.catalogs()
    _, fams = read_fixture(wl.name)
    dd, dr, rr, tot, om = run_gpu(gc, D, R, wl.nbins, wl.bin_width_deg)
    assert list(tot) == [wl.n ** 2] * 3
    check_against(wl.name, (dd, dr, rr), fams, wl.n, wl.n, om)


@pytest.mark.parametrize("name", ["clustered100k_720", "clustered100k_3600", "patch100k_1500"])
def test_full_size_vs_fixture(gc, name):
    """Full 100k + 100k workloads in the default launch plan, against the stored oracle."""
    print(f"[gpu] {name} full vs fixture", flush=True)
    fx = read_fixture(name)
    if fx is None:
        pytest.skip("fixture missing")
    meta, fams = fx
    wl = catalogs.WORKLOADS[name]
    D, R = wl.catalogs()
    assert meta["sha256_D"] == D.sha256() and meta["sha256_R"] == R.sha256()
    dd, dr, rr, tot, om = run_gpu(gc, D, R, wl.nbins, wl.bin_width_deg)
    assert list(tot) == [wl.n ** 2] * 3
    check_against(name, (dd, dr, rr), fams, wl.n, wl.n, om)


def test_symmetry_and_invariances(gc):
    print("[gpu] DR(D,D)==DD, swap, shuffle", flush=True)
    D, R = catalogs.WORKLOADS["clustered100k_720"].catalogs(n=20000)
    dd, dr_self, _, _, _ = run_gpu(gc, D, D, 720, 0.25, same=True)
    np.testing.assert_array_equal(dd, dr_self)
    _, dr1, _, _, _ = run_gpu(gc, D, R, 720, 0.25)
    _, dr2, _, _, _ = run_gpu(gc, R, D, 720, 0.25)
    np.testing.assert_array_equal(dr1, dr2)
    perm = np.random.default_rng(3).permutation(len(D))
    Dp = catalogs.Catalog(D.ra[perm].copy(), D.dec[perm].copy())
    a = run_gpu(gc, D, R, 720, 0.25)
    b = run_gpu(gc, Dp, R, 720, 0.25)
    for x, y in zip(a[:3], b[:3]):
        np.testing.assert_array_equal(x, y)


def test_outputs_overwritten_and_self_pairs(gc):
    print("[gpu] overwrite semantics, self pairs in bin 0", flush=True)
    D, R = catalogs.WORKLOADS["patch100k_1500"].catalogs(n=3000)
    a = run_gpu(gc, D, R, 1500, 0.001, prefill=-1)
    b = run_gpu(gc, D, R, 1500, 0.001, prefill=0)
    for x, y in zip(a[:3], b[:3]):
        np.testing.assert_array_equal(x, y)
    assert a[0][0] >= 3000 and a[2][0] >= 3000
    # coincident D/R points land in bin 0 of DR
    c = run_gpu(gc, D, catalogs.Catalog(D.ra.copy(), D.dec.copy()), 1500, 0.001)
    assert c[1][0] >= 3000


@pytest.mark.parametrize("tuning", [dict(dot_precision=32), dict(dot_precision=64), dict(i_per_lane=4),
                                    dict(blocks_per_cu=1), dict(flush_interval=3),
                                    dict(flush_interval=17, i_per_lane=4, dot_precision=64),
                                    dict(shared_histogram=1), dict(shared_histogram=2),
                                    dict(shared_histogram=2, flush_interval=5),
                                    dict(span_kernel=1), dict(span_kernel=2, i_per_lane=4),
                                    dict(fast_core=1), dict(fast_core=2, i_per_lane=4),
                                    dict(fast_core=2, flush_interval=5),
                                    # the bin table's layouts: histogram columns, workgroup sizes,
                                    # L1 shares, galaxies per lane (2 only here)
                                    dict(hist_columns=1), dict(hist_columns=1, waves_per_group=4, l1_share=3),
                                    dict(hist_columns=16, i_per_lane=8), dict(i_per_lane=2),
                                    dict(i_per_lane=2, l1_share=1, flush_interval=9), dict(waves_per_group=16),
                                    dict(waves_per_group=5, l1_share=3), dict(l1_share=1),
                                    dict(hist_columns=16, waves_per_group=4, flush_interval=2),
                                    dict(l1_share=4)])
def test_tuning_does_not_change_results(gc, tuning):
    print(f"[gpu] tuning {tuning}", flush=True)
    D, R = catalogs.WORKLOADS["clustered100k_720"].catalogs(n=6000)
    fams = oracle_fams(D, R, 720, 0.25)
    base = run_gpu(gc, D, R, 720, 0.25)
    t = run_gpu(gc, D, R, 720, 0.25, tuning=gc.Tuning(**tuning))
    check_against(f"tuning {tuning}", t[:3], fams, len(D), len(R), t[4])
    for x, y in zip(base[:3], t[:3]):
        np.testing.assert_array_equal(x, y)


@pytest.mark.parametrize("tuning", [dict(i_per_lane=2), dict(i_per_lane=8, waves_per_group=8),
                                    dict(waves_per_group=8, flush_interval=4), dict(l1_share=2)])
def test_fine_bin_layouts(gc, tuning):
    """3600 bins of 0.05 deg (a one-column histogram beside the bin table): other
    galaxies per lane, workgroup sizes and an L1 share give the oracle's result and the
    default's, bit for bit."""
    print(f"[gpu] 3600 bins tuning {tuning}", flush=True)
    D, R = catalogs.WORKLOADS["clustered100k_3600"].catalogs(n=6000)
    fams = oracle_fams(D, R, 3600, 0.05)
    base = run_gpu(gc, D, R, 3600, 0.05)
    t = run_gpu(gc, D, R, 3600, 0.05, tuning=gc.Tuning(**tuning))
    check_against(f"3600 bins tuning {tuning}", t[:3], fams, len(D), len(R), t[4])
    for x, y in zip(base[:3], t[:3]):
        np.testing.assert_array_equal(x, y)


@pytest.mark.parametrize("case", [
    ("patch100k_1500", 1500, 0.001, dict(span_kernel=1)),
    ("patch100k_1500", 1500, 0.001, dict(span_kernel=2, i_per_lane=4)),
    ("patch100k_1500", 1500, 0.001, dict(dot_precision=32)),
    ("patch100k_1500", 1500, 0.001, dict(shared_histogram=2, flush_interval=7)),
    # bins ending exactly at 90 deg: every pair past 90 deg goes through the narrow core's
    # x < 0 branch into the last bin
    ("uniform10k_720", 360, 0.25, dict(dot_precision=64, span_kernel=2)),
    ("uniform10k_720", 360, 0.25, dict(dot_precision=64, span_kernel=1)),
])
def test_fp64_span_variants(gc, case):
    name, nbins, w, tuning = case
    print(f"[gpu] {name} nbins={nbins} w={w} tuning {tuning}", flush=True)
    D, R = catalogs.WORKLOADS[name].catalogs(n=6000)
    fams = oracle_fams(D, R, nbins, w)
    t = run_gpu(gc, D, R, nbins, w, tuning=gc.Tuning(**tuning))
    check_against(f"{name} {tuning}", t[:3], fams, len(D), len(R), t[4])
    base = run_gpu(gc, D, R, nbins, w, tuning=gc.Tuning(dot_precision=64))
    for x, y in zip(base[:3], t[:3]):
        np.testing.assert_array_equal(x, y)


def _fast_rects(n_i, n_j, sym, s0, s1, BI):
    """The off-diagonal work units [s0, s1) of one family as rectangles (row0, row1, col0, col1) of
    (i, j) pairs, following the decomposition gc_histogram_part documents: unit s of a cross family
    is i-block s // n_j against j = s % n_j; a self family takes, block by block, j from the end of
    the block to n_j (the upper triangle by blocks).  BI: galaxies per i-block (64 per lane)."""
    rects, s, nbf = [], s0, n_i // BI
    while s < s1:
        if not sym:
            b, j = divmod(s, n_j)
        else:
            lo, hi = 0, nbf - 1
            while lo < hi:  # last block whose first unit is <= s
                mid = (lo + hi + 1) // 2
                if mid * n_j - BI * mid * (mid + 1) // 2 <= s:
                    lo = mid
                else:
                    hi = mid - 1
            b = lo
            j = (b + 1) * BI + (s - (b * n_j - BI * b * (b + 1) // 2))
        take = min(s1 - s, n_j - j)
        rects.append((b * BI, (b + 1) * BI, j, j + take))
        s += take
    return rects


def _part_units(total, p, parts):
    return total * p // parts, total * (p + 1) // parts


def _oracle_rects(A, B, rects, nbins, w, weight):
    h = [np.zeros(nbins, dtype=np.uint64) for _ in range(3)]
    for r0, r1, c0, c1 in rects:
        fam = oracle.family_rows(A.ra[r0:r1], A.dec[r0:r1], B.ra[c0:c1], B.dec[c0:c1], nbins, w)
        for k, x in enumerate((fam.hist, fam.lo, fam.hi)):
            h[k] += x * np.uint64(weight)
    return oracle.FamilyResult(*h)


def test_million_catalogs(gc):
    """1M + 1M (3e12 ordered pairs), clustered D and uniform R at 720 x 0.25 deg, in the default
    launch plan (bench's): exact totals; DD == DR(D, D) and RR == DR(R, R) bitwise (every pair's
    bin is fixed by the pair alone, so the self families' triangle schedule - a binary search over
    the full blocks' prefix sums, 7812 of them at 2 galaxies per lane - must reproduce the cross
    family's full square); and three parts of the same job (gc_histogram_part, 2e6 parts, the same
    plan) against the oracle on exactly the pairs each part covers, with the moved-pair budget
    enforced."""
    import torch
    print("[gpu] clustered1m_720: totals, self == cross, parts against the oracle", flush=True)
    wl = catalogs.WORKLOADS["clustered1m_720"]
    D, R = wl.catalogs()
    n, nbins, w = wl.n, wl.nbins, wl.bin_width_deg
    tun = None
    BI = 64 * gc.launch_plan(n, n, nbins, w)["i_per_lane"]
    dd, dr, rr, tot, om = run_gpu(gc, D, R, nbins, w, tuning=tun)
    assert list(tot) == [n * n] * 3
    pd = gc.prepare(_dev(D.ra), _dev(D.dec))
    pr = gc.prepare(_dev(R.ra), _dev(R.dec))
    out = torch.empty((3, nbins), dtype=torch.int64, device="cuda")
    for prep, self_hist, name in ((pd, dd, "D"), (pr, rr, "R")):
        gc.histogram_dd_dr_rr(prep, n, prep, n, nbins, w, out=out, tuning=tun)
        torch.cuda.synchronize()
        h = out.cpu().numpy().view(np.uint64)
        np.testing.assert_array_equal(h[0], self_hist, err_msg=f"DD({name}) differs between calls")
        np.testing.assert_array_equal(h[0], h[1], err_msg=f"DD({name}) != DR({name}, {name})")
    parts = 2_000_000
    nbf = n // BI
    t_cross = nbf * n
    t_self = nbf * n - BI * nbf * (nbf + 1) // 2
    for p in (0, 1_000_000, parts - 2):  # even p: no diagonal or ragged-block unit in this part
        g0, g1 = _part_units(n, p, parts)  # the diagonal / ragged-block units: n of them in every family
        assert g0 == g1
        out.zero_()
        gc.histogram_part(pd, n, pr, n, nbins, w, p, parts, out, tuning=tun)
        torch.cuda.synchronize()
        h = out.cpu().numpy().view(np.uint64)
        cases = (("DD", D, D, True, t_self, 2), ("DR", D, R, False, t_cross, 1), ("RR", R, R, True, t_self, 2))
        for k, (fam, A, B, sym, total, weight) in enumerate(cases):
            rects = _fast_rects(n, n, sym, *_part_units(total, p, parts), BI)
            ref = _oracle_rects(A, B, rects, nbins, w, weight)
            pairs = weight * sum((r1 - r0) * (c1 - c0) for r0, r1, c0, c1 in rects)
            assert pairs > 0
            rep = oracle.flow_check(h[k], ref, pairs, moved_budget=MOVED_BUDGET)
            assert rep.ok, f"part {p} {fam}: {rep.message}"


@pytest.mark.parametrize("nbins,w", [(720, 0.25), (3600, 0.05), (1440, 0.125)])
def test_bin_table_maps_every_entry(gc, nbins, w):
    """The bin table built on the device: for every entry q (c in [(q - 1/2)/M - 1, (q + 1/2)/M - 1],
    holding e and the row offset of B) and 64 values of c across it, bin = B - [x > e] with
    x = cos(theta) equals the bin of the angle of c, theta = 2 asin(c / sqrt2) (c >= 0) or
    180 - 2 asin(-c / sqrt2) degrees.  Where the table needs no always-recheck entries (720 x 0.25
    deg) the middle entry (q = M) holds both ends of the range in two alias rows, counted as bins 0
    and nbins - 1; for finer bins the entries whose |c| may lie below S* = g_c / margin hold NaN, and
    only those: their pairs are all rechecked."""
    import torch
    print(f"[gpu] bin table entries {nbins} x {w}", flush=True)
    ws = torch.zeros(gc.workspace_bytes(nbins), dtype=torch.uint8, device="cuda")
    x = torch.tensor([0.5], dtype=torch.float32, device="cuda")
    bins = torch.empty(1, dtype=torch.int32, device="cuda")
    trip = torch.empty(1, dtype=torch.uint8, device="cuda")
    import ctypes
    _ptr = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    st = gc.load().gc_eval_angle_core(_ptr(x), None, 1, nbins, w, 32, _ptr(bins), _ptr(trip), None, None,
                                      _ptr(ws), ws.numel(), None)
    assert st == 0
    torch.cuda.synchronize()
    w_rad = np.radians(w)
    # M: ceil(4 / w), or the largest sound M >= 2.5 / w that lets two one-column workgroups share a
    # compute unit (3600 x 0.05 deg)
    m = int(gc.launch_plan(1000, 1000, nbins, w)["lut_m"])
    assert np.ceil(2.5 / w_rad) <= m <= np.ceil(4 / w_rad)
    if nbins == 720:
        assert m == np.ceil(4 / w_rad)
    off = ((nbins + 1) * 8 + 255) // 256 * 256
    tab = ws[off: off + (2 * m + 1) * 8].cpu().numpy().view(np.uint32).reshape(-1, 2)
    e = tab[:, 0].view(np.float32).astype(np.float64)
    nan = np.isnan(e)
    # row offsets: 4 bytes a row (one column) or 64 (sixteen columns, the layout chosen when two
    # workgroups' histograms fit in LDS); the alias rows follow the spare rows of that layout
    unit = 64 if nbins * 16 * 4 * 2 < 160 * 1024 else 4
    alias = nbins + 2 if unit == 64 else nbins + 65
    assert np.all(tab[:, 1] % unit == 0)
    b = tab[:, 1].astype(np.int64) // unit
    # the entries that must hold NaN: smallest |c| of the entry below S* (plan_lut's reading)
    q = np.arange(2 * m + 1)
    c_lo, c_hi = (q - 0.5) / m - 1, (q + 0.5) / m - 1
    s_min = np.where((c_lo <= 0) & (c_hi >= 0), 0.0, np.minimum(np.abs(c_lo), np.abs(c_hi)))
    c_edges = np.sqrt(2) * np.sin(np.arange(1, nbins + 1) * w_rad / 2)
    c_edges = np.where(np.arange(1, nbins + 1) * w <= 90, c_edges, -np.sqrt(2) * np.cos(np.arange(1, nbins + 1) * w_rad / 2))
    if nan.any():
        assert nan[m]
        s_star = s_min[nan].max()
        assert np.all(nan == (s_min <= s_star)) and s_star < 0.05
    else:
        assert e[m] == 0.0 and b[m] == alias
    frac = np.linspace(0.0, 1.0, 65)[:-1]
    c = (q[:, None] + frac[None, :] - 0.5) / m - 1.0
    c = np.clip(c, -1.0, 1.0)
    th = np.where(c >= 0, 2 * np.degrees(np.arcsin(np.minimum(c, 1) / np.sqrt(2))),
                  180 - 2 * np.degrees(np.arcsin(np.minimum(-c, 1) / np.sqrt(2))))
    xs = np.cos(np.radians(th))
    want = np.minimum(np.floor(th / w).astype(np.int64), nbins - 1)
    got = b[:, None] - (xs > e[:, None])
    if not nan.any():
        got = np.where(got == alias - 1, 0, np.where(got == alias, nbins - 1, got))
    # a sample within the fp32 rounding of the stored edge cosine may fall either way
    near = np.abs(xs - e[:, None]) < 1e-7
    ok = (got == want) | near | nan[:, None]
    assert np.all(ok), int((~ok).sum())
    # every edge is held by the entry its c rounds to (or that entry always rechecks)
    for k in range(1, nbins):
        th_e = k * w
        ce = np.sqrt(2) * np.sin(np.radians(th_e) / 2) if th_e <= 90 else -np.sqrt(2) * np.cos(np.radians(th_e) / 2)
        qe = int(np.rint(m * (ce + 1)))
        if nan[qe]:
            continue
        assert abs(e[qe] - np.cos(np.radians(th_e))) < 1e-7 and b[qe] == k, (k, qe, e[qe], b[qe])


@pytest.mark.parametrize("nbins,w", [(720, 0.25), (3600, 0.05), (1440, 0.125), (1500, 0.001)])
def test_duplicates_and_antipodes(gc, nbins, w):
    """Exact duplicate galaxies (cosine 1: separation 0) and exact antipodes (cosine -1: 180 deg)
    exercise each fast core's ends: the bin table's middle entry (both ends at once, in its alias
    rows at 720 bins, always rechecked at 3600 and 1440 bins), the series core's t = 0 and x < 0."""
    print(f"[gpu] duplicates and antipodes nbins={nbins}", flush=True)
    rng = np.random.default_rng(nbins)
    base = catalogs.uniform_sphere(400, seed=nbins) if nbins * w >= 180 else catalogs.Catalog(
        rng.uniform(0, 60, 400).astype(np.float32), rng.uniform(-60, 60, 400).astype(np.float32))

    def build(idx, flip):
        ra = base.ra[idx].astype(np.float64)
        dec = base.dec[idx].astype(np.float64)
        ra = np.where(flip, np.mod(ra + 10800.0, 21600.0), ra)
        dec = np.where(flip, -dec, dec)
        return catalogs.Catalog(ra.astype(np.float32), dec.astype(np.float32))

    idx_d = rng.integers(0, 400, 2200)
    idx_r = rng.integers(0, 400, 1900)
    D = build(idx_d, rng.random(2200) < 0.3)
    R = build(idx_r, rng.random(1900) < 0.5)
    fams = oracle_fams(D, R, nbins, w)
    t = run_gpu(gc, D, R, nbins, w)
    check_against(f"duplicates {nbins}", t[:3], fams, len(D), len(R))
    # one point and its antipode only: DD all at 0, DR all in the last bin
    P = build(np.zeros(700, np.int64), np.zeros(700, bool))
    Q = build(np.zeros(600, np.int64), np.ones(600, bool))
    dd, dr, rr, tot, _ = run_gpu(gc, P, Q, nbins, w)
    assert dd[0] == 700 * 700 and dr[nbins - 1] == 700 * 600 and rr[0] == 600 * 600
    assert list(tot) == [700 * 700, 700 * 600, 600 * 600]


@pytest.mark.parametrize("nbins,w,want", [
    (720, 0.25, dict(core=2, i_per_lane=2, hist_columns=16, waves_per_group=16, l1_share=1, always_recheck=0)),
    (3600, 0.05, dict(core=2, i_per_lane=2, hist_columns=1, waves_per_group=16, l1_share=4, lut_m=3167,
                      always_recheck=1)),
    (1440, 0.125, dict(core=2, i_per_lane=2, hist_columns=1, waves_per_group=16, l1_share=3, lut_m=1834)),
    (1500, 0.001, dict(core=2, dot_precision=64, i_per_lane=4, lut_m=0)),
])
def test_launch_plan_choices(gc, nbins, w, want):
    """The planner's choices for representative bins (each the fastest layout measured for its
    case): the sixteen-column table at 720 bins with every read from LDS; for finer bins one
    column in two workgroups of 16 waves per compute unit, the 3600-bin table shrunk to M = 3167
    so that they fit, with three sixteenths (51 KB table) or a quarter (29 KB) of the reads
    through the L1; the fp64 series core for the patch's 0.001 deg bins.  The results do not depend on these
    choices (the tuning tests); this pins the choices themselves."""
    p = gc.launch_plan(100000, 100000, nbins, w)
    print(f"[gpu] launch plan {nbins} x {w}: {p}", flush=True)
    for k, v in want.items():
        assert p[k] == v, (k, p)
    if p["hist_columns"] == 1 and p["i_per_lane"] == 2:
        assert 2 * p["lds_bytes"] <= 160 * 1024 and p["blocks_per_cu"] % 2 == 0  # two workgroups per CU


@pytest.mark.parametrize("nbins,w,tuning", [(3600, 0.05, dict(fast_core=1)), (3600, 0.05, dict(i_per_lane=4)),
                                            (3600, 0.05, dict(i_per_lane=2)), (3600, 0.05, dict(waves_per_group=8)),
                                            (3600, 0.05, dict(l1_share=2)), (3600, 0.05, dict(l1_share=3, i_per_lane=4)),
                                            (3600, 0.05, dict(l1_share=4)), (3600, 0.05, dict(l1_share=4, i_per_lane=4)),
                                            (3600, 0.05, dict(flush_interval=5)), (3600, 0.05, dict(dot_precision=64)),
                                            (3601, 0.0499972, dict(fast_core=1))])
def test_fine_bin_table_tuning_invariance(gc, nbins, w, tuning):
    """Bins through the fine bin table (one-column histogram in workgroups of 16 waves, entries near
    0 and 180 deg always rechecked) against the arccos core, other galaxies per lane (2, 4; K = 4
    takes the table of M = ceil(4 / w), the default a smaller one), other workgroup sizes and L1
    shares, frequent flushes and the fp64 dot: the same histograms, all within the oracle's edge
    flow; 3601 x 0.0499972 deg puts the edges off the round angles."""
    print(f"[gpu] fine bin table nbins={nbins} w={w} tuning {tuning}", flush=True)
    D, R = catalogs.WORKLOADS["clustered100k_3600"].catalogs(n=5000)
    fams = oracle_fams(D, R, nbins, w)
    base = run_gpu(gc, D, R, nbins, w)
    check_against("fine bin table", base[:3], fams, len(D), len(R), base[4])
    t = run_gpu(gc, D, R, nbins, w, tuning=gc.Tuning(**tuning))
    for x, y in zip(base[:3], t[:3]):
        np.testing.assert_array_equal(x, y)


def test_concurrent_streams_and_threads(gc):
    """Two host threads, each with its own stream, workspace and outputs, run whole jobs at once
    (the launch planner's device cache is shared); every result equals the sequential one."""
    import threading
    import torch
    print("[gpu] concurrent streams and threads", flush=True)
    jobs = []
    for name, nbins, w in [("clustered100k_720", 720, 0.25), ("patch100k_1500", 1500, 0.001),
                           ("clustered100k_3600", 3600, 0.05)]:
        D, R = catalogs.WORKLOADS[name].catalogs(n=3000)
        jobs.append((D, R.subset(0, 2500), nbins, w))
    want = [run_gpu(gc, D, R, nbins, w) for D, R, nbins, w in jobs]
    got = [[None] * len(jobs) for _ in range(2)]
    errors = []

    def worker(t):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for q in range(3):  # several rounds, so the two threads overlap
                    for k, (D, R, nbins, w) in enumerate(jobs):
                        pd = gc.prepare(_dev(D.ra), _dev(D.dec))
                        pr = gc.prepare(_dev(R.ra), _dev(R.dec))
                        out = torch.empty((3, nbins), dtype=torch.int64, device="cuda")
                        gc.histogram_dd_dr_rr(pd, len(D), pr, len(R), nbins, w, out=out)
                        om = gc.omega(out[0], out[1], out[2], len(D), len(R))
                        s.synchronize()
                        got[t][k] = (out.cpu().numpy().view(np.uint64).copy(), om.cpu().numpy())
        except Exception as e:  # reported by the main thread
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(2)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    assert not errors, errors
    for t in range(2):
        for k in range(len(jobs)):
            h, om = got[t][k]
            for f in range(3):
                assert np.array_equal(h[f], want[k][f]), (t, k, f)
            assert np.array_equal(np.isnan(om), np.isnan(want[k][4]))
            ok = ~np.isnan(om)
            assert np.array_equal(om[ok], want[k][4][ok])


@pytest.mark.parametrize("name,nbins,w", [("clustered100k_720", 720, 0.25), ("clustered100k_3600", 3600, 0.05),
                                          ("patch100k_1500", 1500, 0.001)])
def test_hip_graph_replay(gc, name, nbins, w):
    """The whole job (prepare x2, histograms, totals, omega) captured once in a HIP graph: the
    library makes no allocation, memset or synchronisation, so every call only enqueues kernels.
    Each replay, with eager work and synchronisation between replays, equals the eager result,
    also after the input buffers receive other catalogs."""
    import torch
    print(f"[gpu] HIP graph replay {name}", flush=True)
    n_d, n_r = 3000, 2500
    D, R = catalogs.WORKLOADS[name].catalogs(n=n_d)
    R = R.subset(0, n_r)
    D2, R2 = catalogs.WORKLOADS[name].catalogs(n=2 * n_d)
    D2, R2 = D2.subset(n_d, 2 * n_d), R2.subset(n_d, n_d + n_r)
    ra_d, dec_d, ra_r, dec_r = (_dev(a) for a in (D.ra, D.dec, R.ra, R.dec))
    pd = torch.empty(gc.prepared_bytes(n_d), dtype=torch.uint8, device="cuda")
    pr = torch.empty(gc.prepared_bytes(n_r), dtype=torch.uint8, device="cuda")
    out = torch.empty((3, nbins), dtype=torch.int64, device="cuda")
    ws = torch.empty(gc.workspace_bytes(nbins), dtype=torch.uint8, device="cuda")
    tot = torch.empty(3, dtype=torch.int64, device="cuda")
    om = torch.empty(nbins, dtype=torch.float64, device="cuda")

    def job():
        gc.prepare(ra_d, dec_d, out=pd)
        gc.prepare(ra_r, dec_r, out=pr)
        gc.histogram_dd_dr_rr(pd, n_d, pr, n_r, nbins, w, out=out, workspace=ws)
        gc.histogram_totals(out[0], out[1], out[2], out=tot)
        gc.omega(out[0], out[1], out[2], n_d, n_r, out=om)

    def state():
        torch.cuda.synchronize()
        return out.cpu().numpy().copy(), tot.cpu().numpy().copy(), om.cpu().numpy().copy()

    def same(a, b):
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
        assert np.array_equal(np.isnan(a[2]), np.isnan(b[2]))
        ok = ~np.isnan(a[2])
        assert np.array_equal(a[2][ok], b[2][ok])

    job()  # eager, also fills the planner's device cache before capture
    ref = state()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        job()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        job()
    for rep in range(3):
        out.fill_(-1)
        tot.fill_(-1)
        om.fill_(0.0)
        torch.cuda.synchronize()
        g.replay()
        got = state()
        same(got, ref)
        assert [int(t) for t in got[1]] == [n_d * n_d, n_d * n_r, n_r * n_r], rep
    # other catalogs in the same buffers: the replay follows them
    for dst, src in zip((ra_d, dec_d, ra_r, dec_r), (D2.ra, D2.dec, R2.ra, R2.dec)):
        dst.copy_(_dev(src))
    job()
    ref2 = state()
    assert not np.array_equal(ref2[0], ref[0])
    for rep in range(2):
        out.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        same(state(), ref2)


def test_identical_galaxies_past_the_flush_interval(gc):
    """2.4M copies of one galaxy: every DD pair lands in bin 0 (weight 2 off the diagonal), so a
    shared histogram word grows at the largest possible rate and the automatic flush interval
    (about 5.2e5 j-steps a wave between flushes) is crossed several times; DD[0] = N^2 exactly."""
    import torch
    n = 2_400_000
    print(f"[gpu] {n} identical galaxies", flush=True)
    ra = torch.full((n,), 1234.5, dtype=torch.float32, device="cuda")
    dec = torch.full((n,), -321.25, dtype=torch.float32, device="cuda")
    pd = gc.prepare(ra, dec)
    dd, dr, rr = gc.histogram_dd_dr_rr(pd, n, None, 0, 720, 0.25)
    torch.cuda.synchronize()
    h = dd.cpu().numpy().view(np.uint64)
    assert int(h[0]) == n * n and int(h[1:].sum()) == 0
    assert int(dr.cpu().numpy().view(np.uint64).sum()) == 0 and int(rr.cpu().numpy().view(np.uint64).sum()) == 0


def test_library_loaded_before_torch(gc):
    """A program that loads the library before it imports torch still runs on the GPU (the
    binding imports torch first, so that the process holds one HIP runtime)."""
    import subprocess
    import sys
    print("[gpu] load order", flush=True)
    code = ("import numpy as np\n"
            "import two_point_angular_amd as g\n"
            "g.load()\n"
            "import torch\n"
            "ra = torch.tensor([0.0, 70.0], device='cuda'); dec = torch.zeros(2, device='cuda')\n"
            "p = g.prepare(ra, dec)\n"
            "dd, dr, rr = g.histogram_dd_dr_rr(p, 2, p, 2, 720, 0.25)\n"
            "h = dd.cpu().numpy()\n"
            "assert int(h[0]) == 2 and int(h[4]) == 2 and int(h.sum()) == 4, h\n"
            "print('ok')\n")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120,
                       cwd=os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    print(r.stdout, r.stderr[-2000:], flush=True)
    assert r.returncode == 0 and "ok" in r.stdout
