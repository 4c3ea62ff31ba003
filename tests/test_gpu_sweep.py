"""A seeded sweep of bin counts, widths and catalog shapes against the fp64 oracle.

Each case draws a regime (bins covering 180 degrees, fine bins on a narrow range, bins covering
part of the sky or reaching far past 180 degrees, widths that divide 90 degrees and widths just
off them), sizes from 1 to 1500 galaxies (R may be empty) and catalogs (clustered, uniform or a
2 x 2 degree patch), so that every core and launch plan the library chooses is met at shapes
no other test fixes.  Every family must pass the edge-flow check (totals exact, every net move
between bins explained by pairs within 1e-5 degrees of the edge, at most 1e-6 N_a N_b moved pairs).
Only the two tests of bins narrower than the window, over near-duplicate galaxies, waive the
moved-pair budget, for the reason their docstrings give."""
import numpy as np
import pytest

from oracle import oracle
from two_point_angular_amd import catalogs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gc():
    import torch
    import two_point_angular_amd as gcm
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gcm.load()
    return gcm


def draw_case(rng):
    regime = int(rng.integers(0, 5))
    if regime == 0:    # bins covering 180 degrees, 2 .. 8192 of them
        nbins = int(rng.integers(2, 8193))
        w = 180.0 / nbins * float(rng.uniform(1.0, 1.002))
    elif regime == 1:  # fine bins on a narrow range (fp64 dot)
        nbins = int(rng.integers(1, 8193))
        w = float(10 ** rng.uniform(-4, -2))
    elif regime == 2:  # part of the sky, or far past 180 degrees
        nbins = int(rng.integers(1, 4000))
        w = float(rng.uniform(0.01, 1.0))
    elif regime == 3:  # widths that divide 90 degrees
        w = float(rng.choice([0.05, 0.1, 0.125, 0.25, 0.5, 1.0, 2.0, 5.0]))
        nbins = int(np.ceil(180 / w))
    else:              # widths just off round values
        w = float(rng.choice([0.05, 0.1, 0.25])) * float(1 + rng.uniform(-1e-4, 1e-4))
        nbins = int(np.ceil(180 / w - 0.5))
    nbins = max(1, min(nbins, 8192))
    n_d, n_r = int(rng.integers(1, 1500)), int(rng.integers(0, 1500))
    kind = int(rng.integers(0, 3))
    if kind == 0:
        D = catalogs.clustered(n_d, int(rng.integers(1, 1000)))
        R = catalogs.uniform_sphere(max(n_r, 1), int(rng.integers(1, 1000))).subset(0, n_r)
    elif kind == 1:
        D = catalogs.uniform_sphere(n_d, int(rng.integers(1, 1000)))
        R = catalogs.uniform_sphere(max(n_r, 1), int(rng.integers(1, 1000))).subset(0, n_r)
    else:
        D = catalogs.Catalog(rng.uniform(0, 120, n_d).astype(np.float32), rng.uniform(0, 120, n_d).astype(np.float32))
        R = catalogs.Catalog(rng.uniform(0, 120, n_r).astype(np.float32), rng.uniform(0, 120, n_r).astype(np.float32))
    return regime, kind, nbins, w, D, R


MOVED_BUDGET = 1e-6


def run_case(gc, nbins, w, D, R, budget=MOVED_BUDGET):
    import torch
    n_d, n_r = len(D), len(R)
    pd = gc.prepare(torch.from_numpy(D.ra).cuda(), torch.from_numpy(D.dec).cuda())
    pr = gc.prepare(torch.from_numpy(R.ra).cuda(), torch.from_numpy(R.dec).cuda()) if n_r else None
    dd, dr, rr = gc.histogram_dd_dr_rr(pd, n_d, pr, n_r, nbins, w)
    torch.cuda.synchronize()
    h = [x.cpu().numpy().view(np.uint64).astype(np.int64) for x in (dd, dr, rr)]
    res = oracle.histograms(D.ra, D.dec, R.ra, R.dec, nbins, w)
    want = {"DD": n_d * n_d, "DR": n_d * n_r, "RR": n_r * n_r}
    return [(f, oracle.flow_check(h[k], res.family(f), want[f], moved_budget=budget))
            for k, f in enumerate(oracle.FAMILIES)]


@pytest.mark.parametrize("seed", [1, 2, 3, 4, 5, 6])
def test_seeded_sweep(gc, seed):
    rng = np.random.default_rng(seed)
    for c in range(30):
        regime, kind, nbins, w, D, R = draw_case(rng)
        print(f"[gpu] sweep seed {seed} case {c}: regime {regime} kind {kind} nbins {nbins} w {w!r} "
              f"n {len(D)},{len(R)}", flush=True)
        for f, rep in run_case(gc, nbins, w, D, R):
            assert rep.ok, f"seed {seed} case {c} (nbins {nbins}, w {w!r}) {f}: {rep.message}"


@pytest.mark.parametrize("nbins,w,kind", [
    (2994, 0.7881125095716911, "uniform"),    # x < 0 in the bin table's middle entry: the bin of 180 deg
    (3991, 0.5715292422229417, "clustered"),  # an edge past 180 deg must not enter the bin table
    (1735, 0.6798535794426259, "uniform"),
    (800, 0.3, "clustered"),                  # 240 deg of bins, 180 / w an integer (no bin table)
])
def test_bins_reaching_past_180_degrees(gc, nbins, w, kind):
    """Bins that reach far past 180 degrees: every pair still lands in the bin of its angle (the
    largest angles in bin floor(180 / w), none past it)."""
    print(f"[gpu] bins past 180 deg: {nbins} x {w}", flush=True)
    base = catalogs.uniform_sphere(1000, 41) if kind == "uniform" else catalogs.clustered(1000, 43)
    # near-antipodes and near-duplicates of the first 200 galaxies: pairs within a fraction of a
    # degree of 0 and of 180 degrees, the bin table's middle entry
    a, d = base.ra[:200].astype(np.float64), base.dec[:200].astype(np.float64)
    anti_ra, anti_dec = (a + 10800.0 + 0.2) % 21600.0, -d
    dup_ra, dup_dec = (a + 0.3) % 21600.0, d
    D = catalogs.Catalog(np.concatenate([base.ra, anti_ra.astype(np.float32), dup_ra.astype(np.float32)]),
                         np.concatenate([base.dec, anti_dec.astype(np.float32), dup_dec.astype(np.float32)]))
    R0 = catalogs.uniform_sphere(900, 42)
    R = catalogs.Catalog(np.concatenate([R0.ra, anti_ra.astype(np.float32)]),
                         np.concatenate([R0.dec, anti_dec.astype(np.float32)]))
    for f, rep in run_case(gc, nbins, w, D, R):
        assert rep.ok, f"{f}: {rep.message}"


@pytest.mark.parametrize("nbins,w", [(3, 1e-7), (100, 1e-7), (8192, 1e-7), (100, 1e-6), (1, 1e-7)])
def test_bins_narrower_than_the_parity_window(gc, nbins, w):
    """Bins far narrower than the 1e-5 deg parity window, over near-duplicate galaxies (offsets
    down to 1e-5 arcmin, most of them rounded to an fp32 neighbour or to the same value): the
    fp64 angle itself cannot place such pairs (1 - cos is a few fp64 ulps), so the GPU may put
    them in any bin within the window of their oracle angle, and the check counts each pair at
    every edge within that window.  For the same reason the 1e-6 N_a N_b budget on moved pairs is
    waived here: the fp64 angle of a near-duplicate pair is itself uncertain by more than a bin, so
    how many of them land across an edge is not fixed by the definition (every move must still be
    explained by pairs within 1e-5 deg of that edge)."""
    print(f"[gpu] bins narrower than the window: {nbins} x {w}", flush=True)
    rng = np.random.default_rng(nbins)
    base = catalogs.uniform_sphere(800, 51)
    ra, dec = base.ra.astype(np.float64), base.dec.astype(np.float64)
    j = rng.integers(0, 100, 400)
    ra[100:500] = ra[j] + rng.normal(0, 1, 400) * 10 ** rng.uniform(-5, 0, 400)
    dec[100:500] = np.clip(dec[j] + rng.normal(0, 1, 400) * 10 ** rng.uniform(-5, 0, 400), -5400, 5400)
    D = catalogs.Catalog(ra.astype(np.float32), dec.astype(np.float32))
    R = catalogs.uniform_sphere(600, 52)
    for f, rep in run_case(gc, nbins, w, D, R, budget=1.0):
        assert rep.ok, f"{f}: {rep.message}"


def test_seeded_sweep_mid_sizes(gc):
    """Eight draws of 3k to 20k galaxies (R of 0 to 20k), where the grid holds from a part of one
    round of workgroups to several, every family has full i-blocks and a ragged one, and the
    workgroups' step shares and chunks cross block boundaries: the workloads' bin counts (180 to
    7200 bins over 180 degrees, and widths of 0.01 to 0.5 deg that stop short of it), over
    clustered, uniform and 2 x 2 degree catalogs.  Every family passes the edge-flow check within
    the 1e-6 N_a N_b moved-pair budget."""
    rng = np.random.default_rng(303)
    for c in range(8):
        n_d, n_r = int(rng.integers(3000, 20000)), int(rng.integers(0, 20000))
        nbins = int(rng.choice([180, 360, 720, 1440, 1500, 3600, 7200]))
        w = 180.0 / nbins if rng.random() < 0.7 else float(rng.uniform(0.01, 0.5))
        kind = int(rng.integers(0, 3))
        seed = int(rng.integers(1, 10**6))
        if kind == 0:
            D = catalogs.clustered(n_d, seed)
        elif kind == 1:
            D = catalogs.uniform_sphere(n_d, seed)
        else:
            D = catalogs.patch(n_d, seed)
        R = catalogs.uniform_sphere(max(n_r, 1), int(rng.integers(1, 10**6))).subset(0, n_r)
        print(f"[gpu] mid-size sweep case {c}: nbins {nbins} w {w!r} kind {kind} n {n_d},{n_r} "
              f"plan {gc.launch_plan(n_d, n_r, nbins, w)}", flush=True)
        for f, rep in run_case(gc, nbins, w, D, R):
            assert rep.ok, f"case {c} (nbins {nbins}, w {w!r}, n {n_d},{n_r}) {f}: {rep.message}"


def test_seeded_sweep_narrow_widths(gc):
    """20 random widths, log-uniform over 1e-7 .. 0.03 deg, and 1 .. 8192 bins, over catalogs half
    made of near-duplicates (offsets 1e-6 .. 1 arcmin around an eighth of the galaxies), R of 0 to
    1200 galaxies: every family passes the edge-flow check.  The moved-pair budget is waived as in
    the test above: half of each catalog is near-duplicates, whose fp64 angles are uncertain by
    more than the narrowest bins (the check still requires every move to lie within 1e-5 deg of
    its edge)."""
    rng = np.random.default_rng(201)
    for c in range(20):
        w = float(10 ** rng.uniform(-7, -1.5))
        nbins = int(rng.integers(1, 8193))
        n = int(rng.integers(200, 1500))
        seed = int(rng.integers(1, 10**6))
        base = catalogs.uniform_sphere(n, seed) if rng.random() < 0.5 else catalogs.clustered(n, seed)
        ra, dec = base.ra.astype(np.float64), base.dec.astype(np.float64)
        m = n // 2
        j = rng.integers(0, n // 8, m)
        lo_exp = rng.uniform(-6, -2)
        ra[n - m:] = ra[j] + rng.normal(0, 1, m) * 10 ** rng.uniform(lo_exp, 0, m)
        dec[n - m:] = np.clip(dec[j] + rng.normal(0, 1, m) * 10 ** rng.uniform(lo_exp, 0, m), -5400, 5400)
        D = catalogs.Catalog(ra.astype(np.float32), dec.astype(np.float32))
        n_r = int(rng.integers(0, 1200))
        R = catalogs.uniform_sphere(max(n_r, 1), int(rng.integers(1, 10**6))).subset(0, n_r)
        print(f"[gpu] narrow sweep case {c}: nbins {nbins} w {w!r} n {n},{n_r}", flush=True)
        for f, rep in run_case(gc, nbins, w, D, R, budget=1.0):
            assert rep.ok, f"case {c} (nbins {nbins}, w {w!r}) {f}: {rep.message}"


def test_seeded_sweep_tunings_and_parts(gc):
    """The same draws under random launch-plan overrides (dot precision, galaxies per lane,
    workgroups per CU, histogram placement, span core, fast core, flush interval, and the bin
    table's histogram columns, workgroup size and L1 share), as one call
    or as 2 to 40 additive parts.  An override the bins cannot take is refused with
    GC_ERR_INVALID_ARGUMENT; every accepted case passes the edge-flow check."""
    import torch
    rng = np.random.default_rng(21)
    accepted = 0
    for c in range(90):
        regime, kind, nbins, w, D, R = draw_case(rng)
        tun = {}
        if rng.random() < 0.7:
            tun = dict(dot_precision=int(rng.choice([0, 32, 64])), i_per_lane=int(rng.choice([0, 2, 4, 8])),
                       blocks_per_cu=int(rng.choice([0, 0, 1, 2, 3])), shared_histogram=int(rng.choice([0, 1, 2])),
                       span_kernel=int(rng.choice([0, 1, 2])), fast_core=int(rng.choice([0, 1, 2])),
                       flush_interval=int(rng.choice([0, 0, 1, 7, 100])),
                       hist_columns=int(rng.choice([0, 0, 1, 16])), waves_per_group=int(rng.choice([0, 0, 4, 8, 16])),
                       l1_share=int(rng.choice([0, 1, 2, 3, 4])))
        parts = int(rng.choice([1, 1, 1, 2, 3, 7, 40]))
        print(f"[gpu] sweep+tuning case {c}: nbins {nbins} w {w!r} n {len(D)},{len(R)} parts {parts} {tun}",
              flush=True)
        n_d, n_r = len(D), len(R)
        pd = gc.prepare(torch.from_numpy(D.ra).cuda(), torch.from_numpy(D.dec).cuda())
        pr = gc.prepare(torch.from_numpy(R.ra).cuda(), torch.from_numpy(R.dec).cuda()) if n_r else None
        t = gc.Tuning(**tun)
        try:
            if parts == 1:
                out = torch.empty((3, nbins), dtype=torch.int64, device="cuda")
                gc.histogram_dd_dr_rr(pd, n_d, pr, n_r, nbins, w, out=out, tuning=t)
            else:
                out = torch.zeros((3, nbins), dtype=torch.int64, device="cuda")
                for p in range(parts):
                    gc.histogram_part(pd, n_d, pr, n_r, nbins, w, p, parts, out=out, tuning=t)
        except gc.GCError as e:
            assert e.status == 1, e  # an override these bins cannot take
            continue
        accepted += 1
        torch.cuda.synchronize()
        h = [x.astype(np.int64) for x in out.cpu().numpy().view(np.uint64)]
        res = oracle.histograms(D.ra, D.dec, R.ra, R.dec, nbins, w)
        want = {"DD": n_d * n_d, "DR": n_d * n_r, "RR": n_r * n_r}
        for k, f in enumerate(oracle.FAMILIES):
            rep = oracle.flow_check(h[k], res.family(f), want[f], moved_budget=MOVED_BUDGET)
            assert rep.ok, f"case {c} (nbins {nbins}, w {w!r}, parts {parts}, {tun}) {f}: {rep.message}"
    assert accepted >= 60


def test_seeded_core_sweep_on_exact_cosines(gc):
    """For drawn bins and widths, the angle-to-bin core the planner picks, on fp32 and fp64
    cosines within 64 units in the last place of 400 edge cosines and on uniform ones: a fast bin
    the guard lets through equals the bin of the cosine's fp64 arccos, and so does the exact
    recheck's bin, except within 1e-5 degrees of an edge (where either side is right)."""
    import torch
    rng = np.random.default_rng(51)
    for c in range(30):
        regime, kind, nbins, w, D, R = draw_case(rng)
        print(f"[gpu] core sweep case {c}: nbins {nbins} w {w!r}", flush=True)
        e = np.arange(1, nbins)
        e = e[e * w < 180.0]
        if len(e) > 400:
            e = rng.choice(e, 400, replace=False)
        ce = np.cos(np.radians(e * w))
        offs = np.arange(-64, 65)
        for dtype in (np.float32, np.float64):
            base = ce.astype(dtype)
            if dtype == np.float32:
                bits = base.view(np.int32).astype(np.int64)
                allb = (bits[:, None] + np.where(base[:, None] >= 0, offs[None, :], -offs[None, :])).ravel()
                x = allb[(allb >= -2**31) & (allb < 2**31)].astype(np.int32).view(np.float32)
            else:
                x = (base[:, None] * (1 + offs[None, :] * 2.0**-50)).ravel()
            x = np.concatenate([x, rng.uniform(-1, 1, 20000).astype(dtype), np.array([1, -1, 0], dtype=dtype)])
            x = np.ascontiguousarray(x[np.isfinite(x) & (np.abs(x) <= 1.0)])
            b, trip, exact, _ = gc.eval_angle_core(torch.from_numpy(x).cuda(), nbins, w)
            torch.cuda.synchronize()
            b, trip, exact = (v.cpu().numpy().astype(np.int64) for v in (b, trip, exact))
            t = np.degrees(np.arccos(x.astype(np.float64))) / w
            truth = np.minimum(np.floor(t), nbins - 1).astype(np.int64)
            near = np.abs(t - np.round(t)) * w < 1e-5
            assert not ((exact != truth) & ~near).any(), (c, nbins, w, np.dtype(dtype).name)
            assert not ((trip == 0) & (b != truth) & ~near).any(), (c, nbins, w, np.dtype(dtype).name)
