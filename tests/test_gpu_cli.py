"""The end-to-end program galaxy_gc on the GPU: text catalogs in, the page's omega.out out.

Its result file must equal, byte for byte, the file written from the library path's histograms
and omega for the same catalogs; those histograms must pass the edge-flow check against the
fp64 oracle; and every row of the file must agree with the oracle's counts where the oracle has
RR > 0 (a bin with RR = 0 has no row, as in the page's writer).
"""
import os
import subprocess

import numpy as np
import pytest

from oracle import oracle
from two_point_angular_amd import catalogs

pytestmark = pytest.mark.gpu

HEADER = "bin start\t\tomega\t        hist_DD\t        hist_DR\t        hist_RR"


@pytest.fixture(scope="module")
def gc():
    import torch
    import two_point_angular_amd as gcm
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gcm.load()
    if not os.path.exists(gcm.CLI_PATH):
        pytest.fail("galaxy_gc is not built (python -m two_point_angular_amd.build)")
    return gcm


def parse_result(path, nbins, w):
    lines = open(path).read().split("\n")
    assert lines[0] == HEADER and lines[-1] == ""
    hist = np.zeros((3, nbins), dtype=np.int64)
    om = np.full(nbins, np.nan)
    present = np.zeros(nbins, dtype=bool)
    for ln in lines[1:-1]:
        f = ln.split("\t")
        k = int(round(float(f[0]) / w))
        present[k] = True
        om[k] = float(f[1])
        hist[:, k] = [int(x) for x in f[2:]]
    return hist, om, present


@pytest.mark.parametrize("name,n,nbins,w", [("clustered100k_720", 3000, 720, 0.25),
                                            ("patch100k_1500", 3000, 1500, 0.001)])
def test_cli_end_to_end(gc, tmp_path, name, n, nbins, w):
    import torch
    print(f"[gpu] galaxy_gc {name} n={n} nbins={nbins}", flush=True)
    D, R = catalogs.WORKLOADS[name].catalogs(n=n)
    R = R.subset(0, n - 300)                                 # unequal sizes
    dp, rp, out = tmp_path / "D.txt", tmp_path / "R.txt", tmp_path / "omega.out"
    catalogs.write_text(D, str(dp))
    catalogs.write_text(R, str(rp))
    r = subprocess.run([gc.CLI_PATH, "--nbins", str(nbins), "--width", repr(w), str(dp), str(rp), str(out)],
                       capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0 and "(exact)" in r.stdout

    # the library path on the same catalogs, written by the same writer
    dev = "cuda"
    ra_d, dec_d = gc.read_catalog(str(dp))
    ra_r, dec_r = gc.read_catalog(str(rp))
    pd = gc.prepare(torch.from_numpy(ra_d).to(dev), torch.from_numpy(dec_d).to(dev))
    pr = gc.prepare(torch.from_numpy(ra_r).to(dev), torch.from_numpy(dec_r).to(dev))
    dd, dr, rr = gc.histogram_dd_dr_rr(pd, len(ra_d), pr, len(ra_r), nbins, w)
    om = gc.omega(dd, dr, rr, len(ra_d), len(ra_r))
    torch.cuda.synchronize()
    h = [x.cpu().numpy() for x in (dd, dr, rr)]
    ref = tmp_path / "ref.out"
    gc.write_omega(str(ref), *h, om.cpu().numpy(), w)
    assert out.read_bytes() == ref.read_bytes()

    # the library histograms against the oracle, and the file's rows against both
    res = oracle.histograms(D.ra, D.dec, R.ra, R.dec, nbins, w)
    fams = {f: res.family(f) for f in oracle.FAMILIES}
    want = {"DD": len(D) ** 2, "DR": len(D) * len(R), "RR": len(R) ** 2}
    for k, f in enumerate(oracle.FAMILIES):
        rep = oracle.flow_check(h[k].astype(np.int64), fams[f], want[f])
        assert rep.ok, f"{f}: {rep.message}"
    fh, fom, present = parse_result(str(out), nbins, w)
    assert np.array_equal(present, h[2] > 0)
    for k in range(3):
        assert np.array_equal(fh[k][present], h[k].astype(np.int64)[present])
    ora_om = oracle.omega(fams["DD"].hist, fams["DR"].hist, fams["RR"].hist, len(D), len(R))
    sel = present & (fams["RR"].hist >= 1000)
    assert np.all(np.abs(fom[sel] - ora_om[sel]) <= 1e-4 + 5e-7)


@pytest.mark.parametrize("n_d,n_r", [(0, 500), (1, 1), (700, 0)])
def test_cli_degenerate_catalogs(gc, tmp_path, n_d, n_r):
    """Empty and one-galaxy catalogs: the sums N_a N_b still hold (zero for an empty family) and
    the file equals the one written from the library path's histograms."""
    import torch
    print(f"[gpu] galaxy_gc degenerate n_d={n_d} n_r={n_r}", flush=True)
    nbins, w = 720, 0.25
    D, R = catalogs.WORKLOADS["clustered100k_720"].catalogs(n=1000)
    D, R = D.subset(0, n_d), R.subset(0, n_r)
    dp, rp, out = tmp_path / "D.txt", tmp_path / "R.txt", tmp_path / "omega.out"
    catalogs.write_text(D, str(dp))
    catalogs.write_text(R, str(rp))
    r = subprocess.run([gc.CLI_PATH, str(dp), str(rp), str(out)], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0 and "(exact)" in r.stdout
    assert f"DD {n_d * n_d}  DR {n_d * n_r}  RR {n_r * n_r} (exact)" in r.stdout
    dev = "cuda"
    pd = gc.prepare(torch.from_numpy(D.ra).to(dev), torch.from_numpy(D.dec).to(dev))
    pr = gc.prepare(torch.from_numpy(R.ra).to(dev), torch.from_numpy(R.dec).to(dev))
    dd, dr, rr = gc.histogram_dd_dr_rr(pd, n_d, pr, n_r, nbins, w)
    om = gc.omega(dd, dr, rr, n_d, n_r)
    torch.cuda.synchronize()
    ref = tmp_path / "ref.out"
    gc.write_omega(str(ref), *[x.cpu().numpy() for x in (dd, dr, rr)], om.cpu().numpy(), w)
    assert out.read_bytes() == ref.read_bytes()
    if n_r == 1:
        assert out.read_text().split("\n")[1].split("\t")[-1].strip() == "1"  # the one RR pair, bin 0
