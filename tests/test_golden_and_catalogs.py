"""Generators are deterministic and the stored oracle fixtures match them."""
import os

import numpy as np
import pytest

from oracle import oracle
from two_point_angular_amd import catalogs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def read_fixture(name):
    path = os.path.join(GOLDEN, f"oracle_{name}.txt")
    if not os.path.exists(path):
        return None
    meta, rows = {}, []
    with open(path) as f:
        for line in f:
            if line.startswith("#"):
                parts = line[1:].split()
                if len(parts) == 2:
                    meta[parts[0]] = parts[1]
                continue
            rows.append([int(v) for v in line.split()])
    a = np.array(rows, dtype=np.uint64)
    fams = {}
    for k, fam in enumerate(oracle.FAMILIES):
        fams[fam] = oracle.FamilyResult(a[:, 1 + k].copy(), a[:, 4 + 2 * k].copy(), a[:, 5 + 2 * k].copy())
    return meta, fams


def test_catalog_ranges_and_determinism():
    for name, wl in catalogs.WORKLOADS.items():
        D, R = wl.catalogs(n=5000)
        for c in (D, R):
            assert c.ra.dtype == np.float32 and len(c) == 5000
            assert np.all(np.isfinite(c.ra)) and np.all(np.isfinite(c.dec))
            assert c.ra.min() >= 0 and c.ra.max() <= 21600
            assert c.dec.min() >= -5400 and c.dec.max() <= 5400
        if wl.kind == "patch":
            assert D.ra.max() < 120.0001 and D.dec.max() < 120.0001
        D2, R2 = wl.catalogs(n=5000)
        assert D.sha256() == D2.sha256() and R.sha256() == R2.sha256()


def test_clustered_catalog_is_clustered():
    D = catalogs.clustered(20000, 1)
    u = catalogs.uniform_sphere(20000, 1)
    a = np.radians(D.ra / 60.0); d = np.radians(D.dec / 60.0)
    v = np.stack([np.cos(d) * np.cos(a), np.cos(d) * np.sin(a), np.sin(d)], 1)
    # fraction of galaxies with a neighbour within 0.5 deg among the first 2000
    c = v[:2000] @ v.T
    close = (c > np.cos(np.radians(0.5))).sum(1) - 1
    au = np.radians(u.ra / 60.0); du = np.radians(u.dec / 60.0)
    vu = np.stack([np.cos(du) * np.cos(au), np.cos(du) * np.sin(au), np.sin(du)], 1)
    cu = vu[:2000] @ vu.T
    close_u = (cu > np.cos(np.radians(0.5))).sum(1) - 1
    assert (close > 0).mean() > 0.5 > (close_u > 0).mean()


@pytest.mark.parametrize("name", ["uniform10k_720", "clustered100k_720", "clustered100k_3600",
                                  "patch100k_1500"])
def test_fixture_matches_generators(name):
    fx = read_fixture(name)
    if fx is None:
        pytest.skip(f"fixture for {name} not generated")
    meta, fams = fx
    wl = catalogs.WORKLOADS[name]
    D, R = wl.catalogs()
    assert meta["sha256_D"] == D.sha256()
    assert meta["sha256_R"] == R.sha256()
    assert int(meta["nbins"]) == wl.nbins and float(meta["width_deg"]) == wl.bin_width_deg
    for fam in oracle.FAMILIES:
        assert int(fams[fam].hist.sum()) == wl.n * wl.n


def test_small_fixture_reproduces():
    fx = read_fixture("uniform10k_720")
    assert fx is not None
    _, fams = fx
    wl = catalogs.WORKLOADS["uniform10k_720"]
    D, R = wl.catalogs()
    res = oracle.histograms(D.ra, D.dec, R.ra, R.dec, wl.nbins, wl.bin_width_deg)
    for fam in oracle.FAMILIES:
        np.testing.assert_array_equal(res.family(fam).hist, fams[fam].hist)
        np.testing.assert_array_equal(res.family(fam).lo, fams[fam].lo)
        np.testing.assert_array_equal(res.family(fam).hi, fams[fam].hi)
