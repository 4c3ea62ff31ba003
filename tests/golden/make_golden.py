"""Write the oracle's full-size histograms as text fixtures.

Calls only the CPU fp64 oracle (``oracle/``) and the seeded catalog generators.
Each fixture records the workload, the SHA-256 of both catalogs (so a generator
change is detected), and per bin: DD, DR, RR and, per family, the oracle's
near-edge counts lo/hi (ordered pairs within 1e-5 deg below / at-or-above the
bin's lower edge).

Usage: python tests/golden/make_golden.py [workload ...]
"""
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import oracle  # noqa: E402
from two_point_angular_amd import catalogs  # noqa: E402

DEFAULT = ["uniform10k_720", "clustered100k_720", "clustered100k_3600", "patch100k_1500"]


def path_for(name: str) -> str:
    return os.path.join(HERE, f"oracle_{name}.txt")


def write(name: str) -> str:
    wl = catalogs.WORKLOADS[name]
    D, R = wl.catalogs()
    t0 = time.time()
    res = oracle.histograms(D.ra, D.dec, R.ra, R.dec, wl.nbins, wl.bin_width_deg, symmetric=True)
    dt = time.time() - t0
    out = path_for(name)
    with open(out, "w") as f:
        f.write(f"# oracle histograms for workload {name}: n_d = n_r = {wl.n}, "
                f"{wl.nbins} bins of {wl.bin_width_deg} deg, generator kind {wl.kind}\n")
        f.write("# written by tests/golden/make_golden.py (CPU fp64 oracle, symmetric mode)\n")
        f.write(f"# sha256_D {D.sha256()}\n# sha256_R {R.sha256()}\n")
        f.write(f"# nbins {wl.nbins}\n# width_deg {wl.bin_width_deg!r}\n# n {wl.n}\n")
        f.write("# bin DD DR RR loDD hiDD loDR hiDR loRR hiRR\n")
        for b in range(wl.nbins):
            row = [b, res.dd.hist[b], res.dr.hist[b], res.rr.hist[b], res.dd.lo[b], res.dd.hi[b],
                   res.dr.lo[b], res.dr.hi[b], res.rr.lo[b], res.rr.hi[b]]
            f.write(" ".join(str(int(v)) for v in row) + "\n")
    print(f"{name}: {dt:.1f} s -> {out}", flush=True)
    return out


if __name__ == "__main__":
    for name in (sys.argv[1:] or DEFAULT):
        write(name)
