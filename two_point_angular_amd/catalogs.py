"""Seeded synthetic galaxy catalogs (right ascension, declination) in arcminutes.

The workload on "CUDA Deep Dive: 10B Galaxy Pairs on an RTX 5080" (section "The problem")
is two catalogs of 100,000 galaxies each, one observed (D) and one random (R), given
as fp32 right ascension and declination in arcminutes. Those catalog files are not
available here, so these generators stand in for them with the same sizes and dtype.

This module only draws positions. It holds none of the pair-angle or binning
arithmetic, so both the fp64 oracle and the GPU library can be fed from it without
sharing any of the method's code.

Recipes (numpy ``Generator(PCG64(seed))``, fp64 draws, one final rounding to fp32):

* ``uniform_sphere(n, seed)``: u1 = U[0,1)^n, then u2 = U[0,1)^n;
  alpha = 21600 * u1, delta = asin(2*u2 - 1) * 10800/pi.
* ``clustered(n, seed)``: 200 centres drawn first, uniform on the sphere as above;
  then, per galaxy and in this order: membership m = U < 0.6, centre index in
  [0, 200), two tangent-plane Gaussian offsets (east, north) with sigma = 0.5 deg,
  and a uniform-sphere fallback position.  Members are placed at angular distance
  rho = hypot(east, north) along bearing beta = atan2(east, north) from their
  centre (spherical destination-point formula); the other 40 % take the fallback.
* ``patch(n, seed)``: alpha and delta uniform in [0, 120) arcmin (a 2 x 2 deg box).
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass

import numpy as np

ARCMIN_PER_RAD = 10800.0 / np.pi
FULL_CIRCLE_ARCMIN = 21600.0


@dataclass(frozen=True)
class Catalog:
    """One catalog: fp32 arrays of right ascension and declination in arcmin."""

    ra: np.ndarray
    dec: np.ndarray
    name: str = ""

    def __post_init__(self):
        if self.ra.dtype != np.float32 or self.dec.dtype != np.float32:
            raise TypeError("catalog arrays must be float32")
        if self.ra.shape != self.dec.shape or self.ra.ndim != 1:
            raise ValueError("ra and dec must be 1-D arrays of equal length")

    def __len__(self) -> int:
        return int(self.ra.shape[0])

    def sha256(self) -> str:
        h = hashlib.sha256()
        h.update(np.ascontiguousarray(self.ra).tobytes())
        h.update(np.ascontiguousarray(self.dec).tobytes())
        return h.hexdigest()

    def subset(self, start: int, stop: int) -> "Catalog":
        return Catalog(self.ra[start:stop].copy(), self.dec[start:stop].copy(),
                       f"{self.name}[{start}:{stop}]")


def _uniform_sphere_fp64(rng: np.random.Generator, n: int):
    u1 = rng.random(n)
    u2 = rng.random(n)
    ra = FULL_CIRCLE_ARCMIN * u1
    dec = np.arcsin(2.0 * u2 - 1.0) * ARCMIN_PER_RAD
    return ra, dec


def uniform_sphere(n: int, seed: int, name: str = "") -> Catalog:
    rng = np.random.Generator(np.random.PCG64(seed))
    ra, dec = _uniform_sphere_fp64(rng, n)
    return Catalog(ra.astype(np.float32), dec.astype(np.float32), name or f"uniform(n={n},seed={seed})")


def clustered(n: int, seed: int, n_centres: int = 200, member_frac: float = 0.6,
              sigma_deg: float = 0.5, name: str = "") -> Catalog:
    rng = np.random.Generator(np.random.PCG64(seed))
    c_ra, c_dec = _uniform_sphere_fp64(rng, n_centres)
    member = rng.random(n) < member_frac
    centre = rng.integers(0, n_centres, n)
    east = rng.normal(0.0, sigma_deg, n)
    north = rng.normal(0.0, sigma_deg, n)
    f_ra, f_dec = _uniform_sphere_fp64(rng, n)

    rho = np.radians(np.hypot(east, north))
    beta = np.arctan2(east, north)
    a_c = c_ra[centre] / ARCMIN_PER_RAD
    d_c = c_dec[centre] / ARCMIN_PER_RAD
    sin_d = np.sin(d_c) * np.cos(rho) + np.cos(d_c) * np.sin(rho) * np.cos(beta)
    d = np.arcsin(np.clip(sin_d, -1.0, 1.0))
    a = a_c + np.arctan2(np.sin(beta) * np.sin(rho) * np.cos(d_c),
                         np.cos(rho) - np.sin(d_c) * np.sin(d))
    ra_m = np.mod(a * ARCMIN_PER_RAD, FULL_CIRCLE_ARCMIN)
    dec_m = d * ARCMIN_PER_RAD

    ra = np.where(member, ra_m, f_ra)
    dec = np.where(member, dec_m, f_dec)
    return Catalog(ra.astype(np.float32), dec.astype(np.float32),
                   name or f"clustered(n={n},seed={seed})")


def patch(n: int, seed: int, side_arcmin: float = 120.0, name: str = "") -> Catalog:
    rng = np.random.Generator(np.random.PCG64(seed))
    ra = side_arcmin * rng.random(n)
    dec = side_arcmin * rng.random(n)
    return Catalog(ra.astype(np.float32), dec.astype(np.float32), name or f"patch(n={n},seed={seed})")


@dataclass(frozen=True)
class Workload:
    """A named (D, R, binning) configuration."""

    name: str
    n: int
    nbins: int
    bin_width_deg: float
    kind: str  # "uniform", "clustered" or "patch"

    def catalogs(self, n: int | None = None) -> tuple[Catalog, Catalog]:
        n = self.n if n is None else n
        if self.kind == "uniform":
            return uniform_sphere(n, 1, "D"), uniform_sphere(n, 2, "R")
        if self.kind == "clustered":
            return clustered(n, 1, name="D"), uniform_sphere(n, 2, "R")
        if self.kind == "patch":
            return patch(n, 1, name="D"), patch(n, 2, name="R")
        raise ValueError(self.kind)


# The five workloads.  Sizes and binnings follow the 100k + 100k problem statement;
# the small uniform case finishes on the CPU oracle in seconds.
WORKLOADS = {
    "uniform10k_720": Workload("uniform10k_720", 10_000, 720, 0.25, "uniform"),
    "clustered100k_720": Workload("clustered100k_720", 100_000, 720, 0.25, "clustered"),
    "clustered100k_3600": Workload("clustered100k_3600", 100_000, 3600, 0.05, "clustered"),
    "clustered1m_720": Workload("clustered1m_720", 1_000_000, 720, 0.25, "clustered"),
    "patch100k_1500": Workload("patch100k_1500", 100_000, 1500, 0.001, "patch"),
}


def write_text(cat: Catalog, path: str) -> None:
    """Write a catalog in the page's input format: the galaxy count, then one "alpha delta"
    line per galaxy in arcminutes.  Nine significant digits identify every fp32 value, so
    a reader that rounds correctly gets the same fp32 catalog back."""
    with open(path, "w") as f:
        f.write(f"{len(cat)}\n")
        f.write("".join(f"{a:.9g} {d:.9g}\n" for a, d in zip(cat.ra.tolist(), cat.dec.tolist())))


def _main(argv=None) -> int:
    import argparse
    ap = argparse.ArgumentParser(description="Write a workload's D and R catalogs as text files.")
    ap.add_argument("workload", choices=sorted(WORKLOADS))
    ap.add_argument("d_path")
    ap.add_argument("r_path")
    ap.add_argument("-n", type=int, default=None, help="first n galaxies only")
    a = ap.parse_args(argv)
    D, R = WORKLOADS[a.workload].catalogs(n=a.n)
    write_text(D, a.d_path)
    write_text(R, a.r_path)
    return 0


if __name__ == "__main__":
    raise SystemExit(_main())
