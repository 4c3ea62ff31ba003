"""The pair kernel's angle-to-bin core on the GPU, checked exhaustively near every bin edge.

For a pair whose true cosine is x, the kernel sees x~ with |x~ - x| <= g, where g is the
dot-product error bound (fp32 dot of fp32-rounded unit vectors: 5 * 2^-24; fp64 dot of
fp64 unit vectors: well under 1e-14).  The kernel either rechecks the pair in fp64 (trip)
or bins it from x~ alone.  Soundness: for every x~ that does not trip, every x in
[x~ - g, x~ + g] must truncate to the same bin (acos is monotone, so the two ends decide).
The cosines tested are every fp32 value within 4096 ulps of each edge's cosine (fp32
core), a dense fp64 sweep across each edge (fp64 core), and random cosines.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

G32 = 5.0 * 2.0 ** -24 * (1 + 1e-6) + 1e-12
# The bin-table core's fast steps take x~ from the matrix cores (v_mfma_f32_16x16x4f32), whose
# rounding is undocumented; its guard assumes |x~ - x| <= 12 * 2^-24 (five one-ulp roundings plus
# the fp32 rounding of both unit vectors), so its soundness is checked at that radius too.
G_LUT = 12.0 * 2.0 ** -24 * (1 + 1e-6) + 1e-12
G64 = 1e-14
# The exact recheck compares the fp64 cosine with fp64 edge cosines cos(e w).  Rounding
# cos(e w) to fp64 moves the edge by at most 2^-54 / sin(e w) rad (1.8e-10 deg at the first
# 0.001-deg edge), so it may disagree with truncating acos(x) / w only within that distance
# of an edge; 1e-8 deg bounds it for every binning here and is 1000x below 1e-5 deg.
NEAR_DEG = 1e-8


@pytest.fixture(scope="module")
def gc():
    import torch
    import two_point_angular_amd as gcm
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gcm.load()
    return gcm


def true_bins(x, nbins, w_deg):
    t = np.degrees(np.arccos(np.clip(x, -1.0, 1.0))) / w_deg
    return np.minimum(np.floor(t), nbins - 1).astype(np.int64), t


def run_core(gc, x, nbins, w):
    import torch
    xt = torch.from_numpy(x).to("cuda")
    b, trip, exact, _ = gc.eval_angle_core(xt, nbins, w)
    torch.cuda.synchronize()
    return b.cpu().numpy().astype(np.int64), trip.cpu().numpy().astype(bool), exact.cpu().numpy().astype(np.int64)


def edge_neighbourhood_f32(nbins, w_deg, ulps=4096):
    c = np.cos(np.radians(np.arange(1, nbins) * w_deg)).astype(np.float32)
    bits = c.view(np.int32).astype(np.int64)
    offs = np.arange(-ulps, ulps + 1, dtype=np.int64)
    # fp32 bit patterns are monotone in value within one sign; handle negatives separately
    allb = (bits[:, None] + np.where(c[:, None] >= 0, offs[None, :], -offs[None, :])).ravel()
    allb = allb[(allb >= np.int64(np.iinfo(np.int32).min)) & (allb <= np.int64(np.iinfo(np.int32).max))]
    x = allb.astype(np.int32).view(np.float32)
    return x[np.isfinite(x) & (np.abs(x) <= 1.0)]


def check_sound(x_exact_in, b, trip, nbins, w, g):
    keep = ~trip
    xk = x_exact_in[keep]
    lo, _ = true_bins(np.clip(xk + g, -1, 1), nbins, w)   # larger cosine -> smaller angle
    hi, _ = true_bins(np.clip(xk - g, -1, 1), nbins, w)
    bad = (lo != b[keep]) | (hi != b[keep])
    assert not bad.any(), (int(bad.sum()), xk[bad][:5], b[keep][bad][:5], lo[bad][:5], hi[bad][:5])


# (nbins, width): 720 x 0.25 deg bins through the bin table; 1440 x 0.125 and 3600 x 0.05 deg
# through the bin table with always-recheck entries near 0 and 180 deg, and 3601 x 0.0499972 deg,
# where the edges fall off the round angles; 1500 x 0.001 deg through the clamped arccos core.
FP32_CASES = [(720, 0.25), (1440, 0.125), (3600, 0.05), (3601, 0.0499972), (1500, 0.001)]


def uses_table(nbins, w):
    """The bin table serves fp32 bins covering 180 deg whose table (2 ceil(4 / w_rad) + 1 entries)
    fits its 14337-entry limit: widths down to about 0.032 deg."""
    return (nbins + 0.5) * w >= 180 and 2 * np.ceil(4 / np.radians(w)) + 1 <= 14337


@pytest.mark.parametrize("nbins,w", FP32_CASES)
def test_fp32_core_sound_near_edges(gc, nbins, w):
    print(f"[gpu] fp32 core near edges nbins={nbins}", flush=True)
    rng = np.random.default_rng(nbins)
    x = np.concatenate([edge_neighbourhood_f32(nbins, w),
                        rng.uniform(-1, 1, 2_000_000).astype(np.float32),
                        (1 - rng.random(200_000) * 1e-4).astype(np.float32),
                        np.array([1.0, -1.0, 0.0, -0.0, 0.5, -0.5], np.float32)])
    b, trip, exact = run_core(gc, x, nbins, w)
    xd = x.astype(np.float64)
    assert b.min() >= 0 and b.max() <= nbins - 1
    check_sound(xd, b, trip, nbins, w, G32)
    if uses_table(nbins, w):
        # every cosine within 4096 ulps of an edge (>= 4096 * 2^-25, far past 12 * 2^-24) is in x
        check_sound(xd, b, trip, nbins, w, G_LUT)
    tb, t = true_bins(xd, nbins, w)
    near = np.abs(t - np.round(t)) * w < NEAR_DEG
    assert np.all((exact == tb) | near)
    if nbins != 1500:
        r = trip[len(x) - 2_200_006: len(x) - 200_006].mean()
        assert r < 1.5e-2, r


# fp64 cores: 720 x 0.25 deg the generic core, 400 x 0.2 deg (80 deg) the narrow-range core,
# 1500 x 0.001 deg the series core.
FP64_CASES = [(720, 0.25), (400, 0.2), (1500, 0.001)]


def series_rho(nbins, w):
    """The series core's relative bound when it applies (bins ending by ~9 deg), else None."""
    th = (nbins + 1) * np.radians(w)
    if th >= np.pi / 2:
        return None
    y = 2 * np.sin(th / 2) ** 2
    q = 2 * np.arcsin(np.sqrt(y / 2)) / np.sqrt(y)
    r = (q - np.sqrt(2) * (1 + y / 12 + 3 * y * y / 160)) / q
    return 1.25 * (r + 7 * 2.0 ** -24) if 0 <= r <= 2e-8 else None


@pytest.mark.parametrize("nbins,w", FP64_CASES)
def test_fp64_core_sound_near_edges(gc, nbins, w):
    print(f"[gpu] fp64 core near edges nbins={nbins}", flush=True)
    rng = np.random.default_rng(nbins + 1)
    e = np.arange(1, nbins)
    u = np.linspace(-0.02, 0.02, 801)
    th = np.radians((e[:, None] + u[None, :]) * w).ravel()
    x = np.concatenate([np.cos(th), rng.uniform(-1, 1, 2_000_000),
                        np.cos(np.radians(rng.uniform(0, 3.0, 1_000_000))),
                        np.array([1.0, -1.0, 0.0, -0.0])])
    b, trip, exact = run_core(gc, x, nbins, w)
    assert b.min() >= 0 and b.max() <= nbins - 1
    check_sound(x, b, trip, nbins, w, G64)
    tb, t = true_bins(x, nbins, w)
    near = np.abs(t - np.round(t)) * w < NEAR_DEG
    assert np.all((exact == tb) | near)
    r = trip[len(th): len(th) + 2_000_000].mean()
    assert r < 1.5e-2, r


def _header_constant(name):
    import os
    path = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                        "two_point_angular_amd", "csrc", "gc_acos_poly.h")
    for line in open(path):
        parts = line.split()
        if len(parts) >= 3 and parts[0] == "#define" and parts[1] == name:
            return float(parts[2])
    raise KeyError(name)


def _core_t(gc, x, nbins, w):
    import torch
    xt = torch.from_numpy(x).to("cuda")
    _, trip, _, t = gc.eval_angle_core(xt, nbins, w, with_exact=False, with_t=True)
    torch.cuda.synchronize()
    return t.cpu().numpy().astype(np.float64), trip.cpu().numpy().astype(bool)


@pytest.mark.parametrize("nbins,w", FP32_CASES)
def test_fp32_core_error_within_model(gc, nbins, w):
    """The fp32 core's coordinate against its exact value for the same fp32 cosine, over every
    64th fp32 value in [-1, 1].  Arccos cores: the guard assumes |t~ - t| <= C(t) with
    C(t) = E_core / w + 2^-24 (t + 2h) (core error with a 1-ulp square root, plus the roundings
    that form t).  Bin-table core: c = copysign(sqrt(1 - |x|), x), and the guard assumes
    |c~ - c| s~ <= 1.5 * 2^-23 for the core's own roundings (subtraction, 1-ulp square root)."""
    print(f"[gpu] fp32 core error model nbins={nbins}", flush=True)
    pos = np.arange(0, np.float32(1.0).view(np.uint32) + 1, 64, dtype=np.uint32).view(np.float32)
    x = np.concatenate([pos, -pos[1:]]).astype(np.float32)
    t, _ = _core_t(gc, x, nbins, w)
    if uses_table(nbins, w):
        xd = x.astype(np.float64)
        c_exact = np.copysign(np.sqrt(1.0 - np.abs(xd)), xd)
        s = np.abs(t)
        ratio = np.abs(t - c_exact) * s / (1.5 * 2.0 ** -23)
        print(f"  max |c~ - c| s = {np.max(np.abs(t - c_exact) * s):.3e}; max ratio to the guard's core "
              f"term {ratio.max():.3f}", flush=True)
        assert ratio.max() <= 0.9
        return
    w_rad = np.radians(w)
    t_exact = np.arccos(x.astype(np.float64)) / w_rad
    err = np.abs(t - t_exact)
    e_core = (_header_constant("GC_ACOS_CORE_ERR") + 2.0 ** -24 * (np.pi / 2)) * 1.25
    h = (np.pi / 2) / w_rad
    bound = e_core / w_rad + 2.0 ** -24 * (t_exact + 2 * h) * 1.01
    ratio = err / bound
    print(f"  max |t~ - t| = {err.max():.3e} bins; max ratio to the guard's bound {ratio.max():.3f}", flush=True)
    assert ratio.max() <= 1.0
    # the margin the guard keeps over what the hardware actually does
    assert ratio.max() <= 0.9


@pytest.mark.parametrize("nbins,w", FP64_CASES)
def test_fp64_core_error_within_model(gc, nbins, w):
    """The fp64-dot core's t against acos(x)/w: the guard assumes a relative error rho.  For
    bins ending by 90 deg the narrow-range core is used; it needs t accurate only for x >= 0,
    and for x < 0 (past 90 deg) only t >= nbins - 1/2, which clamps to the last bin.  For bins
    ending by ~9 deg the series core is used: its bound rho_s holds up to one bin past the
    range, and beyond it t only has to stay at or past the last bin."""
    print(f"[gpu] fp64 core error model nbins={nbins}", flush=True)
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.uniform(-1, 1, 4_000_000), np.cos(rng.uniform(0, 0.05, 2_000_000)),
                        1 - rng.random(100_000) * 1e-12, np.array([0.0, -0.0, -1e-300, -1.0])])
    t, trip = _core_t(gc, x, nbins, w)
    t_exact = np.arccos(np.clip(x, -1, 1)) / np.radians(w)
    rho = ((_header_constant("GC_ACOS_FIT_ERR") + 4 * 2.0 ** -24 * (np.pi / 2)) / 1.41 + 10 * 2.0 ** -24) * 1.25
    narrow = nbins * w <= 90.0
    rho_s = series_rho(nbins, w)
    if rho_s is not None:
        rho = rho_s
    acc = x >= 0 if narrow else np.ones(len(x), bool)
    if rho_s is not None:
        acc = acc & (t_exact <= nbins + 1)
    if narrow:
        assert np.all(t[~acc] >= nbins - 0.5) and not trip[~acc].any()
    sel = acc & (t_exact > 1e-3)
    rel = np.abs(t[sel] - t_exact[sel]) / t_exact[sel]
    print(f"  max relative error {rel.max():.3e}; rho {rho:.3e}; ratio {rel.max() / rho:.3f}", flush=True)
    assert rel.max() <= rho
    small = acc & ~sel
    assert np.all(np.abs(t[small] - t_exact[small]) < 1e-3 * rho + 1e-6)


def test_matrix_core_dot_within_bound(gc):
    """The bin-table core's fast steps take the dot product from v_mfma_f32_16x16x4f32.  Its guard
    assumes |x~ - x.y| <= 10 * 2^-24 for fp32 unit vectors x, y (five roundings of one ulp each:
    three products and two sums, in any order and rounding mode).  Checked against the exact
    (fp64) dot product of the same fp32 vectors: random pairs, nearly parallel and antiparallel
    pairs, near-orthogonal pairs, and vectors along the axes."""
    import torch
    print("[gpu] matrix-core dot product error", flush=True)
    rng = np.random.default_rng(77)
    ntiles = 40000
    n = 16 * ntiles

    def unit(v):
        return (v / np.linalg.norm(v, axis=0)).astype(np.float32)

    a = unit(rng.normal(size=(3, n)))
    b = unit(rng.normal(size=(3, n)))
    q = n // 4
    b[:, :q] = unit(a[:, :q].astype(np.float64) + 1e-4 * rng.normal(size=(3, q)))            # nearly parallel
    b[:, q:2 * q] = unit(-a[:, q:2 * q].astype(np.float64) + 1e-4 * rng.normal(size=(3, q)))  # nearly antiparallel
    ax = np.zeros((3, 16)); ax[0, 0:4] = 1; ax[1, 4:8] = 1; ax[2, 8:12] = 1; ax[:, 12:16] = 1 / np.sqrt(3)
    a[:, -16:] = unit(ax)
    out = gc.eval_dot_mfma(torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda()).cpu().numpy().astype(np.float64)
    A = a.astype(np.float64).reshape(3, ntiles, 16)
    B = b.astype(np.float64).reshape(3, ntiles, 16)
    exact = np.einsum("ctI,ctJ->tIJ", A, B)
    err = np.abs(out - exact) / 2.0 ** -24
    # the tile's own pairs (i == j) hold the biased cases; every other (i, j) is a random pair
    print(f"  max |mfma - exact| = {err.max():.3f} x 2^-24 (bound 10)", flush=True)
    assert err.max() <= 10.0
    diag = err[:, np.arange(16), np.arange(16)]
    assert diag.max() <= 10.0


@pytest.mark.parametrize("nbins,w,dtype", [(720, 0.25, "float32"), (3600, 0.05, "float32"), (90, 1.0, "float32"),
                                           (1500, 0.001, "float64"), (720, 0.25, "float64")])
def test_non_finite_cosines_evaluate_as_one(gc, nbins, w, dtype):
    """Every core evaluates a NaN or infinite cosine as the cosine 1 (bin 0), never indexing its
    table with it."""
    import torch
    print(f"[gpu] non-finite cosines {nbins} x {w} {dtype}", flush=True)
    x = torch.tensor([np.nan, np.inf, -np.inf, 1.0], dtype=getattr(torch, dtype), device="cuda")
    b, trip, exact, _ = gc.eval_angle_core(x, nbins, w)
    b, trip, exact = (v.cpu().numpy() for v in (b, trip, exact))
    assert np.all(b == b[3]) and np.all(trip == trip[3]) and np.all(exact == exact[3]) and exact[3] == 0
