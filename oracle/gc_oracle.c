/*
 * gc_oracle.c -- plain CPU fp64 oracle for the all-pairs angular-separation
 * histograms DD, DR, RR and the Landy-Szalay estimator.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or constant with the GPU library, and the GPU library never
 * calls it.
 *
 * What it computes follows "CUDA Deep Dive: 10B Galaxy Pairs on an RTX 5080"
 * (section "The problem"):
 *   - every galaxy is (alpha, delta) in arcminutes;
 *   - the separation of two galaxies is the angle between their radius vectors,
 *       theta = acos( sin d1 sin d2 + cos d1 cos d2 cos(a1 - a2) ),
 *     the law-of-cosines form printed there;
 *   - each ordered pair (i, j), self-pairs included, adds one count to one of
 *     nbins fixed-width bins, for each of the families DD (D x D), DR (D x R)
 *     and RR (R x R), so every histogram sums to N_a * N_b;
 *   - omega = (DD - 2 DR + RR) / RR per bin.
 * The bin index truncates theta/width and clamps it into [0, nbins-1], as the
 * appendix listing's histogram-index helper does (clamp of the cosine into
 * [-1, 1] first, truncation, clamp of the index).
 *
 * Readings where the page leaves a step open (each also listed in the design
 * notes):
 *   - the fp32 arcminute inputs are taken as exact values and converted to
 *     radians in fp64 (the page converts in fp32 while parsing);
 *   - bin b covers [b*w, (b+1)*w) degrees; theta >= nbins*w goes to nbins-1;
 *   - omega is NaN where RR is zero (the page skips such bins); for unequal
 *     catalog sizes the normalised form
 *       (DD/nD^2 - 2 DR/(nD nR) + RR/nR^2) / (RR/nR^2)
 *     is used, which is the page's formula when nD == nR.
 *
 * Near-edge bookkeeping: for each family the oracle also counts, per inner
 * edge e = 1..nbins-1, the ordered pairs whose fp64 angle lies within
 * EDGE_TOL_DEG = 1e-5 degrees below edge e (lo[e]) or at/above it (hi[e]),
 * "above" meaning that the oracle's bin is e or higher.  Bins narrower than the
 * window put one pair within it of several edges; the pair is counted at each.
 * A GPU histogram may differ from the oracle only by pairs counted there.
 *
 * Symmetric mode evaluates only i <= j for a catalog against itself and
 * counts i < j twice.  That is exact (the page's section "L1: DD/RR symmetry"
 * shows the weights sum to N^2), and bit-identical here because a1 - a2 is
 * exactly -(a2 - a1), cos is even, and the products are formed in the same
 * order for (i, j) and (j, i).  sin/cos of each declination are evaluated once
 * per galaxy; that is the same libm call on the same argument, so every pair
 * sees bit-identical values to a per-pair evaluation.
 *
 * Build: gcc -O2 -fopenmp -fPIC -shared (no -ffast-math), libm sin/cos/acos.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

#define EDGE_TOL_DEG 1e-5

static const double PI = 3.14159265358979323846;

/* arcminutes -> radians, in fp64 */
static double arcmin_to_rad(float arcmin) { return (double)arcmin * (PI / 10800.0); }

/* The angle of one pair, in degrees, straight from the law-of-cosines form. */
double gco_pair_angle_deg(float ra1, float dec1, float ra2, float dec2) {
    double a1 = arcmin_to_rad(ra1), d1 = arcmin_to_rad(dec1);
    double a2 = arcmin_to_rad(ra2), d2 = arcmin_to_rad(dec2);
    double c = sin(d1) * sin(d2) + cos(d1) * cos(d2) * cos(a1 - a2);
    if (c > 1.0) c = 1.0;
    if (c < -1.0) c = -1.0;
    return acos(c) * (180.0 / PI);
}

/* Truncate theta/w, clamp into [0, nbins-1]. */
int64_t gco_bin_index(double theta_deg, double w_deg, int64_t nbins) {
    double q = floor(theta_deg / w_deg);
    if (q < 0.0) q = 0.0;
    if (q > (double)(nbins - 1)) q = (double)(nbins - 1);
    return (int64_t)q;
}

typedef struct {
    double a;     /* right ascension, rad */
    double sind;  /* sin(declination) */
    double cosd;  /* cos(declination) */
} gco_galaxy;

static gco_galaxy *to_galaxies(const float *ra, const float *dec, int64_t n) {
    gco_galaxy *g = (gco_galaxy *)malloc(sizeof(gco_galaxy) * (size_t)(n > 0 ? n : 1));
    if (!g) return NULL;
    for (int64_t k = 0; k < n; ++k) {
        double d = arcmin_to_rad(dec[k]);
        g[k].a = arcmin_to_rad(ra[k]);
        g[k].sind = sin(d);
        g[k].cosd = cos(d);
    }
    return g;
}

/* One ordered pair's contribution of `weight` to hist and to the near-edge
 * counters. */
static void count_pair(const gco_galaxy *p, const gco_galaxy *q, double w_deg, int64_t nbins,
                       uint64_t weight, uint64_t *hist, uint64_t *lo, uint64_t *hi) {
    double c = p->sind * q->sind + p->cosd * q->cosd * cos(p->a - q->a);
    if (c > 1.0) c = 1.0;
    if (c < -1.0) c = -1.0;
    double theta = acos(c) * (180.0 / PI);
    int64_t b = gco_bin_index(theta, w_deg, nbins);
    hist[b] += weight;
    /* Every inner edge within the window, on each side: the pair is above the edges
     * 1..b and below b+1..nbins-1.  The distance to an edge grows as the edge moves
     * away from the pair's own bin, so each walk stops at the first edge outside the
     * window; with bins wider than the window each walk tests one edge. */
    for (int64_t e = b; e >= 1 && theta - (double)e * w_deg < EDGE_TOL_DEG; --e) hi[e] += weight;
    for (int64_t e = b + 1; e < nbins && (double)e * w_deg - theta <= EDGE_TOL_DEG; ++e) lo[e] += weight;
}

/*
 * Histogram of rows [row0, row1) of catalog A against all of catalog B.
 * symmetric != 0 requires A and B to be the same catalog; then only j >= i is
 * evaluated, with weight 2 for j > i and 1 for j == i.
 * hist, lo, hi: nbins uint64 each, overwritten.  Returns 0, or -1 on bad input.
 */
int gco_family_rows(const float *ra_a, const float *dec_a, int64_t n_a,
                    const float *ra_b, const float *dec_b, int64_t n_b,
                    int64_t row0, int64_t row1, int symmetric,
                    int64_t nbins, double w_deg, int nthreads,
                    uint64_t *hist, uint64_t *lo, uint64_t *hi) {
    if (nbins <= 0 || !(w_deg > 0.0) || !isfinite(w_deg) || n_a < 0 || n_b < 0) return -1;
    if (row0 < 0 || row1 > n_a || row0 > row1) return -1;
    if (symmetric && n_a != n_b) return -1;
    memset(hist, 0, sizeof(uint64_t) * (size_t)nbins);
    memset(lo, 0, sizeof(uint64_t) * (size_t)nbins);
    memset(hi, 0, sizeof(uint64_t) * (size_t)nbins);
    if (row1 == row0 || n_b == 0) return 0;
    for (int64_t k = 0; k < n_a; ++k)
        if (!isfinite(ra_a[k]) || !isfinite(dec_a[k])) return -1;
    for (int64_t k = 0; k < n_b; ++k)
        if (!isfinite(ra_b[k]) || !isfinite(dec_b[k])) return -1;

    gco_galaxy *ga = to_galaxies(ra_a, dec_a, n_a);
    gco_galaxy *gb = to_galaxies(ra_b, dec_b, n_b);
    if (!ga || !gb) { free(ga); free(gb); return -1; }
    if (nthreads <= 0) nthreads = omp_get_max_threads();

    int failed = 0;
#pragma omp parallel num_threads(nthreads)
    {
        uint64_t *h = (uint64_t *)calloc((size_t)nbins * 3, sizeof(uint64_t));
        if (!h) {
#pragma omp atomic write
            failed = 1;
        } else {
            uint64_t *l = h + nbins, *u = h + 2 * nbins;
#pragma omp for schedule(dynamic, 16)
            for (int64_t i = row0; i < row1; ++i) {
                if (symmetric) {
                    count_pair(&ga[i], &ga[i], w_deg, nbins, 1, h, l, u);
                    for (int64_t j = i + 1; j < n_b; ++j) count_pair(&ga[i], &ga[j], w_deg, nbins, 2, h, l, u);
                } else {
                    for (int64_t j = 0; j < n_b; ++j) count_pair(&ga[i], &gb[j], w_deg, nbins, 1, h, l, u);
                }
            }
#pragma omp critical
            {
                for (int64_t b = 0; b < nbins; ++b) {
                    hist[b] += h[b];
                    lo[b] += l[b];
                    hi[b] += u[b];
                }
            }
            free(h);
        }
    }
    free(ga);
    free(gb);
    return failed ? -1 : 0;
}

/*
 * DD (D x D), DR (D x R), RR (R x R) over all ordered pairs.
 * edge_lo, edge_hi: [3][nbins] (family order DD, DR, RR), overwritten.
 */
int gco_histograms(const float *ra_d, const float *dec_d, int64_t n_d,
                   const float *ra_r, const float *dec_r, int64_t n_r,
                   int64_t nbins, double w_deg, int symmetric, int nthreads,
                   uint64_t *dd, uint64_t *dr, uint64_t *rr,
                   uint64_t *edge_lo, uint64_t *edge_hi) {
    int rc = gco_family_rows(ra_d, dec_d, n_d, ra_d, dec_d, n_d, 0, n_d, symmetric, nbins, w_deg,
                             nthreads, dd, edge_lo, edge_hi);
    if (rc) return rc;
    rc = gco_family_rows(ra_d, dec_d, n_d, ra_r, dec_r, n_r, 0, n_d, 0, nbins, w_deg, nthreads, dr,
                         edge_lo + nbins, edge_hi + nbins);
    if (rc) return rc;
    return gco_family_rows(ra_r, dec_r, n_r, ra_r, dec_r, n_r, 0, n_r, symmetric, nbins, w_deg,
                           nthreads, rr, edge_lo + 2 * nbins, edge_hi + 2 * nbins);
}

/* Per-pair bins of A x B (row-major n_a x n_b), for brute-force cross-checks
 * on small inputs. */
int gco_pair_bins(const float *ra_a, const float *dec_a, int64_t n_a,
                  const float *ra_b, const float *dec_b, int64_t n_b,
                  int64_t nbins, double w_deg, int64_t *bins_out, double *theta_out) {
    if (nbins <= 0 || !(w_deg > 0.0) || n_a < 0 || n_b < 0) return -1;
    for (int64_t i = 0; i < n_a; ++i)
        for (int64_t j = 0; j < n_b; ++j) {
            double t = gco_pair_angle_deg(ra_a[i], dec_a[i], ra_b[j], dec_b[j]);
            if (theta_out) theta_out[i * n_b + j] = t;
            bins_out[i * n_b + j] = gco_bin_index(t, w_deg, nbins);
        }
    return 0;
}

/* Landy-Szalay omega per bin, fp64; NaN where RR == 0. */
int gco_omega(const uint64_t *dd, const uint64_t *dr, const uint64_t *rr, int64_t nbins,
              int64_t n_d, int64_t n_r, double *omega) {
    if (nbins <= 0 || n_d < 0 || n_r < 0) return -1;
    for (int64_t b = 0; b < nbins; ++b) {
        if (rr[b] == 0) {
            omega[b] = NAN;
        } else if (n_d == n_r) {
            omega[b] = ((double)dd[b] - 2.0 * (double)dr[b] + (double)rr[b]) / (double)rr[b];
        } else {
            double nd = (double)n_d, nr = (double)n_r;
            double fdd = (double)dd[b] / (nd * nd);
            double fdr = (double)dr[b] / (nd * nr);
            double frr = (double)rr[b] / (nr * nr);
            omega[b] = (fdd - 2.0 * fdr + frr) / frr;
        }
    }
    return 0;
}

int gco_max_threads(void) { return omp_get_max_threads(); }
