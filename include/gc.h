/*
 * gc.h -- all-pairs angular-separation histograms (DD, DR, RR) and the
 * Landy-Szalay two-point angular correlation estimator, on one AMD MI355X
 * (gfx950) GPU.
 *
 * The operation is the one stated in "CUDA Deep Dive: 10B Galaxy Pairs on an
 * RTX 5080", section "The problem":
 *   - two catalogs, D (observed) and R (random), each a list of galaxies given
 *     as right ascension alpha and declination delta in arcminutes;
 *   - for every ordered pair of galaxies the angular separation
 *       theta = acos( sin d1 sin d2 + cos d1 cos d2 cos(a1 - a2) ),
 *     i.e. the angle between the two radius vectors;
 *   - theta binned into fixed-width bins for the three families DD (D x D),
 *     DR (D x R) and RR (R x R), each covering every ordered pair including
 *     self-pairs, so each histogram sums to exactly N_a * N_b;
 *   - omega = (DD - 2 DR + RR) / RR per bin.
 * Bin k covers [k*w, (k+1)*w) degrees; theta >= nbins*w goes to bin nbins-1
 * (truncation and clamping as in the appendix listing's histogram-index
 * helper).  Results equal an fp64 evaluation except for pairs whose fp64 angle
 * lies within rounding (well under 1e-5 degrees) of a bin edge.
 *
 * Conventions shared by every call:
 *   - Pointers named d_* or documented "device" are device pointers on the
 *     current HIP device; the caller owns every buffer and keeps it alive until
 *     the work enqueued on `stream` has completed.
 *   - Calls are asynchronous on `stream` (a hipStream_t; 0 is the null stream).
 *   - The library allocates no device memory, prints nothing and never exits.
 *   - Arguments are validated on the host before anything is enqueued.  On any
 *     error status nothing has been enqueued and the outputs are untouched.
 *   - Thread-safe: the only state is a per-device property cache filled once,
 *     and a per-thread record of the last HIP error.
 */
#ifndef GC_H_
#define GC_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t *gc_stream_t; /* the same type as hipStream_t */

typedef enum {
    GC_OK = 0,
    GC_ERR_INVALID_ARGUMENT = 1, /* null pointer, negative size, nbins <= 0, width <= 0 or not
                                    finite, misaligned buffer, bad tuning field */
    GC_ERR_UNSUPPORTED = 2,      /* nbins above GC_MAX_BINS, n above GC_MAX_GALAXIES */
    GC_ERR_WORKSPACE = 3,        /* workspace smaller than gc_workspace_bytes() */
    GC_ERR_DEVICE = 4,           /* a HIP call or kernel launch failed; see gc_last_device_error() */
    GC_ERR_IO = 5                /* a file could not be opened, mapped, parsed or written (gc_io.h) */
} gc_status;

#define GC_MAX_BINS 8192                 /* bins per histogram (LDS-resident per wavefront) */
#define GC_MAX_GALAXIES 2147483647LL     /* galaxies per catalog (2^31 - 1) */
#define GC_ALIGNMENT 256                 /* required alignment of prepared blobs and workspace */

/* ---------------------------------------------------------------- prepare ----
 * Convert one catalog to the library's prepared form: per galaxy the unit
 * radius vector (cos d cos a, cos d sin a, sin d), computed in fp64 from the
 * exact fp32 arcminute inputs (a = alpha * pi/10800, d = delta * pi/10800),
 * stored as structure-of-arrays in fp32 (correctly rounded) and in fp64.  The
 * angle between two galaxies is the arccos of their vectors' dot product
 * (section "The problem"); precomputing per-galaxy trigonometry is the page's
 * section "L2: precomputed sin/cos", taken one step further.
 *
 *   d_ra_arcmin, d_dec_arcmin : device-accessible, n fp32 values each (device
 *                               memory, or pinned host memory mapped into the
 *                               device, read once over the bus); should be finite:
 *                               a galaxy with a non-finite coordinate is placed at
 *                               alpha = delta = 0 (its pairs' bins are meaningless,
 *                               the totals still hold).
 *   n                         : number of galaxies, 0 <= n <= GC_MAX_GALAXIES.
 *   d_prepared                : device, gc_prepared_bytes(n) bytes, GC_ALIGNMENT-aligned;
 *                               its layout is private to the library.  May be null
 *                               only when n == 0.
 */
size_t gc_prepared_bytes(int64_t n);
gc_status gc_prepare(const float *d_ra_arcmin, const float *d_dec_arcmin, int64_t n,
                     void *d_prepared, gc_stream_t stream);

/* -------------------------------------------------------------- histogram ----
 * DD, DR and RR over all ordered pairs of the prepared catalogs (section "The
 * problem"; DD and RR use the i <= j symmetry of section "L1: DD/RR symmetry",
 * which changes no count).
 *
 *   d_prepared_d, n_d : prepared catalog D (from gc_prepare) and its size.
 *   d_prepared_r, n_r : prepared catalog R and its size.  D and R may be the same
 *                       blob; then DR is the full ordered D x D histogram.
 *   nbins             : 1 <= nbins <= GC_MAX_BINS.
 *   bin_width_deg     : w > 0, finite.  Bin k = [k*w, (k+1)*w) degrees; larger angles
 *                       go to bin nbins-1.
 *   d_dd, d_dr, d_rr  : device, nbins uint64 each, 8-byte aligned; OVERWRITTEN.
 *                       Sums: n_d^2, n_d*n_r, n_r^2.  A family with no pairs is all zero.
 *   d_workspace       : device scratch of at least gc_workspace_bytes(nbins) bytes
 *                       (the fp64 edge cosines and the bin table: at most 177 KiB),
 *                       GC_ALIGNMENT-aligned; contents on entry are ignored.  Must not
 *                       be used by another call until this one has completed.
 * The outputs are zeroed first and the pair kernel's workgroups add their counts
 * into them with 64-bit atomics, so they must not be read or written by other work
 * until the call has completed.
 * Returns GC_OK once the work is enqueued.
 */
size_t gc_workspace_bytes(int32_t nbins);
gc_status gc_histogram_dd_dr_rr(const void *d_prepared_d, int64_t n_d,
                                const void *d_prepared_r, int64_t n_r,
                                int32_t nbins, double bin_width_deg,
                                uint64_t *d_dd, uint64_t *d_dr, uint64_t *d_rr,
                                void *d_workspace, size_t workspace_bytes,
                                gc_stream_t stream);

/* Optional overrides of the launch plan, for tuning sweeps and tests.  Every field
 * 0 means "the library's choice"; gc_histogram_dd_dr_rr is this call with all zeros.
 * The result does not depend on these fields (only speed does). */
typedef struct {
    int32_t dot_precision;   /* 0 auto, 32: fp32 dot product, 64: fp64 dot product */
    int32_t i_per_lane;      /* 0 auto, or 4 or 8 galaxies held per lane (2 as well for the bin table) */
    int32_t blocks_per_cu;   /* 0 auto (occupancy), else 1..8 workgroups per compute unit */
    int32_t shared_histogram; /* 0 auto; 1: one private LDS histogram per wavefront;
                                 2: one LDS histogram per workgroup, shared by its wavefronts */
    int32_t span_kernel;     /* 0 auto; 1: the generic core; 2: the core specialised to the
                                bins' span - fp32 dot: no clamp of the bin coordinate (only
                                valid when (nbins + 1/2) * width >= 180 deg); fp64 dot: no
                                sign handling (only valid when nbins * width <= 90 deg) */
    int32_t fast_core;       /* 0 auto; 1: never use a fast core (the degree-6 arccos
                                cores bin every pair); 2: always - the bin table (fp32 dot,
                                bins covering 180 deg, width >= ~0.032 deg; one histogram
                                shared per workgroup of up to 16 wavefronts) or the series
                                (fp64 dot, bins ending by about 9 deg); invalid where neither
                                applies */
    int64_t flush_interval;  /* 0 auto; else j-steps between flushes of the 32-bit LDS
                                histograms into 64-bit totals (>= 1) */
    int32_t hist_columns;    /* bin-table core: 0 auto; 1 or 16 LDS histogram columns (16: one
                                word per bin for each lane mod 16, so an atomic's 16-lane group
                                never shares a bank; invalid where it does not fit in LDS) */
    int32_t waves_per_group; /* bin-table core: 0 auto, else 4..16 wavefronts per workgroup */
    int32_t l1_share;        /* bin-table core: 0 auto; share of table reads made through the
                                vector L1 instead of LDS: 1 none, 2 an eighth, 3 a quarter,
                                4 three sixteenths (one-column histogram only).  Auto: none,
                                except in the one-column layout of two workgroups per compute
                                unit, where the share depends on the table's size */
    int32_t reserved_;       /* must be 0 */
} gc_tuning;

gc_status gc_histogram_dd_dr_rr_tuned(const void *d_prepared_d, int64_t n_d,
                                      const void *d_prepared_r, int64_t n_r,
                                      int32_t nbins, double bin_width_deg,
                                      uint64_t *d_dd, uint64_t *d_dr, uint64_t *d_rr,
                                      void *d_workspace, size_t workspace_bytes,
                                      const gc_tuning *tuning, gc_stream_t stream);

/* ------------------------------------------------------------------ parts ----
 * One part of the histogram job, for catalogs too large to process in one call
 * (N >> 10^6), for checkpointing, or for spreading the job over several devices or
 * processes.  The histograms are additive over any partition of the pairs (section
 * "L1: DD/RR symmetry" sums weighted pairs; nothing else couples them), so the job is
 * cut into `parts` pieces: part p takes, in each of DD, DR and RR and in each of its
 * two kinds of work unit (off-diagonal and diagonal/ragged), the units
 * floor(T p / parts) .. floor(T (p+1) / parts) of the T units the single call uses.
 * Each pair's bin depends on that pair alone, so the parts of one job, in any order
 * and on any device, sum exactly to gc_histogram_dd_dr_rr's result.
 *
 * Unlike gc_histogram_dd_dr_rr this call ACCUMULATES: it adds the part's counts to
 * d_dd, d_dr, d_rr (zero them before part 0).  Arguments are those of
 * gc_histogram_dd_dr_rr_tuned (tuning may be null), plus:
 *   part, parts : 1 <= parts <= GC_MAX_PARTS, 0 <= part < parts.  Every part of one
 *                 job must use the same catalogs, bins and tuning, and the same build of
 *                 this library: the work units are those of the launch plan (their size
 *                 follows its galaxies per lane, gc_launch_plan's i_per_lane).
 * A part that holds no work for a family adds nothing to it.  Calls that add into the
 * same outputs must be ordered (the same stream, or synchronised).
 */
#define GC_MAX_PARTS (1LL << 40)
gc_status gc_histogram_part(const void *d_prepared_d, int64_t n_d,
                            const void *d_prepared_r, int64_t n_r,
                            int32_t nbins, double bin_width_deg,
                            int64_t part, int64_t parts,
                            uint64_t *d_dd, uint64_t *d_dr, uint64_t *d_rr,
                            void *d_workspace, size_t workspace_bytes,
                            const gc_tuning *tuning, gc_stream_t stream);

/* ------------------------------------------------- allocation-free variant ----
 * For callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  gc_histogram_dd_dr_rr
 * without the workspace argument: its scratch (the edge cosines and the bin table)
 * is an array of GC_STATIC_SCRATCH_BYTES in the library's own device memory, one
 * per GPU, held until the process ends.  The call allocates nothing; its first
 * call on a device resolves that device's array address (a runtime query that
 * enqueues nothing).  The results are those of gc_histogram_dd_dr_rr, bit for bit.
 *
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents (ignored on entry: every word a call reads, it has written first).
 * Calls that overlap on one GPU -- different streams, or threads without
 * ordering -- RACE and return wrong counts; order them on one stream.
 * Arguments, results and errors are those of gc_histogram_dd_dr_rr;
 * GC_ERR_UNSUPPORTED if a job's tables would not fit the array (the library checks
 * at build time that those of every nbins <= GC_MAX_BINS do).
 */
#define GC_STATIC_SCRATCH_BYTES (256u << 10)
gc_status gc_histogram_dd_dr_rr_noalloc(const void *d_prepared_d, int64_t n_d,
                                        const void *d_prepared_r, int64_t n_r,
                                        int32_t nbins, double bin_width_deg,
                                        uint64_t *d_dd, uint64_t *d_dr, uint64_t *d_rr,
                                        gc_stream_t stream);

/* ----------------------------------------------------------------- totals ----
 * The three histogram sums, for the exact-total check of section "The problem"
 * (each family must sum to N_a * N_b).  d_totals: device, 3 uint64 (DD, DR, RR
 * order), overwritten. */
gc_status gc_histogram_totals(const uint64_t *d_dd, const uint64_t *d_dr, const uint64_t *d_rr,
                              int32_t nbins, uint64_t *d_totals, gc_stream_t stream);

/* ------------------------------------------------------------------ omega ----
 * Landy-Szalay estimator per bin in fp64 (section "The problem"):
 *   omega = (DD - 2 DR + RR) / RR                       when n_d == n_r,
 *   omega = (DD/n_d^2 - 2 DR/(n_d n_r) + RR/n_r^2) / (RR/n_r^2)   otherwise,
 * and NaN where RR == 0 (the page's program skips such bins) and in every bin when
 * n_d == 0 < n_r (the normalised DD and DR are then 0/0).
 *   d_dd, d_dr, d_rr : device, nbins uint64 each.   d_omega: device, nbins fp64, overwritten. */
gc_status gc_omega(const uint64_t *d_dd, const uint64_t *d_dr, const uint64_t *d_rr,
                   int32_t nbins, int64_t n_d, int64_t n_r, double *d_omega, gc_stream_t stream);

/* ----------------------------------------------------------------- status ----
 * The kernels' diagnostics (the angle-to-bin core on given cosines, the matrix-core dot
 * products) and the measured ceilings of the resources the pair kernel uses are declared in
 * gc_diag.h; they are not part of the histogram computation. */
const char *gc_status_string(gc_status status);
int gc_last_device_error(void); /* last hipError_t seen by this thread (0 if none) */
const char *gc_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GC_H_ */
