/*
 * gc_ladder.h -- the ablation ladder of "CUDA Deep Dive: 10B Galaxy Pairs on an
 * RTX 5080" (section "The ladder" and the sections "L1: DD/RR symmetry" to
 * "L5: the last 8%", "Tile size sweep" and "What didn't pay off"), rebuilt as
 * HIP kernels for gfx950 so that each of the page's steps can be timed, and its
 * effect on the counts measured, on this GPU.
 *
 * Each rung adds one change to the previous one; all rungs compute DD, DR and RR
 * with the page's fp32 arithmetic (law of cosines on (alpha, delta) converted to
 * radians in fp32), not the certified path of gc.h, so their counts may differ
 * from the exact histograms near bin edges.  That difference is part of what the
 * ladder measures.
 *
 *   rung 0  one thread per (i, j) pair in 32 x 32 blocks; per pair the sines and
 *           cosines of both declinations, cos of the right-ascension difference,
 *           and acosf; no symmetry.  Every block keeps 3 histograms in LDS and
 *           adds its non-zero bins to the outputs with 64-bit global atomics.
 *   rung 1  + symmetry: DD and RR only for j >= i, weight 2 off the diagonal
 *           (section "L1: DD/RR symmetry").
 *   rung 2  + sin/cos of each declination computed once per galaxy (a prepass
 *           into the workspace) instead of per pair ("L2: precomputed sin/cos").
 *   rung 3  + tiling: one thread per i galaxy, a block of `tile` threads, the
 *           j-tile of `tile` galaxies of both catalogs staged in LDS as 16-byte
 *           records, one broadcast read per catalog and pair ("L3: block tiling").
 *   rung 4  + a polynomial arccos in place of acosf ("L4: fast acos"): the
 *           handbook approximation of Abramowitz and Stegun, formula 4.4.45,
 *           acos(x) ~ sqrt(1 - x) (a0 + a1 x + a2 x^2 + a3 x^3) on [0, 1], whose
 *           error the handbook bounds by 6.7e-5 rad; reflected for x < 0.
 *   rung 5  + inner loop unrolled by 8, launch bounds fixed to the tile, and DD/RR
 *           skipped for blocks wholly below the diagonal ("L5: the last 8%").
 *
 * The arccos of any rung can be overridden (acos_kind): GC_LADDER_ACOS_LIBM
 * (acosf), GC_LADDER_ACOS_HANDBOOK (formula 4.4.45), GC_LADDER_ACOS_FIT6 (the
 * degree-6 fit of gc.h's fp32 core, without its guard); -1 keeps the rung's own
 * (libm for rungs 0-3, handbook for rungs 4-5).
 *
 * Conventions are those of gc.h (device pointers, asynchronous on `stream`, no
 * allocation, host-side validation with nothing enqueued on error).
 */
#ifndef GC_LADDER_H_
#define GC_LADDER_H_

#include "gc.h"

#ifdef __cplusplus
extern "C" {
#endif

#define GC_LADDER_RUNGS 6
#define GC_LADDER_ACOS_RUNG (-1)
#define GC_LADDER_ACOS_LIBM 0
#define GC_LADDER_ACOS_HANDBOOK 1
#define GC_LADDER_ACOS_FIT6 2
#define GC_LADDER_MAX_GALAXIES 2000000LL /* grid-dimension limit of the one-thread-per-pair rungs */

/* Workspace bytes for catalogs of n_d and n_r galaxies: three fp32 arrays (sin delta,
 * cos delta, alpha in radians) per catalog, each 256-byte aligned.  0 on bad sizes. */
size_t gc_ladder_workspace_bytes(int64_t n_d, int64_t n_r);

/* DD, DR, RR of one ladder rung.
 *   rung          0..5 as listed above.
 *   acos_kind     -1 (the rung's own) or one of GC_LADDER_ACOS_*.
 *   tile          rungs 3-5: threads per block and j-tile width, a power of two in
 *                 64..1024, or 0 for 512; rungs 0-2: must be 0.
 *   bin_stride    LDS words between the three per-block histograms: 0 for nbins, or
 *                 any value >= nbins (the padding of section "What didn't pay off").
 *   d_ra_*, d_dec_*  device fp32 arrays of n_* galaxies, arcminutes.  Not modified.
 *   n_d, n_r      0..GC_LADDER_MAX_GALAXIES.
 *   nbins, bin_width_deg  as in gc.h (1..GC_MAX_BINS; width > 0, finite).
 *   d_dd, d_dr, d_rr  device uint64[nbins] each, 8-byte aligned; OVERWRITTEN.
 *   d_workspace   gc_ladder_workspace_bytes(n_d, n_r) bytes, 256-byte aligned.
 * Errors: GC_ERR_INVALID_ARGUMENT (bad rung, acos_kind, tile, stride, null or
 * misaligned pointer, bad bins), GC_ERR_UNSUPPORTED (n or nbins too large, or the
 * LDS footprint, 12 stride + 32 tile bytes, above 160 KiB), GC_ERR_WORKSPACE,
 * GC_ERR_DEVICE. */
gc_status gc_ladder_histogram(int32_t rung, int32_t acos_kind, int32_t tile, int32_t bin_stride,
                              const float *d_ra_d, const float *d_dec_d, int64_t n_d,
                              const float *d_ra_r, const float *d_dec_r, int64_t n_r,
                              int32_t nbins, double bin_width_deg,
                              uint64_t *d_dd, uint64_t *d_dr, uint64_t *d_rr,
                              void *d_workspace, size_t workspace_bytes, gc_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* GC_LADDER_H_ */
