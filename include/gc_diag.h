/*
 * gc_diag.h -- diagnostics and measured ceilings of libgc (include/gc.h).  Not part of the
 * histogram computation: these calls evaluate the pair kernel's per-pair core on given inputs,
 * for checking its guard numerically, and measure the rates of the GPU resources the pair
 * kernel uses (vector ALU, LDS, vector L1), for reading its speed against what this GPU
 * sustains.  The conventions of gc.h apply: device pointers, asynchronous on `stream`, host-side
 * validation before anything is enqueued, status codes.
 */
#ifndef GC_DIAG_H_
#define GC_DIAG_H_

#include "gc.h"

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------- the core ----
 * Evaluate the pair kernel's per-pair angle-to-bin core on given cosines, exactly as
 * the pair kernel does, for numerical verification of its guard.
 *   dot_precision 32: reads d_x32 (n fp32 cosines); 64: reads d_x64 (n fp64 cosines).
 *   d_bin_out  : device, n int32: the fast-path bin.
 *   d_trip_out : device, n uint8: 1 where the guard sends the pair to the exact recheck.
 *   d_exact_out: device, n int32, or null: the exact recheck's bin of the same cosine
 *                (fp32 cosines are widened exactly), found from the fast-path bin by the
 *                kernel's own edge-cosine search.
 *   d_t_out    : device, n fp32, or null: the fast path's coordinate before binning, for
 *                measuring the core's error: theta / width (arccos cores), or
 *                c = copysign(sqrt(1 - |x|), x) (the bin-table core).
 *   d_workspace: at least gc_workspace_bytes(nbins) bytes, GC_ALIGNMENT-aligned; needed when
 *                d_exact_out is given or the core bins through a table (may be null otherwise).
 * The core is the one gc_histogram_dd_dr_rr would use for these bins with default tuning.
 * A non-finite cosine is evaluated as 1 (a pair kernel never sees one: gc_prepare's vectors
 * are unit vectors). */
gc_status gc_eval_angle_core(const float *d_x32, const double *d_x64, int64_t n,
                             int32_t nbins, double bin_width_deg, int32_t dot_precision,
                             int32_t *d_bin_out, uint8_t *d_trip_out, int32_t *d_exact_out,
                             float *d_t_out, void *d_workspace, size_t workspace_bytes,
                             gc_stream_t stream);

/* The dot products of the bin-table core's fast steps, computed on the matrix cores exactly as
 * the pair kernel computes them (v_mfma_f32_16x16x4f32, components x, y, z and 0), for
 * measuring their error against the guard's assumption.  Tile t holds 16 a-vectors and 16
 * b-vectors: d_ax[16 t + i], d_ay[...], d_az[...] and likewise for b (device, fp32, 16 ntiles
 * each); d_out (device, 256 ntiles fp32) receives out[256 t + 16 i + j] = a_(16t+i) . b_(16t+j).
 * Returns GC_ERR_INVALID_ARGUMENT for ntiles < 0 or a null pointer with ntiles > 0,
 * GC_ERR_UNSUPPORTED for ntiles >= 2^31. */
gc_status gc_eval_dot_mfma(const float *d_ax, const float *d_ay, const float *d_az, const float *d_bx,
                           const float *d_by, const float *d_bz, int64_t ntiles, float *d_out, gc_stream_t stream);

/* --------------------------------------------------------------- ceilings ----
 * Microbenchmarks of the two resources the pair kernel uses, for reading its measured
 * rate against what this GPU sustains (not part of the histogram computation).  Each
 * launches 2048 workgroups of 256 threads on `stream`; the caller times the launch (HIP
 * events on the same stream) and divides *ops_out / *atomics_out by the time.
 *   gc_ceiling_valu: kind 0 = fp32 FMA, 1 = fp32 square root, 2 = fp64 FMA; 8 independent
 *     chains per lane, `iters` iterations; *ops_out = lane operations executed.
 *   gc_ceiling_lds_atomic: every lane adds 1 to its wavefront's private LDS histogram of
 *     nbins words, 16 x iters times, at 16 pseudo-random bins (same_bin = 0) or always bin 0;
 *     *atomics_out = lane atomics executed.
 *   d_sink: device scratch of gc_ceiling_sink_bytes() bytes (results are discarded).
 *   ops_out, atomics_out: host pointers. */
size_t gc_ceiling_sink_bytes(void);
gc_status gc_ceiling_valu(int32_t kind, int64_t iters, void *d_sink, size_t sink_bytes,
                          uint64_t *ops_out, gc_stream_t stream);
gc_status gc_ceiling_lds_atomic(int32_t nbins, int32_t same_bin, int64_t iters, void *d_sink,
                                size_t sink_bytes, uint64_t *atomics_out, gc_stream_t stream);

/* LDS access probes: 2048 workgroups of `threads` (256, 512 or 1024) threads share one LDS table
 * of `words` 32-bit words (128 <= words, a multiple of 128, at most 160 KiB with kind 6's extra
 * 1024-word histogram); every active lane issues 16 x iters operations of one kind at addresses
 * drawn once from a hash: 0 ds_add_u32, 1 ds_add_rtn_u32, 2 ds_add_u64, 3 ds_add_rtn_u64,
 * 4 ds_read_b32, 5 ds_read_b64, 6 ds_read_b64 then ds_add_u32 at the histogram word the entry
 * names, 7 ds_add_u32 from one lane in `sparse` (>= 1).  cols = 0 draws the index from the whole
 * table; cols = C (a power of two <= 64) draws a row of a C-column table and takes the lane's index
 * mod C as the column.  *wave_instructions_out = the 64-lane LDS instructions issued (kind 6: pairs
 * of them); divide by the launch's time. */
gc_status gc_ceiling_lds(int32_t kind, int32_t words, int32_t threads, int32_t sparse, int32_t cols,
                         int64_t iters, void *d_sink, size_t sink_bytes, uint64_t *wave_instructions_out,
                         gc_stream_t stream);

/* The vector-memory counterpart: every lane loads 16 x iters random 8-byte entries of a table of
 * `words` 32-bit words (128 <= words, a multiple of 128) held in the first bytes of d_sink (device
 * memory; contents arbitrary), which needs gc_ceiling_sink_bytes() bytes more than the table. */
gc_status gc_ceiling_l1(int32_t words, int32_t threads, int64_t iters, void *d_sink, size_t sink_bytes,
                        uint64_t *wave_instructions_out, gc_stream_t stream);

/* ------------------------------------------------------------------ plan ----
 * The launch plan gc_histogram_dd_dr_rr_tuned would use for these sizes, bins and overrides
 * (tuning may be null), without enqueuing anything: for reading a measurement against the
 * occupancy and layout it ran with.  Needs the device (occupancy queries).  A job with no pairs
 * reports only core, dot_precision and i_per_lane (everything else 0). */
typedef struct {
    int32_t core;              /* 0 arccos (generic), 1 arccos (span-specialised), 2 bin table
                                  (fp32 dot) or series (fp64 dot) */
    int32_t dot_precision;     /* 32 or 64 */
    int32_t i_per_lane;        /* 2, 4 or 8 */
    int32_t hist_columns;      /* 1 or 16 */
    int32_t waves_per_group;   /* wavefronts per workgroup */
    int32_t l1_share;          /* bin table: 1 none, 2 an eighth, 3 a quarter, 4 three
                                  sixteenths; else 0 */
    int32_t shared_histogram;  /* 1: one histogram per workgroup */
    int32_t blocks_per_cu;     /* workgroups per compute unit the grid was sized for */
    int32_t workgroups;        /* grid size */
    int32_t lds_bytes;         /* LDS per workgroup */
    int64_t flush_interval;    /* j-steps between flushes of the 32-bit LDS histograms */
    int32_t always_recheck;    /* bin table: 1 when entries near 0 and 180 deg always recheck */
    int32_t lut_m;             /* bin table: M, the table holding 2 M + 1 entries; else 0 */
} gc_plan;

gc_status gc_launch_plan(int64_t n_d, int64_t n_r, int32_t nbins, double bin_width_deg, const gc_tuning *tuning,
                         gc_plan *plan);

#ifdef __cplusplus
}
#endif

#endif /* GC_DIAG_H_ */
