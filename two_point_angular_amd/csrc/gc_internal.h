// Internal declarations shared by the HIP kernels (gc_kernels.hip) and the C ABI
// (gc_api.cpp).  Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gc {

constexpr int kWave = 64;            // CDNA wavefront width
constexpr int kWavesPerWG = 4;       // pair-kernel workgroup of the arccos and fp64 cores
constexpr int kWGThreads = kWave * kWavesPerWG;
constexpr int kMaxWavesPerWG = 16;   // the bin-table core's workgroups: up to 16 waves sharing one table
// Per-wave recheck queue, 8-byte entries.  Full batches of 64 are drained after every j-step
// and, within a step, after every D pairs per lane (D = drain_span), so a drain point leaves
// fewer than 64 pending and the next appends at most 64 D: 64 (D + 1) entries suffice.  D = 2
// for the bin-table core (its queues share the LDS with the table and the histogram; the
// matrix-core steps drain after every two of a lane's four pairs), D = 1 for it at K = 2 (sixteen
// waves' queues beside its table and histogram), else half a K = 8 step or a whole K = 4 step.
constexpr int drain_span(int k, int core, bool d64) {
  return (core == 2 && !d64) ? (k == 2 ? 1 : 2) : (k > 4 ? k / 2 : k);
}
constexpr int queue_words(int k, int core, bool d64) { return 2 * kWave * (drain_span(k, core, d64) + 1); }
constexpr int kMaxWorkgroups = 8192; // pair-kernel grid limit
constexpr int kMaxBins = 8192;       // GC_MAX_BINS (include/gc.h; gc_api.cpp checks they agree)
constexpr int kMaxBlocksPerCU = 8;
constexpr int kOversubscribe = 4;      // workgroups launched per resident workgroup slot
constexpr int kMinStepsPerWave = 256;  // j-steps per wave below which the grid shrinks

// ---- prepared catalog layout ---------------------------------------------------
// Six structure-of-arrays vectors of `padded` elements each: fp32 x, y, z then fp64
// x, y, z of the unit radius vector.  padded = roundup(n, 64) + 64 keeps every array
// 256-byte aligned and lets wave-uniform batches of j read a few elements past n.
inline int64_t padded_count(int64_t n) { return ((n + 63) / 64) * 64 + 64; }
inline size_t prepared_bytes_for(int64_t n) { return (size_t)padded_count(n) * 36u; }

struct Prepared {
  const float *x, *y, *z;
  const double *x64, *y64, *z64;
};

inline Prepared prepared_view(const void *blob, int64_t n) {
  const int64_t p = padded_count(n);
  const char *b = static_cast<const char *>(blob);
  Prepared v;
  v.x = reinterpret_cast<const float *>(b);
  v.y = v.x + p;
  v.z = v.y + p;
  v.x64 = reinterpret_cast<const double *>(b + 12 * p);
  v.y64 = v.x64 + p;
  v.z64 = v.y64 + p;
  return v;
}

// ---- binning constants -----------------------------------------------------------
// Bin k = [k w, (k+1) w).  The fast path works in units of bins: t = theta / w.
struct BinParams {
  float invw;    // 1 / w_rad                       (fp32)
  float h;       // (pi/2) / w_rad                   (fp32)
  float pinvw;   // pi / w_rad                       (fp32)
  float tmax;    // nbins - 0.5: clamp of t before truncation (plus the lane index in the pair kernel)
  float g32;     // fp32-dot guard: recheck iff |t - round(t)| * s < g32
  float g64k1;   // fp64-dot guard: recheck iff |t - round(t)| * s < g64k1 * s + g64k2
  float g64k2;
  float g64c;    // fp64-dot guard of the narrow and series cores: recheck iff |t - round(t)| < g64c
  float pw[7];   // acos polynomial coefficients times 1 / w_rad (fp32): narrow-range fp64 core
  float ps[3];   // series core (fp64 dot, narrow bins): sqrt2 (1, 1/12, 3/160) / w_rad
  float lut_m;   // bin-table core: entries per unit of c (M); the table has 2 M + 1 entries
  float lut_mb;  // M + 2^23: fma(c, M, M + 2^23) holds round(M (c + 1)) in its low mantissa bits
  float lut_g;   // bin-table core guard: recheck iff |cos(edge) - x| < lut_g
  int32_t lut_n; // 2 M (last entry index), or 0 when the bin table is not used
  int32_t lut_sh;  // log2 of the bytes per histogram row (2; 6 with sixteen columns): an argument, so
                   // that the compiler keeps (sign << lut_sh) + address as one shift-and-add
  int32_t lut_alias;  // bin-table core: the middle entry's row for x < 0 (x > 0: the row before)
  int32_t nbins;
  int32_t b180;  // the bin of the angles just below 180 deg: min(nbins - 1, floor(180 / w))
  int32_t b90;   // the bin holding 90 deg: min(nbins - 1, floor(90 / w))
};

// Bin-table core (fp32 dot, bins covering 0..180 deg): the table lives in the workspace and is
// copied into LDS by each workgroup; entry q = {cos(edge) (fp32 bits, or NaN: always recheck),
// byte offset of the histogram row of the bin above the edge}.  In LDS the second word becomes the
// byte address of that row.  Up to 14337 entries (112 KiB): M = ceil(4 / w_rad) <= 7168, widths
// down to about 0.032 deg.
constexpr int kLutMaxEntries = 14337;
// The table's middle entry (c within 1/(2M) of 0) holds both the smallest angles (x near 1)
// and the largest (x near -1).  When the table needs no always-recheck entries it stores e = 0 and
// the row lut_alias (BinParams), so x > 0 lands in row lut_alias - 1 (counted as bin 0) and x < 0
// in row lut_alias (counted as bin b180, the bin of the angles just below 180 deg, which is
// nbins - 1 unless the bins reach past 180 deg).  (The host admits that form only when no edge
// lies within the middle entry's reach, so each row stands for one bin.)  One-column histograms
// keep 64 spare rows past the last bin, so the alias rows are nbins + 64 and nbins + 65; the
// sixteen-column histogram of the bin-table core has one spare row (nbins) and the alias rows
// nbins + 1 and nbins + 2.
constexpr int kLutAliasWords = 2;
// Histogram columns of the bin-table core: one, or sixteen - row b holds one word per lane mod 16,
// so the 16 lanes an LDS atomic serves together always hit 16 different banks.
constexpr int kHistCols = 16;
// The bin-table core's bound on |x~ - x| in units of 2^-24 (see plan_lut in gc_api.cpp).
constexpr double kLutDotErr = 12.0;
// ---- pair-kernel work description ---------------------------------------------------
// One family (DD, DR or RR): the i catalog is held in registers, the j catalog streamed.
// Its work is a list of "j-steps": one j galaxy against one i-block of 64*K galaxies.
// Block b (i in [b*BI, b*BI + BI)) has j in [0, n_j) (cross family) or [b*BI, n_j)
// (self family, i <= j).  The steps fall into a fast segment (off-diagonal steps of full
// blocks) and a generic one (the diagonal steps of a self family, all steps of a ragged
// block); the family's workgroups [wg_begin, wg_end) split each segment evenly among their
// wavefronts.
struct FamilyWork {
  Prepared ci, cj;
  int64_t n_i, n_j;
  // This launch's j-steps in the family's two segments (a part of the job may start past 0):
  // fast steps [fast_begin, fast_begin + fast_steps) - off-diagonal steps of full i-blocks;
  // generic steps [gen_begin, gen_begin + gen_steps) - diagonal steps and the ragged block.
  int64_t fast_begin, fast_steps;
  int64_t gen_begin, gen_steps;
  int32_t sym;       // 1: self family (j >= i, weight 2 off the diagonal, 1 on it)
  int32_t wg_begin, wg_end;
  int32_t pad_;
};

struct PairArgs {
  FamilyWork fam[3];           // DD, DR, RR
  BinParams bp;
  const uint2 *lut;            // bin table (lut_n + 1 entries) in the workspace, or null
  uint64_t *out[3];            // DD, DR, RR outputs [nbins]; flushes add into them
  const double *edge_cos;      // [nbins + 1] cos(e w) in fp64, for the exact recheck
  int64_t flush_interval;      // j-steps between flushes of the 32-bit LDS histograms
  int32_t nbins;
  int32_t hist_words;          // LDS words of one histogram (rows x columns, rounded up to 64)
  int32_t shared_hist;         // 0: one histogram per wave; 1: one per workgroup
  int32_t waves;               // waves per workgroup (kWavesPerWG, or up to kMaxWavesPerWG for the bin table)
};

// The bin-table kernel's variants: histogram columns (1 or kHistCols) and the share of table
// reads made through the vector L1 instead of LDS (0: none; 1: an eighth; 2: a quarter; 3: three
// sixteenths, one column only).
struct LutVariant {
  int cols = 1;
  int l1 = 2;
};

// LDS bytes of one pair-kernel workgroup: histogram(s), the core's table (table_words, shared-
// histogram mode only), one recheck queue per wave and the workgroup's 64-bit step cursor.
constexpr int kCursorWords = 2;
inline size_t pairs_lds_bytes(int32_t hist_words, bool shared_hist, int k, int core, bool d64, int waves,
                              int32_t table_words = 0) {
  const size_t qw = static_cast<size_t>(queue_words(k, core, d64));
  const size_t words = shared_hist ? hist_words + static_cast<size_t>(table_words) + static_cast<size_t>(waves) * qw
                                   : static_cast<size_t>(waves) * (hist_words + qw);
  return (words + kCursorWords) * sizeof(uint32_t);
}
// Histogram words of the bin-table core: one column with 64 spare rows and the two alias rows, or
// kHistCols columns of nbins + 3 rows (one spare row, two alias rows).
inline int32_t lut_hist_words(int32_t nbins, int cols) {
  return cols == 1 ? (nbins + kWave + kLutAliasWords + 63) / 64 * 64 : (cols * (nbins + 3) + 63) / 64 * 64;
}
// Words of the core's table in LDS: the bin table (2 per entry).
inline int32_t table_words(int32_t lut_n, bool dot64, int core) { return (!dot64 && core == 2) ? 2 * (lut_n + 1) : 0; }

// Records a failed HIP call for gc_last_device_error() (gc_api.cpp).
void record_hip_error(hipError_t e);

// ---- launchers (gc_kernels.hip) ----------------------------------------------------------
hipError_t launch_prepare(const float *ra, const float *dec, int64_t n, void *blob, hipStream_t s);
// dot64: fp64 dot-product variant; k: galaxies per lane (4 or 8); core: 0 the generic core;
// 1 the one specialised to the bins' span - fp32 dot: nbins w covers 180 deg (no clamp of t,
// spare bin instead); fp64 dot: nbins w <= 90 deg (no sign handling); 2 - fp32 dot: the
// bin-table core (full span, shared histogram); fp64 dot: the series core (bins ending by ~9 deg)
// lv: the bin-table kernel's variant (core 2, fp32 dot only).
hipError_t launch_pairs(const PairArgs &a, int num_wg, bool dot64, int k, int core, LutVariant lv, hipStream_t s);
hipError_t pairs_occupancy(bool dot64, int k, int core, LutVariant lv, size_t lds_bytes, int threads,
                           int *blocks_per_cu);
// The bin table: 2 m + 1 entries; cols: the histogram's columns (scales the row offsets);
// alias: the middle entry's row when it holds no recheck zone; s_star > 0: entries whose |c| may
// lie below s_star hold NaN (always recheck).
hipError_t launch_eval_dot_mfma(const float *ax, const float *ay, const float *az, const float *bx, const float *by,
                                const float *bz, int64_t ntiles, float *out, hipStream_t s);
// accumulate: add the sums to the outputs instead of overwriting them
hipError_t launch_totals(const uint64_t *dd, const uint64_t *dr, const uint64_t *rr, int32_t nbins,
                         uint64_t *totals, hipStream_t s);
hipError_t launch_omega(const uint64_t *dd, const uint64_t *dr, const uint64_t *rr, int32_t nbins,
                        int64_t n_d, int64_t n_r, double *omega, hipStream_t s);
// The edge cosines c[e] = cos(e w) (e = 0..nbins, -inf past 180 deg), the bin table when
// lut is set (entries 0..2m) and, when out[0] is set, zeroed outputs (DD, DR, RR): one launch.
struct TablesArgs {
  int32_t nbins = 0;
  double w_deg = 0.0;
  double *edge_cos = nullptr;
  uint2 *lut = nullptr;
  int32_t m = 0, cols = 1, alias = 0;
  double margin = 0.0, s_star = 0.0;
  uint64_t *out[3] = {nullptr, nullptr, nullptr};
  int32_t edge_blocks = 0;  // set by launch_tables
};
hipError_t launch_tables(const TablesArgs &t, hipStream_t s);
hipError_t launch_eval_core(const float *x32, const double *x64, int64_t n, const BinParams &bp,
                            bool dot64, int core, const uint2 *lut, const double *edge_cos, int32_t *bin_out,
                            uint8_t *trip_out, int32_t *exact_out, float *t_out, hipStream_t s);

// Workspace layout: the edge-cosine table, then the bin table.
inline size_t edge_table_bytes(int32_t nbins) {
  return ((static_cast<size_t>(nbins) + 1) * sizeof(double) + 255) / 256 * 256;
}
constexpr size_t kLutBytes = (static_cast<size_t>(kLutMaxEntries) * 8 + 255) / 256 * 256;

}  // namespace gc
