// Internal declarations shared by the HIP kernels (gc_kernels.hip) and the C ABI
// (gc_api.cpp).  Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gc {

constexpr int kWave = 64;            // CDNA wavefront width
constexpr int kWavesPerWG = 4;       // pair-kernel workgroup = 4 independent wavefronts
constexpr int kWGThreads = kWave * kWavesPerWG;
// Per-wave recheck queue, 8-byte entries.  Full batches of 64 are drained after every j-step
// and, within a step, after every D pairs per lane (D = drain_span: 4, i.e. once in the middle
// of a K = 8 step; 2 for the edge-table core, whose table leaves less LDS for queues), so a
// drain point leaves fewer than 64 pending and the next appends at most 64 D: 64 (D + 1)
// entries suffice.  (Halving the queue of K = 8 lets a fifth workgroup fit in LDS beside the
// bin table or a 3600-bin shared histogram.)
constexpr int drain_span(int k, int core) { return core >= 3 ? 2 : (k > 4 ? k / 2 : k); }
constexpr int queue_words(int k, int core) { return 2 * kWave * (drain_span(k, core) + 1); }
constexpr int kMaxWorkgroups = 2048; // partial-histogram slots held by the workspace
constexpr int kMaxBlocksPerCU = 8;

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
  float etab_hk; // edge-table core with an integral h: h + 2^23 (exact), so that one fma gives the key
  int32_t lut_n; // 2 M (last entry index), or 0 when the bin table is not used
  int32_t lut_sh;  // 2, log2 of the bytes per histogram word: an argument, so that the compiler
                   // keeps (sign << 2) + address as one shift-and-add
  int32_t nbins;
  int32_t b180;  // the bin of the angles just below 180 deg: min(nbins - 1, floor(180 / w))
};

// Bin-table core (fp32 dot, bins covering 0..180 deg): the table lives in the workspace and is
// copied into LDS by each workgroup; entry q = {cos(edge) (fp32 bits), 4 x the bin above the
// edge}.  In LDS the second word becomes the byte address of the bin's histogram word.
constexpr int kLutMaxEntries = 2049;
// The table's middle entry (c within 1/(2M) of 0) holds both the smallest angles (x near 1)
// and the largest (x near -1).  It stores e = 0 and bin word nbins + 65, so x > 0 lands in word
// nbins + 64 (counted as bin 0) and x < 0 in word nbins + 65 (counted as bin b180, the bin of
// the angles just below 180 deg, which is nbins - 1 unless the bins reach past 180 deg): two
// histogram words past the 64 spare ones.  (The host admits the table only when no edge lies
// within the middle entry's range, so each word stands for one bin.)
constexpr int kLutAliasWords = 2;
// The bin-table core's bound on |x~ - x| in units of 2^-24 (see plan_lut in gc_api.cpp).
constexpr double kLutDotErr = 12.0;
// Edge-table core (fp32 dot, bins covering 0..180 deg, too fine for the bin table): the cosine
// of edge r (fp32, or NaN where the pair must be rechecked) for r = 0 .. nbins + 1, built in
// the bin table's workspace area.  In LDS: [e_r (kEtabTableWords words) | histogram of bins
// -1 .. nbins + 63 | 4 queues]; bin -1 is reachable only by rechecked pairs (the recheck moves
// them out).

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
  unsigned long long *slots;   // [num_workgroups][nbins] 64-bit partial histograms
  const double *edge_cos;      // [nbins + 1] cos(e w) in fp64, for the exact recheck
  int64_t flush_interval;      // j-steps between flushes of the 32-bit LDS histograms
  int32_t nbins;
  int32_t hist_words;          // LDS words of one histogram (>= nbins + 64: 64 spare bins)
  int32_t shared_hist;         // 0: one histogram per wave; 1: one per workgroup (4 waves)
};

// LDS bytes of one pair-kernel workgroup.
// LDS bytes of one pair-kernel workgroup: histogram(s), the bin table (lut_entries 8-byte
// entries, shared-histogram mode only) and the four recheck queues.
inline size_t pairs_lds_bytes(int32_t hist_words, bool shared_hist, int k, int core, int32_t table_words = 0) {
  const size_t qw = static_cast<size_t>(queue_words(k, core));
  const size_t words = shared_hist ? hist_words + static_cast<size_t>(table_words) +
                                         static_cast<size_t>(kWavesPerWG) * qw
                                   : static_cast<size_t>(kWavesPerWG) * (hist_words + qw);
  return words * sizeof(uint32_t);
}
// Histogram words of the edge-table core: bins -1 .. nbins + 63 (64 spares, as in core32).
inline int32_t etab_hist_words(int32_t nbins) { return (nbins + 1 + 64 + 63) / 64 * 64; }
// The edge table's LDS region (words): e_r at word r, the histogram right after it, so that
// the count of bin r sits a fixed 4 (kEtabTableWords + 1) bytes past e_r (bin -1 first), an
// offset the LDS atomic carries in its instruction.
constexpr int kEtabTableWords = 4096;
// Words of the core's table in LDS: the bin table (2 per entry), or the edge-table region.
inline int32_t table_words(const PairArgs &a, bool dot64, int core) {
  if (dot64) return 0;
  if (core == 2) return 2 * (a.bp.lut_n + 1);
  if (core >= 3) return kEtabTableWords;
  return 0;
}

// Records a failed HIP call for gc_last_device_error() (gc_api.cpp).
void record_hip_error(hipError_t e);

// ---- launchers (gc_kernels.hip) ----------------------------------------------------------
hipError_t launch_prepare(const float *ra, const float *dec, int64_t n, void *blob, hipStream_t s);
// dot64: fp64 dot-product variant; k: galaxies per lane (4 or 8); core: 0 the generic core;
// 1 the one specialised to the bins' span - fp32 dot: nbins w covers 180 deg (no clamp of t,
// spare bin instead); fp64 dot: nbins w <= 90 deg (no sign handling); 2 - fp32 dot: the
// bin-table core (full span, shared histogram); fp64 dot: the series core (bins ending by ~9 deg)
hipError_t launch_pairs(const PairArgs &a, int num_wg, bool dot64, int k, int core, hipStream_t s);
hipError_t pairs_occupancy(bool dot64, int k, int core, size_t lds_bytes, int *blocks_per_cu);
hipError_t launch_lut(int32_t nbins, double w_deg, int32_t m, double margin, uint2 *lut, hipStream_t s);
hipError_t launch_eval_dot_mfma(const float *ax, const float *ay, const float *az, const float *bx, const float *by,
                                const float *bz, int64_t ntiles, float *out, hipStream_t s);
hipError_t launch_etab(int32_t nbins, double w_deg, double g_x, double e3, uint32_t *et, hipStream_t s);
// accumulate: add the sums to the outputs instead of overwriting them
hipError_t launch_merge(const unsigned long long *slots, int32_t nbins, const int32_t wg_begin[3],
                        const int32_t wg_end[3], uint64_t *out[3], bool accumulate, hipStream_t s);
hipError_t launch_totals(const uint64_t *dd, const uint64_t *dr, const uint64_t *rr, int32_t nbins,
                         uint64_t *totals, hipStream_t s);
hipError_t launch_omega(const uint64_t *dd, const uint64_t *dr, const uint64_t *rr, int32_t nbins,
                        int64_t n_d, int64_t n_r, double *omega, hipStream_t s);
hipError_t launch_edges(int32_t nbins, double w_deg, double *edge_cos, hipStream_t s);
hipError_t launch_eval_core(const float *x32, const double *x64, int64_t n, const BinParams &bp,
                            bool dot64, int core, const uint2 *lut, const double *edge_cos, int32_t *bin_out,
                            uint8_t *trip_out, int32_t *exact_out, float *t_out, hipStream_t s);

// Workspace layout: the edge-cosine table, the bin table, then the per-workgroup 64-bit
// partial histograms.
inline size_t edge_table_bytes(int32_t nbins) {
  return ((static_cast<size_t>(nbins) + 1) * sizeof(double) + 255) / 256 * 256;
}
constexpr size_t kLutBytes = (static_cast<size_t>(kLutMaxEntries) * 8 + 255) / 256 * 256;

}  // namespace gc
