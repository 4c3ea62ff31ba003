// C ABI of libgc: argument validation, launch planning and kernel launches.
// Every check runs on the host before any HIP call, so every error path is reachable
// without a GPU.
#include <math.h>
#include <mutex>
#include <string.h>

#include "../../include/gc_diag.h"
#include "gc_acos_poly.h"
#include "gc_internal.h"

static_assert(GC_MAX_BINS == gc::kMaxBins, "the kernels' bin limit is GC_MAX_BINS");

namespace gc {
namespace {

thread_local int t_last_hip_error = 0;

gc_status device_error(hipError_t e) {
  t_last_hip_error = static_cast<int>(e);
  return GC_ERR_DEVICE;
}

}  // namespace

void record_hip_error(hipError_t e) { t_last_hip_error = static_cast<int>(e); }

namespace {

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// ---- per-device cache: CU count and pair-kernel occupancy -----------------------------
struct DeviceInfo {
  bool valid = false;
  int cus = 0;
  // occupancy per (kernel variant, bin-table variant, lds bytes, threads)
  struct Occ { int vi, cols, l1; size_t lds; int threads, blocks; };
  static constexpr int kSlots = 96;
  Occ occ[kSlots];
  int nocc = 0;
};
constexpr int kMaxDevices = 64;
std::mutex g_mu;
DeviceInfo g_dev[kMaxDevices];

hipError_t device_info(int *cus, bool dot64, int k, int core, LutVariant lv, size_t lds, int threads,
                       int *blocks_per_cu) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  DeviceInfo &d = g_dev[dev];
  if (!d.valid) {
    int n = 0;
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    d.cus = n;
    d.valid = true;
  }
  *cus = d.cus;
  if (!blocks_per_cu) return hipSuccess;
  const int vi = ((dot64 ? 5 : 0) + core) * 3 + (k == 8 ? 2 : (k == 4 ? 1 : 0));  // fp32 cores 0..4, fp64 0..2
  const bool lut = core == 2 && !dot64;
  const int cols = lut ? lv.cols : 1, l1 = lut ? lv.l1 : 2;
  for (int q = 0; q < d.nocc; ++q) {
    const DeviceInfo::Occ &o = d.occ[q];
    if (o.vi == vi && o.cols == cols && o.l1 == l1 && o.lds == lds && o.threads == threads) {
      *blocks_per_cu = o.blocks;
      return hipSuccess;
    }
  }
  int blocks = 0;
  e = pairs_occupancy(dot64, k, core, lv, lds, threads, &blocks);
  if (e != hipSuccess) return e;
  if (d.nocc < DeviceInfo::kSlots) d.occ[d.nocc++] = {vi, cols, l1, lds, threads, blocks};
  *blocks_per_cu = blocks;
  return hipSuccess;
}

// ---- binning constants and the certified guard -----------------------------------------
// Error model (all in units of bins, t = theta / w):
//  fp32 dot: the unit vectors are fp32 roundings of fp64 ones (|e| <= 2^-24 per component)
//    and the dot product takes three fp32 roundings, so |x~ - x| <= g_x = 5 * 2^-24 (+ the
//    fp64 prep error).  Since acos(1 - y) has derivative <= 1/sqrt(y), a cosine error g_x
//    moves theta by at most 2 g_x / s, s = sqrt(1 - |x~|) as computed (2.02 covers the
//    rounding of s).  The arccos core adds at most E_core (rad), and forming t in fp32
//    adds 2^-24 (t + 2h) (roundings of 1/w, (pi/2)/w and the final fma).  The kernel
//    rechecks iff |t - round(t)| * s < g32 = 2.02 g_x / w + C, C = E_core / w + 2^-24 (nbins
//    + 1 + 2h), which is implied by |t - round(t)| < 2.02 g_x / (s w) + C because s <= 1.
//  fp64 dot: the cosine error is ~1e-15, so the dominant error is the fp32 core, relative
//    to t: |t~ - t| <= rho t with rho covering sqrt, polynomial, narrowing and t roundings
//    (two more units of 2^-24 for the narrow-range core, whose coefficients are rounded
//    after scaling by 1 / w: sum |C_i| / P_min = 1.39 units).
//    Recheck iff |t - round(t)| * s < g64k1 * s + g64k2, g64k1 = rho (nbins + 1),
//    g64k2 = 2.02 g64 / w.  The narrow-range and series cores bin no angle near 180 deg, and
//    every edge lies at t >= 1, where s >= s_lo = 0.95 sqrt2 sin(w/4) (a pair with t~ < 1/2
//    is clamped to t = 1/2, which never trips, and is more than half a bin from any edge).
//    There g64k2 / s <= g64k2 / s_lo, so they recheck iff |t - round(t)| < g64c = g64k1 +
//    g64k2 / s_lo: one compare instead of a subtraction, a multiply and a compare.
constexpr double kTwoM24 = 5.9604644775390625e-08;  // 2^-24
constexpr double kPi = 3.14159265358979323846;

void set_fp64_guard(BinParams &bp, double rho, int32_t nbins, double w_rad) {
  const double g64 = 1e-14;
  const double k1 = rho * (static_cast<double>(nbins) + 1.0), k2 = 2.02 * g64 / w_rad;
  const double s_lo = 0.95 * 1.41421356237309504880 * sin(0.25 * w_rad);
  bp.g64k1 = static_cast<float>(k1 * (1.0 + 1e-6));
  bp.g64k2 = static_cast<float>(k2 * (1.0 + 1e-6));
  bp.g64c = static_cast<float>((k1 + k2 / s_lo) * (1.0 + 1e-6));
}

BinParams make_bins(int32_t nbins, double w_deg) {
  const double w_rad = w_deg * (kPi / 180.0);
  BinParams bp;
  bp.nbins = nbins;
  {
    const double b = floor(180.0 / w_deg);
    bp.b180 = b < static_cast<double>(nbins - 1) ? static_cast<int32_t>(b) : nbins - 1;
    const double b9 = floor(90.0 / w_deg);
    bp.b90 = b9 < static_cast<double>(nbins - 1) ? static_cast<int32_t>(b9) : nbins - 1;
  }
  bp.invw = static_cast<float>(1.0 / w_rad);
  bp.h = static_cast<float>((kPi / 2.0) / w_rad);
  bp.pinvw = static_cast<float>(kPi / w_rad);
  bp.tmax = static_cast<float>(nbins) - 0.5f;
  // fp32-dot guard
  const double g_x = 5.0 * kTwoM24 * (1.0 + 1e-6) + 1e-12;
  // core error: the exhaustive fp32 bound (computed with a correctly rounded square root)
  // plus the extra half ulp a 1-ulp hardware square root may add, times P <= pi/2; 25 % margin
  const double e_core = (GC_ACOS_CORE_ERR + kTwoM24 * (kPi / 2.0)) * 1.25;
  const double h = (kPi / 2.0) / w_rad;
  const double c = e_core / w_rad + kTwoM24 * (static_cast<double>(nbins) + 1.0 + 2.0 * h) * 1.01;
  bp.g32 = static_cast<float>((2.02 * g_x / w_rad + c) * (1.0 + 1e-6));
  // fp64-dot guard
  const double rho = ((GC_ACOS_FIT_ERR + 4.0 * kTwoM24 * (kPi / 2.0)) / 1.41 + 10.0 * kTwoM24) * 1.25;
  set_fp64_guard(bp, rho, nbins, w_rad);
  const double coef[7] = {GC_ACOS_C0, GC_ACOS_C1, GC_ACOS_C2, GC_ACOS_C3, GC_ACOS_C4, GC_ACOS_C5, GC_ACOS_C6};
  for (int q = 0; q < 7; ++q) bp.pw[q] = static_cast<float>(static_cast<double>(coef[q]) / w_rad);
  return bp;
}

// ---- bin-table core -------------------------------------------------------------------------
// The fp32-dot core of the full span can bin through a table instead of an arccos (core_lut in
// gc_kernels.hip): c = copysign(sqrt(1 - |x|), x) grows with the angle on each half (c =
// sqrt2 sin(theta/2) up to 90 deg, -sqrt2 cos(theta/2) beyond), entry q = round(M (c + 1))
// covers c in [(q - 1/2)/M - 1, (q + 1/2)/M - 1] widened by a margin, and holds the one edge in
// that range as its cosine e (fp32); the pair's side of the edge is the sign of e - x.
// Guard (in the cosine): |x~ - x| <= g_x, |e - cos| <= 2^-25 (fp32 rounding of a cosine in
// [-1, 1]); recheck iff |e - x~| < lut_g = 1.1 (g_x + 2^-25).  (The test's subtraction rounds
// monotonically and lut_g is an fp32 number, so a computed |e - x~| >= lut_g means the exact one
// is too, up to the 10 % margin.)  g_x = kLutDotErr 2^-24: the fp32 rounding of the unit vectors
// (2 units) plus the dot product's arithmetic, taken as up to five roundings of one ulp each
// (three products, two sums) for the matrix-core dot of the fast steps, whatever order and
// rounding mode the instruction uses; the scalar fma chain of the other steps needs 3.
// Selecting the entry: y = 1 - |x~| is exact for |x~| >= 1/2, so |c~ - c| s~ <= g_x + 2^-23 s~^2
// (the dot product through sqrt, whose derivative is 1 / (2 sqrt); the 1-ulp square root);
// g_c = 1.1 (g_x + 2^-23) (for |x~| < 1/2, s > 0.7 and the subtraction's 2^-25 fits the 10 %).
// The table is sound when
//  (a) no widened entry range can hold two edges: 1/M + 2 margin < the smallest gap between
//      consecutive edges in c (M = ceil(4 / w_rad) unless the layout asks for a smaller table,
//      margin = 0.45 (gap - 1/M));
//  (b) where the error of c may exceed the margin (s~ < S* = g_c / margin), no pair can reach an
//      edge: 1 - |x| <= y + g_x <= s~^2 (1 + 2^-22) + g_x, so |c| <= sqrt(S*^2 (1 + 2^-22) + g_x)
//      must stay below the |c| of the first and last edges;
//  (c) the middle entry (q = M: c within 1/(2M) of 0, i.e. both the smallest angles and the
//      largest) holds no edge: 1/(2M) + margin < |c| of the first and last edges.  It stores
//      e = 0 and sends x > 0 to a histogram word counted as bin 0 and x < 0 to one counted as
//      bin nbins - 1 (|x~| > 1 - 1/(4 M^2) there, so it never trips).
// Then every edge within the error of c~ lies in c~'s entry, which holds it.
struct LutPlan {
  bool ok = false;
  int32_t m = 0;
  double margin = 0.0;
  double s_star = 0.0;  // > 0: entries whose |c| may lie below s_star hold NaN (always recheck)
  float g = 0.0f;
};

// Where (b) or (c) fails (bins narrower than about 0.22 deg), the table still serves every pair
// whose c~ the error bound pins within the margin: an entry whose smallest |c| is at least
// S* = g_c / margin has |c~ - c| <= g_c / s~ <= margin for every pair in it, so (a) alone makes its
// edge the only one the pair can be near.  Entries closer to c = 0 (angles within about
// 2 asin(S* / sqrt2) of 0 or 180 deg, the middle entry among them) hold NaN, and their pairs are
// rechecked; S* is kept at or below 0.05 (about 4 deg), so the rechecked share stays small.
// m: the table's M, or 0 for ceil(4 / w_rad).
LutPlan plan_lut(int32_t nbins, double w_deg, int32_t m = 0) {
  LutPlan p;
  if (!((static_cast<double>(nbins) + 0.5) * w_deg >= 180.0) || nbins < 2) return p;
  const double w = w_deg * (kPi / 180.0);
  const double md = m > 0 ? static_cast<double>(m) : ceil(4.0 / w);
  if (2.0 * md + 1.0 > static_cast<double>(kLutMaxEntries)) return p;
  const double sqrt2 = 1.41421356237309504880;
  auto c_right = [&](int e) { return sqrt2 * sin(0.5 * e * w); };
  auto c_left = [&](int e) { return -sqrt2 * cos(0.5 * e * w); };
  double gap = 1e300, c_edge_min = 1e300;
  for (int e = 1; e < nbins; ++e) {
    const double th = e * w_deg;
    if (th > 180.0) break;
    if (th <= 90.0) c_edge_min = fmin(c_edge_min, fabs(c_right(e)));
    if (th >= 90.0) c_edge_min = fmin(c_edge_min, fabs(c_left(e)));
    if (e + 1 < nbins && (e + 1) * w_deg <= 180.0) {
      if ((e + 1) * w_deg <= 90.0) gap = fmin(gap, c_right(e + 1) - c_right(e));
      if (th >= 90.0) gap = fmin(gap, c_left(e + 1) - c_left(e));
    }
  }
  const double margin = 0.45 * (gap - 1.0 / md);
  if (!(margin > 0.0)) return p;
  const double g_x = kLutDotErr * kTwoM24 * (1.0 + 1e-6) + 1e-12;
  const double g_c = 1.1 * (g_x + 2.0 * kTwoM24);
  const double s_star = g_c / margin;
  const double reach = sqrt(s_star * s_star * (1.0 + 4.0 * kTwoM24) + g_x);
  if (!(reach < 0.95 * c_edge_min) || !(0.5 / md + margin < 0.95 * c_edge_min)) {
    if (!(s_star <= 0.05)) return p;
    p.s_star = s_star * (1.0 + 1e-6);
  }
  p.ok = true;
  p.m = static_cast<int32_t>(md);
  p.margin = margin;
  p.g = static_cast<float>(1.1 * (g_x + 0.5 * kTwoM24) * (1.0 + 1e-6));
  return p;
}

// The bin-table kernel's histogram rows: cols 16 keeps one spare row (nbins) and the alias rows
// nbins + 1, nbins + 2; one column keeps 64 spare words and the alias words nbins + 64, nbins + 65.
void apply_lut(BinParams &bp, const LutPlan &lp, int cols, int32_t nbins) {
  bp.lut_m = static_cast<float>(lp.m);
  bp.lut_mb = static_cast<float>(lp.m) + 8388608.0f;  // exact: M < 2^23
  bp.lut_g = lp.g;
  bp.lut_n = 2 * lp.m;
  bp.lut_sh = cols == kHistCols ? 6 : 2;
  bp.lut_alias = cols == kHistCols ? nbins + 2 : nbins + kWave + 1;
}

bool lut_layout(const LutPlan &lp, int32_t nbins, int k, const gc_tuning &tu, LutVariant *lv, int *waves);

// LDS of one compute unit on gfx950.
constexpr size_t kLdsPerCU = 160 * 1024;

// The bin-table kernel's K and layout, unless overridden: K = 2 where the sixteen-column
// histogram fits (two workgroups of 16 waves: eight per SIMD).  Else one column: K = 2 with two
// workgroups of 16 waves per compute unit where they fit beside the table, taking, where the
// table of ceil(4 / w) entries leaves no room for them, the largest sound table that does, down
// to M = 2.5 / w (a smaller M widens the always-recheck zone near 0 and 180 deg: S* grows as
// 1 / margin); else K = 4 with one workgroup of 16 waves (its 80 VGPRs would allow six waves per
// SIMD, the LDS not two workgroups).  With the waves of a workgroup sharing its steps through the
// cursor, the larger groups measured fastest: 100k + 100k at 720 bins 6.35 ms at K = 2 against
// 6.41 at K = 4 and 7.15 at K = 8.  3600 bins: K = 4 with M = 4 / w 8.39 ms; two workgroups of
// K = 2 with M = 2.5 / w 8.21 ms (M = 2.5 / w with one workgroup: 8.61, the rechecks alone).
// lp may be replaced by the smaller table's plan; *k receives the K chosen.
bool lut_choose(LutPlan &lp, int32_t nbins, double w_deg, const gc_tuning &tu, int *k, LutVariant *lv,
                int *waves) {
  if (tu.i_per_lane) {
    *k = tu.i_per_lane;
    return lut_layout(lp, nbins, *k, tu, lv, waves);
  }
  *k = 2;
  if (lut_layout(lp, nbins, 2, tu, lv, waves) && lv->cols == kHistCols) return true;
  if (tu.hist_columns == 0 && tu.waves_per_group == 0) {
    const size_t base = pairs_lds_bytes(lut_hist_words(nbins, 1), true, 2, 2, false, kMaxWavesPerWG, 0);
    if (2 * base < kLdsPerCU) {
      const int64_t tw_max = static_cast<int64_t>((kLdsPerCU / 2 - base) / sizeof(uint32_t));
      const int64_t m_fit = (tw_max / 2 - 1) / 2;  // 2 (2 M + 1) table words
      const double w = w_deg * (kPi / 180.0);
      if (static_cast<double>(m_fit) >= ceil(2.5 / w)) {
        const LutPlan p2 = m_fit < lp.m ? plan_lut(nbins, w_deg, static_cast<int32_t>(m_fit)) : lp;
        gc_tuning t2 = tu;
        t2.hist_columns = 1;
        t2.waves_per_group = kMaxWavesPerWG;
        // With two workgroups per CU the LDS is the tighter resource, and a share of the table
        // reads goes through the vector L1: a quarter while the table stays mostly in its 32 KB,
        // three sixteenths for larger ones.  Measured, an eighth / three sixteenths / a quarter:
        // 1440 x 0.125 deg (29 KB table) 7.46 / 7.26 / 7.08 ms; 1800 x 0.1 (37 KB) 7.48 / 7.28 /
        // 7.13; 2400 x 0.075 (49 KB) 7.57 / 7.37 / 7.32; 3600 x 0.05 (51 KB) 7.92 / 7.75 / 7.83
        // (none: 8.30 at 3600 bins).
        if (t2.l1_share == 0) t2.l1_share = 8 * (2 * static_cast<size_t>(p2.m) + 1) <= 40 * 1024 ? 3 : 4;
        LutVariant lv2;
        int w2 = 0;
        if (p2.ok && lut_layout(p2, nbins, 2, t2, &lv2, &w2)) {
          lp = p2;
          *lv = lv2;
          *waves = w2;
          return true;
        }
      }
    }
  }
  *k = 4;
  return lut_layout(lp, nbins, 4, tu, lv, waves);
}

// The bin-table kernel's layout at a given K: sixteen histogram columns when two workgroups of 8
// waves (12 at K = 4, 16 at K = 2) fit in a compute unit's LDS beside their tables and queues;
// else one column in workgroups of 16 waves (lut_choose sizes the table so that two of them fit
// where it can).  Every table read goes to LDS unless overridden (or unless
// lut_choose picks the one-column layout of two workgroups per CU): a share through the vector
// L1 measured slower where the VALU is as busy as the LDS (720 bins: an eighth 6.40 against
// 6.35 ms) and with one workgroup per CU (3600 bins: an eighth 9.46 against 8.76 ms).  Overrides
// may pick any layout that fits.
// Returns false when none fits.
bool lut_layout(const LutPlan &lp, int32_t nbins, int k, const gc_tuning &tu, LutVariant *lv, int *waves) {
  const int32_t tw = 2 * (2 * lp.m + 1);
  auto lds = [&](int cols, int nw) { return pairs_lds_bytes(lut_hist_words(nbins, cols), true, k, 2, false, nw, tw); };
  // two workgroups per compute unit, each a whole number of waves per SIMD, as many as the
  // registers allow: 8 waves at K = 8 (<= 96 VGPRs: five per SIMD, four used), 12 at K = 4
  // (<= 80: six), 16 at K = 2 (<= 64: eight)
  const int nw2 = k == 2 ? 16 : (k == 4 ? 12 : 8);
  int cols = tu.hist_columns, nw = tu.waves_per_group;
  if (cols == 0) cols = 2 * lds(kHistCols, nw ? nw : nw2) <= kLdsPerCU ? kHistCols : 1;
  if (nw == 0) nw = cols == kHistCols ? nw2 : kMaxWavesPerWG;
  if (lds(cols, nw) > kLdsPerCU) return false;
  lv->cols = cols;
  lv->l1 = tu.l1_share ? tu.l1_share - 1 : 0;
  if (cols == kHistCols && lv->l1 == 3) return false;  // three sixteenths: the one-column layout only
  *waves = nw;
  return true;
}

// ---- series core ---------------------------------------------------------------------------
// fp64 dot, bins ending by about 9 deg: t = s (q0 + q1 y + q2 y^2) / w with y = 1 - x, the
// quadratic truncation of acos(1 - y) / sqrt(y) = sqrt2 (1 + y/12 + 3y^2/160 + 5y^3/896 + ...).
// All omitted terms are positive, so the relative truncation error R grows with y; it is taken
// at y_max = 1 - cos((nbins + 1) w), one bin past the range (beyond it the guard never needs t:
// the quadratic grows with y, so those pairs land at or past the last bin).  The core's
// relative error: R plus roundings of the three scaled coefficients (1 unit of 2^-24), the two
// fmas (2), narrowing y (half a unit through the square root), the 1-ulp square root (2) and
// the product (1): rho_s = 1.25 (R + 7 * 2^-24).  Used when R <= 2e-8.
struct SeriesPlan;
void apply_series(BinParams &bp, const SeriesPlan &sp, int32_t nbins, double w_deg);

struct SeriesPlan {
  bool ok = false;
  float ps[3] = {0.0f, 0.0f, 0.0f};
  double rho = 0.0;
};

SeriesPlan plan_series(int32_t nbins, double w_deg) {
  SeriesPlan p;
  const double w = w_deg * (kPi / 180.0);
  const double th = (static_cast<double>(nbins) + 1.0) * w;
  if (!(th < kPi / 2.0)) return p;
  const double sh = sin(0.5 * th);
  const double y = 2.0 * sh * sh;                       // 1 - cos(th), without cancellation
  const double q_exact = 2.0 * asin(sqrt(0.5 * y)) / sqrt(y);
  const double sqrt2 = 1.41421356237309504880;
  const double q_trunc = sqrt2 * (1.0 + y / 12.0 + 3.0 * y * y / 160.0);
  const double r = (q_exact - q_trunc) / q_exact;
  if (!(r >= 0.0 && r <= 2e-8)) return p;
  p.ok = true;
  p.ps[0] = static_cast<float>(sqrt2 / w);
  p.ps[1] = static_cast<float>(sqrt2 / 12.0 / w);
  p.ps[2] = static_cast<float>(3.0 * sqrt2 / 160.0 / w);
  p.rho = 1.25 * (r + 7.0 * kTwoM24);
  return p;
}

void apply_series(BinParams &bp, const SeriesPlan &sp, int32_t nbins, double w_deg) {
  for (int q = 0; q < 3; ++q) bp.ps[q] = sp.ps[q];
  set_fp64_guard(bp, sp.rho, nbins, w_deg * (kPi / 180.0));
}

// Spans the specialised cores accept: the fp32 core without a clamp needs nbins w to reach
// 180 deg within half a bin; the fp64 core without sign handling needs nbins w <= 90 deg.
bool span_full(int32_t nbins, double w_deg) { return (static_cast<double>(nbins) + 0.5) * w_deg >= 180.0; }
bool span_narrow(int32_t nbins, double w_deg) { return static_cast<double>(nbins) * w_deg <= 90.0; }

// ---- validation ------------------------------------------------------------------------------
gc_status check_bins(int32_t nbins, double w) {
  if (nbins <= 0 || !(w > 0.0) || !isfinite(w)) return GC_ERR_INVALID_ARGUMENT;
  if (nbins > GC_MAX_BINS) return GC_ERR_UNSUPPORTED;
  return GC_OK;
}

gc_status check_catalog(const void *prep, int64_t n) {
  if (n < 0) return GC_ERR_INVALID_ARGUMENT;
  if (n > GC_MAX_GALAXIES) return GC_ERR_UNSUPPORTED;
  if (n > 0 && (!prep || !aligned(prep, GC_ALIGNMENT))) return GC_ERR_INVALID_ARGUMENT;
  return GC_OK;
}

// Scratch of a histogram call: the edge cosines and the bin table.
size_t workspace_bytes(int32_t nbins) { return edge_table_bytes(nbins) + kLutBytes; }

// j-steps of one family in its two segments.  Cross: fast = full blocks x n_j, generic = the
// ragged block's n_j steps.  Self (upper triangle by blocks): fast = sum over full blocks b of
// n - (b+1) BI, generic = n (the diagonal blocks, ragged block included, tile [0, n)).
void family_steps(int64_t n_i, int64_t n_j, bool sym, int k, int64_t *fast, int64_t *generic) {
  *fast = *generic = 0;
  if (n_i == 0 || n_j == 0) return;
  const int64_t bi = static_cast<int64_t>(kWave) * k;
  const int64_t nbf = n_i / bi;
  if (!sym) {
    *fast = nbf * n_j;
    *generic = (n_i % bi) ? n_j : 0;
  } else {
    *fast = nbf * n_j - bi * nbf * (nbf + 1) / 2;
    *generic = n_j;
  }
}

}  // namespace
}  // namespace gc

using namespace gc;

extern "C" {

const char *gc_version(void) { return "gc 0.1 (gfx950)"; }

const char *gc_status_string(gc_status s) {
  switch (s) {
    case GC_OK: return "ok";
    case GC_ERR_INVALID_ARGUMENT: return "invalid argument";
    case GC_ERR_UNSUPPORTED: return "unsupported size";
    case GC_ERR_WORKSPACE: return "workspace too small";
    case GC_ERR_DEVICE: return "device error";
    case GC_ERR_IO: return "file input/output error";
  }
  return "unknown status";
}

int gc_last_device_error(void) { return t_last_hip_error; }

size_t gc_prepared_bytes(int64_t n) {
  if (n < 0 || n > GC_MAX_GALAXIES) return 0;
  return prepared_bytes_for(n);
}

gc_status gc_prepare(const float *ra, const float *dec, int64_t n, void *prepared, gc_stream_t stream) {
  if (n < 0) return GC_ERR_INVALID_ARGUMENT;
  if (n > GC_MAX_GALAXIES) return GC_ERR_UNSUPPORTED;
  if (n > 0 && (!ra || !dec)) return GC_ERR_INVALID_ARGUMENT;
  if (!prepared) return n == 0 ? GC_OK : GC_ERR_INVALID_ARGUMENT;
  if (!aligned(prepared, GC_ALIGNMENT)) return GC_ERR_INVALID_ARGUMENT;
  hipError_t e = launch_prepare(ra, dec, n, prepared, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? GC_OK : device_error(e);
}

size_t gc_workspace_bytes(int32_t nbins) {
  if (nbins <= 0 || nbins > GC_MAX_BINS) return 0;
  return workspace_bytes(nbins);
}

}  // extern "C"

namespace gc {
namespace {

// The histogram call and its parts.  Part p of P takes, in each segment of every family, the
// j-steps floor(T p / P) .. floor(T (p+1) / P) of the same decomposition; with accumulate the
// outputs are not zeroed first, so the pair kernel's flushes add to them.  Every pair's bin is
// fixed by the pair alone (the lane always holds the lower index of a self pair, and the recheck
// is exact), so the parts sum to the single call's result.
// plan_out non-null: only plan (sizes and tuning are checked; the pointers may be null) and
// describe the launch in *plan_out; nothing is enqueued.
gc_status histogram_impl(const void *prep_d, int64_t n_d, const void *prep_r, int64_t n_r, int32_t nbins,
                         double w_deg, uint64_t *dd, uint64_t *dr, uint64_t *rr, void *workspace, size_t ws_bytes,
                         const gc_tuning *tuning, int64_t part, int64_t parts, bool accumulate, gc_stream_t stream,
                         gc_plan *plan_out = nullptr) {
  gc_status st;
  if ((st = check_bins(nbins, w_deg)) != GC_OK) return st;
  if (plan_out) {
    if (n_d < 0 || n_r < 0) return GC_ERR_INVALID_ARGUMENT;
    if (n_d > GC_MAX_GALAXIES || n_r > GC_MAX_GALAXIES) return GC_ERR_UNSUPPORTED;
  } else {
    if ((st = check_catalog(prep_d, n_d)) != GC_OK) return st;
    if ((st = check_catalog(prep_r, n_r)) != GC_OK) return st;
    if (!dd || !dr || !rr || !aligned(dd, 8) || !aligned(dr, 8) || !aligned(rr, 8))
      return GC_ERR_INVALID_ARGUMENT;
    if (!workspace || !aligned(workspace, GC_ALIGNMENT)) return GC_ERR_INVALID_ARGUMENT;
    if (ws_bytes < workspace_bytes(nbins)) return GC_ERR_WORKSPACE;
  }
  gc_tuning tu;
  memset(&tu, 0, sizeof(tu));
  if (tuning) tu = *tuning;
  if ((tu.dot_precision != 0 && tu.dot_precision != 32 && tu.dot_precision != 64) ||
      (tu.i_per_lane != 0 && tu.i_per_lane != 2 && tu.i_per_lane != 4 && tu.i_per_lane != 8) || tu.blocks_per_cu < 0 ||
      tu.blocks_per_cu > kMaxBlocksPerCU || tu.shared_histogram < 0 || tu.shared_histogram > 2 ||
      tu.span_kernel < 0 || tu.span_kernel > 2 || tu.fast_core < 0 || tu.fast_core > 2 ||
      tu.flush_interval < 0 || (tu.hist_columns != 0 && tu.hist_columns != 1 && tu.hist_columns != kHistCols) ||
      (tu.waves_per_group != 0 && (tu.waves_per_group < kWavesPerWG || tu.waves_per_group > kMaxWavesPerWG)) ||
      tu.l1_share < 0 || tu.l1_share > 4 || tu.reserved_ != 0)
    return GC_ERR_INVALID_ARGUMENT;

  // Plan.  Bins narrower than 0.01 deg put most pairs where the fp32 dot product cannot
  // certify the bin; those use the fp64 dot-product instantiation.
  const bool dot64 = tu.dot_precision == 64 || (tu.dot_precision == 0 && w_deg < 0.01);
  // Galaxies per lane: 8 for the fp32 arccos kernels; 4 for the fp64 kernel, whose fp64
  // i-galaxies at K = 8 leave room for only three waves per SIMD; the bin-table core picks its
  // own (lut_choose: 2, or 4 where neither the sixteen-column histogram nor two workgroups of the
  // one-column one fit).
  int k = tu.i_per_lane ? tu.i_per_lane : (dot64 ? 4 : 8);
  // Span-specialised cores: when the bins reach 180 deg (up to half a bin), t cannot exceed
  // nbins + 1 and the fp32 kernel needs no clamp of t (a spare bin takes t = nbins); when they
  // end by 90 deg, the fp64 kernel needs no sign handling (x < 0 is the last bin).
  const bool span_ok = dot64 ? span_narrow(nbins, w_deg) : span_full(nbins, w_deg);
  if (tu.span_kernel == 2 && !span_ok) return GC_ERR_INVALID_ARGUMENT;
  const bool span = span_ok && tu.span_kernel != 1;
  // The arccos-free cores where they are sound: the bin table (fp32 dot, full span, shared
  // histogram) and the series (fp64 dot, bins ending by ~9 deg).
  LutPlan lp = dot64 ? LutPlan() : plan_lut(nbins, w_deg);
  const SeriesPlan sp = dot64 ? plan_series(nbins, w_deg) : SeriesPlan();
  LutVariant lv;
  int lut_waves = kWavesPerWG;
  int k_lut = k;
  const bool lut_fits = lp.ok && lut_choose(lp, nbins, w_deg, tu, &k_lut, &lv, &lut_waves);
  if (lp.ok && !lut_fits && (tu.hist_columns || tu.waves_per_group)) return GC_ERR_INVALID_ARGUMENT;
  const bool lut_ok = lut_fits && span && tu.shared_histogram != 1;
  const bool series_ok = sp.ok && span;
  if (tu.fast_core == 2 && !lut_ok && !series_ok) return GC_ERR_INVALID_ARGUMENT;
  const bool use_lut = lut_ok && tu.fast_core != 1;
  const bool use_series = series_ok && tu.fast_core != 1;
  const int core = (use_lut || use_series) ? 2 : (span ? 1 : 0);
  if (use_lut) k = k_lut;
  if (k == 2 && !use_lut) return GC_ERR_INVALID_ARGUMENT;  // K = 2 is built for the bin-table core only
  const hipStream_t hs = reinterpret_cast<hipStream_t>(stream);

  PairArgs a;
  memset(&a, 0, sizeof(a));
  a.nbins = nbins;
  a.waves = use_lut ? lut_waves : kWavesPerWG;
  a.hist_words = (nbins + kWave + 63) / 64 * 64;  // 64 spare bins past the last (see core32)
  a.bp = make_bins(nbins, w_deg);
  if (use_series) apply_series(a.bp, sp, nbins, w_deg);
  if (use_lut) {
    a.hist_words = lut_hist_words(nbins, lv.cols);
    apply_lut(a.bp, lp, lv.cols, nbins);
  }
  uint2 *lut_dev = reinterpret_cast<uint2 *>(static_cast<char *>(workspace) + edge_table_bytes(nbins));
  a.lut = use_lut ? lut_dev : nullptr;
  double *edge_cos = static_cast<double *>(workspace);
  a.edge_cos = edge_cos;
  a.out[0] = dd;
  a.out[1] = dr;
  a.out[2] = rr;

  const Prepared pd = prepared_view(prep_d, n_d), pr = prepared_view(prep_r, n_r);
  const int64_t nn[3][2] = {{n_d, n_d}, {n_d, n_r}, {n_r, n_r}};
  const Prepared cc[3][2] = {{pd, pd}, {pd, pr}, {pr, pr}};
  int64_t steps[3], total = 0;
  for (int f = 0; f < 3; ++f) {
    const bool sym = f != 1;
    int64_t all_fast = 0, all_gen = 0;
    family_steps(nn[f][0], nn[f][1], sym, k, &all_fast, &all_gen);
    auto cut = [&](int64_t all, int64_t q) {
      return static_cast<int64_t>(static_cast<__int128>(all) * q / parts);
    };
    FamilyWork &fw = a.fam[f];
    fw.fast_begin = cut(all_fast, part);
    fw.fast_steps = cut(all_fast, part + 1) - fw.fast_begin;
    fw.gen_begin = cut(all_gen, part);
    fw.gen_steps = cut(all_gen, part + 1) - fw.gen_begin;
    steps[f] = fw.fast_steps + fw.gen_steps;
    total += steps[f];
    fw.ci = cc[f][0];
    fw.cj = cc[f][1];
    fw.n_i = nn[f][0];
    fw.n_j = nn[f][1];
    fw.sym = sym ? 1 : 0;
  }

  int32_t wb[3] = {0, 0, 0}, we[3] = {0, 0, 0};
  int num_wg = 0;
  if (total > 0) {
    // Histogram placement: one private histogram per wave unless sharing one per workgroup
    // lets more workgroups fit in LDS.
    int cus = 0, occ = 0, occ_shared = 0;
    const int threads = a.waves * kWave;
    const int32_t tw = table_words(a.bp.lut_n, dot64, core);
    // (a layout that exceeds the compute unit's LDS has occupancy 0 and is not asked about)
    const bool must_share = use_lut || tu.shared_histogram == 2;
    const size_t lds_private = pairs_lds_bytes(a.hist_words, false, k, core, dot64, a.waves);
    const size_t lds_shared = pairs_lds_bytes(a.hist_words, true, k, core, dot64, a.waves, tw);
    hipError_t e = device_info(&cus, dot64, k, core, lv, 0, threads, nullptr);
    if (e != hipSuccess) return device_error(e);
    if (!must_share && lds_private <= kLdsPerCU) {
      e = device_info(&cus, dot64, k, core, lv, lds_private, threads, &occ);
      if (e != hipSuccess) return device_error(e);
    }
    if (tu.shared_histogram != 1 && lds_shared <= kLdsPerCU) {
      e = device_info(&cus, dot64, k, core, lv, lds_shared, threads, &occ_shared);
      if (e != hipSuccess) return device_error(e);
    }
    bool shared = must_share || (tu.shared_histogram == 0 && occ_shared > occ);
    if (shared) occ = occ_shared;
    a.shared_hist = shared ? 1 : 0;
    // Between two flushes a bin must stay within +-2^31: each j-step adds at most 2 * 64 K
    // per wave, and in shared mode every wave of the workgroup adds to the same histogram.  A
    // wave tests the interval after every batch of j-steps (up to 16 with the matrix-core dot),
    // so it may run 15 steps past it; the margin of 32 covers that.
    const int64_t max_inc = 2ll * kWave * k * (shared ? a.waves : 1);
    const int64_t auto_flush = static_cast<int64_t>(0x7fffffffll / max_inc) - 32;
    a.flush_interval = tu.flush_interval ? (tu.flush_interval < auto_flush ? tu.flush_interval : auto_flush)
                                         : auto_flush;
    // Workgroups: kOversubscribe times as many as fit on the compute units at once (whole
    // rounds).  Each takes a static share of its family's steps; as workgroups finish, the
    // dispatcher starts the waiting ones on the freed slots, so the families' unequal cost per
    // step (and the ragged end of the triangles) leaves a tail of one short workgroup instead of
    // one whole persistent share (100k + 100k at 720 bins: 7.39 -> 6.85 ms).  Four rounds measured
    // best overall: 720 bins 6.14 ms with three, 6.12 with four or five, 6.15 with eight; 3600 bins
    // 7.59 / 7.53 / 7.49; the patch (six resident per CU) 7.54 with three, 7.45 with four.
    if (occ < 1 && !tu.blocks_per_cu) return GC_ERR_UNSUPPORTED;
    const int per_cu = tu.blocks_per_cu ? tu.blocks_per_cu : kOversubscribe * occ;
    int64_t g = static_cast<int64_t>(per_cu) * cus;
    if (g > kMaxWorkgroups) g = kMaxWorkgroups;
    // at least kMinStepsPerWave j-steps per wave: a small job takes fewer workgroups, so each
    // one's fixed cost (table copy, histogram zeroing, final flush) spreads over more pairs
    // (rounded to whole rounds of one workgroup per CU: 261 workgroups on 256 CUs left five CUs
    // with two, and the job waited for them: 0.236 against 0.195 ms for 10k + 10k)
    int64_t want = (total + kMinStepsPerWave * a.waves - 1) / (kMinStepsPerWave * a.waves);
    if (cus > 0 && want >= cus / 2) want = (want + cus / 2) / cus * cus;
    if (g > want) g = want;
    int nonzero = 0;
    for (int f = 0; f < 3; ++f) nonzero += steps[f] > 0;
    if (g < nonzero) g = nonzero;
    // split workgroups among families in proportion to their j-steps
    int64_t gf[3];
    int64_t used = 0;
    double frac[3];
    for (int f = 0; f < 3; ++f) {
      const double exact = static_cast<double>(g) * static_cast<double>(steps[f]) / static_cast<double>(total);
      gf[f] = steps[f] > 0 ? static_cast<int64_t>(exact) : 0;
      if (steps[f] > 0 && gf[f] < 1) gf[f] = 1;
      frac[f] = exact - static_cast<double>(gf[f]);
      used += gf[f];
    }
    while (used < g) {
      int best = -1;
      for (int f = 0; f < 3; ++f)
        if (steps[f] > 0 && (best < 0 || frac[f] > frac[best])) best = f;
      gf[best] += 1;
      frac[best] -= 1.0;
      ++used;
    }
    while (used > g) {  // only when the minimum of one workgroup per family overshot
      int best = -1;
      for (int f = 0; f < 3; ++f)
        if (gf[f] > 1 && (best < 0 || frac[f] < frac[best])) best = f;
      gf[best] -= 1;
      frac[best] += 1.0;
      --used;
    }
    int32_t cur = 0;
    for (int f = 0; f < 3; ++f) {
      wb[f] = cur;
      cur += static_cast<int32_t>(gf[f]);
      we[f] = cur;
      a.fam[f].wg_begin = wb[f];
      a.fam[f].wg_end = we[f];
    }
    num_wg = cur;
    if (plan_out) {
      plan_out->core = core;
      plan_out->dot_precision = dot64 ? 64 : 32;
      plan_out->i_per_lane = k;
      plan_out->hist_columns = use_lut ? lv.cols : 1;
      plan_out->waves_per_group = a.waves;
      plan_out->l1_share = use_lut ? lv.l1 + 1 : 0;
      plan_out->shared_histogram = a.shared_hist;
      plan_out->blocks_per_cu = per_cu;
      plan_out->workgroups = num_wg;
      plan_out->lds_bytes = static_cast<int32_t>(shared ? lds_shared : lds_private);
      plan_out->flush_interval = a.flush_interval;
      plan_out->always_recheck = use_lut && lp.s_star > 0.0 ? 1 : 0;
      plan_out->lut_m = use_lut ? lp.m : 0;
      return GC_OK;
    }
  }
  if (plan_out) {
    if (total == 0) {  // no work: nothing to launch but the zeroing of the outputs
      memset(plan_out, 0, sizeof(*plan_out));
      plan_out->core = core;
      plan_out->dot_precision = dot64 ? 64 : 32;
      plan_out->i_per_lane = k;
    }
    return GC_OK;
  }
  // One launch builds the tables and, unless the call accumulates, zeroes the outputs that the
  // pair kernel's flushes then add into; the pair kernel follows on the same stream.
  if (total > 0 || !accumulate) {
    TablesArgs t;
    t.nbins = nbins;
    t.w_deg = w_deg;
    t.edge_cos = edge_cos;
    if (use_lut && total > 0) {
      t.lut = lut_dev;
      t.m = lp.m;
      t.margin = lp.margin;
      t.cols = lv.cols;
      t.alias = a.bp.lut_alias;
      t.s_star = lp.s_star;
    }
    if (!accumulate) {
      t.out[0] = dd;
      t.out[1] = dr;
      t.out[2] = rr;
    }
    hipError_t e = launch_tables(t, hs);
    if (e != hipSuccess) return device_error(e);
  }
  if (total > 0) {
    hipError_t e = launch_pairs(a, num_wg, dot64, k, core, lv, hs);
    if (e != hipSuccess) return device_error(e);
  }
  return GC_OK;
}

}  // namespace
}  // namespace gc

extern "C" {

gc_status gc_histogram_dd_dr_rr_tuned(const void *prep_d, int64_t n_d, const void *prep_r, int64_t n_r,
                                      int32_t nbins, double w_deg, uint64_t *dd, uint64_t *dr,
                                      uint64_t *rr, void *workspace, size_t ws_bytes,
                                      const gc_tuning *tuning, gc_stream_t stream) {
  return histogram_impl(prep_d, n_d, prep_r, n_r, nbins, w_deg, dd, dr, rr, workspace, ws_bytes, tuning, 0, 1, false,
                        stream);
}

gc_status gc_histogram_part(const void *prep_d, int64_t n_d, const void *prep_r, int64_t n_r, int32_t nbins,
                            double w_deg, int64_t part, int64_t parts, uint64_t *dd, uint64_t *dr, uint64_t *rr,
                            void *workspace, size_t ws_bytes, const gc_tuning *tuning, gc_stream_t stream) {
  if (parts < 1 || parts > GC_MAX_PARTS || part < 0 || part >= parts) return GC_ERR_INVALID_ARGUMENT;
  return histogram_impl(prep_d, n_d, prep_r, n_r, nbins, w_deg, dd, dr, rr, workspace, ws_bytes, tuning, part, parts,
                        true, stream);
}

gc_status gc_launch_plan(int64_t n_d, int64_t n_r, int32_t nbins, double w_deg, const gc_tuning *tuning,
                         gc_plan *plan) {
  if (!plan) return GC_ERR_INVALID_ARGUMENT;
  return histogram_impl(nullptr, n_d, nullptr, n_r, nbins, w_deg, nullptr, nullptr, nullptr, nullptr, 0, tuning, 0, 1,
                        false, nullptr, plan);
}

}  // extern "C"

// The allocation-free entry point's scratch: one array per GPU, in device memory that the runtime
// sets up with the library's code, held until the process ends.  In host code `scratch` names a
// host-side stand-in, never the device array: its device address is taken once per device with
// hipGetSymbolAddress (that device current), and only that address reaches kernels.
static __device__ __align__(256) unsigned char scratch[GC_STATIC_SCRATCH_BYTES];
static_assert(((GC_MAX_BINS + 1) * sizeof(double) + 255) / 256 * 256 + gc::kLutBytes <= GC_STATIC_SCRATCH_BYTES,
              "the static scratch holds the tables of every bin count");

namespace gc {
namespace {

void *g_scratch[kMaxDevices];  // the current device's array address, guarded by g_mu

hipError_t static_scratch(void **ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p || !aligned(p, GC_ALIGNMENT)) return hipErrorInvalidSymbol;
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return hipSuccess;
}

}  // namespace
}  // namespace gc

extern "C" {

gc_status gc_histogram_dd_dr_rr_noalloc(const void *prep_d, int64_t n_d, const void *prep_r, int64_t n_r,
                                        int32_t nbins, double w_deg, uint64_t *dd, uint64_t *dr, uint64_t *rr,
                                        gc_stream_t stream) {
  // the checks of histogram_impl that precede any HIP call, so a bad call reaches none
  gc_status st;
  if ((st = check_bins(nbins, w_deg)) != GC_OK) return st;
  if ((st = check_catalog(prep_d, n_d)) != GC_OK) return st;
  if ((st = check_catalog(prep_r, n_r)) != GC_OK) return st;
  if (!dd || !dr || !rr || !aligned(dd, 8) || !aligned(dr, 8) || !aligned(rr, 8)) return GC_ERR_INVALID_ARGUMENT;
  // the tables of every bin count the library accepts fit the array (checked at compile time)
  if (workspace_bytes(nbins) > GC_STATIC_SCRATCH_BYTES) return GC_ERR_UNSUPPORTED;
  void *ws = nullptr;
  const hipError_t e = static_scratch(&ws);
  if (e != hipSuccess) return device_error(e);
  return histogram_impl(prep_d, n_d, prep_r, n_r, nbins, w_deg, dd, dr, rr, ws, GC_STATIC_SCRATCH_BYTES, nullptr, 0,
                        1, false, stream);
}

gc_status gc_histogram_dd_dr_rr(const void *prep_d, int64_t n_d, const void *prep_r, int64_t n_r,
                                int32_t nbins, double w_deg, uint64_t *dd, uint64_t *dr, uint64_t *rr,
                                void *workspace, size_t ws_bytes, gc_stream_t stream) {
  return gc_histogram_dd_dr_rr_tuned(prep_d, n_d, prep_r, n_r, nbins, w_deg, dd, dr, rr, workspace,
                                     ws_bytes, nullptr, stream);
}

gc_status gc_histogram_totals(const uint64_t *dd, const uint64_t *dr, const uint64_t *rr, int32_t nbins,
                              uint64_t *totals, gc_stream_t stream) {
  if (nbins <= 0) return GC_ERR_INVALID_ARGUMENT;
  if (nbins > GC_MAX_BINS) return GC_ERR_UNSUPPORTED;
  if (!dd || !dr || !rr || !totals || !aligned(dd, 8) || !aligned(dr, 8) || !aligned(rr, 8) ||
      !aligned(totals, 8))
    return GC_ERR_INVALID_ARGUMENT;
  hipError_t e = launch_totals(dd, dr, rr, nbins, totals, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? GC_OK : device_error(e);
}

gc_status gc_omega(const uint64_t *dd, const uint64_t *dr, const uint64_t *rr, int32_t nbins, int64_t n_d,
                   int64_t n_r, double *omega, gc_stream_t stream) {
  if (nbins <= 0 || n_d < 0 || n_r < 0) return GC_ERR_INVALID_ARGUMENT;
  if (nbins > GC_MAX_BINS) return GC_ERR_UNSUPPORTED;
  if (!dd || !dr || !rr || !omega || !aligned(dd, 8) || !aligned(dr, 8) || !aligned(rr, 8) ||
      !aligned(omega, 8))
    return GC_ERR_INVALID_ARGUMENT;
  hipError_t e = launch_omega(dd, dr, rr, nbins, n_d, n_r, omega, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? GC_OK : device_error(e);
}

gc_status gc_eval_angle_core(const float *x32, const double *x64, int64_t n, int32_t nbins, double w_deg,
                             int32_t dot_precision, int32_t *bin_out, uint8_t *trip_out, int32_t *exact_out,
                             float *t_out, void *workspace, size_t ws_bytes, gc_stream_t stream) {
  gc_status st;
  if ((st = check_bins(nbins, w_deg)) != GC_OK) return st;
  if (n < 0 || (dot_precision != 32 && dot_precision != 64)) return GC_ERR_INVALID_ARGUMENT;
  const bool d64 = dot_precision == 64;
  if (n > 0 && ((d64 && !x64) || (!d64 && !x32) || !bin_out || !trip_out)) return GC_ERR_INVALID_ARGUMENT;
  // the same core the histogram call would use for these bins
  const bool span = d64 ? span_narrow(nbins, w_deg) : span_full(nbins, w_deg);
  LutPlan lp = d64 ? LutPlan() : plan_lut(nbins, w_deg);
  const SeriesPlan sp = d64 ? plan_series(nbins, w_deg) : SeriesPlan();
  gc_tuning tu0;
  memset(&tu0, 0, sizeof(tu0));
  LutVariant lv;
  int lut_waves = 0, lut_k = 0;
  const bool use_lut = lp.ok && span && lut_choose(lp, nbins, w_deg, tu0, &lut_k, &lv, &lut_waves);
  const bool use_series = sp.ok && span;
  const int core = (use_lut || use_series) ? 2 : (span ? 1 : 0);
  if (n == 0) return GC_OK;
  const bool need_ws = exact_out || use_lut;
  if (need_ws && (!workspace || !aligned(workspace, GC_ALIGNMENT))) return GC_ERR_INVALID_ARGUMENT;
  if (need_ws && ws_bytes < edge_table_bytes(nbins) + kLutBytes) return GC_ERR_WORKSPACE;
  BinParams bp = make_bins(nbins, w_deg);
  if (use_series) apply_series(bp, sp, nbins, w_deg);
  const hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  double *edge_cos = static_cast<double *>(workspace);
  uint2 *lut = need_ws ? reinterpret_cast<uint2 *>(static_cast<char *>(workspace) + edge_table_bytes(nbins)) : nullptr;
  hipError_t e = hipSuccess;
  if (use_lut) apply_lut(bp, lp, lv.cols, nbins);
  if (need_ws) {
    TablesArgs t;
    t.nbins = nbins;
    t.w_deg = w_deg;
    t.edge_cos = edge_cos;
    if (use_lut) {
      t.lut = lut;
      t.m = lp.m;
      t.margin = lp.margin;
      t.cols = lv.cols;
      t.alias = bp.lut_alias;
      t.s_star = lp.s_star;
    }
    e = launch_tables(t, hs);
  }
  if (e == hipSuccess)
    e = launch_eval_core(x32, x64, n, bp, d64, core, lut, exact_out ? edge_cos : nullptr, bin_out, trip_out,
                         exact_out, t_out, hs);
  return e == hipSuccess ? GC_OK : device_error(e);
}

gc_status gc_eval_dot_mfma(const float *ax, const float *ay, const float *az, const float *bx, const float *by,
                           const float *bz, int64_t ntiles, float *out, gc_stream_t stream) {
  if (ntiles < 0) return GC_ERR_INVALID_ARGUMENT;
  if (ntiles == 0) return GC_OK;
  if (!ax || !ay || !az || !bx || !by || !bz || !out) return GC_ERR_INVALID_ARGUMENT;
  if (ntiles > 0x7fffffff) return GC_ERR_UNSUPPORTED;
  const hipError_t e =
      launch_eval_dot_mfma(ax, ay, az, bx, by, bz, ntiles, out, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? GC_OK : device_error(e);
}

}  // extern "C"
