// HIP kernels for gfx950 (MI355X): all-pairs angular-separation histograms.
//
// The operation ("CUDA Deep Dive: 10B Galaxy Pairs on an RTX 5080", section "The
// problem"): for every ordered pair of galaxies, theta = the angle between their
// radius vectors, binned into nbins bins of width w, for the families DD, DR, RR.
//
// Kernels:
//   prepare_kernel - (alpha, delta) arcmin -> unit radius vector, fp64 math, stored
//                    as SoA fp32 (correctly rounded) and fp64.
//   tables_kernel  - the fp64 edge cosines and the bin table; zeroes the outputs.
//   pairs_kernel   - the hot loop.  Each workgroup takes an even share of its family's
//                    "j-steps" (one j galaxy against an i-block of 64*K galaxies held K per
//                    lane in VGPRs), which its waves split among themselves in chunks; the
//                    grid holds several rounds of workgroups.  j is wave-uniform, so it is
//                    streamed through the scalar unit (s_load into SGPRs, used directly
//                    as VALU operands) instead of being staged in LDS; the bin-table core
//                    instead takes its dot products from the matrix cores, 16 i x 16 j at a
//                    time.  Per pair: dot product, then one of the cores (an arccos of
//                    sqrt times a fitted polynomial; the bin table; the series), bin index,
//                    certified guard; ds_add_u32 into an LDS histogram.
//                    Pairs the guard cannot certify are queued in LDS and re-binned in fp64,
//                    64 at a time with all lanes busy.  A workgroup's histogram is added
//                    into the 64-bit outputs with atomics.
//   totals_kernel  - per-family sums (wave-shuffle reduction) for the exact N^2 check.
//   omega_kernel   - Landy-Szalay estimator in fp64.
//   eval_core_kernel - the pair kernel's angle-to-bin core on given cosines (diagnostic).
#include "gc_acos_poly.h"
#include "gc_internal.h"

namespace gc {
namespace {

static_assert(GC_ACOS_DEGREE == 6, "acos core is written for a degree-6 polynomial");

typedef __attribute__((address_space(4))) const float cfloat_t;
typedef __attribute__((address_space(4))) const double cdouble_t;

// Reads through the constant address space: with a wave-uniform index these become
// scalar-unit loads (s_load_*) whose results feed VALU instructions as SGPR operands.
// Valid because the prepared catalogs are never written while a pair kernel runs.
__device__ __forceinline__ float ld_uniform(const float *p, int64_t i) {
  return ((const cfloat_t *)p)[i];
}
__device__ __forceinline__ double ld_uniform(const double *p, int64_t i) {
  return ((const cdouble_t *)p)[i];
}

constexpr float kHalfPiF = 1.57079632679489661923f;
typedef float float4v __attribute__((ext_vector_type(4)));  // an MFMA accumulator

// P(a) with acos(a) ~= sqrt(1 - a) * P(a) on [0, 1] (Horner, fp32 FMA).
__device__ __forceinline__ float acos_poly(float a) {
  float p = GC_ACOS_C6;
  p = fmaf(p, a, GC_ACOS_C5);
  p = fmaf(p, a, GC_ACOS_C4);
  p = fmaf(p, a, GC_ACOS_C3);
  p = fmaf(p, a, GC_ACOS_C2);
  p = fmaf(p, a, GC_ACOS_C1);
  p = fmaf(p, a, GC_ACOS_C0);
  return p;
}

// A wave-uniform constant held in a VGPR.  A VALU instruction on this target reads at most
// one scalar operand, so fma(a, sgpr, sgpr) needs one constant in a VGPR; the opaque move
// keeps the compiler from re-materialising it (one v_mov per use) inside the pair loop.
__device__ __forceinline__ float in_vgpr(float v) {
  float r;
  asm("v_mov_b32 %0, %1" : "=v"(r) : "s"(v));
  return r;
}

// fp32-dot core.  x is the fp32 dot product of the two fp32 unit vectors.
//   s  = sqrt(1 - |x|) (clamped at 0),  q = pi/2 - s P(|x|) = pi/2 - acos(|x|)
//   theta = pi/2 - sign(x) q,  t = theta / w,  tc = clamp(t, 0.5, tmax_v)
//   k = trunc(tc); recheck iff |tc - round(tc)| * s < g32, i.e. iff an inner bin edge
//   lies within the certified error bound 2.02 g_x / (s w) + C of t.
// tmax_v = nbins - 1/2 + lane: past the last bin each lane clamps into a spare bin of its
// own (bins nbins .. nbins + 63, folded into bin nbins - 1 by the flush), so a wave whose
// pairs all lie beyond the binned range adds to 64 different LDS words instead of one.
// The integers nbins .. nbins + 63 are edges of spare bins only; a pair the guard flags
// near one is rechecked into bin nbins - 1, where it already counts.
// FULL_SPAN (nbins w >= 180 deg - w/2): t stays below nbins + 1, so the clamp is dropped;
// t = nbins lands in spare bin nbins, and t in (-1, 0) truncates to 0.  Without the clamp
// the guard can only trip more often (near t = 0 and t = nbins, where no inner edge lies),
// never less.
// h_v is (pi/2)/w held in a VGPR (see in_vgpr).
template <bool FULL_SPAN>
__device__ __forceinline__ void core32(float x, const BinParams &bp, float h_v, float tmax_v, uint32_t &k,
                                       bool &trip, float &t_raw) {
  const float a = fabsf(x);
  const float s = __builtin_amdgcn_sqrtf(__builtin_amdgcn_fmed3f(1.0f - a, 0.0f, 1.0f));
  const float q = fmaf(-s, acos_poly(a), kHalfPiF);
  const float t = fmaf(copysignf(q, x), -bp.invw, h_v);
  t_raw = t;
  const float tc = FULL_SPAN ? t : __builtin_amdgcn_fmed3f(t, 0.5f, tmax_v);
  k = static_cast<uint32_t>(tc);
  trip = fabsf(tc - __builtin_rintf(tc)) * s < bp.g32;
}

// fp64-dot core.  x is the fp64 dot product of the fp64 unit vectors; 1 - |x| is formed
// in fp64 before narrowing, so small angles keep full relative precision.
//   r = sqrt(1 - |x|) P(|x|) = acos(|x|);  t = r / w (x >= 0) or (pi - r) / w (x < 0).
//   recheck iff |tc - round(tc)| * s < g64k1 * s + g64k2 (NARROW and SERIES: iff
//   |tc - round(tc)| < g64c, the same window where an edge can be).
// NARROW (nbins w <= 90 deg): a pair with x < 0 is past 90 degrees and belongs to the last
// bin, so no sign handling is needed.  The signed x goes through the same expression with
// 1 - x clamped to [0, 1]: for a in [-1, 0] every term of P(a) is positive (the
// coefficients alternate in sign), so P(a) >= P(0) ~ pi/2 (1 - 1.3e-7) and, with s = 1,
// t >= nbins (1 - 1e-6) > nbins - 1/2, which truncates to the last bin or a spare bin past
// it (the guard may flag it near a spare bin's edge; the recheck keeps it in the last bin).  The coefficients come pre-scaled by 1 / w (bp.pw; the
// highest one in a VGPR, pw6_v), so t = s P'(x) without a final multiply.  tmax_v: as in
// core32, each lane's own spare bin past the last bin.
// SERIES (bins ending by about 9 deg): with y = 1 - x formed in fp64, acos(1 - y) / sqrt(y) =
// sqrt2 (1 + y/12 + 3 y^2/160 + 5 y^3/896 + ...), all terms positive; over the binned range
// (y <= 1 - cos((nbins + 1) w)) the quadratic truncation is within its next term, far below the
// guard's rho, so t = s (q0 + q1 y + q2 y^2) / w (coefficients pre-scaled, q2 in a VGPR).  The
// quadratic grows with y, so every pair past the range, x < 0 included (y clamped to 1), lands
// at or past the last bin.
// SERIES takes y = 1 - x itself: the pair kernel forms it inside the dot product,
// fma(-x_i, x_j, fma(-y_i, y_j, fma(-z_i, z_j, 1))), three fp64 roundings of values in [0, 2]
// (< 7e-16 absolute, inside the guard's 1e-14 allowance for the cosine) and no subtraction.
template <int MODE>  // 0: generic, 1: NARROW, 2: SERIES
__device__ __forceinline__ void core64(double x, const BinParams &bp, float pw6_v, float tmax_v, uint32_t &k,
                                       bool &trip, float &t_raw) {
  float s, t;
  if constexpr (MODE == 2) {
    const float y = __builtin_amdgcn_fmed3f(static_cast<float>(x), 0.0f, 1.0f);  // x holds y = 1 - cos
    s = __builtin_amdgcn_sqrtf(y);
    t = s * fmaf(fmaf(pw6_v, y, bp.ps[1]), y, bp.ps[0]);
  } else if constexpr (MODE == 1) {
    s = __builtin_amdgcn_sqrtf(__builtin_amdgcn_fmed3f(static_cast<float>(1.0 - x), 0.0f, 1.0f));
    const float a = static_cast<float>(x);
    float p = fmaf(pw6_v, a, bp.pw[5]);
    p = fmaf(p, a, bp.pw[4]);
    p = fmaf(p, a, bp.pw[3]);
    p = fmaf(p, a, bp.pw[2]);
    p = fmaf(p, a, bp.pw[1]);
    p = fmaf(p, a, bp.pw[0]);
    t = s * p;
  } else {
    const double ax = fabs(x);
    const float y = static_cast<float>(fmax(1.0 - ax, 0.0));
    const float a = static_cast<float>(ax);
    s = __builtin_amdgcn_sqrtf(y);
    const float r = s * acos_poly(a);
    const int hi = __double2hiint(x);
    const float cr = copysignf(r, __int_as_float(hi));
    const float off = __int_as_float((hi >> 31) & __float_as_int(bp.pinvw));
    t = fmaf(cr, bp.invw, off);
  }
  t_raw = t;
  const float tc = __builtin_amdgcn_fmed3f(t, 0.5f, tmax_v);
  k = static_cast<uint32_t>(tc);
  if constexpr (MODE == 0) {
    // |tc - round(tc)| * s < g64k1 * s + g64k2, arranged so that each instruction reads one
    // scalar constant
    trip = (fabsf(tc - __builtin_rintf(tc)) - bp.g64k1) * s < bp.g64k2;
  } else {
    // no edge near 180 deg: s is bounded below near every edge, and the window is constant
    trip = fabsf(tc - __builtin_rintf(tc)) < bp.g64c;
  }
}

// Bin-table core (fp32 dot, bins covering 0..180 deg).  The table entry is chosen by
//   c = copysign(sqrt(1 - |x|), x),
// which increases with the angle on each half: c in [0, 1] for 0..90 deg (c = sqrt2 sin(theta/2)),
// c in [-1, 0) for 90..180 deg (c = -sqrt2 cos(theta/2)), so equal steps of c are steps of
// comparable angle.  Entry q = round(M (c + 1)) holds the one bin edge whose c lies in the
// entry's range widened by a margin, as e = cos(edge angle) in fp32, and B = the bin above the
// edge; with no edge in range, e = 4 (beyond every cosine) and B = the entry's bin.  A pair lies
// below the edge iff x > e, so bin = B - [e - x < 0], and it is rechecked iff |e - x| < lut_g,
// which bounds the dot product's error plus the rounding of e.  The side of the edge is thus
// decided on the cosine itself; c only selects the edge, and the host checks that the error of c
// can never select an entry without the edge a pair is near.
// lut_key: fma(c, M, M + 2^23) is 2^23 + q exactly (one rounding of M (c + 1) + 2^23 to an
// integer), so q is the key's bit pattern minus that of 2^23.
// mb: M + 2^23 (bp.lut_mb); the pair kernel passes it held in a VGPR.
__device__ __forceinline__ float lut_key(float x, const BinParams &bp, float mb, float &c) {
  const float s = __builtin_amdgcn_sqrtf(__builtin_amdgcn_fmed3f(1.0f - fabsf(x), 0.0f, 1.0f));
  c = copysignf(s, x);
  return fmaf(c, bp.lut_m, mb);
}
constexpr uint32_t kLutKeyBias = 0x4B000000u;  // bit pattern of 2^23

// The core with the table in global memory (diagnostic kernel): entry = {e bits, row offset of B}.
// A NaN e (an always-recheck entry) fails the guard's comparison, so the pair trips.
__device__ __forceinline__ void core_lut(float x, const BinParams &bp, const uint2 *tab, uint32_t &k, bool &trip,
                                         float &c_raw) {
  float c;
  const uint2 ent = tab[__float_as_uint(lut_key(x, bp, bp.lut_mb, c)) - kLutKeyBias];
  const float d = __uint_as_float(ent.x) - x;
  trip = !(fabsf(d) >= bp.lut_g);
  k = (ent.y >> bp.lut_sh) - (__float_as_uint(d) >> 31);
  c_raw = c;
}

// The pair kernel's form, with the table in LDS: entry = {e bits, byte address of bin B's
// histogram word}.  Entry q sits at LDS byte tab + 8 q = (key bits << 3) + tab_bias with
// tab_bias = tab - (bits of 2^23 << 3) (mod 2^32): one shift-and-add per lookup.  The histogram
// word to add to is (sign of e - x, as 0 or -1) << 2 plus the entry's address: one more.
typedef __attribute__((address_space(3))) const unsigned long long lds_entry_t;
typedef __attribute__((address_space(3))) uint32_t lds_word_t;
__device__ __forceinline__ uint32_t lds_address(const void *p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const char *)p));
}
__device__ __forceinline__ uint2 lut_read_lds(float key, uint32_t tab_bias) {
  const unsigned long long v =
      *reinterpret_cast<lds_entry_t *>(static_cast<uintptr_t>((__float_as_uint(key) << 3) + tab_bias));
  return make_uint2(static_cast<uint32_t>(v), static_cast<uint32_t>(v >> 32));
}
// The histogram word of a bin-table pair from d = e - x: the entry's row (bin B) for x <= e, the
// row below it (bin B - 1) for x > e (d < 0, whose sign bit becomes a one-row step down).
__device__ __forceinline__ uint32_t lut_signed_address(float d, uint32_t row, const BinParams &bp) {
  return (static_cast<uint32_t>(__float_as_int(d) >> 31) << bp.lut_sh) + row;
}
__device__ __forceinline__ uint32_t lut_word_address(float x, uint2 ent, const BinParams &bp, bool &trip) {
  const float d = __uint_as_float(ent.x) - x;
  trip = !(fabsf(d) >= bp.lut_g);  // NaN e (always-recheck entry): trips
  return lut_signed_address(d, ent.y, bp);
}

// Exact recheck in the cosine domain.  theta >= e w  <=>  x <= cos(e w), so bin k holds x
// iff c[k+1] < x <= c[k], with c[e] = cos(e w) in fp64 (c[0] = 1; c[e] = -inf past 180
// degrees).  Starting from the fast-path bin k, walk to the bin that satisfies this.  The
// result differs from truncating the fp64 angle only for x within fp64 rounding of an
// edge cosine (angles within ~1e-11 degrees of an edge).
__device__ __forceinline__ uint32_t exact_bin(double x, uint32_t k, const double *__restrict__ c,
                                              int32_t nbins) {
  while (k > 0 && x > c[k]) --k;
  while (k + 1 < static_cast<uint32_t>(nbins) && x <= c[k + 1]) ++k;
  return k;
}

// A value the whole wave holds, made visibly so (a scalar register) for the compiler.
__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(static_cast<uint64_t>(v) >> 32));
  return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

__device__ __forceinline__ double dot64(const Prepared &a, int64_t i, const Prepared &b, int64_t j) {
  return fma(a.x64[i], b.x64[j], fma(a.y64[i], b.y64[j], a.z64[i] * b.z64[j]));
}

// ----------------------------------------------------------------------------- prepare
__global__ void __launch_bounds__(256) prepare_kernel(const float *__restrict__ ra,
                                                      const float *__restrict__ dec, int64_t n,
                                                      int64_t padded, float *x, float *y, float *z,
                                                      double *x64, double *y64, double *z64) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= padded) return;
  double ux = 0.0, uy = 0.0, uz = 0.0;
  if (idx < n) {
    const double arcmin = 3.14159265358979323846 / 10800.0;
    // A non-finite coordinate would make a NaN vector, whose cosines could index the pair
    // kernels' tables anywhere; such a galaxy is placed at alpha = delta = 0 instead.
    const bool ok = __builtin_isfinite(ra[idx]) && __builtin_isfinite(dec[idx]);
    const double a = ok ? static_cast<double>(ra[idx]) * arcmin : 0.0;
    const double d = ok ? static_cast<double>(dec[idx]) * arcmin : 0.0;
    double sa, ca, sd, cd;
    sincos(a, &sa, &ca);
    sincos(d, &sd, &cd);
    ux = cd * ca;
    uy = cd * sa;
    uz = sd;
  }
  x[idx] = static_cast<float>(ux);
  y[idx] = static_cast<float>(uy);
  z[idx] = static_cast<float>(uz);
  x64[idx] = ux;
  y64[idx] = uy;
  z64[idx] = uz;
}

// ------------------------------------------------------------------------------- pairs
struct FastTag { static constexpr bool value = false; };
struct GenericTag { static constexpr bool value = true; };

template <bool D64> struct Real;
template <> struct Real<false> { typedef float T; };
template <> struct Real<true> { typedef double T; };

// Re-bin the c <= 64 queued pairs in entries [first, first + c) exactly in fp64 (one pair
// per lane) and move their counts from the fast-path row to the exact bin's row.  Entry e:
// word 2e = j, word 2e+1 = (i - i0) << 16 | (fast-path row + 1); both fields fit in 16 bits
// (i - i0 < 64 K <= 512 and rows < kMaxBins + 66, checked at compile time).
// A fast-path row >= nbins is a spare row standing for bin nbins - 1.  The counts move in the lane's own column of a
// multi-column histogram (any column serves: the flush sums them).  The walk to the exact bin
// starts from the fast-path row, or, when that row lies on the other side of 90 deg from the pair
// (an always-recheck table entry near 0 or 180 deg), from the end of the range on the pair's side.
// The rows of i and j are clamped into their catalogs and the fast-path row into the histogram's
// rows, so even a corrupted entry cannot read or write past them.
template <int COLS>
__device__ __forceinline__ void drain_queue(uint32_t *hist, const uint32_t *queue, int first, int c,
                                            const Prepared &ci, const Prepared &cj, int64_t i0, int64_t n_i,
                                            int64_t n_j, uint32_t w, const double *edge_cos, int32_t nbins, int32_t b90,
                                            int32_t b180, int32_t rows) {
  const int lane = threadIdx.x & (kWave - 1);
  __builtin_amdgcn_wave_barrier();
  if (lane < c) {
    const int e = first + lane;
    const int64_t jq = queue[2 * e];
    const int64_t jj = jq < n_j ? jq : n_j - 1;
    const uint32_t p = queue[2 * e + 1];
    int kf = static_cast<int>(p & 0xffffu) - 1;
    kf = kf < rows ? kf : rows - 1;
    const int last = nbins - 1;
    int kr = kf < 0 ? 0 : (kf < last ? kf : last);
    int64_t ig = i0 + static_cast<int64_t>(p >> 16);
    ig = ig < n_i ? ig : n_i - 1;
    const double x = dot64(ci, ig, cj, jj);
    // a start on the wrong side of 90 deg (b90: the bin holding 90 deg) jumps to that side's end
    if (x < 0.0 && kr < b90) kr = b180;
    if (x > 0.0 && kr > b90) kr = 0;
    const int ke = static_cast<int>(exact_bin(x, static_cast<uint32_t>(kr), edge_cos, nbins));
    if (ke != kf) {
      const int col = COLS > 1 ? (lane & (COLS - 1)) : 0;
      atomicSub(hist + kf * COLS + col, w);
      atomicAdd(hist + ke * COLS + col, w);
    }
  }
  __builtin_amdgcn_wave_barrier();
}

// CORE 0: the generic core; 1: the core specialised to the bins' span (fp32 dot, full span;
// fp64 dot, narrow range); 2: fp32 dot, the bin-table core on the fast steps (matrix-core dot
// products, a shared histogram and the table in LDS), fp64 dot, the series core.  The generic
// steps of the bin-table core use the full-span core.  Register budgets: K = 4 builds for six
// waves per SIMD (<= 80 VGPRs), fp32 K = 8 for five (<= 96; its 24 fp32 i-coordinates, or the
// 32 matrix-core tiles), fp64 K = 8 for four (48 VGPRs of fp64 i-coordinates).  Measured on
// the 100k workloads, each step up in waves per SIMD outweighed the few spills it costs outside
// the pair loop.  The bin-table core also builds at K = 2 for eight waves per SIMD (<= 64 VGPRs).
// The bin-table core (CORE 2, fp32 dot) also takes COLS, its histogram's columns (1 or
// kHistCols), and L1S, the share of its table reads made through the vector L1 (0 none, 1 an
// eighth, 2 a quarter); its workgroups hold up to kMaxWavesPerWG waves (A.waves), all sharing
// one table and one histogram.  The other cores run kWavesPerWG waves per workgroup.
template <int K, bool D64, int CORE, int COLS = 1, int L1S = 2>
__global__ void __launch_bounds__((CORE == 2 && !D64) ? kMaxWavesPerWG * kWave : kWGThreads)
__attribute__((amdgpu_waves_per_eu(K == 2 ? 8 : (K == 4 ? 6 : (D64 ? 4 : 5)))))
pairs_kernel(const PairArgs A) {
  typedef typename Real<D64>::T real;
  constexpr bool SPAN = CORE != 0;
  constexpr bool LUT = CORE == 2 && !D64;  // fp64 dot: CORE 2 is the series core
  constexpr int BI = kWave * K;       // i-block: galaxies per wave
  constexpr int JB = D64 ? 4 : 8;     // j galaxies per scalar batch
  static_assert(COLS == 1 || (LUT && COLS == kHistCols), "multi-column histograms belong to the bin-table core");
  static_assert(L1S == 2 || LUT, "the L1 share is a bin-table core variant");
  static_assert(L1S != 3 || COLS == 1, "three sixteenths through the L1: the one-column layout only");
  // queue entries pack (i - i0) and the fast-path row + 1 into 16 bits each
  static_assert(BI <= 0x10000 && kMaxBins + kWave + kLutAliasWords + 1 < 0x10000, "queue fields overflow");
  extern __shared__ uint32_t lds[];

  const int lane = threadIdx.x & (kWave - 1);
  // The wave index is the same in every lane; readfirstlane tells the compiler so, which keeps
  // the step range, the loop counters and every j index in SGPRs (scalar loads of j, scalar
  // branches).
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int nw = A.waves;  // waves per workgroup (blockDim.x / 64)
  const int nthreads = nw * kWave;
  // LDS: private mode, per wave [histogram | queue]; shared mode, [histogram | bin table |
  // one queue per wave] (the table only with the bin-table core).
  const bool shared_hist = LUT || A.shared_hist != 0;
  constexpr int QW = queue_words(K, CORE, D64);
  const int tab_words = LUT ? 2 * (A.bp.lut_n + 1) : 0;
  uint32_t *const hist = shared_hist ? lds : lds + wv * (A.hist_words + QW);
  uint2 *const tab = reinterpret_cast<uint2 *>(lds + A.hist_words);
  uint32_t *const queue = shared_hist ? lds + A.hist_words + tab_words + wv * QW : hist + A.hist_words;
  // the workgroup's cursor into its fast steps (64-bit, after the queues; every offset before it
  // is an even number of words)
  unsigned long long *const cursor = reinterpret_cast<unsigned long long *>(
      shared_hist ? lds + A.hist_words + tab_words + nw * QW : lds + nw * (A.hist_words + QW));
  const uint32_t hist_addr = lds_address(hist);
  // a multi-column histogram: this lane's column, and its byte offset within a row
  const int colw = COLS > 1 ? (lane & (COLS - 1)) : 0;
  const uint32_t col4 = static_cast<uint32_t>(4 * colw);
  const uint32_t tab_bias = lds_address(tab) - (kLutKeyBias << 3);
  // the global table's copy: entry q at byte (key bits << 3) - (bits of 2^23 << 3), a 32-bit offset
  // (one shift-and-add) that the load adds to the table's address held in scalar registers
  const char *const lut_l1 = reinterpret_cast<const char *>(A.lut);
  auto lut_read_l1 = [&](float key) __attribute__((always_inline)) {
    const uint32_t off = (__float_as_uint(key) << 3) - (kLutKeyBias << 3);
    return *reinterpret_cast<const uint2 *>(lut_l1 + off);
  };
  const int g = blockIdx.x;
  auto in_family = [&](int f) { return g >= A.fam[f].wg_begin && g < A.fam[f].wg_end; };
  const int fi = in_family(0) ? 0 : (in_family(1) ? 1 : 2);
  const FamilyWork &F = A.fam[fi];
  const BinParams &bp = A.bp;
  const uint32_t W = F.sym ? 2u : 1u;
  // the one wave-uniform constant each core needs in a VGPR, and this lane's clamp
  const float c_v = in_vgpr(D64 ? (CORE == 2 ? bp.ps[2] : bp.pw[6]) : bp.h);
  // the bin table's key addend M + 2^23, in a VGPR of its own (a VALU fma reads one scalar operand;
  // c_v = h serves the generic steps' arccos core)
  const float mb_v = in_vgpr(LUT ? bp.lut_mb : 0.0f);
  const float tmax_v = bp.tmax + static_cast<float>(lane);

  // the family's output histogram: every flush adds into it with 64-bit atomics (it was zeroed
  // before the launch, or holds the counts that a part adds to)
  unsigned long long *const slot = reinterpret_cast<unsigned long long *>(A.out[fi]);
  if (shared_hist) {
    for (int b = threadIdx.x; b < A.hist_words; b += nthreads) hist[b] = 0u;
    if constexpr (LUT)
      for (int q = threadIdx.x; q <= A.bp.lut_n; q += nthreads) {
        const uint2 e = A.lut[q];
        tab[q] = make_uint2(e.x, hist_addr + e.y);
      }
  } else {
    for (int b = lane; b < A.hist_words; b += kWave) hist[b] = 0u;
  }
  if (threadIdx.x == 0) *cursor = 0ull;
  // (A device-scope fence before this barrier, which writes back the L2 on gfx950, cost each
  // workgroup ~20 us: an eighth of the 10k + 10k job.  Nothing here needs one: the set-up writes
  // only LDS.)
  __syncthreads();

  // The family's j-steps form two segments:
  //   fast    - the off-diagonal steps of full i-blocks: batched, unrolled, no per-pair checks;
  //   generic - the diagonal steps j in [i0, i0 + BI) of a self family and every step of a
  //             ragged last i-block: per-pair weights and validity, a rolled loop, slower.
  // The generic steps are split evenly among the family's waves (V of them; this is wave v), so
  // every wave gets the same share of the slower work.  The fast steps are split evenly among the
  // family's workgroups (U; this is workgroup u), and the waves of a workgroup take them in chunks
  // from its cursor, so they end together however fast each one runs: a workgroup holds its LDS
  // until its last wave ends, and with equal fixed shares the waves of one workgroup ended up to
  // 40 % apart (per-wave timestamps, 100k + 100k at 720 bins).
  const int64_t U = F.wg_end - F.wg_begin, u = g - F.wg_begin;
  const int64_t V = U * nw, v = u * nw + wv;
  auto share = [](int64_t begin, int64_t total, int64_t parts, int64_t idx, int64_t &lo, int64_t &hi)
      __attribute__((always_inline)) {
    const int64_t q = total / parts, r = total % parts;
    lo = begin + q * idx + (r * idx) / parts;
    hi = begin + q * (idx + 1) + (r * (idx + 1)) / parts;
  };
  int64_t fs, fe, gs, ge;
  share(F.fast_begin, F.fast_steps, U, u, fs, fe);
  share(F.gen_begin, F.gen_steps, V, v, gs, ge);
  const int64_t nbf = F.n_i / BI;  // full i-blocks

  // j-steps since the last flush, and the interval, as 32-bit wave-uniform values so that the
  // test stays on the scalar unit (the host caps the interval near 2^31 / (2 * 64 K * waves),
  // at most ~8.4e6 steps)
  int32_t since_flush = 0;
  const int32_t flush_every = __builtin_amdgcn_readfirstlane(
      static_cast<int32_t>(A.flush_interval < 0x7fff0000 ? A.flush_interval : 0x7fff0000));
  int qcount = 0;  // queue entries [0, qcount) are pending
  // histogram rows: bins, spare rows and the bin table's alias rows
  const int hist_rows = COLS > 1 ? A.nbins + 3 : A.hist_words;
  const uint32_t lane_tag = static_cast<uint32_t>(lane) << 16;
  int64_t i0 = 0;
  real ix[K], iy[K], iz[K];

  // The queue is drained (64 at a time, from the top) after every j-step and within it after
  // every drain_span pairs per lane, so it never holds more than 64 (drain_span + 1) entries.
  auto drain = [&](int c) __attribute__((always_inline)) {
    drain_queue<COLS>(hist, queue, qcount - c, c, F.ci, F.cj, i0, F.n_i, F.n_j, W, A.edge_cos, A.nbins, A.bp.b90,
                      A.bp.b180, hist_rows);
    qcount -= c;
  };
  auto drain_all = [&]() __attribute__((always_inline)) {
    while (qcount > 0) drain(qcount < kWave ? qcount : kWave);
  };
  // Drain full-wave batches: leaves fewer than 64 entries pending.
  auto drain_full = [&]() __attribute__((always_inline)) {
    while (__builtin_expect(qcount >= kWave, 0)) drain(kWave);
  };
  // The bin a histogram row counts for: bins 0 .. nbins - 1 themselves; the spare rows past the
  // last bin count for bin nbins - 1; the bin table's two alias rows for bins 0 and b180.
  auto row_bin = [&](int row) __attribute__((always_inline)) {
    if (row < A.nbins) return row;
    if (LUT && row == A.bp.lut_alias - 1) return 0;
    if (LUT && row == A.bp.lut_alias) return static_cast<int>(A.bp.b180);
    return A.nbins - 1;
  };
  // Add the LDS histogram into the family's 64-bit output.  Each word is taken with an
  // atomic exchange, so in shared mode other waves may keep adding meanwhile; the value is
  // read as signed because a pending recheck may have moved a count out of a bin that an
  // earlier flush already emptied (the flush interval keeps every word within +-2^31).  The
  // rows past nbins are added to the bins they stand for.
  auto flush = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_wave_barrier();
    if constexpr (COLS > 1) {
      for (int row = lane; row < hist_rows; row += kWave) {
        long long c = 0;
#pragma unroll
        for (int q = 0; q < COLS; ++q) c += static_cast<int>(atomicExch(hist + row * COLS + q, 0u));
        if (c) atomicAdd(slot + row_bin(row), static_cast<unsigned long long>(c));
      }
    } else {
      for (int bb = lane; bb < A.nbins; bb += kWave) {
        const uint32_t c = atomicExch(hist + bb, 0u);
        if (c) atomicAdd(slot + bb, static_cast<unsigned long long>(static_cast<long long>(static_cast<int>(c))));
      }
      long long spare = static_cast<int>(atomicExch(hist + A.nbins + lane, 0u));
      if constexpr (LUT) {
        // the middle table entry's two words: bin 0 and bin b180 (the angles just below 180 deg)
        if (lane < kLutAliasWords) {
          const long long a = static_cast<int>(atomicExch(hist + A.nbins + kWave + lane, 0u));
          if (a) atomicAdd(slot + (lane == 0 ? 0 : A.bp.b180), static_cast<unsigned long long>(a));
        }
      }
#pragma unroll
      for (int off = kWave / 2; off > 0; off >>= 1) spare += __shfl_xor(spare, off, kWave);
      if (lane == 0 && spare) atomicAdd(slot + (A.nbins - 1), static_cast<unsigned long long>(spare));
    }
    __builtin_amdgcn_wave_barrier();
  };
  // The last flush of a shared histogram: once every wave of the workgroup is done adding, the
  // rows are split among all of its threads (each row read once) instead of each wave taking the
  // whole histogram in turn.
  auto final_flush = [&]() __attribute__((always_inline)) {
    if (!shared_hist) {
      flush();
      return;
    }
    __syncthreads();
    for (int row = threadIdx.x; row < hist_rows; row += nthreads) {
      long long c = 0;
#pragma unroll
      for (int q = 0; q < COLS; ++q) c += static_cast<int>(hist[row * COLS + q]);
      if (c) atomicAdd(slot + row_bin(row), static_cast<unsigned long long>(c));
    }
  };
  auto load_j = [&](int64_t jj, real &x, real &y, real &z) __attribute__((always_inline)) {
    if constexpr (D64) {
      x = ld_uniform(F.cj.x64, jj); y = ld_uniform(F.cj.y64, jj); z = ld_uniform(F.cj.z64, jj);
    } else {
      x = ld_uniform(F.cj.x, jj); y = ld_uniform(F.cj.y, jj); z = ld_uniform(F.cj.z, jj);
    }
  };

  // One j against this lane's K i-galaxies.  Pairs the guard flags are appended to the
  // wave's queue right after their atomic (each bin index dies at once), and the queue is
  // drained in full-wave batches after the step.
  // Append a flagged pair (this lane's k-th i against j) to the wave's queue; kslot = its
  // fast-path row + 1.
  // (The flag, drain and flush tests are marked unlikely, so that the common path falls through
  // them instead of taking a branch a pair: 1-3 % on every core.)
  auto enqueue = [&](bool tp, uint32_t kslot, int k, int64_t jg) __attribute__((always_inline)) {
    const unsigned long long m = __ballot(tp);
    if (__builtin_expect(m != 0, 0)) {
      if (tp) {
        // slot = pending count + number of flagged lanes below this one
        const uint32_t e = __builtin_amdgcn_mbcnt_hi(
            static_cast<uint32_t>(m >> 32),
            __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), static_cast<uint32_t>(qcount)));
        queue[2 * e] = static_cast<uint32_t>(jg);
        queue[2 * e + 1] = (lane_tag + (static_cast<uint32_t>(kWave * k) << 16)) | kslot;
      }
      qcount += __popcll(m);
    }
  };

  // The same for a pair of a matrix-core tile, whose j varies across the wave: i_local = i - i0 =
  // 16 t + 4 comp + r (comp = lane / 16).  The compiler keeps the lane's part in a register
  // across the tile loop, and the kernels spill it, so an enqueue reloads it from scratch and
  // waits.  The one-column layout enqueues after every pair, and with four waves per SIMD those
  // waits cost time (3600 bins: 8.63 -> 8.41 ms), so there the caller passes il = 16 t + r and the
  // lane id is recomputed here: two ALU instructions in a volatile asm statement, which (unlike
  // the equivalent builtins) the compiler cannot hoist out of this rare branch.  The
  // sixteen-column layout passes the whole i_local: it enqueues rarely at eight waves per SIMD,
  // and the other form measured slower there (720 bins: 6.20 against 6.26 ms).
  auto enqueue_ij = [&](bool tp, uint32_t kslot, uint32_t il, int64_t jl) __attribute__((always_inline)) {
    const unsigned long long m = __ballot(tp);
    if (__builtin_expect(m != 0, 0)) {
      if (tp) {
        const uint32_t e = __builtin_amdgcn_mbcnt_hi(
            static_cast<uint32_t>(m >> 32),
            __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), static_cast<uint32_t>(qcount)));
        uint32_t i_local = il;
        if constexpr (COLS == 1) {
          uint32_t ln;
          asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
          i_local += (ln >> 4) << 2;
        }
        queue[2 * e] = static_cast<uint32_t>(jl);
        queue[2 * e + 1] = (i_local << 16) | kslot;
      }
      qcount += __popcll(m);
    }
  };

  // Which of a lane's table reads go through the vector L1 (the rest read the LDS copy): a random
  // 64-lane LDS read costs ~7 CU cycles, the same read through the vector L1 ~37, and the LDS also
  // takes every pair's atomic, so a share of the reads may go to the L1.  Scalar-j steps: pairs
  // k = 1, 5 (a quarter) or k = 1 of 8 (an eighth, and for three sixteenths); matrix-core tiles:
  // result r = 1 (a quarter), r = 1 of odd tiles (an eighth), and with it r = 3 of tiles 1 and 5
  // of every 8 (three sixteenths).
  auto l1_scalar = [](int k) constexpr {
    return L1S == 2 ? k % 4 == 1 : ((L1S == 1 || L1S == 3) ? k % 8 == 1 : false);
  };
  auto l1_tile = [](int r, int t) constexpr {
    return L1S == 2 ? r == 1
                    : (L1S == 1 ? r == 1 && (t & 1)
                                : (L1S == 3 ? (r == 1 && (t & 1)) || (r == 3 && (t & 3) == 1) : false));
  };
  // The histogram row address of a bin-table pair: (sign of e - x) << lut_sh plus the entry's row
  // address, plus this lane's column; an L1 entry holds the row's offset, the LDS copy its address.
  const uint32_t l1_base = hist_addr + col4;
  auto lut_row_address = [&](float x, uint2 ent, bool from_l1, bool &trip) __attribute__((always_inline)) {
    return lut_word_address(x, ent, bp, trip) + (from_l1 ? l1_base : col4);
  };

  auto step = [&](real xj, real yj, real zj, int64_t jg, auto generic_tag) __attribute__((always_inline)) {
    constexpr bool GENERIC = decltype(generic_tag)::value;
    if constexpr (LUT && !GENERIC) {
      // all K table reads first, so one LDS wait covers them
      float xv[K];
      uint2 ev[K];
#pragma unroll
      for (int k = 0; k < K; ++k) {
        float c_unused;
        xv[k] = fmaf(ix[k], xj, fmaf(iy[k], yj, iz[k] * zj));
        const float key = lut_key(xv[k], bp, mb_v, c_unused);
        if (l1_scalar(k)) ev[k] = lut_read_l1(key);
        else ev[k] = lut_read_lds(key, tab_bias);
      }
#pragma unroll
      for (int k = 0; k < K; ++k) {
        bool tp;
        const uint32_t a = lut_row_address(xv[k], ev[k], l1_scalar(k), tp);
        __hip_atomic_fetch_add(reinterpret_cast<lds_word_t *>(static_cast<uintptr_t>(a)), W, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_WORKGROUP);
        enqueue(tp, ((a - hist_addr) >> bp.lut_sh) + 1, k, jg);
        if ((k + 1) % drain_span(K, CORE, D64) == 0 && k + 1 < K) drain_full();
      }
    } else {
#pragma unroll
      for (int k = 0; k < K; ++k) {
        uint32_t kk;
        bool tp;
        real x;
        if constexpr (D64 && CORE == 2) x = fma(-ix[k], xj, fma(-iy[k], yj, fma(-iz[k], zj, 1.0)));  // 1 - cos
        else x = fma(ix[k], xj, fma(iy[k], yj, iz[k] * zj));
        float t_unused;
        if constexpr (D64) core64<CORE>(x, bp, c_v, tmax_v, kk, tp, t_unused);
        else core32<SPAN>(x, bp, c_v, tmax_v, kk, tp, t_unused);
        if constexpr (GENERIC) {
          const int64_t ig = i0 + lane + kWave * k;
          const bool valid = ig < F.n_i && (!F.sym || jg >= ig);
          const bool self = F.sym && jg == ig;  // only a self family pairs a galaxy with itself
          if (self) kk = 0u;                     // separation 0
          tp = tp && valid && !self;
          if (valid) atomicAdd(hist + kk * COLS + colw, self ? 1u : W);
        } else {
          atomicAdd(hist + kk * COLS + colw, W);
        }
        enqueue(tp, kk + 1, k, jg);
        if ((k + 1) % drain_span(K, CORE, D64) == 0 && k + 1 < K) drain_full();
      }
    }
    drain_full();
  };

  auto check_flush = [&]() __attribute__((always_inline)) {
    if (__builtin_expect(since_flush >= flush_every, 0)) {
      drain_all();
      flush();
      since_flush = 0;
    }
  };

  // Diagonal / ragged j-steps: per-pair weights; rare, so a rolled loop.
  auto run_generic = [&](int64_t ja, int64_t jb) __attribute__((always_inline)) {
#pragma unroll 1
    for (int64_t jj = ja; jj < jb; ++jj) {
      real xs, ys, zs;
      load_j(jj, xs, ys, zs);
      step(xs, ys, zs, jj, GenericTag());
      since_flush += 1;
      check_flush();
    }
  };

  // Off-diagonal j-steps of a full i-block: batches of JB j galaxies read by the scalar
  // unit, the next batch requested before the current one is processed.  The j index is a
  // wave-uniform base plus a 32-bit offset (a range never exceeds one catalog), so the loop's
  // control and the scalar loads' addresses stay on the scalar unit (with a 64-bit index the
  // compiler formed them on the VALU: ~12 instructions per batch).
  auto run_fast = [&](int64_t ja, int64_t jb) __attribute__((always_inline)) {
    const int64_t j_base = uniform64(ja);
    const int32_t n = __builtin_amdgcn_readfirstlane(static_cast<int32_t>(jb - ja));
    int32_t u = 0;
    if (JB <= n) {
      real xs[JB], ys[JB], zs[JB];
#pragma unroll
      for (int v = 0; v < JB; ++v) load_j(j_base + v, xs[v], ys[v], zs[v]);
      while (true) {
        const bool more = u + 2 * JB <= n;
        real nx[JB], ny[JB], nz[JB];
        if (more) {
#pragma unroll
          for (int v = 0; v < JB; ++v) load_j(j_base + u + JB + v, nx[v], ny[v], nz[v]);
        }
#pragma unroll
        for (int v = 0; v < JB; ++v) step(xs[v], ys[v], zs[v], j_base + u + v, FastTag());
        u += JB;
        since_flush += JB;
        check_flush();
        if (!more) break;
#pragma unroll
        for (int v = 0; v < JB; ++v) {
          xs[v] = nx[v]; ys[v] = ny[v]; zs[v] = nz[v];
        }
      }
    }
#pragma unroll 1
    for (; u < n; ++u) {
      real xs, ys, zs;
      load_j(j_base + u, xs, ys, zs);
      step(xs, ys, zs, j_base + u, FastTag());
      since_flush += 1;
      check_flush();
    }
  };

  // Bin-table core, fast steps: the dot products on the matrix cores.  v_mfma_f32_16x16x4f32
  // multiplies a 16 x 4 tile of i-galaxies (lane l: component l / 16 of galaxy i0 + 16 t + l % 16,
  // component 3 = 0) by a 4 x 16 tile of j-galaxies (lane l: component l / 16 of j0 + l % 16);
  // lane l receives the dot products of i = i0 + 16 t + 4 (l / 16) + r, r = 0..3, with
  // j = j0 + l % 16.  The i-block of BI galaxies is BI / 16 such tiles, held as one VGPR each; a
  // chunk of 16 j-galaxies takes one vector load per lane.  The matrix cores run beside the VALU,
  // which keeps only the binning.
  constexpr int NT = LUT ? BI / 16 : 1;
  const int comp = lane >> 4, sub = lane & 15;
  float at[NT];
  auto load_tiles = [&](int64_t b) __attribute__((always_inline)) {
    i0 = b * BI;
    const float *src = comp == 0 ? F.ci.x : (comp == 1 ? F.ci.y : F.ci.z);
#pragma unroll
    for (int t = 0; t < NT; ++t) at[t] = comp < 3 ? src[i0 + 16 * t + sub] : 0.0f;
  };
  // Full chunks of 16 j in [ja, jb) (fewer than 16 remain; the caller runs them the usual way).
  // The chunk count is a wave-uniform 32-bit value, so the loop's control runs on the scalar unit
  // (with 64-bit j bounds the compiler kept it on the VALU: ~8 instructions per chunk); each lane's
  // j pointer advances by 16, and its j index is formed only where a pair is queued.
  auto run_fast_mfma = [&](int64_t ja, int64_t jb) __attribute__((always_inline)) {
    const float *jp = (comp == 0 ? F.cj.x : (comp == 1 ? F.cj.y : F.cj.z)) + ja + sub;
    const float4v zero = {0.0f, 0.0f, 0.0f, 0.0f};
    const int32_t nch = __builtin_amdgcn_readfirstlane(static_cast<int32_t>((jb - ja) >> 4));
    for (int32_t ch = 0; ch < nch; ++ch) {
      const int64_t jl = ja + 16 * static_cast<int64_t>(ch) + sub;
      const float bj = comp < 3 ? jp[16 * ch] : 0.0f;
      // each tile's product is requested one tile ahead, so its latency overlaps the binning
      float4v dn = __builtin_amdgcn_mfma_f32_16x16x4f32(at[0], bj, zero, 0, 0, 0);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const float4v d = dn;
        if (t + 1 < NT) dn = __builtin_amdgcn_mfma_f32_16x16x4f32(at[t + 1 < NT ? t + 1 : t], bj, zero, 0, 0, 0);
        uint2 ev[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float c_unused;
          const float key = lut_key(d[r], bp, mb_v, c_unused);
          if (l1_tile(r, t)) ev[r] = lut_read_l1(key);
          else ev[r] = lut_read_lds(key, tab_bias);
        }
        if constexpr (COLS > 1) {
          float dl[4];
          uint32_t a[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            dl[r] = __uint_as_float(ev[r].x) - d[r];
            a[r] = lut_signed_address(dl[r], ev[r].y, bp) + (l1_tile(r, t) ? l1_base : col4);
            __hip_atomic_fetch_add(reinterpret_cast<lds_word_t *>(static_cast<uintptr_t>(a[r])), W, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_WORKGROUP);
          }
          // One guard test for the four pairs: the smallest |e - x| of them (v_minimum3_f32, which
          // returns NaN if any operand is NaN, so an always-recheck entry still trips).  Only when
          // some lane's four hold a flagged pair are they tested one by one and queued, with a
          // drain point after every drain_span pairs.  (Measured with the sixteen-column
          // histogram: 6.89 -> 6.74 ms on 100k + 100k at 720 bins; with one column the per-pair
          // form below measured faster with one workgroup per CU and level with two.)
          const float dmin = __builtin_elementwise_minimum(
              __builtin_elementwise_minimum(fabsf(dl[0]), fabsf(dl[1])),
              __builtin_elementwise_minimum(fabsf(dl[2]), fabsf(dl[3])));
          if (__builtin_expect(__ballot(!(dmin >= bp.lut_g)) != 0, 0)) {
            constexpr int DS = drain_span(K, CORE, D64);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              enqueue_ij(!(fabsf(dl[r]) >= bp.lut_g), ((a[r] - hist_addr) >> bp.lut_sh) + 1,
                         static_cast<uint32_t>(16 * t + 4 * comp + r), jl);
              if ((r + 1) % DS == 0) drain_full();
            }
          }
        } else {
          auto bin_pair = [&](int r) __attribute__((always_inline)) {
            bool tp;
            const uint32_t a = lut_row_address(d[r], ev[r], l1_tile(r, t), tp);
            __hip_atomic_fetch_add(reinterpret_cast<lds_word_t *>(static_cast<uintptr_t>(a)), W, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_WORKGROUP);
            enqueue_ij(tp, ((a - hist_addr) >> bp.lut_sh) + 1, static_cast<uint32_t>(16 * t + r), jl);
          };
          // a drain point after every drain_span pairs of the lane's four (one or two)
          constexpr int DS = drain_span(K, CORE, D64);
          bin_pair(0);
          if (DS == 1) drain_full();
          bin_pair(1);
          drain_full();
          bin_pair(2);
          if (DS == 1) drain_full();
          bin_pair(3);
          drain_full();
        }
      }
      since_flush += 16;
      check_flush();
    }
  };

  auto load_i_block = [&](int64_t b) __attribute__((always_inline)) {
    i0 = b * BI;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int64_t ig = i0 + lane + kWave * k;
      const int64_t il = ig < F.n_i ? ig : i0;
      if constexpr (D64) {
        ix[k] = F.ci.x64[il]; iy[k] = F.ci.y64[il]; iz[k] = F.ci.z64[il];
      } else {
        ix[k] = F.ci.x[il]; iy[k] = F.ci.y[il]; iz[k] = F.ci.z[il];
      }
    }
  };

  // Generic segment.  Self family: block b holds steps [b BI, b BI + min(BI, n - b BI)), so step
  // s is block s / BI, j = s.  Cross family: only the ragged block nbf, j = s.
  {
    int64_t s = gs;
    while (s < ge) {
      const int64_t b = F.sym ? s / BI : nbf;
      const int64_t j = s;
      const int64_t jend = F.sym ? ((b + 1) * BI < F.n_j ? (b + 1) * BI : F.n_j) : F.n_j;
      const int64_t nsteps = (ge - s) < (jend - j) ? (ge - s) : (jend - j);
      if (nsteps <= 0) break;  // unreachable for consistent step counts; keeps every wave finite
      load_i_block(b);
      run_generic(j, j + nsteps);
      drain_all();
      s += nsteps;
    }
  }

  // Fast segment over the full blocks.  Cross family: block b has steps j in [0, n_j), prefix
  // b n_j.  Self family: block b has j in [(b+1) BI, n), prefix Pf(b) = b n - BI b (b+1) / 2.
  // One chunk [s0, s1) of the workgroup's range may span blocks; the i-tiles (and the scalar-j
  // i-block) stay loaded while the next chunk is in the same block.
  int64_t tiles_b = -1, iblk_b = -1;
  auto run_fast_range = [&](int64_t s0, int64_t s1) __attribute__((always_inline)) {
    int64_t s = s0, b = 0, j = 0;
    if (!F.sym) {
      b = s / F.n_j;
      j = s - b * F.n_j;
    } else {
      int64_t lo = 0, hi = nbf - 1;
      while (lo < hi) {
        const int64_t mid = (lo + hi + 1) >> 1;
        const int64_t pm = mid * F.n_j - static_cast<int64_t>(BI) * mid * (mid + 1) / 2;
        if (pm <= s) lo = mid; else hi = mid - 1;
      }
      b = lo;
      j = (b + 1) * BI + (s - (b * F.n_j - static_cast<int64_t>(BI) * b * (b + 1) / 2));
    }
    while (s < s1) {
      const int64_t nsteps = (s1 - s) < (F.n_j - j) ? (s1 - s) : (F.n_j - j);
      if (nsteps <= 0) break;  // unreachable for consistent step counts; keeps every wave finite
      if constexpr (LUT) {
        const int64_t full = nsteps & ~static_cast<int64_t>(15);
        if (full > 0) {
          if (b != tiles_b) {
            load_tiles(b);
            tiles_b = b;
          }
          i0 = b * BI;
          run_fast_mfma(j, j + full);
        }
        if (full < nsteps) {
          if (b != iblk_b) {
            load_i_block(b);
            iblk_b = b;
          }
          i0 = b * BI;
          run_fast(j + full, j + nsteps);
        }
      } else {
        if (b != iblk_b) {
          load_i_block(b);
          iblk_b = b;
        }
        i0 = b * BI;
        run_fast(j, j + nsteps);
      }
      drain_all();
      s += nsteps;
      ++b;
      j = F.sym ? (b + 1) * BI : 0;
    }
  };
  {
    // chunks of a multiple of 16 steps (whole matrix-core j-tiles), about 8 per wave, at least 32
    // (100k + 100k at 720 bins: 6.34 ms with 24 per wave, 6.16-6.19 with 6, 8 or 12)
    const int64_t len = fe - fs;
    const int64_t per = len / (static_cast<int64_t>(nw) * 8);
    const int64_t CH = per < 32 ? 32 : (per + 15) & ~static_cast<int64_t>(15);
    while (true) {
      unsigned long long c = 0;
      if (lane == 0)
        c = __hip_atomic_fetch_add(cursor, static_cast<unsigned long long>(CH), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_WORKGROUP);
      const int64_t c0 = static_cast<int64_t>(
          (static_cast<uint64_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(c >> 32))) << 32) |
          __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(c)));
      if (c0 >= len) break;
      run_fast_range(fs + c0, fs + c0 + CH < fe ? fs + c0 + CH : fe);
    }
  }
  final_flush();
}

// ------------------------------------------------------------------------------- edges
// c[e] = cos(e w) for e = 0..nbins (fp64); -inf where e w exceeds 180 degrees.
__device__ __forceinline__ void edge_entry(int e, int32_t nbins, double w_deg, double *c) {
  if (e > nbins) return;
  const double deg = static_cast<double>(e) * w_deg;
  c[e] = deg <= 180.0 ? cos(deg * (3.14159265358979323846 / 180.0)) : -__builtin_inf();
}

// ------------------------------------------------------------------------------ bin table
// Entry q of the bin-table core (q = 0 .. 2M): c in [(q - 1/2)/M - 1, (q + 1/2)/M - 1] (the
// index rounds), widened by `margin` on both sides.  An edge at angle e w (e = 1 .. nbins-1) sits
// at c = sqrt2 sin(e w / 2) when e w <= 90 deg and at c = -sqrt2 cos(e w / 2) when e w >= 90 deg
// (both for exactly 90).  With one edge in range: {cos(e w) rounded to fp32, the byte offset of the
// histogram row of the bin above the edge}; with none: {4, the row of the bin of the entry's
// middle}.  A row offset is 4 x cols x the row (cols: the histogram's columns).  s_star > 0: an
// entry whose |c| may lie below s_star, where the error of c can exceed the margin, holds NaN
// (every pair in it is rechecked) and the row of its middle's bin, bin 0 for the middle entry;
// s_star == 0: the middle entry holds {0, row `alias`}.  The host only selects this core when no
// widened range can hold two edges (and nbins >= 2, so rows 0 and 1 exist).
__device__ __forceinline__ double lut_angle_deg(double c) {  // inverse of the map above
  constexpr double kSqrtHalf = 0.70710678118654752440, kDeg = 57.295779513082320877;
  return c >= 0.0 ? 2.0 * asin(fmin(c, 1.0) * kSqrtHalf) * kDeg : 180.0 - 2.0 * asin(fmin(-c, 1.0) * kSqrtHalf) * kDeg;
}

__device__ __forceinline__ void lut_entry(int q, int32_t nbins, double w_deg, int32_t m, double margin, int32_t cols,
                                          int32_t alias, double s_star, uint2 *lut) {
  if (q > 2 * m) return;
  constexpr double kSqrt2 = 1.41421356237309504880, kRad = 3.14159265358979323846 / 180.0;
  const uint32_t row_bytes = 4u * static_cast<uint32_t>(cols);
  const double lo = (static_cast<double>(q) - 0.5) / m - 1.0 - margin;
  const double hi = (static_cast<double>(q) + 0.5) / m - 1.0 + margin;
  int count = 0, edge = 0;
  // right half (0 .. 90 deg): c in [max(lo, 0), min(hi, 1)]
  if (hi >= 0.0 && lo <= 1.0) {
    const int e0 = static_cast<int>(floor(lut_angle_deg(fmax(lo, 0.0)) / w_deg)) - 1;
    const int e1 = static_cast<int>(ceil(lut_angle_deg(fmin(hi, 1.0)) / w_deg)) + 1;
    for (int e = e0 < 1 ? 1 : e0; e <= e1 && e < nbins; ++e) {
      const double th = static_cast<double>(e) * w_deg;
      if (th > 90.0) break;
      const double c = kSqrt2 * sin(0.5 * th * kRad);
      if (c >= lo && c <= hi) {
        ++count;
        edge = e;
      }
    }
  }
  // left half (90 .. 180 deg): c in [max(lo, -1), min(hi, 0))
  if (lo < 0.0 && hi >= -1.0) {
    const int e0 = static_cast<int>(floor(lut_angle_deg(fmax(lo, -1.0)) / w_deg)) - 1;
    const int e1 = static_cast<int>(ceil(lut_angle_deg(fmin(hi, -1e-300)) / w_deg)) + 1;
    for (int e = e0 < 1 ? 1 : e0; e <= e1 && e < nbins; ++e) {
      const double th = static_cast<double>(e) * w_deg;
      if (th < 90.0) continue;
      if (th > 180.0) break;  // no angle reaches an edge past 180 deg (its c would wrap positive)
      const double c = -kSqrt2 * cos(0.5 * th * kRad);
      if (c >= lo && c <= hi) {
        ++count;
        edge = e;
      }
    }
  }
  // the smallest |c| of the entry's own (unwidened) range
  const double c_lo = (static_cast<double>(q) - 0.5) / m - 1.0, c_hi = (static_cast<double>(q) + 0.5) / m - 1.0;
  const double s_min = (c_lo <= 0.0 && c_hi >= 0.0) ? 0.0 : fmin(fabs(c_lo), fabs(c_hi));
  auto mid_bin = [&]() {
    const double mid = fmin(fmax(static_cast<double>(q) / m - 1.0, -1.0), 1.0);
    int b = static_cast<int>(floor(lut_angle_deg(mid) / w_deg));
    return b < 0 ? 0 : (b > nbins - 1 ? nbins - 1 : b);
  };
  uint2 ent;
  if (s_star > 0.0 && s_min < s_star) {
    // always recheck; the row is at least 1, so that B - 1 is a row too whatever sign e - x takes
    // (the recheck moves the count from either to the exact bin)
    ent.x = __float_as_uint(__builtin_nanf(""));
    const int b = q == m ? 1 : mid_bin();
    ent.y = row_bytes * static_cast<uint32_t>(b < 1 ? 1 : b);
  } else if (q == m && count == 0) {
    ent.x = __float_as_uint(0.0f);                        // the middle entry (x near +-1)
    ent.y = row_bytes * static_cast<uint32_t>(alias);     // x < 0: row alias; x > 0: row alias - 1
  } else if (count >= 1) {
    ent.x = __float_as_uint(static_cast<float>(cos(static_cast<double>(edge) * w_deg * kRad)));
    ent.y = row_bytes * static_cast<uint32_t>(edge);  // the bin above the edge; the one below is edge - 1
  } else {
    ent.x = __float_as_uint(4.0f);  // e - x > 0 for every cosine: bin = B
    ent.y = row_bytes * static_cast<uint32_t>(mid_bin());
  }
  lut[q] = ent;
}

// ------------------------------------------------------------------------------ tables
// One launch before the pair kernel: blocks [0, edge_blocks) write the edge cosines and, when
// the call overwrites its outputs, zero them (the pair kernel's flushes add into them); the
// blocks after them build the bin table when there is one.
__global__ void __launch_bounds__(256) tables_kernel(const TablesArgs T) {
  if (static_cast<int>(blockIdx.x) < T.edge_blocks) {
    const int e = blockIdx.x * blockDim.x + threadIdx.x;
    edge_entry(e, T.nbins, T.w_deg, T.edge_cos);
    if (T.out[0] && e < T.nbins) {
      T.out[0][e] = 0;
      T.out[1][e] = 0;
      T.out[2][e] = 0;
    }
  } else {
    const int q = (blockIdx.x - T.edge_blocks) * blockDim.x + threadIdx.x;
    lut_entry(q, T.nbins, T.w_deg, T.m, T.margin, T.cols, T.alias, T.s_star, T.lut);
  }
}

// ------------------------------------------------------------------------------ totals
__global__ void __launch_bounds__(256) totals_kernel(const uint64_t *dd, const uint64_t *dr,
                                                     const uint64_t *rr, int32_t nbins,
                                                     uint64_t *totals) {
  __shared__ unsigned long long part[4];
  const int f = blockIdx.x;
  const uint64_t *h = f == 0 ? dd : (f == 1 ? dr : rr);
  unsigned long long acc = 0ull;
  for (int bb = threadIdx.x; bb < nbins; bb += 256) acc += h[bb];
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, kWave);
  if ((threadIdx.x & (kWave - 1)) == 0) part[threadIdx.x / kWave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) totals[f] = part[0] + part[1] + part[2] + part[3];
}

// ------------------------------------------------------------------------------- omega
__global__ void __launch_bounds__(256) omega_kernel(const uint64_t *dd, const uint64_t *dr,
                                                    const uint64_t *rr, int32_t nbins, int64_t n_d,
                                                    int64_t n_r, double *omega) {
  const int bb = blockIdx.x * blockDim.x + threadIdx.x;
  if (bb >= nbins) return;
  const double d = static_cast<double>(dd[bb]);
  const double m = static_cast<double>(dr[bb]);
  const double r = static_cast<double>(rr[bb]);
  double w;
  if (rr[bb] == 0) {
    w = __builtin_nan("");
  } else if (n_d == n_r) {
    w = (d - 2.0 * m + r) / r;
  } else {
    const double nd = static_cast<double>(n_d), nr = static_cast<double>(n_r);
    const double frr = r / (nr * nr);
    w = (d / (nd * nd) - 2.0 * (m / (nd * nr)) + frr) / frr;
  }
  omega[bb] = w;
}

// -------------------------------------------------------------------------- eval core
template <int CORE>
__global__ void __launch_bounds__(256) eval_core_kernel(const float *x32, const double *x64,
                                                        int64_t n, const BinParams bp, int dot64, const uint2 *lut,
                                                        const double *edge_cos, int32_t *bin_out,
                                                        uint8_t *trip_out, int32_t *exact_out, float *t_out) {
  constexpr bool SPAN = CORE != 0;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= n) return;
  uint32_t k;
  bool trip;
  double xe;
  float t;
  if (dot64) {
    xe = x64[idx];
    if (!__builtin_isfinite(xe)) xe = 1.0;  // (a dot product of unit vectors is finite)
    core64<CORE>(CORE == 2 ? 1.0 - xe : xe, bp, CORE == 2 ? bp.ps[2] : bp.pw[6], bp.tmax, k, trip, t);
  } else {
    const float xf = __builtin_isfinite(x32[idx]) ? x32[idx] : 1.0f;  // never index a table with NaN
    xe = static_cast<double>(xf);
    if constexpr (CORE == 2) {
      core_lut(xf, bp, lut, k, trip, t);  // (fp32 dot: CORE 2 is the table)
    } else {
      core32<SPAN>(xf, bp, bp.h, bp.tmax, k, trip, t);
    }
  }
  // k >= nbins: the full-span kernel's spare bins, which the flush folds into bin nbins - 1;
  // the table's alias rows lut_alias - 1 and lut_alias are bins 0 and b180
  const uint32_t last = static_cast<uint32_t>(bp.nbins - 1);
  if (CORE == 2 && !dot64 && k == static_cast<uint32_t>(bp.lut_alias - 1)) k = 0;
  if (CORE == 2 && !dot64 && k == static_cast<uint32_t>(bp.lut_alias)) k = static_cast<uint32_t>(bp.b180);
  k = k < last ? k : last;
  bin_out[idx] = static_cast<int32_t>(k);
  trip_out[idx] = trip ? 1 : 0;
  if (exact_out) exact_out[idx] = static_cast<int32_t>(exact_bin(xe, k, edge_cos, bp.nbins));
  if (t_out) t_out[idx] = t;
}

}  // namespace

// ------------------------------------------------------------------------- eval dot (MFMA)
// One wave per tile, the pair kernel's operand layout: lane l supplies component l / 16 of a-
// and b-vector l % 16 (component 3 = 0) and receives a_(4 (l/16) + r) . b_(l % 16), r = 0..3.
__global__ void __launch_bounds__(64) eval_dot_mfma_kernel(const float *ax, const float *ay, const float *az,
                                                           const float *bx, const float *by, const float *bz,
                                                           int64_t ntiles, float *out) {
  const int64_t t = blockIdx.x;
  if (t >= ntiles) return;
  const int l = threadIdx.x, comp = l >> 4, sub = l & 15;
  const int64_t v = 16 * t + sub;
  const float a = comp == 0 ? ax[v] : (comp == 1 ? ay[v] : (comp == 2 ? az[v] : 0.0f));
  const float b = comp == 0 ? bx[v] : (comp == 1 ? by[v] : (comp == 2 ? bz[v] : 0.0f));
  const float4v zero = {0.0f, 0.0f, 0.0f, 0.0f};
  const float4v d = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, zero, 0, 0, 0);
#pragma unroll
  for (int r = 0; r < 4; ++r) out[256 * t + 16 * (4 * comp + r) + sub] = d[r];
}

// ---------------------------------------------------------------------------- launchers
hipError_t launch_prepare(const float *ra, const float *dec, int64_t n, void *blob, hipStream_t st) {
  const int64_t p = padded_count(n);
  char *b = static_cast<char *>(blob);
  float *x = reinterpret_cast<float *>(b);
  double *x64 = reinterpret_cast<double *>(b + 12 * p);
  const int64_t blocks = (p + 255) / 256;
  hipLaunchKernelGGL(prepare_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, ra, dec, n,
                     p, x, x + p, x + 2 * p, x64, x64 + p, x64 + 2 * p);
  return hipGetLastError();
}

template <int K, bool D64, int CORE, int COLS = 1, int L1S = 2> static const void *pairs_fn() {
  return reinterpret_cast<const void *>(&pairs_kernel<K, D64, CORE, COLS, L1S>);
}

template <int K> static const void *select_lut(LutVariant lv) {
  if (lv.cols == kHistCols) {
    if (lv.l1 == 2) return pairs_fn<K, false, 2, kHistCols, 2>();
    if (lv.l1 == 1) return pairs_fn<K, false, 2, kHistCols, 1>();
    return pairs_fn<K, false, 2, kHistCols, 0>();
  }
  if (lv.l1 == 3) return pairs_fn<K, false, 2, 1, 3>();
  if (lv.l1 == 2) return pairs_fn<K, false, 2, 1, 2>();
  if (lv.l1 == 1) return pairs_fn<K, false, 2, 1, 1>();
  return pairs_fn<K, false, 2, 1, 0>();
}

// Instantiations: K in {4, 8} x {fp32, fp64 dot} x {generic, span-specialised core}, the fp64
// series core and the fp32 bin-table core's variants (columns x L1 share),
// the bin-table core also at K = 2 (<= 64 VGPRs: eight waves per SIMD).
static const void *select_pairs(bool dot64, int k, int core, LutVariant lv) {
  if (dot64) {
    if (core == 2) return k == 4 ? pairs_fn<4, true, 2>() : pairs_fn<8, true, 2>();
    if (core) return k == 4 ? pairs_fn<4, true, 1>() : pairs_fn<8, true, 1>();
    return k == 4 ? pairs_fn<4, true, 0>() : pairs_fn<8, true, 0>();
  }
  if (core == 2) return k == 2 ? select_lut<2>(lv) : (k == 4 ? select_lut<4>(lv) : select_lut<8>(lv));
  if (core) return k == 4 ? pairs_fn<4, false, 1>() : pairs_fn<8, false, 1>();
  return k == 4 ? pairs_fn<4, false, 0>() : pairs_fn<8, false, 0>();
}

hipError_t pairs_occupancy(bool dot64, int k, int core, LutVariant lv, size_t lds_bytes, int threads,
                           int *blocks_per_cu) {
  const void *fn = select_pairs(dot64, k, core, lv);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     static_cast<int>(lds_bytes));
  if (e != hipSuccess) return e;
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, fn, threads, lds_bytes);
}

hipError_t launch_pairs(const PairArgs &a, int num_wg, bool dot64, int k, int core, LutVariant lv, hipStream_t st) {
  const bool table = core >= 2 && !dot64;
  const size_t lds = pairs_lds_bytes(a.hist_words, table || a.shared_hist != 0, k, core, dot64, a.waves,
                                     table_words(a.bp.lut_n, dot64, core));
  const void *fn = select_pairs(dot64, k, core, lv);
  void *args[] = {const_cast<PairArgs *>(&a)};
  return hipLaunchKernel(fn, dim3(num_wg), dim3(a.waves * kWave), args, lds, st);
}

hipError_t launch_totals(const uint64_t *dd, const uint64_t *dr, const uint64_t *rr, int32_t nbins,
                         uint64_t *totals, hipStream_t st) {
  hipLaunchKernelGGL(totals_kernel, dim3(3), dim3(256), 0, st, dd, dr, rr, nbins, totals);
  return hipGetLastError();
}

hipError_t launch_omega(const uint64_t *dd, const uint64_t *dr, const uint64_t *rr, int32_t nbins,
                        int64_t n_d, int64_t n_r, double *omega, hipStream_t st) {
  hipLaunchKernelGGL(omega_kernel, dim3((nbins + 255) / 256), dim3(256), 0, st, dd, dr, rr, nbins, n_d,
                     n_r, omega);
  return hipGetLastError();
}

hipError_t launch_eval_dot_mfma(const float *ax, const float *ay, const float *az, const float *bx, const float *by,
                                const float *bz, int64_t ntiles, float *out, hipStream_t st) {
  hipLaunchKernelGGL(eval_dot_mfma_kernel, dim3(static_cast<unsigned>(ntiles)), dim3(64), 0, st, ax, ay, az, bx, by,
                     bz, ntiles, out);
  return hipGetLastError();
}

hipError_t launch_tables(const TablesArgs &t, hipStream_t st) {
  TablesArgs a = t;
  a.edge_blocks = (a.nbins + 1 + 255) / 256;
  const int lut_blocks = a.lut ? (2 * a.m + 1 + 255) / 256 : 0;
  hipLaunchKernelGGL(tables_kernel, dim3(a.edge_blocks + lut_blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_eval_core(const float *x32, const double *x64, int64_t n, const BinParams &bp,
                            bool dot64, int core, const uint2 *lut, const double *edge_cos, int32_t *bin_out,
                            uint8_t *trip_out, int32_t *exact_out, float *t_out, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>((n + 255) / 256));
  const int d = dot64 ? 1 : 0;
  if (core == 2)
    hipLaunchKernelGGL(eval_core_kernel<2>, grid, dim3(256), 0, st, x32, x64, n, bp, d, lut, edge_cos, bin_out,
                       trip_out, exact_out, t_out);
  else if (core == 1)
    hipLaunchKernelGGL(eval_core_kernel<1>, grid, dim3(256), 0, st, x32, x64, n, bp, d, lut, edge_cos, bin_out,
                       trip_out, exact_out, t_out);
  else
    hipLaunchKernelGGL(eval_core_kernel<0>, grid, dim3(256), 0, st, x32, x64, n, bp, d, lut, edge_cos, bin_out,
                       trip_out, exact_out, t_out);
  return hipGetLastError();
}

}  // namespace gc
