// The ablation ladder of "CUDA Deep Dive: 10B Galaxy Pairs on an RTX 5080" (section "The
// ladder" and the sections it lists), as HIP kernels for gfx950.  Each rung changes one thing
// relative to the previous one; see include/gc_ladder.h for the list.  These kernels exist to
// be timed and to have their counts compared with the exact histograms: they use the page's
// fp32 arithmetic (law of cosines on angles converted to radians in fp32) and no guard.
#include "../../include/gc_ladder.h"
#include "gc_acos_poly.h"
#include "gc_internal.h"

namespace gc {
namespace {

constexpr float kArcminToRadF = static_cast<float>(3.14159265358979323846 / 10800.0);
constexpr float kPiF = 3.14159265358979323846f;
constexpr int kPairBlock = 32;                    // rungs 0-2: 32 x 32 threads, one per (i, j)
constexpr size_t kMaxLdsBytes = 160 * 1024;       // LDS per workgroup on gfx950

struct LadderCat {
  const float *ra, *dec;   // arcmin (rungs 0-1 read these per pair)
  float *s, *c, *a;        // sin delta, cos delta, alpha in radians (prepass, rungs 2-5)
};

struct LadderArgs {
  LadderCat d, r;
  int64_t n_d, n_r;
  unsigned long long *out[3];  // DD, DR, RR
  float t_per_rad;             // bins per radian: (180 / pi) / w
  int32_t nbins, stride;
};

struct Gal {
  float s, c, a;
};

// Per-galaxy values from the raw catalog (what rungs 0 and 1 do once per pair).
__device__ __forceinline__ Gal raw_gal(const LadderCat &cat, int64_t k) {
  const float d = cat.dec[k] * kArcminToRadF;
  Gal g;
  g.s = sinf(d);
  g.c = cosf(d);
  g.a = cat.ra[k] * kArcminToRadF;
  return g;
}

__device__ __forceinline__ Gal prep_gal(const LadderCat &cat, int64_t k) {
  Gal g;
  g.s = cat.s[k];
  g.c = cat.c[k];
  g.a = cat.a[k];
  return g;
}

// The page's angle formula ("The problem"), written with one explicit fma so that every rung
// rounds it the same way: cos theta = sin d1 sin d2 + cos d1 cos d2 cos(a1 - a2), clamped.
// Symmetric in its two galaxies bit for bit: products commute, a2 - a1 = -(a1 - a2) exactly and
// cosf is even.
__device__ __forceinline__ float law_of_cosines(const Gal &p, float sj, float cj, float aj) {
  const float x = fmaf(p.s, sj, (p.c * cj) * cosf(p.a - aj));
  return fminf(fmaxf(x, -1.0f), 1.0f);
}

// Arccos variants.  0: acosf (ROCm's device library).  1: Abramowitz and Stegun 4.4.45,
// sqrt(1 - a) times a cubic in a = |x|, reflected as pi - acos(|x|) for x < 0.  2: the degree-6
// fit of the fp32 pair kernel's core (gc_acos_poly.h), same form, no guard.
template <int KIND>
__device__ __forceinline__ float ladder_acos(float x) {
  if constexpr (KIND == 0) {
    return acosf(x);
  } else {
    const float a = fabsf(x);
    float p;
    if constexpr (KIND == 1) {
      p = fmaf(fmaf(fmaf(-0.0187293f, a, 0.0742610f), a, -0.2121144f), a, 1.5707288f);
    } else {
      p = GC_ACOS_C6;
      p = fmaf(p, a, GC_ACOS_C5);
      p = fmaf(p, a, GC_ACOS_C4);
      p = fmaf(p, a, GC_ACOS_C3);
      p = fmaf(p, a, GC_ACOS_C2);
      p = fmaf(p, a, GC_ACOS_C1);
      p = fmaf(p, a, GC_ACOS_C0);
    }
    // the hardware square root (1 ulp), as the page's fast-math build and the pair kernel use
    const float r = __builtin_amdgcn_sqrtf(1.0f - a) * p;
    return x < 0.0f ? kPiF - r : r;
  }
}

// Truncate theta / w and clamp into the last bin (the appendix listing's index helper).
// (A negative or out-of-range conversion becomes a large unsigned value and lands in the last
// bin, so the index stays inside the histogram whatever the width.)
template <int ACOS>
__device__ __forceinline__ uint32_t ladder_bin(float cos_theta, const LadderArgs &A) {
  const uint32_t k = static_cast<uint32_t>(static_cast<int>(ladder_acos<ACOS>(cos_theta) * A.t_per_rad));
  const uint32_t last = static_cast<uint32_t>(A.nbins - 1);
  return k < last ? k : last;
}

// Add a workgroup's three LDS histograms (DD | DR | RR, A.stride words apart) to the outputs,
// taking the 3 stride words as one run: padding words (bin >= nbins) and zero words are skipped.
__device__ __forceinline__ void flush_block(const uint32_t *h, const LadderArgs &A, int tid, int nthreads) {
  for (int q = tid; q < 3 * A.stride; q += nthreads) {
    const int f = q / A.stride, bin = q - f * A.stride;
    const uint32_t v = h[q];
    if (bin < A.nbins && v != 0u) atomicAdd(A.out[f] + bin, static_cast<unsigned long long>(v));
  }
}

__global__ void __launch_bounds__(256) ladder_prep_kernel(const float *ra, const float *dec, int64_t n, float *s,
                                                          float *c, float *a) {
  const int64_t k = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (k >= n) return;
  const float d = dec[k] * kArcminToRadF;
  s[k] = sinf(d);
  c[k] = cosf(d);
  a[k] = ra[k] * kArcminToRadF;
}

__global__ void __launch_bounds__(256) ladder_zero_kernel(unsigned long long *o0, unsigned long long *o1,
                                                          unsigned long long *o2, int32_t nbins) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= nbins) return;
  o0[b] = 0ull;
  o1[b] = 0ull;
  o2[b] = 0ull;
}

// Rungs 0-2: one thread per (i, j); i = x, j = y.  Each thread evaluates DD(i, j), DR(i, j)
// and RR(i, j) where they exist.  RUNG >= 1 keeps DD and RR only for j >= i (weight 2 off the
// diagonal); RUNG >= 2 reads precomputed per-galaxy values.
template <int RUNG, int ACOS>
__global__ void __launch_bounds__(kPairBlock *kPairBlock) ladder_pair_kernel(const LadderArgs A) {
  extern __shared__ uint32_t h[];
  const int tid = threadIdx.y * kPairBlock + threadIdx.x;
  constexpr int kThreads = kPairBlock * kPairBlock;
  for (int b = tid; b < 3 * A.stride; b += kThreads) h[b] = 0u;
  __syncthreads();
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kPairBlock + threadIdx.x;
  const int64_t j = static_cast<int64_t>(blockIdx.y) * kPairBlock + threadIdx.y;
  auto gal = [&](const LadderCat &cat, int64_t k) __attribute__((always_inline)) {
    if constexpr (RUNG >= 2) return prep_gal(cat, k);
    else return raw_gal(cat, k);
  };
  const bool di = i < A.n_d, dj = j < A.n_d, ri = i < A.n_r, rj = j < A.n_r;
  Gal gdi = {0.0f, 0.0f, 0.0f}, gdj = gdi, gri = gdi, grj = gdi;
  if (di) gdi = gal(A.d, i);
  if (dj) gdj = gal(A.d, j);
  if (ri) gri = gal(A.r, i);
  if (rj) grj = gal(A.r, j);
  const bool sym_ok = RUNG == 0 || j >= i;
  const uint32_t inc = RUNG == 0 ? 1u : 1u + (j != i ? 1u : 0u);
  if (di && dj && sym_ok) atomicAdd(h + 0 * A.stride + ladder_bin<ACOS>(law_of_cosines(gdi, gdj.s, gdj.c, gdj.a), A), inc);
  if (di && rj) atomicAdd(h + 1 * A.stride + ladder_bin<ACOS>(law_of_cosines(gdi, grj.s, grj.c, grj.a), A), 1u);
  if (ri && rj && sym_ok) atomicAdd(h + 2 * A.stride + ladder_bin<ACOS>(law_of_cosines(gri, grj.s, grj.c, grj.a), A), inc);
  __syncthreads();
  flush_block(h, A, tid, kThreads);
}

// Rungs 3-5 (sections "L3: block tiling", "L4: fast acos", "L5: the last 8%").  A workgroup of
// TILE threads takes tile column x (i = x TILE + thread, one galaxy per thread, its values kept in
// registers) against tile row y (TILE consecutive j).  The row's per-galaxy values of both
// catalogs are staged once in LDS as 16-byte records {sin delta, cos delta, alpha, 0}, so a pair
// reads its j values with one broadcast ds_read_b128 per catalog; the three histograms follow the
// records.  DD and RR keep the per-pair upper-triangle test of rung 1.  TUNED (rung 5): the j loop
// unrolled by 8, launch bounds of exactly TILE threads, and a workgroup whose row lies wholly
// before its column (y < x: every j of the row is below every i) does no DD/RR work at all.
template <int TILE, int ACOS, bool TUNED>
__global__ void __launch_bounds__(TUNED ? TILE : 1024) ladder_tile_kernel(const LadderArgs A) {
  extern __shared__ float4 rec[];
  float4 *const rec_d = rec;          // [TILE] D records of the row
  float4 *const rec_r = rec + TILE;   // [TILE] R records of the row
  uint32_t *const hist = reinterpret_cast<uint32_t *>(rec + 2 * TILE);  // DD | DR | RR, A.stride apart
  const int t = threadIdx.x;
  const int64_t row0 = static_cast<int64_t>(blockIdx.y) * TILE;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * TILE + t;
  for (int q = t; q < 3 * A.stride; q += TILE) hist[q] = 0u;
  auto stage = [&](const LadderCat &cat, int64_t n, float4 *dst) __attribute__((always_inline)) {
    const int64_t k = row0 + t;
    dst[t] = k < n ? make_float4(cat.s[k], cat.c[k], cat.a[k], 0.0f) : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  };
  stage(A.d, A.n_d, rec_d);
  stage(A.r, A.n_r, rec_r);
  const bool in_d = i < A.n_d, in_r = i < A.n_r;
  const Gal none = {0.0f, 0.0f, 0.0f};
  const Gal gi_d = in_d ? prep_gal(A.d, i) : none;
  const Gal gi_r = in_r ? prep_gal(A.r, i) : none;
  const int64_t n_max = A.n_d > A.n_r ? A.n_d : A.n_r;
  const int len = static_cast<int>(n_max - row0 < TILE ? n_max - row0 : TILE);  // ragged last row
  const bool upper_possible = !TUNED || blockIdx.y >= blockIdx.x;
  uint32_t *const h_dd = hist, *const h_dr = hist + A.stride, *const h_rr = hist + 2 * A.stride;
  __syncthreads();
  auto count = [&](uint32_t *h, const Gal &g, const float4 &r, uint32_t weight) __attribute__((always_inline)) {
    atomicAdd(h + ladder_bin<ACOS>(law_of_cosines(g, r.x, r.y, r.z), A), weight);
  };
  auto visit = [&](int u) __attribute__((always_inline)) {
    const int64_t j = row0 + u;
    const float4 rr = rec_r[u];
    if (in_d && j < A.n_r) count(h_dr, gi_d, rr, 1u);
    if (upper_possible && j >= i) {
      const uint32_t weight = j == i ? 1u : 2u;  // the diagonal once, every other pair for both orders
      if (in_d && j < A.n_d) count(h_dd, gi_d, rec_d[u], weight);
      if (in_r && j < A.n_r) count(h_rr, gi_r, rr, weight);
    }
  };
  if constexpr (TUNED) {
#pragma unroll 8
    for (int u = 0; u < len; ++u) visit(u);
  } else {
#pragma unroll 1
    for (int u = 0; u < len; ++u) visit(u);
  }
  __syncthreads();
  flush_block(hist, A, t, TILE);
}

template <int RUNG, int ACOS> const void *pair_fn() {
  return reinterpret_cast<const void *>(&ladder_pair_kernel<RUNG, ACOS>);
}
template <int TILE, int ACOS, bool TUNED> const void *tile_fn() {
  return reinterpret_cast<const void *>(&ladder_tile_kernel<TILE, ACOS, TUNED>);
}

template <int RUNG> const void *pair_by_acos(int acos_kind) {
  return acos_kind == 0 ? pair_fn<RUNG, 0>() : (acos_kind == 1 ? pair_fn<RUNG, 1>() : pair_fn<RUNG, 2>());
}
template <int TILE, bool TUNED> const void *tile_by_acos(int acos_kind) {
  return acos_kind == 0 ? tile_fn<TILE, 0, TUNED>()
                        : (acos_kind == 1 ? tile_fn<TILE, 1, TUNED>() : tile_fn<TILE, 2, TUNED>());
}
template <bool TUNED> const void *tile_by_size(int tile, int acos_kind) {
  switch (tile) {
    case 64: return tile_by_acos<64, TUNED>(acos_kind);
    case 128: return tile_by_acos<128, TUNED>(acos_kind);
    case 256: return tile_by_acos<256, TUNED>(acos_kind);
    case 512: return tile_by_acos<512, TUNED>(acos_kind);
    default: return tile_by_acos<1024, TUNED>(acos_kind);
  }
}

const void *select_ladder(int rung, int acos_kind, int tile) {
  switch (rung) {
    case 0: return pair_by_acos<0>(acos_kind);
    case 1: return pair_by_acos<1>(acos_kind);
    case 2: return pair_by_acos<2>(acos_kind);
    case 3:
    case 4: return tile_by_size<false>(tile, acos_kind);
    default: return tile_by_size<true>(tile, acos_kind);
  }
}

size_t aligned_floats(int64_t n) { return (static_cast<size_t>(n) * sizeof(float) + 255) / 256 * 256; }

bool aligned_to(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

}  // namespace
}  // namespace gc

using namespace gc;

extern "C" {

size_t gc_ladder_workspace_bytes(int64_t n_d, int64_t n_r) {
  if (n_d < 0 || n_r < 0 || n_d > GC_LADDER_MAX_GALAXIES || n_r > GC_LADDER_MAX_GALAXIES) return 0;
  return 3 * (aligned_floats(n_d) + aligned_floats(n_r));
}

gc_status gc_ladder_histogram(int32_t rung, int32_t acos_kind, int32_t tile, int32_t bin_stride,
                              const float *ra_d, const float *dec_d, int64_t n_d, const float *ra_r,
                              const float *dec_r, int64_t n_r, int32_t nbins, double w_deg, uint64_t *dd,
                              uint64_t *dr, uint64_t *rr, void *workspace, size_t ws_bytes, gc_stream_t stream) {
  if (rung < 0 || rung >= GC_LADDER_RUNGS) return GC_ERR_INVALID_ARGUMENT;
  if (acos_kind < GC_LADDER_ACOS_RUNG || acos_kind > GC_LADDER_ACOS_FIT6) return GC_ERR_INVALID_ARGUMENT;
  if (nbins <= 0 || !(w_deg > 0.0) || !(w_deg < 1e300)) return GC_ERR_INVALID_ARGUMENT;
  if (nbins > GC_MAX_BINS) return GC_ERR_UNSUPPORTED;
  if (n_d < 0 || n_r < 0) return GC_ERR_INVALID_ARGUMENT;
  if (n_d > GC_LADDER_MAX_GALAXIES || n_r > GC_LADDER_MAX_GALAXIES) return GC_ERR_UNSUPPORTED;
  const bool tiled = rung >= 3;
  if (!tiled && tile != 0) return GC_ERR_INVALID_ARGUMENT;
  if (tiled && tile != 0 && tile != 64 && tile != 128 && tile != 256 && tile != 512 && tile != 1024)
    return GC_ERR_INVALID_ARGUMENT;
  if (bin_stride != 0 && bin_stride < nbins) return GC_ERR_INVALID_ARGUMENT;
  const int t = tiled ? (tile ? tile : 512) : 0;
  const int stride = bin_stride ? bin_stride : nbins;
  // rungs 0-2: three histograms; rungs 3-5: also two rows of 16-byte records
  const size_t lds = 3 * static_cast<size_t>(stride) * sizeof(uint32_t) + 2 * static_cast<size_t>(t) * sizeof(float4);
  if (lds > kMaxLdsBytes) return GC_ERR_UNSUPPORTED;
  if ((n_d > 0 && (!ra_d || !dec_d || !aligned_to(ra_d, 4) || !aligned_to(dec_d, 4))) ||
      (n_r > 0 && (!ra_r || !dec_r || !aligned_to(ra_r, 4) || !aligned_to(dec_r, 4))))
    return GC_ERR_INVALID_ARGUMENT;
  if (!dd || !dr || !rr || !aligned_to(dd, 8) || !aligned_to(dr, 8) || !aligned_to(rr, 8))
    return GC_ERR_INVALID_ARGUMENT;
  const bool need_ws = rung >= 2 && (n_d > 0 || n_r > 0);
  if (need_ws && (!workspace || !aligned_to(workspace, GC_ALIGNMENT))) return GC_ERR_INVALID_ARGUMENT;
  if (need_ws && ws_bytes < gc_ladder_workspace_bytes(n_d, n_r)) return GC_ERR_WORKSPACE;
  const int kind = acos_kind == GC_LADDER_ACOS_RUNG ? (rung >= 4 ? GC_LADDER_ACOS_HANDBOOK : GC_LADDER_ACOS_LIBM)
                                                    : acos_kind;

  const hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  LadderArgs a;
  a.n_d = n_d;
  a.n_r = n_r;
  a.out[0] = reinterpret_cast<unsigned long long *>(dd);
  a.out[1] = reinterpret_cast<unsigned long long *>(dr);
  a.out[2] = reinterpret_cast<unsigned long long *>(rr);
  a.t_per_rad = static_cast<float>((180.0 / 3.14159265358979323846) / w_deg);
  a.nbins = nbins;
  a.stride = stride;
  a.d.ra = ra_d;
  a.d.dec = dec_d;
  a.r.ra = ra_r;
  a.r.dec = dec_r;
  char *ws = static_cast<char *>(workspace);
  const size_t fd = aligned_floats(n_d), fr = aligned_floats(n_r);
  a.d.s = need_ws ? reinterpret_cast<float *>(ws) : nullptr;
  a.d.c = need_ws ? reinterpret_cast<float *>(ws + fd) : nullptr;
  a.d.a = need_ws ? reinterpret_cast<float *>(ws + 2 * fd) : nullptr;
  a.r.s = need_ws ? reinterpret_cast<float *>(ws + 3 * fd) : nullptr;
  a.r.c = need_ws ? reinterpret_cast<float *>(ws + 3 * fd + fr) : nullptr;
  a.r.a = need_ws ? reinterpret_cast<float *>(ws + 3 * fd + 2 * fr) : nullptr;

  hipLaunchKernelGGL(ladder_zero_kernel, dim3((nbins + 255) / 256), dim3(256), 0, hs, a.out[0], a.out[1], a.out[2],
                     nbins);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && need_ws) {
    if (n_d > 0)
      hipLaunchKernelGGL(ladder_prep_kernel, dim3(static_cast<unsigned>((n_d + 255) / 256)), dim3(256), 0, hs, ra_d,
                         dec_d, n_d, a.d.s, a.d.c, a.d.a);
    if (n_r > 0)
      hipLaunchKernelGGL(ladder_prep_kernel, dim3(static_cast<unsigned>((n_r + 255) / 256)), dim3(256), 0, hs, ra_r,
                         dec_r, n_r, a.r.s, a.r.c, a.r.a);
    e = hipGetLastError();
  }
  const int64_t nmax = n_d > n_r ? n_d : n_r;
  if (e == hipSuccess && nmax > 0) {
    const void *fn = select_ladder(rung, kind, t);
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e == hipSuccess) {
      void *args[] = {&a};
      if (tiled) {
        const unsigned g = static_cast<unsigned>((nmax + t - 1) / t);
        e = hipLaunchKernel(fn, dim3(g, g), dim3(t), args, lds, hs);
      } else {
        const unsigned g = static_cast<unsigned>((nmax + kPairBlock - 1) / kPairBlock);
        e = hipLaunchKernel(fn, dim3(g, g), dim3(kPairBlock, kPairBlock), args, lds, hs);
      }
    }
  }
  if (e != hipSuccess) {
    record_hip_error(e);
    return GC_ERR_DEVICE;
  }
  return GC_OK;
}

}  // extern "C"
