// Measured ceilings for the pair kernel's two resources on gfx950: VALU issue (independent
// FMA chains, fp32 square roots, fp64 FMA chains) and LDS atomic increments into per-wave
// histograms (random bins, and every lane on one bin).  A roofline read against a vendor
// number alone can hide what this part actually sustains; these kernels give the measured
// ceiling beside it.  The caller times a launch with events on its stream.
#include "../../include/gc_diag.h"
#include "gc_internal.h"

namespace gc {
namespace {

constexpr int kCeilBlocks = 2048;
constexpr int kCeilThreads = 256;
constexpr int kChains = 8;

// Eight independent dependency chains per lane; each loop iteration issues 8 VALU ops.
__global__ void __launch_bounds__(kCeilThreads) fma32_kernel(float *sink, int64_t iters, float m, float c) {
  float a[kChains];
#pragma unroll
  for (int q = 0; q < kChains; ++q) a[q] = static_cast<float>(threadIdx.x + q);
  for (int64_t i = 0; i < iters; ++i) {
#pragma unroll
    for (int q = 0; q < kChains; ++q) a[q] = fmaf(a[q], m, c);
  }
  float s = 0.0f;
#pragma unroll
  for (int q = 0; q < kChains; ++q) s += a[q];
  sink[blockIdx.x * kCeilThreads + threadIdx.x] = s;
}

__global__ void __launch_bounds__(kCeilThreads) sqrt32_kernel(float *sink, int64_t iters, float m, float c) {
  float a[kChains];
#pragma unroll
  for (int q = 0; q < kChains; ++q) a[q] = static_cast<float>(threadIdx.x + q + 2);
  for (int64_t i = 0; i < iters; ++i) {
#pragma unroll
    for (int q = 0; q < kChains; ++q) a[q] = __builtin_amdgcn_sqrtf(a[q]);
  }
  float s = 0.0f;
#pragma unroll
  for (int q = 0; q < kChains; ++q) s += a[q];
  sink[blockIdx.x * kCeilThreads + threadIdx.x] = fmaf(s, m, c);
}

__global__ void __launch_bounds__(kCeilThreads) fma64_kernel(float *sink, int64_t iters, float m, float c) {
  double a[kChains];
  const double md = m, cd = c;
#pragma unroll
  for (int q = 0; q < kChains; ++q) a[q] = static_cast<double>(threadIdx.x + q);
  for (int64_t i = 0; i < iters; ++i) {
#pragma unroll
    for (int q = 0; q < kChains; ++q) a[q] = fma(a[q], md, cd);
  }
  double s = 0.0;
#pragma unroll
  for (int q = 0; q < kChains; ++q) s += a[q];
  sink[blockIdx.x * kCeilThreads + threadIdx.x] = static_cast<float>(s);
}

// Every lane adds 1 to a bin of its wave's private LDS histogram 16 x iters times.  Each
// lane cycles through 16 bins drawn once from a hash (over the largest power of two
// <= nbins), or uses bin 0 only, so the loop is nothing but ds_add_u32 instructions: the
// LDS atomic throughput for spread or fully colliding addresses.
template <bool SAME_BIN>
__global__ void __launch_bounds__(kCeilThreads) lds_atomic_kernel(uint32_t *sink, int64_t iters, int32_t nbins,
                                                                  int32_t shift) {
  extern __shared__ uint32_t lds[];
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x / kWave;
  uint32_t *hist = lds + wv * nbins;
  for (int b = lane; b < nbins; b += kWave) hist[b] = 0u;
  __builtin_amdgcn_wave_barrier();
  const uint32_t tid = blockIdx.x * kCeilThreads + threadIdx.x;
  uint32_t bins[16];
  uint32_t state = tid * 2654435761u + 12345u;
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    state ^= state << 13;
    state ^= state >> 17;
    state ^= state << 5;
    bins[q] = SAME_BIN ? 0u : (state >> shift);
  }
#pragma unroll 1
  for (int64_t i = 0; i < iters; ++i) {
#pragma unroll
    for (int q = 0; q < 16; ++q) atomicAdd(hist + bins[q], 1u);
  }
  __builtin_amdgcn_wave_barrier();
  uint32_t total = 0;
  for (int b = lane; b < nbins; b += kWave) total += hist[b];
  sink[tid] = total;
}


// LDS access probes, to read the pair kernel's LDS time against: every lane issues 16 x iters
// LDS operations of one kind at addresses drawn once from a hash, into one table of `words`
// 32-bit words shared by the workgroup (so the bank pattern is that of random keys, as in the
// pair kernel).  KIND: 0 ds_add_u32, 1 ds_add_rtn_u32, 2 ds_add_u64, 3 ds_add_rtn_u64,
// 4 ds_read_b32, 5 ds_read_b64, 6 ds_read_b64 of an entry, then ds_add_u32 into a 1024-word
// histogram at the word the entry names (the bin-table core's pair of accesses), 7 ds_add_u32
// issued by one lane in `sparse` (the rest masked off).  cols = 0: the index is drawn from the
// whole table; cols = C (a power of two <= 64): the table is C columns of words / C rows, the row
// is drawn and the column is the lane's index mod C (a histogram replicated per lane group).
constexpr int kProbeHist = 1024;
template <int KIND>
__global__ void __launch_bounds__(1024) lds_probe_kernel(uint32_t *sink, int64_t iters, int32_t words,
                                                         int32_t sparse, int32_t cols) {
  extern __shared__ uint32_t lds[];
  constexpr bool WIDE = KIND == 2 || KIND == 3 || KIND == 5 || KIND == 6;
  const uint32_t tid = blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t *hist = lds + words;
  for (int q = threadIdx.x; q < words; q += blockDim.x)
    lds[q] = KIND == 6 ? ((static_cast<uint32_t>(q) * 2654435761u) >> 22) : 0u;  // < kProbeHist
  if (KIND == 6)
    for (int q = threadIdx.x; q < kProbeHist; q += blockDim.x) hist[q] = 0u;
  __syncthreads();
  const uint32_t n = WIDE ? static_cast<uint32_t>(words / 2) : static_cast<uint32_t>(words);
  uint32_t idx[16];
  uint32_t state = tid * 2654435761u + 12345u;
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    state ^= state << 13;
    state ^= state >> 17;
    state ^= state << 5;
    if (cols == 0) {
      idx[q] = static_cast<uint32_t>((static_cast<uint64_t>(state) * n) >> 32);  // < n
    } else {
      const uint32_t c = static_cast<uint32_t>(cols), rows = n / c;
      idx[q] = static_cast<uint32_t>((static_cast<uint64_t>(state) * rows) >> 32) * c + (threadIdx.x & (c - 1));
    }
  }
  const bool active = KIND != 7 || (tid % static_cast<uint32_t>(sparse)) == 0u;
  unsigned long long *lds64 = reinterpret_cast<unsigned long long *>(lds);
  unsigned long long acc = 0ull;
  if (active) {
#pragma unroll 1
    for (int64_t i = 0; i < iters; ++i) {
      if constexpr (KIND == 0 || KIND == 7) {
#pragma unroll
        for (int q = 0; q < 16; ++q) atomicAdd(lds + idx[q], 1u);
      } else if constexpr (KIND == 1) {
        uint32_t r[16];
#pragma unroll
        for (int q = 0; q < 16; ++q)
          r[q] = __hip_atomic_fetch_add(lds + idx[q], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
#pragma unroll
        for (int q = 0; q < 16; ++q) acc += r[q];
      } else if constexpr (KIND == 2) {
#pragma unroll
        for (int q = 0; q < 16; ++q) atomicAdd(lds64 + idx[q], 1ull);
      } else if constexpr (KIND == 3) {
        unsigned long long r[16];
#pragma unroll
        for (int q = 0; q < 16; ++q)
          r[q] = __hip_atomic_fetch_add(lds64 + idx[q], 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
#pragma unroll
        for (int q = 0; q < 16; ++q) acc += r[q];
      } else if constexpr (KIND == 4) {
        // (the index's low bit flips with i, so the reads cannot be hoisted out of the loop; n is even)
        const uint32_t flip = static_cast<uint32_t>(i & 1);
        uint32_t v[16];
#pragma unroll
        for (int q = 0; q < 16; ++q) v[q] = lds[idx[q] ^ flip];
#pragma unroll
        for (int q = 0; q < 16; ++q) acc += v[q];
      } else if constexpr (KIND == 5) {
        const uint32_t flip = static_cast<uint32_t>(i & 1);
        unsigned long long v[16];
#pragma unroll
        for (int q = 0; q < 16; ++q) v[q] = lds64[idx[q] ^ flip];
#pragma unroll
        for (int q = 0; q < 16; ++q) acc += v[q];
      } else {
        const uint32_t flip = static_cast<uint32_t>(i & 1);
        const uint2 *tab = reinterpret_cast<const uint2 *>(lds);
        uint2 v[16];
#pragma unroll
        for (int q = 0; q < 16; ++q) v[q] = tab[idx[q] ^ flip];
#pragma unroll
        for (int q = 0; q < 16; ++q) atomicAdd(hist + ((v[q].x + v[q].y) & (kProbeHist - 1)), 1u);
      }
    }
  }
  __syncthreads();
  uint32_t total = static_cast<uint32_t>(acc) + static_cast<uint32_t>(acc >> 32);
  for (int q = threadIdx.x; q < words; q += blockDim.x) total += lds[q];
  sink[tid] = total;
}

// The same access pattern through the vector memory path: every lane loads 16 x iters random
// 8-byte entries of a table of `words` words in global memory (L1-resident for small tables),
// the way the pair kernel reads part of its bin table.
__global__ void __launch_bounds__(1024) l1_probe_kernel(const uint2 *__restrict__ tab, uint32_t *sink, int64_t iters,
                                                        int32_t words) {
  const uint32_t tid = blockIdx.x * blockDim.x + threadIdx.x;
  const uint32_t n = static_cast<uint32_t>(words / 2);
  uint32_t idx[16];
  uint32_t state = tid * 2654435761u + 12345u;
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    state ^= state << 13;
    state ^= state >> 17;
    state ^= state << 5;
    idx[q] = static_cast<uint32_t>((static_cast<uint64_t>(state) * n) >> 32);  // < n
  }
  uint32_t acc = 0;
#pragma unroll 1
  for (int64_t i = 0; i < iters; ++i) {
    const uint32_t flip = static_cast<uint32_t>(i & 1);  // n even: idx ^ 1 < n
    uint2 v[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) v[q] = tab[idx[q] ^ flip];
#pragma unroll
    for (int q = 0; q < 16; ++q) acc += v[q].x ^ v[q].y;
  }
  sink[tid] = acc;
}

}  // namespace
}  // namespace gc

using namespace gc;

extern "C" {

size_t gc_ceiling_sink_bytes(void) { return static_cast<size_t>(kCeilBlocks) * 1024u * 4u; }

gc_status gc_ceiling_valu(int32_t kind, int64_t iters, void *d_sink, size_t sink_bytes, uint64_t *ops_out,
                          gc_stream_t stream) {
  if (kind < 0 || kind > 2 || iters <= 0 || !d_sink || !ops_out) return GC_ERR_INVALID_ARGUMENT;
  if (sink_bytes < gc_ceiling_sink_bytes()) return GC_ERR_WORKSPACE;
  const hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  float *sink = static_cast<float *>(d_sink);
  const float m = 0.999999f, c = 1e-7f;
  if (kind == 0) hipLaunchKernelGGL(fma32_kernel, dim3(kCeilBlocks), dim3(kCeilThreads), 0, hs, sink, iters, m, c);
  if (kind == 1) hipLaunchKernelGGL(sqrt32_kernel, dim3(kCeilBlocks), dim3(kCeilThreads), 0, hs, sink, iters, m, c);
  if (kind == 2) hipLaunchKernelGGL(fma64_kernel, dim3(kCeilBlocks), dim3(kCeilThreads), 0, hs, sink, iters, m, c);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return GC_ERR_DEVICE;
  *ops_out = static_cast<uint64_t>(kCeilBlocks) * kCeilThreads * static_cast<uint64_t>(iters) * kChains;
  return GC_OK;
}

gc_status gc_ceiling_lds_atomic(int32_t nbins, int32_t same_bin, int64_t iters, void *d_sink, size_t sink_bytes,
                                uint64_t *atomics_out, gc_stream_t stream) {
  if (nbins <= 0 || nbins > GC_MAX_BINS || iters <= 0 || !d_sink || !atomics_out) return GC_ERR_INVALID_ARGUMENT;
  if (sink_bytes < gc_ceiling_sink_bytes()) return GC_ERR_WORKSPACE;
  const size_t lds = static_cast<size_t>(kCeilThreads / kWave) * nbins * sizeof(uint32_t);
  int shift = 32;  // bins = state >> shift covers [0, 2^(32 - shift)), the largest power of two <= nbins
  while (shift > 0 && (1ll << (32 - shift + 1)) <= nbins) --shift;
  if (shift == 32) shift = 31;  // nbins == 1: bins 0..1 would overflow; use bin 0 only
  const hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  uint32_t *sink = static_cast<uint32_t *>(d_sink);
  if (same_bin || nbins == 1)
    hipLaunchKernelGGL(lds_atomic_kernel<true>, dim3(kCeilBlocks), dim3(kCeilThreads), lds, hs, sink, iters, nbins,
                       shift);
  else
    hipLaunchKernelGGL(lds_atomic_kernel<false>, dim3(kCeilBlocks), dim3(kCeilThreads), lds, hs, sink, iters, nbins,
                       shift);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return GC_ERR_DEVICE;
  *atomics_out = static_cast<uint64_t>(kCeilBlocks) * kCeilThreads * static_cast<uint64_t>(iters) * 16u;
  return GC_OK;
}


gc_status gc_ceiling_lds(int32_t kind, int32_t words, int32_t threads, int32_t sparse, int32_t cols, int64_t iters,
                         void *d_sink, size_t sink_bytes, uint64_t *wave_instructions_out, gc_stream_t stream) {
  if (kind < 0 || kind > 7 || iters <= 0 || !d_sink || !wave_instructions_out) return GC_ERR_INVALID_ARGUMENT;
  if (words < 128 || words % 128 != 0 || (threads != 256 && threads != 512 && threads != 1024) || sparse < 1)
    return GC_ERR_INVALID_ARGUMENT;
  if (cols < 0 || cols > 64 || (cols & (cols - 1)) != 0) return GC_ERR_INVALID_ARGUMENT;
  const size_t lds = (static_cast<size_t>(words) + (kind == 6 ? kProbeHist : 0)) * sizeof(uint32_t);
  if (lds > 160u * 1024u) return GC_ERR_UNSUPPORTED;
  if (sink_bytes < static_cast<size_t>(kCeilBlocks) * 1024u * 4u) return GC_ERR_WORKSPACE;
  const hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  uint32_t *sink = static_cast<uint32_t *>(d_sink);
  const void *fns[8] = {reinterpret_cast<const void *>(&lds_probe_kernel<0>),
                        reinterpret_cast<const void *>(&lds_probe_kernel<1>),
                        reinterpret_cast<const void *>(&lds_probe_kernel<2>),
                        reinterpret_cast<const void *>(&lds_probe_kernel<3>),
                        reinterpret_cast<const void *>(&lds_probe_kernel<4>),
                        reinterpret_cast<const void *>(&lds_probe_kernel<5>),
                        reinterpret_cast<const void *>(&lds_probe_kernel<6>),
                        reinterpret_cast<const void *>(&lds_probe_kernel<7>)};
  hipError_t e = hipFuncSetAttribute(fns[kind], hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  if (e != hipSuccess) return GC_ERR_DEVICE;
  void *args[] = {&sink, &iters, &words, &sparse, &cols};
  e = hipLaunchKernel(fns[kind], dim3(kCeilBlocks), dim3(threads), args, lds, hs);
  if (e != hipSuccess) return GC_ERR_DEVICE;
  *wave_instructions_out =
      static_cast<uint64_t>(kCeilBlocks) * static_cast<uint64_t>(threads / kWave) * static_cast<uint64_t>(iters) * 16u;
  return GC_OK;
}


gc_status gc_ceiling_l1(int32_t words, int32_t threads, int64_t iters, void *d_sink, size_t sink_bytes,
                        uint64_t *wave_instructions_out, gc_stream_t stream) {
  if (iters <= 0 || !d_sink || !wave_instructions_out) return GC_ERR_INVALID_ARGUMENT;
  if (words < 128 || words % 128 != 0 || (threads != 256 && threads != 512 && threads != 1024))
    return GC_ERR_INVALID_ARGUMENT;
  // the table is the sink's first `words` words, the results go after it
  const size_t tab_bytes = (static_cast<size_t>(words) * 4u + 255u) / 256u * 256u;
  if (sink_bytes < tab_bytes + static_cast<size_t>(kCeilBlocks) * 1024u * 4u) return GC_ERR_WORKSPACE;
  const hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  const uint2 *tab = static_cast<const uint2 *>(d_sink);
  uint32_t *sink = reinterpret_cast<uint32_t *>(static_cast<char *>(d_sink) + tab_bytes);
  hipLaunchKernelGGL(l1_probe_kernel, dim3(kCeilBlocks), dim3(threads), 0, hs, tab, sink, iters, words);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return GC_ERR_DEVICE;
  *wave_instructions_out =
      static_cast<uint64_t>(kCeilBlocks) * static_cast<uint64_t>(threads / kWave) * static_cast<uint64_t>(iters) * 16u;
  return GC_OK;
}

}  // extern "C"
