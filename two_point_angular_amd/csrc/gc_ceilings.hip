// Measured ceilings for the pair kernel's two resources on gfx950: VALU issue (independent
// FMA chains, fp32 square roots, fp64 FMA chains) and LDS atomic increments into per-wave
// histograms (random bins, and every lane on one bin).  A roofline read against a vendor
// number alone can hide what this part actually sustains; these kernels give the measured
// ceiling beside it.  The caller times a launch with events on its stream.
#include "../../include/gc.h"
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

}  // namespace
}  // namespace gc

using namespace gc;

extern "C" {

size_t gc_ceiling_sink_bytes(void) { return static_cast<size_t>(kCeilBlocks) * kCeilThreads * 4u; }

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

}  // extern "C"
