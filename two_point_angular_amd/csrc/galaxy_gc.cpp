// galaxy_gc: the end-to-end program of "CUDA Deep Dive: 10B Galaxy Pairs on an RTX 5080" (the
// appendix listing's driver: read two catalogs, build DD, DR and RR on the GPU, check the sums,
// write omega.out), over libgc.  Usage:
//
//   galaxy_gc [--nbins N] [--width DEG] [--quiet] D.txt R.txt omega.out
//
// Catalog and result formats: include/gc_io.h.  Defaults: 720 bins of 0.25 degrees (every
// separation from 0 to 180 degrees).  Prints the phase times (read, staging, GPU work,
// write) and the pair rate; exits 0 on success, 1 on any error (message on stderr), 2 on bad
// usage.  Runs on the current HIP device (HIP_VISIBLE_DEVICES selects it).
#include <hip/hip_runtime.h>
#include <inttypes.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <chrono>
#include <string>
#include <thread>
#include <vector>

#include "../../include/gc.h"
#include "../../include/gc_io.h"

namespace {

using Clock = std::chrono::steady_clock;

double ms_since(Clock::time_point t0) {
  return std::chrono::duration<double, std::milli>(Clock::now() - t0).count();
}

int usage() {
  fprintf(stderr, "usage: galaxy_gc [--nbins N] [--width DEG] [--quiet] D.txt R.txt omega.out\n");
  return 2;
}

bool check(gc_status s, const char *what) {
  if (s == GC_OK) return true;
  fprintf(stderr, "galaxy_gc: %s: %s", what, gc_status_string(s));
  if (s == GC_ERR_DEVICE) fprintf(stderr, " (HIP error %d)", gc_last_device_error());
  fprintf(stderr, "\n");
  return false;
}

bool check_hip(hipError_t e, const char *what) {
  if (e == hipSuccess) return true;
  fprintf(stderr, "galaxy_gc: %s: %s\n", what, hipGetErrorString(e));
  return false;
}

bool read_catalog(const char *path, std::vector<float> &ra, std::vector<float> &dec) {
  int64_t n = 0;
  if (!check(gc_catalog_count(path, &n), path)) return false;
  ra.resize(static_cast<size_t>(n));
  dec.resize(static_cast<size_t>(n));
  int64_t got = 0;
  return check(gc_catalog_read(path, ra.data(), dec.data(), n, &got), path);
}

// One device block for everything, freed at scope exit.
struct DeviceBlock {
  char *p = nullptr;
  size_t used = 0;
  ~DeviceBlock() {
    if (p) (void)hipFree(p);
  }
  // carve `bytes` (rounded up to 256) out of the block
  void *take(size_t bytes) {
    void *r = p + used;
    used += (bytes + 255) / 256 * 256;
    return r;
  }
};

// One pinned host block, mapped into the device's address space: the catalogs go in and the
// results come out through it, read and written by kernels (no copy engine, whose first use in a
// process costs several milliseconds).  Freed at scope exit.
struct HostBlock {
  char *p = nullptr;
  char *dev = nullptr;  // the block's device address
  ~HostBlock() {
    if (p) (void)hipHostFree(p);
  }
};

size_t round256(size_t b) { return (b + 255) / 256 * 256; }

// dst[0, n) = src[0, n), 8-byte words; a grid-stride loop.
__global__ void copy_words(const uint64_t *__restrict__ src, uint64_t *__restrict__ dst, int64_t n) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) dst[i] = src[i];
}

hipError_t launch_copy(const uint64_t *src, uint64_t *dst, int64_t n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256;
  copy_words<<<static_cast<unsigned>(blocks < 1024 ? blocks : 1024), 256, 0, st>>>(src, dst, n);
  return hipGetLastError();
}

}  // namespace

int main(int argc, char **argv) {
  int32_t nbins = 720;
  double width = 0.25;
  bool quiet = false;
  std::vector<const char *> pos;
  for (int a = 1; a < argc; ++a) {
    if (!strcmp(argv[a], "--nbins") && a + 1 < argc) {
      char *e = nullptr;
      const long v = strtol(argv[++a], &e, 10);
      if (*e || v <= 0 || v > GC_MAX_BINS) return usage();
      nbins = static_cast<int32_t>(v);
    } else if (!strcmp(argv[a], "--width") && a + 1 < argc) {
      char *e = nullptr;
      width = strtod(argv[++a], &e);
      if (*e || !(width > 0.0) || width > 360.0) return usage();
    } else if (!strcmp(argv[a], "--quiet")) {
      quiet = true;
    } else if (argv[a][0] == '-' && argv[a][1] == '-') {
      return usage();
    } else {
      pos.push_back(argv[a]);
    }
  }
  if (pos.size() != 3) return usage();

  const auto t_all = Clock::now();
  // The catalog sizes first (the count line only), so that the helper thread can start the HIP
  // runtime, allocate the device and host blocks for the whole job and run a one-galaxy job of the
  // same bins (which loads the kernels and caches the launch plan) while this thread parses.
  int64_t n_d = 0, n_r = 0;
  if (!check(gc_catalog_count(pos[0], &n_d), pos[0]) || !check(gc_catalog_count(pos[1], &n_r), pos[1])) return 1;
  const size_t fd = static_cast<size_t>(n_d) * sizeof(float), fr = static_cast<size_t>(n_r) * sizeof(float);
  // results, one run of 8-byte words: DD, DR, RR (nbins each), the three sums, omega (nbins)
  const int64_t res_words = 4 * static_cast<int64_t>(nbins) + 3;
  const size_t res_bytes = static_cast<size_t>(res_words) * sizeof(uint64_t);
  const size_t ws_bytes = gc_workspace_bytes(nbins);
  const size_t dev_total = round256(gc_prepared_bytes(n_d)) + round256(gc_prepared_bytes(n_r)) +
                           round256(gc_prepared_bytes(1)) + round256(res_bytes) + round256(ws_bytes);
  // host block: D (alpha, delta), R (alpha, delta), the one-galaxy input, the results
  const size_t h_rd = 0, h_rr = round256(2 * fd), h_one = h_rr + round256(2 * fr), h_res = h_one + 256;
  const size_t host_total = h_res + round256(res_bytes);
  hipStream_t st = nullptr;
  DeviceBlock blk;
  HostBlock hb;
  gc_status warm_status = GC_OK;
  hipError_t init_err = hipSuccess;
  double init_ms = 0.0;
  void *prep_d = nullptr, *prep_r = nullptr, *prep1 = nullptr, *ws = nullptr;
  uint64_t *res = nullptr;
  std::thread init([&] {
    const auto ti = Clock::now();
    init_err = hipStreamCreate(&st);
    if (init_err == hipSuccess) init_err = hipMalloc(&blk.p, dev_total);
    if (init_err == hipSuccess) init_err = hipHostMalloc(&hb.p, host_total, hipHostMallocMapped | hipHostMallocCoherent);
    if (init_err == hipSuccess) init_err = hipHostGetDevicePointer(reinterpret_cast<void **>(&hb.dev), hb.p, 0);
    if (init_err != hipSuccess) {
      init_ms = ms_since(ti);
      return;
    }
    prep_d = blk.take(gc_prepared_bytes(n_d));
    prep_r = blk.take(gc_prepared_bytes(n_r));
    prep1 = blk.take(gc_prepared_bytes(1));
    res = static_cast<uint64_t *>(blk.take(res_bytes));
    ws = blk.take(ws_bytes);
    // The one-galaxy job: (0, 0) against itself, read from and written back to the host block
    // like the real job.
    float *one = reinterpret_cast<float *>(hb.p + h_one);
    one[0] = one[1] = 0.0f;
    const float *one_dev = reinterpret_cast<const float *>(hb.dev + h_one);
    const gc_stream_t gs = reinterpret_cast<gc_stream_t>(st);
    warm_status = gc_prepare(one_dev, one_dev + 1, 1, prep1, gs);
    if (warm_status == GC_OK)
      warm_status = gc_histogram_dd_dr_rr(prep1, 1, prep1, 1, nbins, width, res, res + nbins, res + 2 * nbins, ws,
                                          ws_bytes, gs);
    if (warm_status == GC_OK)
      init_err = launch_copy(res, reinterpret_cast<uint64_t *>(hb.dev + h_res), 3 * static_cast<int64_t>(nbins), st);
    if (init_err == hipSuccess) init_err = hipStreamSynchronize(st);
    init_ms = ms_since(ti);
  });
  auto t0 = Clock::now();
  std::vector<float> ra_d, dec_d, ra_r, dec_r;
  const bool read_ok = read_catalog(pos[0], ra_d, dec_d) && read_catalog(pos[1], ra_r, dec_r);
  const double read_ms = ms_since(t0);
  init.join();
  if (!read_ok || !check_hip(init_err, "HIP start-up") || !check(warm_status, "warm-up job")) return 1;
  if (static_cast<int64_t>(ra_d.size()) != n_d || static_cast<int64_t>(ra_r.size()) != n_r) {
    fprintf(stderr, "galaxy_gc: a catalog changed while it was read\n");
    return 1;
  }

  // The catalogs into the host block, which the preparation kernels read over the bus.
  t0 = Clock::now();
  if (fd) {
    memcpy(hb.p + h_rd, ra_d.data(), fd);
    memcpy(hb.p + h_rd + fd, dec_d.data(), fd);
  }
  if (fr) {
    memcpy(hb.p + h_rr, ra_r.data(), fr);
    memcpy(hb.p + h_rr + fr, dec_r.data(), fr);
  }
  const double stage_ms = ms_since(t0);
  const float *d_ra_d = reinterpret_cast<const float *>(hb.dev + h_rd), *d_dec_d = d_ra_d + n_d;
  const float *d_ra_r = reinterpret_cast<const float *>(hb.dev + h_rr), *d_dec_r = d_ra_r + n_r;
  uint64_t *dd = res, *dr = res + nbins, *rr = res + 2 * nbins, *tot = res + 3 * nbins;
  double *om = reinterpret_cast<double *>(res + 3 * nbins + 3);
  const gc_stream_t gs = reinterpret_cast<gc_stream_t>(st);

  hipEvent_t e0, e1;
  if (!check_hip(hipEventCreate(&e0), "event") || !check_hip(hipEventCreate(&e1), "event")) return 1;
  t0 = Clock::now();
  if (!check_hip(hipEventRecord(e0, st), "event") ||
      !check(gc_prepare(d_ra_d, d_dec_d, n_d, prep_d, gs), "gc_prepare D") ||
      !check(gc_prepare(d_ra_r, d_dec_r, n_r, prep_r, gs), "gc_prepare R") ||
      !check(gc_histogram_dd_dr_rr(prep_d, n_d, prep_r, n_r, nbins, width, dd, dr, rr, ws, ws_bytes, gs),
             "gc_histogram_dd_dr_rr") ||
      !check(gc_histogram_totals(dd, dr, rr, nbins, tot, gs), "gc_histogram_totals") ||
      !check(gc_omega(dd, dr, rr, nbins, n_d, n_r, om, gs), "gc_omega") ||
      !check_hip(launch_copy(res, reinterpret_cast<uint64_t *>(hb.dev + h_res), res_words, st), "result copy") ||
      !check_hip(hipEventRecord(e1, st), "event") || !check_hip(hipStreamSynchronize(st), "histograms"))
    return 1;
  float gpu_ms = 0.0f;
  (void)hipEventElapsedTime(&gpu_ms, e0, e1);
  const double hist_wall_ms = ms_since(t0);
  const uint64_t *h = reinterpret_cast<const uint64_t *>(hb.p + h_res), *totals = h + 3 * nbins;
  const double *omega = reinterpret_cast<const double *>(h + 3 * nbins + 3);
  // The page's guardrail: every family sums to exactly N_a * N_b.
  const uint64_t want[3] = {static_cast<uint64_t>(n_d) * static_cast<uint64_t>(n_d),
                            static_cast<uint64_t>(n_d) * static_cast<uint64_t>(n_r),
                            static_cast<uint64_t>(n_r) * static_cast<uint64_t>(n_r)};
  const char *fam[3] = {"DD", "DR", "RR"};
  for (int f = 0; f < 3; ++f) {
    if (totals[f] != want[f]) {
      fprintf(stderr, "galaxy_gc: %s histogram sums to %" PRIu64 ", expected %" PRIu64 "\n", fam[f], totals[f],
              want[f]);
      return 1;
    }
  }

  t0 = Clock::now();
  if (!check(gc_omega_write(pos[2], h, h + nbins, h + 2 * nbins, omega, nbins, width), pos[2]))
    return 1;
  const double write_ms = ms_since(t0);
  const double total_ms = ms_since(t_all);
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);

  if (!quiet) {
    const double ordered = static_cast<double>(want[0]) + static_cast<double>(want[1]) + static_cast<double>(want[2]);
    printf("galaxy_gc: %" PRId64 " + %" PRId64 " galaxies, %d bins of %g deg\n", n_d, n_r, nbins, width);
    printf("  sums   DD %" PRIu64 "  DR %" PRIu64 "  RR %" PRIu64 " (exact)\n", totals[0], totals[1], totals[2]);
    printf("  read %.2f ms (alongside: HIP start-up, allocation and a one-galaxy warm-up job %.2f ms) | into "
           "pinned memory %.2f ms | preparation, histograms, omega and results back %.3f ms (GPU events; %.3f ms "
           "wall) | write %.2f ms | total %.2f ms\n",
           read_ms, init_ms, stage_ms, gpu_ms, hist_wall_ms, write_ms, total_ms);
    printf("  %.3e ordered pairs/s on the GPU\n", ordered / (gpu_ms / 1e3));
  }
  return 0;
}
