// galaxy_gc: the end-to-end program of "CUDA Deep Dive: 10B Galaxy Pairs on an RTX 5080" (the
// appendix listing's driver: read two catalogs, build DD, DR and RR on the GPU, check the sums,
// write omega.out), over libgc.  Usage:
//
//   galaxy_gc [--nbins N] [--width DEG] [--quiet] D.txt R.txt omega.out
//
// Catalog and result formats: include/gc_io.h.  Defaults: 720 bins of 0.25 degrees (every
// separation from 0 to 180 degrees).  Prints the phase times (read, upload, histograms, download,
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

// Device buffers, freed at scope exit.
struct DeviceBuffer {
  void *p = nullptr;
  ~DeviceBuffer() {
    if (p) (void)hipFree(p);
  }
  bool alloc(size_t bytes, const char *what) { return check_hip(hipMalloc(&p, bytes ? bytes : 256), what); }
};

struct PinnedBuffer {
  void *p = nullptr;
  ~PinnedBuffer() {
    if (p) (void)hipHostFree(p);
  }
  bool alloc(size_t bytes) { return check_hip(hipHostMalloc(&p, bytes, hipHostMallocDefault), "pinned host buffer"); }
};

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
  // The HIP runtime takes tens of milliseconds to start; start it on a helper thread while this
  // one parses the catalogs.
  hipStream_t st = nullptr;
  hipError_t init_err = hipSuccess;
  double init_ms = 0.0;
  std::thread init([&] {
    const auto ti = Clock::now();
    init_err = hipStreamCreate(&st);
    init_ms = ms_since(ti);
  });
  auto t0 = Clock::now();
  std::vector<float> ra_d, dec_d, ra_r, dec_r;
  const bool read_ok = read_catalog(pos[0], ra_d, dec_d) && read_catalog(pos[1], ra_r, dec_r);
  const double read_ms = ms_since(t0);
  init.join();
  if (!read_ok || !check_hip(init_err, "hipStreamCreate")) return 1;
  const int64_t n_d = static_cast<int64_t>(ra_d.size()), n_r = static_cast<int64_t>(ra_r.size());

  t0 = Clock::now();
  const gc_stream_t gs = reinterpret_cast<gc_stream_t>(st);
  DeviceBuffer in_d, in_r, prep_d, prep_r, hist, ws, om, tot;
  const size_t fd = static_cast<size_t>(n_d) * sizeof(float), fr = static_cast<size_t>(n_r) * sizeof(float);
  if (!in_d.alloc(2 * fd, "device catalog D") || !in_r.alloc(2 * fr, "device catalog R") ||
      !prep_d.alloc(gc_prepared_bytes(n_d), "prepared D") || !prep_r.alloc(gc_prepared_bytes(n_r), "prepared R") ||
      !hist.alloc(3 * static_cast<size_t>(nbins) * sizeof(uint64_t), "histograms") ||
      !ws.alloc(gc_workspace_bytes(nbins), "workspace") ||
      !om.alloc(static_cast<size_t>(nbins) * sizeof(double), "omega") || !tot.alloc(3 * sizeof(uint64_t), "totals"))
    return 1;
  float *d_ra_d = static_cast<float *>(in_d.p), *d_dec_d = d_ra_d + n_d;
  float *d_ra_r = static_cast<float *>(in_r.p), *d_dec_r = d_ra_r + n_r;
  if (!check_hip(hipMemcpyAsync(d_ra_d, ra_d.data(), fd, hipMemcpyHostToDevice, st), "upload") ||
      !check_hip(hipMemcpyAsync(d_dec_d, dec_d.data(), fd, hipMemcpyHostToDevice, st), "upload") ||
      !check_hip(hipMemcpyAsync(d_ra_r, ra_r.data(), fr, hipMemcpyHostToDevice, st), "upload") ||
      !check_hip(hipMemcpyAsync(d_dec_r, dec_r.data(), fr, hipMemcpyHostToDevice, st), "upload") ||
      !check_hip(hipStreamSynchronize(st), "upload"))
    return 1;
  const double upload_ms = ms_since(t0);

  hipEvent_t e0, e1;
  if (!check_hip(hipEventCreate(&e0), "event") || !check_hip(hipEventCreate(&e1), "event")) return 1;
  uint64_t *dd = static_cast<uint64_t *>(hist.p), *dr = dd + nbins, *rr = dr + nbins;
  t0 = Clock::now();
  if (!check_hip(hipEventRecord(e0, st), "event") ||
      !check(gc_prepare(d_ra_d, d_dec_d, n_d, prep_d.p, gs), "gc_prepare D") ||
      !check(gc_prepare(d_ra_r, d_dec_r, n_r, prep_r.p, gs), "gc_prepare R") ||
      !check(gc_histogram_dd_dr_rr(prep_d.p, n_d, prep_r.p, n_r, nbins, width, dd, dr, rr, ws.p,
                                   gc_workspace_bytes(nbins), gs),
             "gc_histogram_dd_dr_rr") ||
      !check(gc_histogram_totals(dd, dr, rr, nbins, static_cast<uint64_t *>(tot.p), gs), "gc_histogram_totals") ||
      !check(gc_omega(dd, dr, rr, nbins, n_d, n_r, static_cast<double *>(om.p), gs), "gc_omega") ||
      !check_hip(hipEventRecord(e1, st), "event") || !check_hip(hipStreamSynchronize(st), "histograms"))
    return 1;
  float gpu_ms = 0.0f;
  (void)hipEventElapsedTime(&gpu_ms, e0, e1);
  const double hist_wall_ms = ms_since(t0);

  t0 = Clock::now();
  // one pinned host block for everything that comes back: histograms, totals, omega
  const size_t hbytes = (3 * static_cast<size_t>(nbins) + 3) * sizeof(uint64_t) + static_cast<size_t>(nbins) * 8;
  PinnedBuffer back;
  if (!back.alloc(hbytes)) return 1;
  uint64_t *h = static_cast<uint64_t *>(back.p), *totals = h + 3 * static_cast<size_t>(nbins);
  double *omega = reinterpret_cast<double *>(totals + 3);
  if (!check_hip(hipMemcpyAsync(h, dd, 3 * static_cast<size_t>(nbins) * sizeof(uint64_t), hipMemcpyDeviceToHost, st),
                 "download") ||
      !check_hip(hipMemcpyAsync(totals, tot.p, 3 * sizeof(uint64_t), hipMemcpyDeviceToHost, st), "download") ||
      !check_hip(hipMemcpyAsync(omega, om.p, static_cast<size_t>(nbins) * sizeof(double), hipMemcpyDeviceToHost, st),
                 "download") ||
      !check_hip(hipStreamSynchronize(st), "download"))
    return 1;
  const double download_ms = ms_since(t0);
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
  (void)hipStreamDestroy(st);

  if (!quiet) {
    const double ordered = static_cast<double>(want[0]) + static_cast<double>(want[1]) + static_cast<double>(want[2]);
    printf("galaxy_gc: %" PRId64 " + %" PRId64 " galaxies, %d bins of %g deg\n", n_d, n_r, nbins, width);
    printf("  sums   DD %" PRIu64 "  DR %" PRIu64 "  RR %" PRIu64 " (exact)\n", totals[0], totals[1], totals[2]);
    printf("  read %.2f ms (HIP start-up %.2f ms alongside) | upload %.2f ms | histograms %.3f ms (GPU events; "
           "%.3f ms wall) | download %.2f ms | write %.2f ms | total %.2f ms\n",
           read_ms, init_ms, upload_ms, gpu_ms, hist_wall_ms, download_ms, write_ms, total_ms);
    printf("  %.3e ordered pairs/s on the GPU\n", ordered / (gpu_ms / 1e3));
  }
  return 0;
}
