// Host-side text input and output of the end-to-end program: the memory-mapped catalog reader
// and the result writer of "CUDA Deep Dive: 10B Galaxy Pairs on an RTX 5080" (section "mmap +
// hand-rolled parser vs. fscanf" and the appendix listing).  The file formats are stated in
// include/gc_io.h.  The number parser is this file's own: it collects up to 19 significant
// digits and a decimal exponent, converts exactly-representable cases with one correctly
// rounded multiplication or division by a power of ten (Clinger's fast path), and hands every
// other token to strtod; the double is then narrowed to float.
#include <errno.h>
#include <fcntl.h>
#include <inttypes.h>
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include <sys/mman.h>
#include <sys/stat.h>
#include <unistd.h>

#include <string>

#include "../../include/gc_io.h"

namespace gc {
namespace {

// 10^0 .. 10^22: every one is exactly representable as a double.
constexpr double kPow10[23] = {1e0,  1e1,  1e2,  1e3,  1e4,  1e5,  1e6,  1e7,  1e8,  1e9,  1e10, 1e11,
                               1e12, 1e13, 1e14, 1e15, 1e16, 1e17, 1e18, 1e19, 1e20, 1e21, 1e22};

inline bool is_space(char c) { return c == ' ' || c == '\n' || c == '\r' || c == '\t' || c == '\v' || c == '\f'; }
inline bool is_digit(char c) { return c >= '0' && c <= '9'; }

struct Cursor {
  const char *p, *end;
  void skip_space() {
    while (p < end && is_space(*p)) ++p;
  }
  bool at_token_end() const { return p >= end || is_space(*p); }
};

// A read-only private mapping of a whole file; unmapped on destruction.
struct MappedFile {
  const char *data = nullptr;
  size_t size = 0;
  bool ok = false;
  explicit MappedFile(const char *path) {
    const int fd = open(path, O_RDONLY | O_CLOEXEC);
    if (fd < 0) return;
    struct stat st;
    if (fstat(fd, &st) != 0 || !S_ISREG(st.st_mode)) {
      close(fd);
      return;
    }
    size = static_cast<size_t>(st.st_size);
    if (size > 0) {
      void *m = mmap(nullptr, size, PROT_READ, MAP_PRIVATE, fd, 0);
      if (m == MAP_FAILED) {
        close(fd);
        size = 0;
        return;
      }
      madvise(m, size, MADV_SEQUENTIAL);
      data = static_cast<const char *>(m);
    }
    close(fd);
    ok = true;
  }
  ~MappedFile() {
    if (data) munmap(const_cast<char *>(data), size);
  }
  MappedFile(const MappedFile &) = delete;
  MappedFile &operator=(const MappedFile &) = delete;
};

// Leading count: [+|-]digits, followed by whitespace or the end of the file.
bool parse_count(Cursor &c, int64_t *out) {
  c.skip_space();
  bool neg = false;
  if (c.p < c.end && (*c.p == '+' || *c.p == '-')) {
    neg = *c.p == '-';
    ++c.p;
  }
  if (c.p >= c.end || !is_digit(*c.p)) return false;
  int64_t v = 0;
  while (c.p < c.end && is_digit(*c.p)) {
    const int d = *c.p - '0';
    if (v > (INT64_MAX - d) / 10) return false;
    v = v * 10 + d;
    ++c.p;
  }
  if (!c.at_token_end()) return false;
  *out = neg ? -v : v;
  return true;
}

// One number of the catalog grammar, converted to the nearest double.
bool parse_number(Cursor &c, double *out) {
  c.skip_space();
  const char *const start = c.p;
  bool neg = false;
  if (c.p < c.end && (*c.p == '+' || *c.p == '-')) {
    neg = *c.p == '-';
    ++c.p;
  }
  uint64_t mant = 0;   // first 19 significant digits
  int kept = 0;        // significant digits in mant
  int64_t e10 = 0;     // decimal exponent of mant's last digit
  bool exact = true;   // no non-zero digit was dropped
  bool any = false;
  while (c.p < c.end && is_digit(*c.p)) {
    const int d = *c.p++ - '0';
    any = true;
    if (kept == 0 && d == 0) continue;
    if (kept < 19) {
      mant = mant * 10 + static_cast<uint64_t>(d);
      ++kept;
    } else {
      ++e10;
      exact = exact && d == 0;
    }
  }
  if (c.p < c.end && *c.p == '.') {
    ++c.p;
    while (c.p < c.end && is_digit(*c.p)) {
      const int d = *c.p++ - '0';
      any = true;
      if (kept == 0 && d == 0) {
        --e10;
        continue;
      }
      if (kept < 19) {
        mant = mant * 10 + static_cast<uint64_t>(d);
        ++kept;
        --e10;
      } else {
        exact = exact && d == 0;
      }
    }
  }
  if (!any) return false;
  if (c.p < c.end && (*c.p == 'e' || *c.p == 'E')) {
    ++c.p;
    bool eneg = false;
    if (c.p < c.end && (*c.p == '+' || *c.p == '-')) {
      eneg = *c.p == '-';
      ++c.p;
    }
    if (c.p >= c.end || !is_digit(*c.p)) return false;
    int64_t ex = 0;
    while (c.p < c.end && is_digit(*c.p)) {
      if (ex < 1000000) ex = ex * 10 + (*c.p - '0');
      ++c.p;
    }
    e10 += eneg ? -ex : ex;
  }
  if (!c.at_token_end()) return false;
  if (mant == 0) {
    *out = neg ? -0.0 : 0.0;
    return true;
  }
  if (exact && mant <= (1ull << 53) && e10 >= -22 && e10 <= 22) {
    const double m = static_cast<double>(mant);
    const double v = e10 < 0 ? m / kPow10[-e10] : m * kPow10[e10];
    *out = neg ? -v : v;
    return true;
  }
  // everything else: the C library's correctly rounded conversion of the same token
  const std::string tok(start, static_cast<size_t>(c.p - start));
  char *endp = nullptr;
  errno = 0;
  const double v = strtod(tok.c_str(), &endp);
  if (endp != tok.c_str() + tok.size()) return false;
  *out = v;
  return true;
}

}  // namespace
}  // namespace gc

using namespace gc;

extern "C" {

gc_status gc_catalog_count(const char *path, int64_t *n_out) {
  if (!path || !n_out) return GC_ERR_INVALID_ARGUMENT;
  MappedFile f(path);
  if (!f.ok) return GC_ERR_IO;
  Cursor c{f.data, f.data + f.size};
  int64_t n = 0;
  if (!parse_count(c, &n) || n < 0) return GC_ERR_IO;
  if (n > GC_MAX_GALAXIES) return GC_ERR_UNSUPPORTED;
  *n_out = n;
  return GC_OK;
}

gc_status gc_catalog_read(const char *path, float *ra, float *dec, int64_t capacity, int64_t *n_out) {
  if (!path || !n_out || capacity < 0) return GC_ERR_INVALID_ARGUMENT;
  MappedFile f(path);
  if (!f.ok) return GC_ERR_IO;
  Cursor c{f.data, f.data + f.size};
  int64_t n = 0;
  if (!parse_count(c, &n) || n < 0) return GC_ERR_IO;
  if (n > GC_MAX_GALAXIES) return GC_ERR_UNSUPPORTED;
  *n_out = n;
  if (n > capacity || (n > 0 && (!ra || !dec))) return GC_ERR_INVALID_ARGUMENT;
  for (int64_t i = 0; i < n; ++i) {
    double a, d;
    if (!parse_number(c, &a) || !parse_number(c, &d)) return GC_ERR_IO;
    const float af = static_cast<float>(a), df = static_cast<float>(d);
    if (!isfinite(af) || !isfinite(df)) return GC_ERR_IO;
    ra[i] = af;
    dec[i] = df;
  }
  c.skip_space();
  if (c.p != c.end) return GC_ERR_IO;
  return GC_OK;
}

gc_status gc_omega_write(const char *path, const uint64_t *dd, const uint64_t *dr, const uint64_t *rr,
                         const double *omega, int32_t nbins, double w_deg) {
  if (!path || !dd || !dr || !rr || !omega || nbins <= 0 || !(w_deg > 0.0) || !isfinite(w_deg))
    return GC_ERR_INVALID_ARGUMENT;
  FILE *out = fopen(path, "w");
  if (!out) return GC_ERR_IO;
  bool ok = fputs("bin start\t\tomega\t        hist_DD\t        hist_DR\t        hist_RR\n", out) >= 0;
  for (int32_t k = 0; ok && k < nbins; ++k) {
    if (rr[k] == 0) continue;
    ok = fprintf(out, "%6.3f\t%15f\t%15" PRIu64 "\t%15" PRIu64 "\t%15" PRIu64 "\n", static_cast<double>(k) * w_deg,
                 omega[k], dd[k], dr[k], rr[k]) > 0;
  }
  ok = (fclose(out) == 0) && ok;
  return ok ? GC_OK : GC_ERR_IO;
}

}  // extern "C"
