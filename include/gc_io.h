/*
 * gc_io.h -- host-side text input and output of the page's end-to-end program
 * ("CUDA Deep Dive: 10B Galaxy Pairs on an RTX 5080", sections "mmap + hand-rolled
 * parser vs. fscanf" and the appendix listing's catalog reader and result writer).
 *
 * Catalog file format (the page's input files): the number of galaxies N as a
 * decimal integer, then N pairs "alpha delta" of decimal numbers in arcminutes,
 * all separated by ASCII whitespace (one pair per line in practice).  Numbers are
 * [+|-]digits[.digits][(e|E)[+|-]digits] with at least one mantissa digit (".5"
 * and "5." are accepted).  Each value is converted to the nearest double and then
 * narrowed to the nearest float (the page's reader also parses in double before
 * narrowing; this one rounds correctly at the first step).  Anything after the
 * 2N numbers other than whitespace is an error, as is a short file.
 *
 * Result file format (the page's omega.out): one header line, then for every bin
 * with RR > 0 a line "%6.3f\t%15f\t%15llu\t%15llu\t%15llu\n" of the bin's lower
 * edge in degrees, omega, DD, DR and RR.  The layout is kept identical to the
 * page's so that its outputs and these can be compared byte for byte; omega here
 * is the fp64 value of gc_omega.
 *
 * All pointers in this header are HOST pointers.  Files are memory-mapped for
 * reading.  Thread-safe; nothing is cached between calls.
 */
#ifndef GC_IO_H_
#define GC_IO_H_

#include "gc.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Galaxy count N of a catalog file (its first token).  *n_out is set on success.
 * Errors: GC_ERR_INVALID_ARGUMENT (null pointer), GC_ERR_IO (cannot open or map the
 * file, no leading integer, N < 0), GC_ERR_UNSUPPORTED (N > GC_MAX_GALAXIES). */
gc_status gc_catalog_count(const char *path, int64_t *n_out);

/* Read a whole catalog into host arrays of `capacity` floats each (alpha, delta in
 * arcminutes, in file order).  *n_out = N on success, and also when capacity < N
 * (then GC_ERR_INVALID_ARGUMENT is returned and nothing is written).
 * Errors: GC_ERR_INVALID_ARGUMENT (null pointer, capacity < N), GC_ERR_IO (cannot
 * open or map the file, a malformed or missing number, trailing non-whitespace),
 * GC_ERR_UNSUPPORTED (N > GC_MAX_GALAXIES).  On error the arrays may hold a prefix of
 * the values. */
gc_status gc_catalog_read(const char *path, float *ra_arcmin, float *dec_arcmin, int64_t capacity,
                          int64_t *n_out);

/* Write the result file for nbins bins of width bin_width_deg from host arrays dd, dr,
 * rr (uint64[nbins]) and omega (double[nbins]).  Replaces the file.
 * Errors: GC_ERR_INVALID_ARGUMENT (null pointer, nbins <= 0, width <= 0 or not finite),
 * GC_ERR_IO (cannot create or write the file). */
gc_status gc_omega_write(const char *path, const uint64_t *dd, const uint64_t *dr, const uint64_t *rr,
                         const double *omega, int32_t nbins, double bin_width_deg);

#ifdef __cplusplus
}
#endif

#endif /* GC_IO_H_ */
