/* Exhaustive FP32 -> FP8 cross-check: a second FP8 encoder that shares no
 * logic with the oracle's (nearest value by binary search over the sorted
 * table of finite magnitudes, ties to the code whose mantissa LSB is 0,
 * magnitudes above the largest value saturate, NaN -> the canonical NaN code
 * 0xFF for E4M3 / 0xFE for E5M2), run over
 * every FP32 bit pattern in [lo, hi) against the oracle's encoder, which is
 * passed in as a function pointer.  Returns the number of mismatches and the
 * first mismatching pattern. */
#include <math.h>
#include <stdint.h>
#include <string.h>

typedef uint8_t (*enc_fn)(float, int);

static uint8_t nearest(float f, const double* v, const uint8_t* c, int n, uint8_t nan_code) {
  uint32_t u;
  memcpy(&u, &f, 4);
  uint8_t sign = (uint8_t)((u >> 31) << 7);
  if (isnan(f)) return nan_code;
  double a = fabs((double)f);
  if (a >= v[n - 1]) return sign | c[n - 1];
  int lo = 0, hi = n - 1;            /* v[lo] <= a < v[hi] */
  while (hi - lo > 1) {
    int mid = (lo + hi) / 2;
    if (v[mid] <= a) lo = mid; else hi = mid;
  }
  double dl = a - v[lo], dh = v[hi] - a;
  if (dl < dh) return sign | c[lo];
  if (dh < dl) return sign | c[hi];
  return sign | ((c[lo] & 1) == 0 ? c[lo] : c[hi]);
}

int64_t fp8_sweep(uint64_t lo, uint64_t hi, int fmt, const double* vals, const uint8_t* codes,
                  int n, void* fn, uint64_t* first_bad) {
  enc_fn enc = (enc_fn)fn;
  int64_t bad = 0;
  uint64_t first = ~0ull;
#pragma omp parallel for schedule(static, 1 << 16) reduction(+ : bad) reduction(min : first)
  for (int64_t i = 0; i < (int64_t)(hi - lo); ++i) {
    uint32_t u = (uint32_t)(lo + (uint64_t)i);
    float f;
    memcpy(&f, &u, 4);
    if (enc(f, fmt) != nearest(f, vals, codes, n, fmt == 0 ? 0xFF : 0xFE)) {
      bad += 1;
      if ((uint64_t)u < first) first = u;
    }
  }
  *first_bad = first;
  return bad;
}
