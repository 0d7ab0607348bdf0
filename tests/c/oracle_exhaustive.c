/*
 * Exhaustive check of the oracle's two conversions (test infrastructure):
 *   e2m1  every fp32 bit pattern except NaN, both signs;
 *   e4m3  every non-negative fp32 bit pattern from +0 to +inf.
 * Each result of oracle_e2m1_encode / oracle_e4m3_encode (linked from the
 * built oracle library) is compared with a nearest-value search written
 * here from the format definitions alone: the table of representable values,
 * a binary search for the neighbours of the input, the nearer one chosen
 * with the distances computed exactly in double, a tie going to the even
 * code, and saturation at the largest finite value (6 for E2M1, 448 = code
 * 0x7E for E4M3FN).  Prints the count of mismatches and the first few;
 * exits 0 only if there are none.
 *
 *   usage: oracle_exhaustive e2m1|e4m3
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

extern int oracle_e2m1_encode(float v);
extern int oracle_e4m3_encode(float t);

static double e2m1_tab[8];
static double e4m3_tab[127];

static float from_bits(uint32_t b) {
  float f;
  memcpy(&f, &b, sizeof f);
  return f;
}

/* index of the nearest table value to a (0 <= a < tab[n-1]), ties to even */
static int nearest(const double* tab, int n, double a) {
  int lo = 0, hi = n - 1; /* tab[lo] <= a < tab[hi] */
  while (hi - lo > 1) {
    const int mid = (lo + hi) / 2;
    if (tab[mid] <= a) lo = mid; else hi = mid;
  }
  const double dlo = a - tab[lo], dhi = tab[hi] - a; /* exact: both fit in double */
  if (dlo < dhi) return lo;
  if (dhi < dlo) return hi;
  return (lo % 2 == 0) ? lo : hi;
}

static int ref_e2m1(float v) {
  const int sign = signbit(v) ? 8 : 0;
  const double a = fabs((double)v);
  if (a >= 6.0) return sign | 7;
  return sign | nearest(e2m1_tab, 8, a);
}

static int ref_e4m3(float t) {
  const double a = (double)t;
  if (a >= 448.0) return 0x7E;
  return nearest(e4m3_tab, 127, a);
}

int main(int argc, char** argv) {
  if (argc != 2 || (strcmp(argv[1], "e2m1") && strcmp(argv[1], "e4m3"))) {
    fprintf(stderr, "usage: %s e2m1|e4m3\n", argv[0]);
    return 2;
  }
  const double grid[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
  for (int c = 0; c < 8; ++c) e2m1_tab[c] = grid[c];
  for (int c = 0; c < 127; ++c) {
    const int e = c >> 3, f = c & 7;
    e4m3_tab[c] = e ? ldexp(1.0 + f / 8.0, e - 7) : ldexp((double)f, -9);
  }
  const int e2m1 = strcmp(argv[1], "e2m1") == 0;
  /* e2m1: all 2^32 patterns (NaN skipped); e4m3: +0 .. +inf */
  const int64_t n = e2m1 ? ((int64_t)1 << 32) : (int64_t)0x7F800000 + 1;
  int64_t bad = 0, checked = 0;
  int shown = 0;
#pragma omp parallel for schedule(static, 1 << 20) reduction(+ : bad, checked)
  for (int64_t i = 0; i < n; ++i) {
    const uint32_t b = (uint32_t)i;
    const float v = from_bits(b);
    if (isnan(v)) continue;
    ++checked;
    const int got = e2m1 ? oracle_e2m1_encode(v) : oracle_e4m3_encode(v);
    const int want = e2m1 ? ref_e2m1(v) : ref_e4m3(v);
    if (got != want) {
      ++bad;
#pragma omp critical
      if (shown < 8) {
        printf("mismatch: bits 0x%08x (%a) oracle %d search %d\n", b, (double)v, got, want);
        ++shown;
      }
    }
  }
  printf("%s: %lld patterns checked, %lld mismatches, %d threads\n", argv[1], (long long)checked,
         (long long)bad, omp_get_max_threads());
  return bad == 0 ? 0 : 1;
}
