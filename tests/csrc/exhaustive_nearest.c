/* Exhaustive check, over every fp32 x in [-1, 1], that counting the
 * thresholds below x picks the nearest NF4 level with ties to the lower
 * index.  The nearest level is found by the definition: the smallest
 * |x - level| (exact in double for the magnitudes where ties can occur),
 * first index on a tie.  Returns the number of mismatches and writes the
 * first mismatching bit pattern to *first_bad. */
#include <math.h>
#include <stdint.h>
#include <string.h>

static float from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

long nearest_mismatches(const float* levels, const float* thr, uint32_t* first_bad) {
  long bad = 0;
  uint32_t first = 0xffffffffu;
  const int64_t top = 0x3F800000; /* bit pattern of 1.0f */
#pragma omp parallel for reduction(+ : bad) schedule(static, 1 << 20)
  for (int64_t u = 0; u <= top; ++u) {
    for (int sgn = 0; sgn < 2; ++sgn) {
      const uint32_t bits = (uint32_t)u | ((uint32_t)sgn << 31);
      const float x = from_bits(bits);
      int best = 0;
      double bd = fabs((double)x - (double)levels[0]);
      for (int i = 1; i < 16; ++i) {
        const double d = fabs((double)x - (double)levels[i]);
        if (d < bd) { bd = d; best = i; }
      }
      int c = 0;
      for (int i = 0; i < 15; ++i) c += (x > thr[i]);
      if (c != best) {
        ++bad;
#pragma omp critical
        { if (bits < first) first = bits; }
      }
    }
  }
  *first_bad = first;
  return bad;
}

/* The same check for a code table in any code order (FP4 has +0 and -0 and
 * descending negative codes): the distinct values are sorted, and counting
 * the nthr thresholds below x must give the index of the nearest distinct
 * value, ties to the lower value. */
long nearest_value_mismatches(const float* values16, const float* thr, int nthr,
                              uint32_t* first_bad) {
  double dist[16];
  int nd = 0;
  for (int i = 0; i < 16; ++i) {
    const double v = (double)values16[i];
    int seen = 0;
    for (int j = 0; j < nd; ++j) seen |= (dist[j] == v);
    if (!seen) dist[nd++] = v;
  }
  for (int i = 1; i < nd; ++i) /* insertion sort, ascending */
    for (int j = i; j > 0 && dist[j - 1] > dist[j]; --j) {
      const double t = dist[j]; dist[j] = dist[j - 1]; dist[j - 1] = t;
    }
  if (nthr != nd - 1) { *first_bad = 0xfffffffeu; return -1; }
  long bad = 0;
  uint32_t first = 0xffffffffu;
  const int64_t top = 0x3F800000;
#pragma omp parallel for reduction(+ : bad) schedule(static, 1 << 20)
  for (int64_t u = 0; u <= top; ++u) {
    for (int sgn = 0; sgn < 2; ++sgn) {
      const uint32_t bits = (uint32_t)u | ((uint32_t)sgn << 31);
      const float x = from_bits(bits);
      int best = 0;
      double bd = fabs((double)x - dist[0]);
      for (int i = 1; i < nd; ++i) {
        const double d = fabs((double)x - dist[i]);
        if (d < bd) { bd = d; best = i; }
      }
      int c = 0;
      for (int i = 0; i < nthr; ++i) c += (x > thr[i]);
      if (c != best) {
        ++bad;
#pragma omp critical
        { if (bits < first) first = bits; }
      }
    }
  }
  *first_bad = first;
  return bad;
}
