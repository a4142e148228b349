/* Host check of the quantizer's bucket rule for a threshold table: buckets
 * split [-1, 1] by sign, binary exponent 2^-6 .. 2^0 and the top 4 mantissa
 * bits, with one bucket per sign for |x| < 2^-6 (1 + 1/16).  Each bucket
 * stores the number of thresholds below all of it and the (at most one)
 * threshold inside it; the count of thresholds below x must equal
 * base + (x > inside) for every fp32 x in [-1, 1].  Returns the number of
 * mismatches (-1 if some bucket holds two thresholds); *first_bad gets the
 * first failing bit pattern. */
#include <math.h>
#include <stdint.h>
#include <string.h>

static float from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

long bucket_mismatches(const float* thr, int nthr, uint32_t* first_bad) {
  float inside[224];
  int base[224];
  for (int t = 0; t < 224; ++t) {
    const int sg = t / 112, ke = (t % 112) / 16, j = t % 16;
    const double lo = (ke == 0 && j == 0) ? 0.0 : ldexp(1.0 + j / 16.0, ke - 6);
    const double hi = ldexp(1.0 + (j + 1) / 16.0, ke - 6);
    int nin = 0;
    base[t] = 0;
    inside[t] = INFINITY;
    for (int i = 0; i < nthr; ++i) {
      const double T = thr[i];
      const int below = sg == 0 ? T < lo : T <= -hi;
      const int in = sg == 0 ? (T >= lo && T < hi) : (T > -hi && T <= -lo);
      base[t] += below;
      if (in) { inside[t] = thr[i]; ++nin; }
    }
    if (nin > 1) { *first_bad = (uint32_t)t; return -1; }
  }
  long bad = 0;
  uint32_t first = 0xffffffffu;
  const int64_t top = 0x3F800000;
#pragma omp parallel for reduction(+ : bad) schedule(static, 1 << 20)
  for (int64_t u = 0; u <= top; ++u) {
    for (int sgn = 0; sgn < 2; ++sgn) {
      const uint32_t bits = (uint32_t)u | ((uint32_t)sgn << 31);
      const float x = from_bits(bits);
      int direct = 0;
      for (int i = 0; i < nthr; ++i) direct += x > thr[i];
      const int e = (int)((bits >> 23) & 0xff);
      const int key = e < 121 ? sgn * 112 : sgn * 112 + (e - 121) * 16 + (int)((bits >> 19) & 15);
      const int got = base[key] + (x > inside[key]);
      if (got != direct) {
        ++bad;
#pragma omp critical
        { if (bits < first) first = bits; }
      }
    }
  }
  *first_bad = first;
  return bad;
}
