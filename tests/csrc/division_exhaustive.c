/* Complete check of the quotient the quantizer uses for blocks with absmax
 * b in [2^-60, 2^126]: from r = fl32(1/b), q = fl32(a r), e = fma(-q, b, a),
 * q' = fma(e, r, q).  Its code must equal the code of the IEEE quotient
 * fl32(a/b) for every |a| <= b.
 *
 * Why checking near the thresholds is enough:
 *  - r has relative error <= 2^-24 and q <= about 2^-23, so q is within two
 *    ulps of a/b, and e is a/b - q times b up to a relative 2^-24 (the
 *    residual has at most 25 significant bits).  Then q + e r (exact inside
 *    the fma) is a/b up to 2^-22 ulp, and q' is a/b rounded to one of its
 *    two fp32 neighbours: |q' - fl32(a/b)| <= 1 ulp.
 *  - Codes compare the quotient with fp32 thresholds T (x > T).  Two fp32
 *    values at most one ulp apart give different answers only if T is the
 *    lower of them, i.e. only if fl32(a/b) lies within one ulp of T.
 * Why one binade of b is enough: multiplying a and b by 2^k multiplies r by
 * 2^-k, leaves q unchanged and multiplies e by 2^k, exactly, as long as no
 * intermediate leaves the normal range.  For quotients near a threshold
 * (|q| >= 2^-5) and 2^-60 <= b <= 2^126, r >= 2^-126 and every nonzero
 * residual is a multiple of 2^(-5-60-46) = 2^-111: all normal.  So the
 * outcome for (a, b) is the outcome for (a 2^-k, b 2^-k) with b 2^-k in
 * [1, 2), and the quotient is the same.
 *
 * The check: every b in [1, 2) (all 2^23 mantissas), every threshold
 * magnitude T given (both signs follow by symmetry: every step is odd in a),
 * and every a whose IEEE quotient lies within 4 ulps of T: q' must equal
 * fl32(a/b) bit for bit.  Returns the number of (a, b) pairs that differ;
 * *first gets the first one as bit patterns, *checked the pairs tested. */
#include <math.h>
#include <stdint.h>
#include <string.h>

static float fb(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t bf(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

long division_exhaustive(const float* thr, int nthr, uint32_t* first, long* checked) {
  long bad = 0, total = 0;
  first[0] = first[1] = 0;
#pragma omp parallel for schedule(static, 4096) reduction(+ : bad, total)
  for (long m = 0; m < (1L << 23); ++m) {
    const float b = fb(0x3f800000u | (uint32_t)m);
    volatile float vb = b;
    const float r = 1.0f / vb;
    for (int t = 0; t < nthr; ++t) {
      const float T = fabsf(thr[t]);
      const uint32_t tb = bf(T);
      const float lo = fb(tb - 4), hi = fb(tb + 4);  /* T -/+ 4 ulps */
      /* dividends around T b: consecutive a move the quotient by at most
       * one ulp of T (a is in T's binade or the next one), so 12 each side
       * cover the window */
      const uint32_t a0 = bf((float)((double)T * (double)b));
      for (int k = -12; k <= 12; ++k) {
        const float a = fb(a0 + (uint32_t)k);
        if (!(a <= b)) continue;
        volatile float va = a;
        const float ieee = va / vb;
        if (ieee < lo || ieee > hi) continue;
        if (k == -12 || k == 12) {  /* the window was not covered */
#pragma omp critical
          if (!first[0] && !first[1]) { first[0] = bf(a); first[1] = bf(b); }
          ++bad;
        }
        const float q = va * r;
        const float e = fmaf(-q, vb, va);
        const float q2 = fmaf(e, r, q);
        ++total;
        if (bf(q2) != bf(ieee)) {
#pragma omp critical
          if (!first[0] && !first[1]) { first[0] = bf(a); first[1] = bf(b); }
          ++bad;
        }
      }
    }
  }
  *checked = total;
  return bad;
}
