/* Host check of the division refinement the quantizer uses for blocks with
 * absmax b >= 2^-80: from r = fl32(1/b), q = fl32(a r), e = fma(-q, b, a),
 * q' = fma(e, r, q) equals the IEEE quotient fl32(a/b) whenever
 * 0.01 <= |a/b| <= 1 (the range in which a code can depend on the last bit
 * of the quotient; every threshold has magnitude >= 0.0398).  Random b over
 * all exponents >= -80, quotients spread over [0.01, 1] with perturbed last
 * bits, both signs.  Returns the number of mismatches; *first gets the
 * first failing (a, b) pair as bit patterns. */
#include <math.h>
#include <stdint.h>
#include <string.h>

static float fb(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t bf(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

long division_mismatches(long samples, uint64_t seed, uint32_t* first) {
  uint64_t s = seed | 1;
  long bad = 0;
  const float bmin = ldexpf(1.0f, -80);
  first[0] = first[1] = 0;
  for (long n = 0; n < samples;) {
    s ^= s << 13; s ^= s >> 7; s ^= s << 17;
    const uint32_t bu = (uint32_t)s & 0x7fffffffu;
    if ((bu >> 23) == 255) continue;
    const float b = fb(bu);
    if (!(b >= bmin)) continue;
    s ^= s << 13; s ^= s >> 7; s ^= s << 17;
    const uint32_t tu = 0x3c23d70au + (uint32_t)((s >> 8) % (0x3f800000u - 0x3c23d70au + 1));
    float a = b * fb(tu);
    a = fb(bf(a) ^ (uint32_t)(s & 7u));
    if (!(fabsf(a) <= b)) a = b;
    if (s & 8u) a = -a;
    volatile float va = a, vb = b;
    const float ieee = va / vb;
    const float r = 1.0f / vb;
    const float q = va * r;
    const float e = fmaf(-q, vb, va);
    const float q2 = fmaf(e, r, q);
    ++n;
    if (bf(q2) != bf(ieee)) {
      if (!bad) { first[0] = bf(a); first[1] = bu; }
      ++bad;
    }
  }
  return bad;
}
