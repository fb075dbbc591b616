// The noise kernel's fp32 log, retyped for the host, against the fp64 libm
// log rounded once to fp32 (the definition the noise uses), over every input
// the Gumbel noise can present: u = (2k + 1) 2^-24 for k < 2^23 and -ln(u).
// Also a strided sweep of fp32 values in [2^-30, 2^30).  Prints the counts,
// and the largest error of the fast path's fp64 value over the noise inputs
// in its own ulps (against the 80-bit long double log).
// Built with g++ -O2 -ffp-contract=off; fma() is the correctly rounded one.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#define __constant__ static const
#include "../markov_bias_chain_amd/csrc/log_table.inc"

static float asf(uint32_t b) { float f; std::memcpy(&f, &b, 4); return f; }
static uint32_t asu(float f) { uint32_t b; std::memcpy(&b, &f, 4); return b; }
static float ref_log(float x) { return (float)std::log((double)x); }
static long fallbacks = 0;
static bool list_fallbacks = false;  // print the inputs the fast path leaves to the library

static int asi(float f) { int b; std::memcpy(&b, &f, 4); return b; }

// Same operations, same order, as the kernel: x = m 2^e from the bit pattern,
// the bucket from the fp32 rounding of m 128 + 1.5 2^23 - 90, r = m c - 1 in
// fp64, ln(1 + r) by Horner in fp64, + e ln2 - ln c, and the test of the 29
// bits below fp32 precision against the rounding midpoint, with the library
// log when it fails.
static double fast_log_y(float x) {
  const uint32_t b = asu(x);
  const int e = (int)(b - 0x3F3504F3u) >> 23;
  const float m = asf(b - ((uint32_t)e << 23));
  const float f = std::fmaf(m, 128.0f, 12582822.0f);
  const LogEntry te = g_log_tab[asi(f) - 0x4B400000];
  const double r = std::fma((double)m, te.c, -1.0);
  double q = std::fma(r, 0.2, -0.25);
  q = std::fma(r, q, 1.0 / 3.0);
  q = std::fma(r, q, -0.5);
  const double lp = std::fma(r * r, q, r);
  return std::fma((double)e, 0x1.62e42fefa39efp-1, te.nlc + lp);
}

static float fast_log(float x) {
  const double y = fast_log_y(x);
  uint64_t yb;
  std::memcpy(&yb, &y, 8);
  const uint32_t low = (uint32_t)yb & 0x1FFFFFFFu;
  if (low - ((1u << 28) - (1u << 12)) > (1u << 13)) return (float)y;
  ++fallbacks;
  if (list_fallbacks) std::printf("%08x\n", asu(x));
  return ref_log(x);
}

// |y - ln x| in ulps of y, against the 80-bit library log.  Below 2^12 ulps
// the midpoint test above is sound on its own: y and ln x then lie on the
// same side of every rounding midpoint that y is more than 2^12 ulps from.
static double max_ulps = 0.0;
static void track_error(float x) {
  const double y = fast_log_y(x);
  const long double t = logl((long double)x);
  if (y == 0.0) return;
  const double ulp = std::ldexp(1.0, std::ilogb(y) - 52);
  const double err = (double)fabsl((long double)y - t) / ulp;
  if (err > max_ulps) max_ulps = err;
}

int main(int argc, char** argv) {
  // --list: only print (one hex bit pattern per line) the noise inputs on
  // which the fast path could not decide the rounding.
  if (argc > 1 && std::strcmp(argv[1], "--list") == 0) {
    list_fallbacks = true;
    for (uint32_t k = 0; k < (1u << 23); ++k) {
      const float u = (float)(2u * k + 1u) * 0x1p-24f;
      fast_log(-fast_log(u));
    }
    return 0;
  }
  long n = 0, bad = 0;
  for (uint32_t k = 0; k < (1u << 23); ++k) {
    const float u = (float)(2u * k + 1u) * 0x1p-24f;
    const float a = ref_log(u);
    bad += asu(fast_log(u)) != asu(a);
    bad += asu(fast_log(-a)) != asu(ref_log(-a));
    n += 2;
    track_error(u);
    track_error(-a);
  }
  const long noise_fallbacks = fallbacks;
  long n2 = 0, bad2 = 0;
  for (uint32_t b = asu(0x1p-30f); b < asu(0x1p30f); b += 7, ++n2)
    bad2 += asu(fast_log(asf(b))) != asu(ref_log(asf(b)));
  std::printf("noise %ld %ld %ld sweep %ld %ld %ld ulps %.1f\n", n, bad, noise_fallbacks, n2, bad2,
              fallbacks - noise_fallbacks, max_ulps);
  return 0;
}
