// Host-side constant tables of libqlora, derived once per codebook from the
// definition of its level set.
//
// Level sets ("LLMs · QLoRA", NormalFloat paragraph and its code listing):
// * NF4: 16 normal quantiles at evenly spaced probabilities in [0.02, 0.98],
//   divided by the largest magnitude.  Each quantile is found in double
//   precision by bisection on the normal CDF Phi(x) = erfc(-x/sqrt 2)/2, and
//   the normalised value is rounded to fp32 once.
// * uniform 4-bit (the comparison grid of the same write-up): 16 evenly
//   spaced values from -1 to 1, each computed in double and rounded to fp32
//   once.
//
// Encoder thresholds: the listing picks the level nearest to x = w/absmax by
// an argmin of |x - L_i| in fp32, the first minimum winning.  For x between
// L_i and L_{i+1} only those two levels can win (every other level is at
// least one level gap, > 0.07, farther), and "L_{i+1} wins" is a monotone
// predicate of x, so the whole rule is code = #{j : x >= T_j} for 15 fp32
// thresholds T_1..T_15.  Each T_j is found exactly by bisection over the
// ordered fp32 values between L_{j-1} and L_j with the same fp32 arithmetic.

#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "internal.h"

namespace qlora {
namespace {

double normal_cdf(double x) { return 0.5 * std::erfc(-x / std::sqrt(2.0)); }

// Phi^-1(p) by bisection to the resolution of double.
double normal_quantile(double p) {
  double lo = -40.0, hi = 40.0;
  for (int it = 0; it < 4000; ++it) {
    double mid = 0.5 * (lo + hi);
    if (mid <= lo || mid >= hi) break;
    if (normal_cdf(mid) < p)
      lo = mid;
    else
      hi = mid;
  }
  double dlo = std::fabs(normal_cdf(lo) - p), dhi = std::fabs(normal_cdf(hi) - p);
  return dlo <= dhi ? lo : hi;
}

uint32_t f2u(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return u;
}
float u2f(uint32_t u) {
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

// Monotone map fp32 -> uint32 (total order on finite values, -0 < +0).
uint32_t order_key(float f) {
  uint32_t u = f2u(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
float from_key(uint32_t k) { return u2f((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k); }

// true if the upper level of the pair wins at x (strictly smaller fp32 distance)
bool upper_wins(float x, float lo, float hi) {
  volatile float dlo = x - lo;   // fp32 subtraction, round to nearest even
  volatile float dhi = hi - x;
  return dhi < dlo;
}

uint16_t bf16_rne(float f) {
  uint32_t u = f2u(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

Tables build_tables(int codebook) {
  Tables t;
  if (codebook == kCodebookUniform4) {
    for (int i = 0; i < 16; ++i) t.L[i] = (float)(-1.0 + 2.0 * i / 15.0);
  } else if (codebook == kCodebookInt4 || codebook == kCodebookInt3 ||
             codebook == kCodebookTernary) {
    // Symmetric integers k / h, |k| <= h, in sign-magnitude form: code 8 + m
    // is +m / h and code 7 - m is -m / h (m = 0..7), so zero appears twice
    // (-0, +0) and magnitudes m > h lie beyond +-1, where x = w / c_b never
    // reaches them.
    const int h = codebook == kCodebookInt4 ? 7 : (codebook == kCodebookInt3 ? 3 : 1);
    for (int m = 0; m < 8; ++m) {
      t.L[8 + m] = (float)((double)m / h);
      t.L[7 - m] = -t.L[8 + m];
    }
  } else {
    double q[16];
    double qmax = 0.0;
    for (int i = 0; i < 16; ++i) {
      double p = (0.02 * (15 - i) + 0.98 * i) / 15.0;
      q[i] = normal_quantile(p);
      qmax = std::fmax(qmax, std::fabs(q[i]));
    }
    for (int i = 0; i < 16; ++i) t.L[i] = (float)(q[i] / qmax);
  }
  // The fused expansions use the magnitudes L[8..15] and a sign bit: the
  // table must be sign-symmetric, L[15 - i] = -L[i] exactly.
  t.symmetric = 1;
  for (int i = 0; i < 16; ++i)
    if (t.L[15 - i] != -t.L[i]) t.symmetric = 0;

  t.T[0] = -INFINITY;
  for (int j = 1; j < 16; ++j) {
    float lo = t.L[j - 1], hi = t.L[j];
    uint32_t a = order_key(lo), b = order_key(hi);   // pred(a) false, pred(b) true
    while (b - a > 1) {
      uint32_t m = a + (b - a) / 2;
      if (upper_wins(from_key(m), lo, hi))
        b = m;
      else
        a = m;
    }
    // hi itself loses when it ties with lo (-0 and +0): the threshold is the
    // next value up
    while (!upper_wins(from_key(b), lo, hi)) ++b;
    t.T[j] = from_key(b);
  }

  for (int m = 0; m < 8; ++m) t.expand.mag[m] = t.L[8 + m];
  // Byte planes of the bf16-rounded magnitudes (bytes 2 and 3 of the fp32
  // pattern): plane[p][w] holds byte p + 2 of m = 4w .. 4w + 3.
  for (int p = 0; p < 2; ++p) {
    for (int w = 0; w < 2; ++w) {
      uint32_t v = 0;
      for (int b = 0; b < 4; ++b) {
        uint32_t bits = (uint32_t)bf16_rne(t.L[8 + 4 * w + b]) << 16;
        v |= ((bits >> (8 * (p + 2))) & 0xffu) << (8 * b);
      }
      t.expand16.plane[p][w] = v;
    }
  }
  // Bucket table of the encoder.  The bucket of x is computed from
  // u = RN(x + 3), which lies at most 2^-23 above x + 3 and never below the
  // bucket of x, so it is exact if no threshold lies within 2^-23 below a
  // bucket boundary; that and "one threshold per bucket" are checked here.
  t.quant.ok = 1;
  for (int i = 0; i < kBuckets; ++i) {
    const double a = -1.0 + i / 32.0, b = (i < 64) ? a + 1.0 / 32.0 : INFINITY;
    BucketEntry &en = t.quant.bucket[i];
    en.T = INFINITY;
    en.base = 0;
    int inside = 0;
    for (int j = 1; j < 16; ++j) {
      const double tj = t.T[j];
      if (tj > 1.0) continue;              // beyond the largest x = w / c_b
      if (tj < a) ++en.base;
      else if (tj < b) {
        en.T = t.T[j];
        ++inside;
      }
      if (i > 0 && tj < a && tj >= a - 0x1p-23) t.quant.ok = 0;
    }
    if (inside > 1) t.quant.ok = 0;
  }
  return t;
}

}  // namespace

const Tables &tables(int codebook) {
  static Tables t[kCodebooks];
  static std::once_flag once[kCodebooks];
  const int cb = (codebook >= 0 && codebook < kCodebooks) ? codebook : 0;
  std::call_once(once[cb], [cb] { t[cb] = build_tables(cb); });
  return t[cb];
}

}  // namespace qlora

extern "C" void qlora_levels(float out[16]) {
  const qlora::Tables &t = qlora::tables(qlora::kCodebookNF4);
  for (int i = 0; i < 16; ++i) out[i] = t.L[i];
}

extern "C" void qlora_thresholds(float out[15]) {
  const qlora::Tables &t = qlora::tables(qlora::kCodebookNF4);
  for (int j = 1; j < 16; ++j) out[j - 1] = t.T[j];
}

extern "C" int qlora_codebook_levels(int codebook, float out[16]) {
  if (codebook < 0 || codebook >= qlora::kCodebooks || !out) return -1;
  const qlora::Tables &t = qlora::tables(codebook);
  for (int i = 0; i < 16; ++i) out[i] = t.L[i];
  return 0;
}

extern "C" int qlora_codebook_thresholds(int codebook, float out[15]) {
  if (codebook < 0 || codebook >= qlora::kCodebooks || !out) return -1;
  const qlora::Tables &t = qlora::tables(codebook);
  for (int j = 1; j < 16; ++j) out[j - 1] = t.T[j];
  return 0;
}
