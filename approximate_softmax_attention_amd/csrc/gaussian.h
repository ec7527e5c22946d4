// Standard normal values from two 64-bit counter-based draws, for the
// Gaussian hyperplanes of the sortLSH hash (HA page, "Algorithm",
// Definition 1, read as signs of projections on Gaussian hyperplanes; the
// page fixes no generator).
//
// Box-Muller (Box and Muller, 1958): g = sqrt(-2 ln u1) cos(2 pi u2) with
// u1 = ((a >> 11) + 1) 2^-53 in (0, 1] and u2 = (b >> 11) 2^-53 in [0, 1).
// The three functions are evaluated with correctly rounded binary64 additions,
// subtractions, multiplications and divisions only, in a fixed order, on
// exactly split exponents: no fused multiply-add (contraction is switched off
// below) and no library transcendental. Every IEEE-754 platform therefore
// computes the same bits, so the device draws the hyperplanes itself from the
// seed and the host (sortlsh_hyperplanes) returns the identical values.
//
//  ln u, u in (0, 1]: u = f 2^e with f in [1, 2); if f > sqrt 2 then f = f/2,
//     e = e + 1; s = (f - 1)/(f + 1), z = s s; p = Horner in z of 1/(2k+1),
//     k = 11..0 (ln f = 2 atanh s); ln u = e ln2 + (2s) p.
//  sqrt y, y > 0: y = m 2^e with m in [1, 2); if e is odd then m = 2m,
//     e = e - 1; x = (1 + m)/2 and six Newton steps x = (x + m/x)/2;
//     sqrt y = x 2^(e/2); y <= 0 gives 0.
//  cos 2 pi u, u = B 2^-53: q = (B + 2^50) >> 51, r = (B - q 2^51) 2^-51 in
//     [-1/2, 1/2), theta = r (pi/2), t = theta^2; C = Horner in t of
//     (-1)^k/(2k)!, k = 9..0; S = theta times Horner in t of (-1)^k/(2k+1)!,
//     k = 8..0; the result is C, -S, -C, S for q mod 4 = 0, 1, 2, 3.
// Constants are the binary64 values nearest to ln 2, sqrt 2, pi/2 and the
// series coefficients.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace ha {

namespace gauss {

constexpr double kLn2 = 0.6931471805599453094;
constexpr double kSqrt2 = 1.4142135623730950488;
constexpr double kPio2 = 1.5707963267948966192;

__host__ __device__ inline uint64_t bits_of(double x) { return __builtin_bit_cast(uint64_t, x); }
__host__ __device__ inline double from_bits(uint64_t u) { return __builtin_bit_cast(double, u); }

// x = f 2^e exactly with f in [1, 2); x positive and normal.
__host__ __device__ inline double split(double x, int& e) {
  const uint64_t u = bits_of(x);
  e = int((u >> 52) & 0x7FF) - 1023;
  return from_bits((u & ((uint64_t(1) << 52) - 1)) | (uint64_t(1023) << 52));
}

// 2^k for a normal exponent k
__host__ __device__ inline double pow2(int k) { return from_bits(uint64_t(k + 1023) << 52); }

__host__ __device__ inline double ln_unit(double u) {
#pragma clang fp contract(off)
  int e;
  double f = split(u, e);
  if (f > kSqrt2) {
    f = f * 0.5;
    e = e + 1;
  }
  const double s = (f - 1.0) / (f + 1.0);
  const double z = s * s;
  double p = 1.0 / 23.0;
  p = p * z + 1.0 / 21.0;
  p = p * z + 1.0 / 19.0;
  p = p * z + 1.0 / 17.0;
  p = p * z + 1.0 / 15.0;
  p = p * z + 1.0 / 13.0;
  p = p * z + 1.0 / 11.0;
  p = p * z + 1.0 / 9.0;
  p = p * z + 1.0 / 7.0;
  p = p * z + 1.0 / 5.0;
  p = p * z + 1.0 / 3.0;
  p = p * z + 1.0;
  const double a = double(e) * kLn2;
  const double b = (2.0 * s) * p;
  return a + b;
}

__host__ __device__ inline double sqrt_newton(double y) {
#pragma clang fp contract(off)
  if (!(y > 0.0)) return 0.0;
  int e;
  double m = split(y, e);
  if (e & 1) {
    m = m * 2.0;
    e = e - 1;
  }
  double x = (1.0 + m) / 2.0;
  for (int i = 0; i < 6; ++i) x = (x + m / x) / 2.0;
  return x * pow2(e / 2);
}

// cos(2 pi B 2^-53) for 0 <= B < 2^53
__host__ __device__ inline double cos_two_pi(uint64_t B) {
#pragma clang fp contract(off)
  const uint64_t q = (B + (uint64_t(1) << 50)) >> 51;
  const int64_t r = int64_t(B) - int64_t(q << 51);
  const double theta = (double(r) * 0x1p-51) * kPio2;
  const double t = theta * theta;
  double c = -1.0 / 6402373705728000.0;      // -1/18!
  c = c * t + 1.0 / 20922789888000.0;         //  1/16!
  c = c * t + -1.0 / 87178291200.0;           // -1/14!
  c = c * t + 1.0 / 479001600.0;              //  1/12!
  c = c * t + -1.0 / 3628800.0;               // -1/10!
  c = c * t + 1.0 / 40320.0;                  //  1/8!
  c = c * t + -1.0 / 720.0;                   // -1/6!
  c = c * t + 1.0 / 24.0;                     //  1/4!
  c = c * t + -1.0 / 2.0;                     // -1/2!
  c = c * t + 1.0;
  double s = 1.0 / 355687428096000.0;         //  1/17!
  s = s * t + -1.0 / 1307674368000.0;         // -1/15!
  s = s * t + 1.0 / 6227020800.0;             //  1/13!
  s = s * t + -1.0 / 39916800.0;              // -1/11!
  s = s * t + 1.0 / 362880.0;                 //  1/9!
  s = s * t + -1.0 / 5040.0;                  // -1/7!
  s = s * t + 1.0 / 120.0;                    //  1/5!
  s = s * t + -1.0 / 6.0;                     // -1/3!
  s = s * t + 1.0;
  s = theta * s;
  switch (q & 3) {
    case 0: return c;
    case 1: return -s;
    case 2: return -c;
    default: return s;
  }
}

// g (binary64) from the draws a and b
__host__ __device__ inline double box_muller(uint64_t a, uint64_t b) {
#pragma clang fp contract(off)
  const double u1 = double((a >> 11) + 1) * 0x1p-53;
  const double rad = sqrt_newton(-2.0 * ln_unit(u1));
  return rad * cos_two_pi(b >> 11);
}

// Nearest bfloat16 (ties to even) of the fp32 rounding of g, as its bits
__host__ __device__ inline uint16_t to_bf16_bits(double g) {
  uint32_t u = __builtin_bit_cast(uint32_t, float(g));
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

}  // namespace gauss

}  // namespace ha
