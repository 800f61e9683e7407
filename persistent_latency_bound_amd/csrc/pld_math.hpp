// Scalar math shared by the kernel and a host build used in the CPU tests.
//
// exp_f64: e^x in fp64 for the router gates (a handful of threads per step). Cody and
// Waite's argument reduction x = k ln2 + r, with ln2 split into a head with trailing zero
// bits and a tail (the two constants fdlibm's exp uses), so k * ln2_head is exact for the
// k that occur and |r| <= ln2 / 2; e^r by its Taylor series to degree 13 in Horner form
// (truncation below 1e-17 relative on that interval), then scaled by 2^k. The constants
// live in an array the caller fills once (the kernel keeps them in LDS: literal fp64
// constants would be hoisted into registers that stay live across every stage).
#pragma once
#include <math.h>

#if defined(__HIPCC__)
#define PLD_HD __host__ __device__
#else
#define PLD_HD
#endif

namespace pld {

constexpr int EXP_TERMS = 13;
constexpr int EXP_CONSTS = 3 + EXP_TERMS;   // dk[0..2] and dk[3..3 + EXP_TERMS)

PLD_HD inline void exp_f64_consts(double* dk) {
  dk[0] = 1.4426950408889634;          // 1/ln2
  dk[1] = 6.93147180369123816490e-01;  // ln2 head (trailing zero bits)
  dk[2] = 1.90821492927058770002e-10;  // ln2 tail
  for (int n = 1; n <= EXP_TERMS; n++) dk[2 + n] = 1.0 / (double)n;
}

PLD_HD inline double exp_f64(double x, const double* dk) {
  if (x > 709.0) return INFINITY;
  if (x < -745.0) return 0.0;
  const double k = rint(x * dk[0]);
  double r = fma(-k, dk[1], x);
  r = fma(-k, dk[2], r);
  double p = 1.0;
  for (int n = EXP_TERMS; n >= 1; n--) p = fma(p, r * dk[2 + n], 1.0);
  return ldexp(p, (int)k);
}

}  // namespace pld
