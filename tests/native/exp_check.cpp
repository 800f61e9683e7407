// Host build of the kernel's fp64 exp (pld_math.hpp) against the C library's exp: prints the
// largest error in units of the last place over the router's range and the edge cases.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "pld_math.hpp"

static double ulp_err(double got, double ref) {
  if (got == ref) return 0.0;
  if (!isfinite(ref) || !isfinite(got) || ref == 0.0) return INFINITY;
  return fabs(got - ref) / (nextafter(fabs(ref), INFINITY) - fabs(ref));
}

int main() {
  double dk[pld::EXP_CONSTS];
  pld::exp_f64_consts(dk);
  double worst = 0.0, at = 0.0;
  uint64_t s = 0x9E3779B97F4A7C15ull;
  for (int i = 0; i < 2000000; i++) {
    s = s * 6364136223846793005ull + 1442695040888963407ull;   // an LCG draw (Knuth's MMIX constants)
    const double u = (double)(s >> 11) * 0x1p-53;
    const double x = i & 1 ? -700.0 + 1400.0 * u : -40.0 + 80.0 * u;   // whole range, and the gates' range
    const double e = ulp_err(pld::exp_f64(x, dk), exp(x));
    if (e > worst) { worst = e; at = x; }
  }
  for (double x = -745.0; x <= 709.0; x += 0.125) {
    const double e = ulp_err(pld::exp_f64(x, dk), exp(x));
    if (e > worst && exp(x) > 1e-300) { worst = e; at = x; }   // (subnormal results are not used)
  }
  const int edges_ok = pld::exp_f64(0.0, dk) == 1.0 && isinf(pld::exp_f64(710.0, dk)) && pld::exp_f64(-746.0, dk) == 0.0;
  printf("max_ulp %.3f at %.17g edges_ok %d\n", worst, at, edges_ok);
  return 0;
}
