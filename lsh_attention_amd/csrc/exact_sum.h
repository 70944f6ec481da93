// Exact comparison of sums of float64 products, for the hash's last-resort
// decision between near-tied rotation columns.  Host and device code (the
// host build serves the CPU test of this arithmetic).
//
// Every product of two bf16 or two fp32 values is exact in float64, and so is
// the sum of two float64 values as the pair (rounded sum, error) from TwoSum
// (Knuth, round to nearest).  An expansion is a list of float64 components,
// nonoverlapping and increasing in magnitude, whose exact sum is its value
// (Shewchuk, "Adaptive precision floating-point arithmetic and fast robust
// geometric predicates", 1997: Grow-Expansion with zero elimination); its sign
// is the sign of its largest (last) nonzero component.  For the products of
// bf16 or fp32 values no underflow can occur: they are at least 2^-298 in
// magnitude, and every partial sum is a multiple of 2^-350, far above
// float64's smallest normal number.
#pragma once

#if defined(__HIPCC__)
#define LSH_HD __host__ __device__
#else
#define LSH_HD
#endif

namespace lsh {

LSH_HD inline double two_sum(double a, double b, double& err) {
  const double s = a + b, bb = s - a;
  err = (a - (s - bb)) + (b - bb);
  return s;
}

// e[0..n) + b -> e[0..m), in place (each component is written at or below the
// index it was read from); returns m >= 1.
LSH_HD inline int grow_expansion(double* e, int n, double b) {
  double q = b;
  int m = 0;
  for (int i = 0; i < n; ++i) {
    double err;
    q = two_sum(q, e[i], err);
    if (err != 0.0) e[m++] = err;
  }
  if (q != 0.0 || m == 0) e[m++] = q;
  return m;
}

LSH_HD inline int expansion_sign(const double* e, int n) {
  for (int i = n - 1; i >= 0; --i)
    if (e[i] != 0.0) return e[i] > 0.0 ? 1 : -1;
  return 0;
}

// Sign of |A| - |B| for A = sum prod_a[0..n), B = sum prod_b[0..n) (n <= 64
// float64 terms, summed exactly), using the scratch expansions ea (n), eb (n)
// and d (2n); sa and sb receive the signs of A and B.
LSH_HD inline int exact_abs_compare(const double* prod_a, const double* prod_b, int n, double* ea, double* eb,
                                    double* d, int& sa, int& sb) {
  int na = 0, nb = 0;
  for (int k = 0; k < n; ++k) na = grow_expansion(ea, na, prod_a[k]);
  for (int k = 0; k < n; ++k) nb = grow_expansion(eb, nb, prod_b[k]);
  sa = expansion_sign(ea, na);
  sb = expansion_sign(eb, nb);
  int nd = 0;
  for (int k = 0; k < na; ++k) nd = grow_expansion(d, nd, sa < 0 ? -ea[k] : ea[k]);
  for (int k = 0; k < nb; ++k) nd = grow_expansion(d, nd, sb < 0 ? eb[k] : -eb[k]);
  return expansion_sign(d, nd);
}

}  // namespace lsh
