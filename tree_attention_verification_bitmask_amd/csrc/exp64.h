// float64 exp for non-positive arguments, shared by the kernels that decide
// in float64 (tree_target_sample, tree_accept_stochastic).
#pragma once

#include <hip/hip_runtime.h>

namespace tv {

// exp(x) for x <= 0 in float64, table-driven (P. T. P. Tang, "Table-driven
// implementation of the exponential function in IEEE floating-point
// arithmetic", ACM TOMS 15(2), 1989): x = (64 m + j) ln2/64 + r with
// |r| <= ln2/128, exp(x) = 2^m * 2^(j/64) * exp(r), where exp(r) - 1 is its
// Taylor polynomial to degree 5 (remainder below r^6/720 < 4e-17).  The
// 64 values 2^(j/64) sit in LDS; ln2/64 is split into hi + lo so that
// x - n*hi is exact under FMA.  x is clamped at -760, below which the result
// underflows to 0 as exp does; -inf and NaN give 0.  Measured on the host
// against extended-precision exp over 2e7 points in [-760, 0]: at most 2 ulps,
// and the same zero and subnormal results.
constexpr int kExpTable = 64;

struct ExpConst {
    double inv_l;  // 64 / ln2
    double l_hi;   // ln2 / 64, rounded to double
    double l_lo;   // ln2 / 64 - l_hi
};

__device__ __forceinline__ void exp_table_fill(double *tab) {
    if (threadIdx.x < kExpTable) tab[threadIdx.x] = exp2((double)threadIdx.x / kExpTable);
}

__device__ __forceinline__ double exp_nonpos(double x, const double *tab, const ExpConst &k) {
    x = fmax(x, -760.0);  // also maps -inf and NaN to -760
    // n = rint(x * 64 / ln2) by the 1.5 * 2^52 shift: the sum's low word holds
    // n in two's complement, and subtracting the shift again gives n exactly
    const double shifted = fma(x, k.inv_l, 6755399441055744.0);
    const int n = (int)__double2loint(shifted);
    const double nf = shifted - 6755399441055744.0;
    double r = fma(-nf, k.l_hi, x);
    r = fma(-nf, k.l_lo, r);
    double p = fma(r, 1.0 / 120.0, 1.0 / 24.0);
    p = fma(p, r, 1.0 / 6.0);
    p = fma(p, r, 0.5);
    p = fma(p, r, 1.0);
    p *= r;  // exp(r) - 1
    const double t = tab[n & (kExpTable - 1)];
    // v in [1, 2); ldexp rounds once, into the subnormal range if need be
    return ldexp(fma(t, p, t), n >> 6);
}

// The constants of exp_nonpos: ln2 / 64 split into a double and its
// remainder (x86 long double carries 64 significand bits, so the remainder is
// exact to ~2^-11 of itself).
inline ExpConst exp_const() {
    const long double ln2 = 0.6931471805599453094172321214581765680755L;
    ExpConst ek;
    ek.l_hi = (double)(ln2 / 64);
    ek.l_lo = (double)(ln2 / 64 - (long double)ek.l_hi);
    ek.inv_l = (double)(64 / ln2);
    return ek;
}

}  // namespace tv
