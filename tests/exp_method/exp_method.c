/* CPU check of the method behind the verification kernels' binary64
 * exponential: Cody and Waite's reduction x = k ln 2 + r with ln 2 held as
 * two doubles (RN(ln 2), RN(ln 2 - RN(ln 2))) and both products by k inside
 * an FMA, the degree-13 Taylor polynomial of e^r with coefficients RN(1/n!)
 * by Horner's rule, then ldexp.  Prints the largest difference in units in
 * the last place from the C library's exp over n pseudo-random arguments in
 * [-746, 0] (four ranges) and a list of edge arguments.
 * Usage: exp_method n */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static double method_exp(double x) {
    const double log2e = 0x1.71547652b82fep+0, ln2_hi = 0x1.62e42fefa39efp-1,
                 ln2_lo = 0x1.abc9e3b39803fp-56;
    if (!(x > -746.0))
        return x != x ? x : 0.0;
    const double k = rint(x * log2e);
    double r = fma(-k, ln2_hi, x);
    r = fma(-k, ln2_lo, r);
    double c[14];
    for (int n = 0; n < 14; ++n) {
        double f = 1.0;
        for (int j = 2; j <= n; ++j) f *= j;
        c[n] = 1.0 / f; /* RN(1/n!): n! is exact in binary64 up to 13! */
    }
    double p = c[13];
    for (int n = 12; n >= 0; --n) p = fma(p, r, c[n]);
    return ldexp(p, (int)k);
}

static double ulp_diff(double a, double b) {
    if (a == b)
        return 0.0;
    if (fabs(a) < 0x1p-1022 || fabs(b) < 0x1p-1022)
        return fabs(a - b) / 0x1p-1074;
    int64_t ia, ib;
    memcpy(&ia, &a, 8);
    memcpy(&ib, &b, 8);
    return fabs((double)(ia - ib));
}

int main(int argc, char **argv) {
    long n = argc > 1 ? atol(argv[1]) : 1000000;
    uint64_t s = 88172645463325252ull;
    double worst = 0.0;
    const double span[4] = {746.0, 40.0, 1.0, 0x1p-30};
    for (long i = 0; i < n; ++i) {
        s ^= s << 13;
        s ^= s >> 7;
        s ^= s << 17;
        const double x = -span[i & 3] * ((double)(s >> 11) * 0x1p-53);
        const double d = ulp_diff(exp(x), method_exp(x));
        if (d > worst)
            worst = d;
    }
    const double edge[] = {0.0, -0.0, -1e-300, -0.34657359027997264, -0.3465735902799727,
                           -708.3964185322641, -709.0, -744.0, -745.1332191019411, -745.9,
                           -746.0, -1000.0, -INFINITY};
    for (unsigned i = 0; i < sizeof edge / sizeof edge[0]; ++i) {
        const double d = ulp_diff(exp(edge[i]), method_exp(edge[i]));
        if (d > worst)
            worst = d;
    }
    printf("%.3f %d\n", worst, isnan(method_exp(NAN)) ? 1 : 0);
    return 0;
}
