// Real-basis Clebsch-Gordan tables for the path planner.
//
// The tensor product contracts two dense feature vectors with a sparse,
// structured coupling tensor ("An Efficient Sparse Kernel Generator for
// O(3)-Equivariant Deep Networks", abstract).  Here that tensor is the
// Clebsch-Gordan coefficient table carried to the real spherical-harmonic basis:
//
//   1. complex coefficients <l1 m1 l2 m2 | l3 m3> through the Wigner 3j symbol,
//        <l1 m1 l2 m2 | L M> = (-1)^(l1 - l2 + M) sqrt(2L+1) (l1 l2 L; m1 m2 -M),
//      with the 3j symbol from Racah's single-sum formula;
//   2. the unitary map from complex to real harmonics, element (real m, complex mu):
//        m > 0:  (-1)^m / sqrt2 at mu = m,   1/sqrt2 at mu = -m
//        m = 0:  1 at mu = 0
//        m < 0:  i / sqrt2 at mu = m,        -i (-1)^m / sqrt2 at mu = -m
//      (real harmonics with the Condon-Shortley phase; l = 1 is ordered y, z, x);
//   3. T[m1,m2,m3] = sum conj(Q1[m1,mu1]) conj(Q2[m2,mu2]) Q3[m3,mu3] <...>, which
//      is purely real for even l1+l2+l3 and purely imaginary for odd; the table is
//      that real or imaginary part, signed so the first non-zero entry in
//      row-major (m1, m2, m3) order is positive, with |value| <= 1e-10 set to 0.
//
// Steps 2-3 fix a convention that any consumer of the real tables must share, so
// the same three rules appear wherever tables are built.
#include <cmath>
#include <complex>
#include <cstdlib>
#include <vector>

#include "planner.hpp"

namespace oeq {
namespace {

double factorial(int n) {
    static const double table[] = {1.0, 1.0, 2.0, 6.0, 24.0, 120.0, 720.0, 5040.0, 40320.0,
                                   362880.0, 3628800.0, 39916800.0, 479001600.0,
                                   6227020800.0, 87178291200.0, 1307674368000.0,
                                   20922789888000.0, 355687428096000.0};
    return (n >= 0 && n < 18) ? table[n] : NAN;
}

// Wigner 3j symbol (j1 j2 j3; m1 m2 m3) for integer arguments.
double wigner_3j(int j1, int j2, int j3, int m1, int m2, int m3) {
    if (m1 + m2 + m3 != 0) return 0.0;
    if (std::abs(m1) > j1 || std::abs(m2) > j2 || std::abs(m3) > j3) return 0.0;
    if (j3 < std::abs(j1 - j2) || j3 > j1 + j2) return 0.0;
    const double tri = factorial(j1 + j2 - j3) * factorial(j1 - j2 + j3) *
                       factorial(-j1 + j2 + j3) / factorial(j1 + j2 + j3 + 1);
    const double mf = factorial(j1 + m1) * factorial(j1 - m1) * factorial(j2 + m2) *
                      factorial(j2 - m2) * factorial(j3 + m3) * factorial(j3 - m3);
    const int kmin = std::max(0, std::max(j2 - j3 - m1, j1 - j3 + m2));
    const int kmax = std::min(j1 + j2 - j3, std::min(j1 - m1, j2 + m2));
    double s = 0.0;
    for (int k = kmin; k <= kmax; ++k) {
        const double den = factorial(k) * factorial(j3 - j2 + k + m1) *
                           factorial(j3 - j1 + k - m2) * factorial(j1 + j2 - j3 - k) *
                           factorial(j1 - k - m1) * factorial(j2 - k + m2);
        s += ((k % 2) ? -1.0 : 1.0) / den;
    }
    const int ph = j1 - j2 - m3;
    return (((ph % 2) + 2) % 2 ? -1.0 : 1.0) * std::sqrt(tri * mf) * s;
}

double clebsch_gordan(int l1, int m1, int l2, int m2, int L, int M) {
    const int ph = l1 - l2 + M;
    return (((ph % 2) + 2) % 2 ? -1.0 : 1.0) * std::sqrt(2.0 * L + 1.0) *
           wigner_3j(l1, l2, L, m1, m2, -M);
}

// Element (real m, complex mu) of the complex -> real harmonic map.
std::complex<double> to_real(int m, int mu) {
    const double h = 1.0 / std::sqrt(2.0);
    const double sm = (std::abs(m) % 2) ? -1.0 : 1.0;
    if (m > 0) {
        if (mu == m) return {sm * h, 0.0};
        if (mu == -m) return {h, 0.0};
        return {0.0, 0.0};
    }
    if (m == 0) return {mu == 0 ? 1.0 : 0.0, 0.0};
    if (mu == m) return {0.0, h};
    if (mu == -m) return {0.0, -sm * h};
    return {0.0, 0.0};
}

}  // namespace

bool cg_real_table(int l1, int l2, int l3, std::vector<double> &out) {
    if (l1 < 0 || l2 < 0 || l3 < 0 || l1 > kLMax || l2 > kLMax || l3 > kLMax) return false;
    if (l3 < std::abs(l1 - l2) || l3 > l1 + l2) return false;
    const int n1 = 2 * l1 + 1, n2 = 2 * l2 + 1, n3 = 2 * l3 + 1;
    const bool even = ((l1 + l2 + l3) % 2) == 0;
    std::vector<double> part(static_cast<size_t>(n1) * n2 * n3, 0.0);
    for (int a = -l1; a <= l1; ++a)
        for (int b = -l2; b <= l2; ++b)
            for (int c = -l3; c <= l3; ++c) {
                std::complex<double> t(0.0, 0.0);
                // complex coefficients vanish unless mu3 = mu1 + mu2
                for (int mu1 = -l1; mu1 <= l1; ++mu1)
                    for (int mu2 = -l2; mu2 <= l2; ++mu2) {
                        const int mu3 = mu1 + mu2;
                        if (std::abs(mu3) > l3) continue;
                        const std::complex<double> q =
                            std::conj(to_real(a, mu1)) * std::conj(to_real(b, mu2)) *
                            to_real(c, mu3);
                        if (q == std::complex<double>(0.0, 0.0)) continue;
                        t += q * clebsch_gordan(l1, mu1, l2, mu2, l3, mu3);
                    }
                part[(static_cast<size_t>(a + l1) * n2 + (b + l2)) * n3 + (c + l3)] =
                    even ? t.real() : t.imag();
            }
    double sign = 0.0;
    for (double v : part)
        if (std::fabs(v) > 1e-10) {
            sign = v > 0 ? 1.0 : -1.0;
            break;
        }
    out.assign(part.size(), 0.0);
    for (size_t i = 0; i < part.size(); ++i) {
        const double v = sign * part[i];
        out[i] = std::fabs(v) > 1e-10 ? v : 0.0;
    }
    return true;
}

}  // namespace oeq
