// codebook.cpp -- the library's float32 codebooks, solved on the host.
//
// The optimal per-coordinate scalar quantiser of the rotated block (the
// article "llama.cpp に TurboQuant を実装", section "TurboQuant の何が違うのか",
// calls it the Lloyd-Max codebook) for a standard normal coordinate: levels
// that are the conditional means of their cells and thresholds that are the
// midpoints of neighbouring levels.  Solved here by alternating the two
// conditions from a uniform start on [-2, 2], in double, symmetrised each
// round; then rounded to float for the kernels.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <mutex>

#include "internal.h"

namespace tq {
namespace {

double phi(double x) { return std::isinf(x) ? 0.0 : std::exp(-0.5 * x * x) * 0.3989422804014327; }
// P(X > x) for X ~ N(0, 1); erfc keeps the upper tail accurate.
double upper_tail(double x) { return 0.5 * std::erfc(x * 0.7071067811865476); }

void lloyd_max(int bits, double *lv, double *th)
{
    const int L = 1 << bits;
    for (int k = 0; k < L; ++k)
        lv[k] = -2.0 + 4.0 * k / (L - 1);
    for (int round = 0; round < 100000; ++round) {
        for (int k = 0; k + 1 < L; ++k)
            th[k] = 0.5 * (lv[k] + lv[k + 1]);
        double change = 0.0;
        double nl[16];
        for (int k = 0; k < L; ++k) {
            double a = k == 0 ? -INFINITY : th[k - 1];
            double b = k == L - 1 ? INFINITY : th[k];
            double mass = upper_tail(a) - upper_tail(b);
            nl[k] = (phi(a) - phi(b)) / mass;
        }
        for (int k = 0; k < L; ++k) {
            double s = 0.5 * (nl[k] - nl[L - 1 - k]);
            change = std::fmax(change, std::fabs(s - lv[k]));
            lv[k] = s;
        }
        if (change < 1e-15)
            break;
    }
    for (int k = 0; k + 1 < L; ++k)
        th[k] = 0.5 * (lv[k] + lv[k + 1]);
    th[L / 2 - 1] = 0.0;
}

// Solve the 3x3 system sum_j M[i][j] c[j] = r[i] by Cramer's rule.
void solve3(const double M[3][3], const double r[3], double c[3])
{
    auto det = [](const double A[3][3]) {
        return A[0][0] * (A[1][1] * A[2][2] - A[1][2] * A[2][1]) -
               A[0][1] * (A[1][0] * A[2][2] - A[1][2] * A[2][0]) +
               A[0][2] * (A[1][0] * A[2][1] - A[1][1] * A[2][0]);
    };
    double d = det(M);
    for (int j = 0; j < 3; ++j) {
        double A[3][3];
        for (int i = 0; i < 3; ++i)
            for (int k = 0; k < 3; ++k)
                A[i][k] = k == j ? r[i] : M[i][k];
        c[j] = det(A) / d;
    }
}

void build(int bits, Codebook *cb)
{
    double lv[16], th[15];
    lloyd_max(bits, lv, th);
    const int L = 1 << bits, P = L / 2;
    cb->bits = bits;
    for (int k = 0; k < 8; ++k)
        cb->levels[k] = k < L ? (float)lv[k] : 0.0f;
    for (int k = 0; k < 7; ++k)
        cb->thresholds[k] = k < L - 1 ? (float)th[k] : 0.0f;
    if (bits == 2) {
        // one positive threshold: g(t) = t / tau_1; clamp keeps F = 2 + g in (0, 4)
        double tau = th[P];
        cb->g1 = (float)(1.0 / tau);
        cb->g2 = cb->g3 = 0.0f;
        cb->clamp_t = (float)(1.9 * tau);   // F in [0.1, 3.9]
    } else {
        // three positive thresholds: g(t) = g1 t + g2 t|t| + g3 t^3 through (tau_k, k)
        double M[3][3], r[3], c[3];
        for (int k = 0; k < 3; ++k) {
            double t = th[P + k];
            M[k][0] = t;
            M[k][1] = t * t;
            M[k][2] = t * t * t;
            r[k] = k + 1;
        }
        solve3(M, r, c);
        cb->g1 = (float)c[0];
        cb->g2 = (float)c[1];
        cb->g3 = (float)c[2];
        // For the Gaussian levels g rises to ~3.6 near t = 2.7 and falls after it;
        // clamping |t| at 2.6 keeps it increasing with |g| < 4 (verified below).
        cb->clamp_t = 2.6f;
    }
    // The decision function must be increasing on [0, clamp_t] and stay below
    // 2^bits/2 there, and its decision points (where it crosses k) must sit on the
    // thresholds: checked in double on the float coefficients the kernels get.  The
    // decision point of threshold k is found by bisection; rounding the coefficients
    // to float moves it by less than 1e-7 (9.4e-8 at the largest turbo3 threshold),
    // and the check allows 2e-7, about one float spacing of the thresholds.
    auto g = [cb](double t) { return t * (cb->g1 + cb->g2 * std::fabs(t) + cb->g3 * t * t); };
    double prev = 0.0;
    bool ok = true;
    for (int i = 1; i <= 100000; ++i) {
        double t = cb->clamp_t * i / 100000.0, v = g(t);
        ok = ok && v > prev;
        prev = v;
    }
    ok = ok && g(cb->clamp_t) < P - 1e-3;
    for (int k = 1; k < P; ++k) {
        const double tau = th[P - 1 + k];
        double a = tau - 1e-3, b = tau + 1e-3;
        ok = ok && g(a) < k && g(b) >= k;
        for (int it = 0; it < 100; ++it) {
            const double c = 0.5 * (a + b);
            (g(c) < k ? a : b) = c;
        }
        ok = ok && std::fabs(0.5 * (a + b) - tau) < 2e-7;
    }
    if (!ok) {
        std::fprintf(stderr, "libtq: encoder decision function check failed (bits=%d)\n", bits);
        std::abort();
    }
}

Codebook g_cb[2];
std::once_flag g_once;

}  // namespace

const Codebook *codebook(int bits)
{
    if (bits != 2 && bits != 3)
        return nullptr;
    std::call_once(g_once, [] {
        build(2, &g_cb[0]);
        build(3, &g_cb[1]);
    });
    return &g_cb[bits - 2];
}

}  // namespace tq
