// w8inv_math.h -- device arithmetic shared by the library's kernels:
// exact format conversions, double-double helpers, and the correctly rounded
// fp32 exponential and logarithm (EXP32 / LOG32) that the blockwise logprob
// and the SwiGLU glue use.
//
// Why correctly rounded: the tokenspeed "Numerics envelopes" page asks that
// the blockwise logprob be one fixed fp32 arithmetic (alignment.trainer
// table, "--logprob-order blockwise"; "Logprobs" section) but does not name
// an exp or a log.  Taking RN32(e^x) and RN32(ln x) makes that arithmetic a
// pure function of its inputs, reproducible by any implementation.
//
// All code here is compiled with -ffp-contract=off: every + - * / is one IEEE
// double or float operation; fused operations appear only as explicit fma.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w8i {

// ------------------------------------------------------------------ formats

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float((uint32_t)b << 16);
}

// fp16 bits -> double, exactly, decoded from the fields (subnormals m*2^-24).
__device__ __forceinline__ double f16_to_f64(uint32_t h) {
    const uint32_t e = (h >> 10) & 31u, m = h & 1023u;
    double v = __builtin_ldexp((double)(e ? (m | 1024u) : m), (e ? (int)e : 1) - 25);
    if (e == 31u) v = m ? __builtin_nan("") : __builtin_inf();
    return (h & 0x8000u) ? -v : v;
}

// Round a float to bf16, nearest-even (NaN stays a quiet NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Round a double to bf16, nearest-even, with a single rounding: the double is
// first rounded to float by round-to-odd (truncate, then set the sticky bit
// when inexact), which keeps 16 extra bits and so cannot create a false tie.
__device__ __forceinline__ uint16_t f64_to_bf16(double d) {
    float f = (float)d;
    uint32_t u = __float_as_uint(f);
    const double back = (double)f;
    if (back != d && (u & 0x7fffffffu) < 0x7f800000u) {
        if (__builtin_fabs(back) > __builtin_fabs(d)) u -= 1u;
        u |= 1u;
    }
    return f32_to_bf16(__uint_as_float(u));
}

// ------------------------------------------------------------ layer glue
// The column-local glue between the projections of one decode layer.  The
// glue kernels and the fused projection epilogues both call these, so a fused
// epilogue gives the bits of the projection followed by the glue kernel.

// residual add: fp32 sum of two bf16 values, rounded to bf16 nearest-even
__device__ __forceinline__ uint16_t add_bf16(uint16_t a, uint16_t b) {
    return f32_to_bf16(bf16_to_f32(a) + bf16_to_f32(b));
}

// SwiGLU: silu(g) * u = g / (1 + e^-g) * u in fp64, rounded once to bf16.  In
// fp64, e^-g of any bf16 gate is finite or its silu is below bf16's range, so
// the final rounding is the only one that matters (in fp32, e^-g overflows
// for g < -88.7 while g e^g u can still be a normal bf16).
__device__ __forceinline__ uint16_t swiglu_bf16(uint16_t gate, uint16_t up) {
    const double g = (double)bf16_to_f32(gate);
    const double u = (double)bf16_to_f32(up);
    const double silu = g / (1.0 + ::exp(-g));
    return f64_to_bf16(silu * u);
}

// ------------------------------------------------------------ double-double

struct dd {
    double hi, lo;
};

__device__ __forceinline__ dd two_sum(double a, double b) {
    const double s = a + b;
    const double bb = s - a;
    const double e = (a - (s - bb)) + (b - bb);
    return {s, e};
}

__device__ __forceinline__ dd fast_two_sum(double a, double b) {  // needs |a| >= |b|
    const double s = a + b;
    return {s, b - (s - a)};
}

__device__ __forceinline__ dd two_prod(double a, double b) {
    const double p = a * b;
    return {p, __builtin_fma(a, b, -p)};
}

__device__ __forceinline__ dd dd_add(dd a, dd b) {
    dd s = two_sum(a.hi, b.hi);
    const dd t = two_sum(a.lo, b.lo);
    s.lo += t.hi;
    s = fast_two_sum(s.hi, s.lo);
    s.lo += t.lo;
    return fast_two_sum(s.hi, s.lo);
}

__device__ __forceinline__ dd dd_mul(dd a, dd b) {
    dd p = two_prod(a.hi, b.hi);
    p.lo += a.hi * b.lo + a.lo * b.hi;
    return fast_two_sum(p.hi, p.lo);
}

// a / n for a small positive integer n (exact remainder by fma).
__device__ __forceinline__ dd dd_div_int(dd a, double n) {
    const double q1 = a.hi / n;
    double r = __builtin_fma(-q1, n, a.hi);
    r += a.lo;
    const double q2 = r / n;
    return fast_two_sum(q1, q2);
}

// ln 2 as a triple-double: hi = RN64(ln 2), lo1 = RN64(ln 2 - hi),
// lo2 = RN64(ln 2 - hi - lo1); derived from 80-digit decimal arithmetic.
constexpr double kLn2Hi = 0x1.62e42fefa39efp-1;
constexpr double kLn2Lo1 = 0x1.abc9e3b39803fp-56;
constexpr double kLn2Lo2 = 0x1.7b57a079a1934p-111;
constexpr double kInvLn2 = 0x1.71547652b82fep+0;

// ------------------------------------------------- correct rounding to fp32

// Distance from the non-negative finite float f to its upper / lower
// neighbour, as a double.  Above FLT_MAX the next grid point is 2^128 (the
// overflow boundary of round-to-nearest sits half way to it).
__device__ __forceinline__ double f32_gap_up(float f) {
    const uint32_t u = __float_as_uint(f);
    if (u == 0x7f7fffffu) return 0x1p104;
    return (double)__uint_as_float(u + 1u) - (double)f;
}
__device__ __forceinline__ double f32_gap_down(float f) {  // f > 0
    return (double)f - (double)__uint_as_float(__float_as_uint(f) - 1u);
}

// RN32 of the non-negative value hi + lo (|lo| tiny against hi): round hi,
// then move one step if hi + lo lies beyond the half-way point (ties to even).
__device__ __forceinline__ float rn32_dd_nonneg(double hi, double lo) {
    float f = (float)hi;
    if (__builtin_isinf(f)) return f;
    const double d = (hi - (double)f) + lo;  // hi - f is exact
    const uint32_t u = __float_as_uint(f);
    if (d > 0.0) {
        const double half = f32_gap_up(f) * 0.5;
        if (d > half || (d == half && (u & 1u)))
            f = (u == 0x7f7fffffu) ? __builtin_inff() : __uint_as_float(u + 1u);
    } else if (d < 0.0 && f > 0.0f) {
        const double half = f32_gap_down(f) * 0.5;
        if (-d > half || (-d == half && (u & 1u))) f = __uint_as_float(u - 1u);
    }
    return f;
}

// ---------------------------------------------------------------- EXP32

// e^r for the double-double r, |r| <= 0.35: Taylor series to degree 23 in the
// nested form 1 + r(1 + r/2(1 + r/3(...))), every step in double-double.
__device__ __noinline__ dd exp_dd_reduced(dd r) {
    dd p = {1.0, 0.0};
    for (int n = 23; n >= 1; --n) {
        p = dd_div_int(dd_mul(p, r), (double)n);
        p = dd_add(p, dd{1.0, 0.0});
    }
    return p;
}

// EXP32(x) = RN32(e^x) for every fp32 x.
//   x < -104 (incl. -inf): e^x < 2^-150, so the result is +0.
//   x > 89: e^x > FLT_MAX + ulp/2, so the result is +inf.
//   Otherwise x = k ln2 + r, k = rint(x / ln2), |r| <= 0.35, where x - k*hi is
//   exact (x is a multiple of 2^-25 whenever k != 0, k*hi a multiple of 2^-53).
//   Fast path: degree-14 Taylor polynomial in double, relative error below
//   2^-50; if the result lies within 2^-48 (relative) of a binary32 rounding
//   boundary it is recomputed in double-double (error ~2^-100) before rounding.
__device__ __forceinline__ float exp32(float xf) {
    if (!(xf >= -104.0f)) return (xf != xf) ? xf : 0.0f;
    if (xf > 89.0f) return __builtin_inff();
    const double x = (double)xf;
    const double k = __builtin_rint(x * kInvLn2);
    const double rh = __builtin_fma(-k, kLn2Hi, x);  // exact
    const double r = __builtin_fma(-k, kLn2Lo1, rh);
    // Taylor polynomial of degree 14, Horner form; 1/n! rounded to double
    double p = 1.0 / 87178291200.0;              // 1/14!
    p = __builtin_fma(p, r, 1.0 / 6227020800.0); // 1/13!
    p = __builtin_fma(p, r, 1.0 / 479001600.0);  // 1/12!
    p = __builtin_fma(p, r, 1.0 / 39916800.0);
    p = __builtin_fma(p, r, 1.0 / 3628800.0);
    p = __builtin_fma(p, r, 1.0 / 362880.0);
    p = __builtin_fma(p, r, 1.0 / 40320.0);
    p = __builtin_fma(p, r, 1.0 / 5040.0);
    p = __builtin_fma(p, r, 1.0 / 720.0);
    p = __builtin_fma(p, r, 1.0 / 120.0);
    p = __builtin_fma(p, r, 1.0 / 24.0);
    p = __builtin_fma(p, r, 1.0 / 6.0);
    p = __builtin_fma(p, r, 0.5);
    p = __builtin_fma(p, r, 1.0);
    p = __builtin_fma(p, r, 1.0);
    const int ki = (int)k;
    const double v = __builtin_ldexp(p, ki);
    const float f = (float)v;
    if (!__builtin_isinf(f)) {
        // distance from v to the binary32 rounding boundary on its side
        const double d = v - (double)f;
        const double half = (d >= 0.0 ? f32_gap_up(f) : f32_gap_down(f)) * 0.5;
        if (half - __builtin_fabs(d) > v * 0x1p-48) return f;
    }
    // hard case: double-double evaluation
    dd rd = two_prod(-k, kLn2Lo1);
    rd.lo += -k * kLn2Lo2;
    rd = dd_add(dd{rh, 0.0}, rd);
    const dd e = exp_dd_reduced(rd);
    return rn32_dd_nonneg(__builtin_ldexp(e.hi, ki), __builtin_ldexp(e.lo, ki));
}

// ---------------------------------------------------------------- LOG32

// ln(m 2^e) in double-double, m in [sqrt(1/2), sqrt(2)): ln x = e ln2 +
// 2 atanh(z), z = (m - 1)/(m + 1), |z| <= 0.1716; atanh by its odd series to
// z^43, Horner in double-double (error ~2^-100).  m - 1 and m + 1 are exact in
// double (m has 24 significant bits).
__device__ __noinline__ dd log_dd_reduced(double m, int ex) {
    const double num = m - 1.0, den = m + 1.0;
    const double q1 = num / den;
    const double rem = __builtin_fma(-q1, den, num);
    const dd z = fast_two_sum(q1, rem / den);
    const dd z2 = dd_mul(z, z);
    // sum_{i=0}^{21} z2^i / (2i + 1), Horner in double-double
    dd p = dd_div_int(dd{1.0, 0.0}, 43.0);
    for (int i = 20; i >= 0; --i) {
        p = dd_mul(p, z2);
        p = dd_add(p, dd_div_int(dd{1.0, 0.0}, (double)(2 * i + 1)));
    }
    dd lnm = dd_mul(z, p);
    lnm.hi *= 2.0;
    lnm.lo *= 2.0;
    const double e = (double)ex;
    dd le = two_prod(e, kLn2Hi);
    le.lo += e * kLn2Lo1;
    return dd_add(le, lnm);
}

// LOG32(x) = RN32(ln x) for every fp32 x.  x = m 2^e as above.
//   Fast path, in double: the same atanh series to z^22 (the 12 terms of
//   s = z^2 from s^0 / 1 to s^11 / 23; the next term is below 2^-65 of the
//   sum), z = RN64((m - 1)/(m + 1)), lnm = 2 z P, v = fma(e, ln2_hi, lnm) +
//   e ln2_lo.  Each of z, s, P (Horner: the last of its 11 fmas dominates,
//   the earlier errors shrink by s <= 0.0295 per step) and z P rounds once:
//   |lnm - ln m| <= 3.2 2^-53 |ln m|; for e != 0, |ln x| >= ln2 - ln sqrt 2 =
//   0.3466 >= |ln m| and the fma and the final add round once each, so
//   |v - ln x| <= 5.5 2^-53 |ln x| < 2^-50 |ln x| (and for e = 0, v = lnm).
//   If v lies farther than 2^-47 |v| (8 times that bound) from the binary32
//   rounding boundary on its side, RN32(v) = RN32(ln x); otherwise (about one
//   input in 2^22) the double-double evaluation decides.
__device__ __forceinline__ float log32(float xf) {
    if (xf != xf || xf < 0.0f) return __builtin_nanf("");
    if (xf == 0.0f) return -__builtin_inff();
    if (__builtin_isinf(xf)) return xf;
    if (xf == 1.0f) return 0.0f;
    int ex;
    double m = __builtin_frexp((double)xf, &ex);  // m in [0.5, 1)
    if (m < 0x1.6a09e667f3bcdp-1) {                // sqrt(1/2)
        m *= 2.0;
        ex -= 1;
    }
    const double z = (m - 1.0) / (m + 1.0);
    const double s = z * z;
    double p = 1.0 / 23.0;
    p = __builtin_fma(p, s, 1.0 / 21.0);
    p = __builtin_fma(p, s, 1.0 / 19.0);
    p = __builtin_fma(p, s, 1.0 / 17.0);
    p = __builtin_fma(p, s, 1.0 / 15.0);
    p = __builtin_fma(p, s, 1.0 / 13.0);
    p = __builtin_fma(p, s, 1.0 / 11.0);
    p = __builtin_fma(p, s, 1.0 / 9.0);
    p = __builtin_fma(p, s, 1.0 / 7.0);
    p = __builtin_fma(p, s, 1.0 / 5.0);
    p = __builtin_fma(p, s, 1.0 / 3.0);
    p = __builtin_fma(p, s, 1.0);
    const double lnm = 2.0 * (z * p);
    const double e = (double)ex;
    const double v = __builtin_fma(e, kLn2Hi, lnm) + e * kLn2Lo1;
    const float f = (float)v;  // RN32(-v) = -RN32(v): the check runs on |v|
    const double a = __builtin_fabs(v);
    const float fa = __builtin_fabsf(f);  // >= 2^-25: ln x != 0 for x != 1
    const double d = a - (double)fa;
    const double half = (d >= 0.0 ? f32_gap_up(fa) : f32_gap_down(fa)) * 0.5;
    if (half - __builtin_fabs(d) > a * 0x1p-47) return f;
    const dd sl = log_dd_reduced(m, ex);
    if (sl.hi < 0.0) return -rn32_dd_nonneg(-sl.hi, -sl.lo);
    return rn32_dd_nonneg(sl.hi, sl.lo);
}

}  // namespace w8i
