// act_math.h -- per-element binary32 math of the activations in libmeswish.
//
// Every activation is written as a struct with the same device interface:
//
//   fwd<P>(x, k, rk)         value at x                       (fast path)
//   bwd<P>(x, dy, k, rk)     dy times the derivative at x     (fast path)
//   rare_thr<P>()            an element is rare where its key exceeds this
//   is_rare<BWD, P>(x, k)    true exactly where the element's key > rare_thr
//   fwd_rare(x, k), bwd_rare(x, dy, k)   the rare branch, taken per wave
//
// x = +-inf gives the limits as x -> +-inf with the parameter fixed (a zero
// Swish alpha or LeakyReLU slope leaves 0 * inf = NaN); NaN gives NaN.
//
// P (precise) is true for binary32 I/O, where results must agree with the
// exact value to 1e-5 relative; bfloat16 I/O needs only 2^-9, so its fast
// paths skip the extra-precision terms.  Each fast path folds the element's
// rare key into the running maximum rk (rk = fmaxf(rk, key); a NaN key is
// never rare, as the comparison it stands for is false).  A vector whose
// maximum exceeds rare_thr<P>() holds at least one rare element, and the
// caller recomputes exactly those where is_rare is true.  One max3 per
// three elements and one comparison per vector replace a comparison per
// element.  Keys must be quiet: a signaling NaN makes the maximum NaN.
//
// Sources, by page title and section:
//   Swish: blog post "Memory efficient Swish" (adeeplearner.github.io),
//     "How is Swish implemented?" (x Sigmoid(alpha x)) and "How is the
//     memory efficient version Swish implemented?" (backward from x alone).
//   The family: "What activations cost, in memory and in arithmetic",
//     Given: ReLU, LeakyReLU, sigmoid, tanh, GELU with erf, GELU with the tanh
//     approximation.  Standard definitions:
//       ReLU(x) = x > 0 ? x : 0            LeakyReLU(x) = x > 0 ? x : a x
//       sigmoid(x) = 1 / (1 + e^-x)        tanh(x)
//       GELU(x) = x Phi(x) = x erfc(-x / sqrt 2) / 2
//       GELU_tanh(x) = x (1 + tanh u) / 2 = x sigmoid(2u),
//                      u = sqrt(2/pi) (x + 0.044715 x^3)
//     Derivatives: 1 or 0; 1 or a; s (1 - s); 1 - tanh^2 = 4E / (1 + E)^2
//     with E = e^-2|x|; Phi(x) + x phi(x); s (1 + x (1 - s) 2u').
//
// Building blocks: the hardware exp2 and reciprocal (v_exp_f32, v_rcp_f32,
// which flush subnormals), exact hi+lo splits of products (fma), and
// frexp/ldexp to apply factors below the binary32 normal range with a
// single rounding at the end.
#pragma once

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

namespace meswish {

enum ActKind {
    kSwish = 0,
    kRelu = 1,
    kLeakyRelu = 2,
    kSigmoid = 3,
    kTanh = 4,
    kGeluErf = 5,
    kGeluTanh = 6,
    kActCount = 7,
    // Swish with alpha exactly 1: the same results by a shorter backward
    // (internal to the library; callers name kSwish).
    kSwishUnit = 8
};

// Coefficients prepared on the host (make_coef in meswish.hip).
struct Coef {
    float p;       // alpha (Swish) or negative slope (LeakyReLU); unused otherwise
    float c_hi;    // binary32 nearest to the exponent coefficient C (per activation)
    float c_lo;    // C - c_hi
    float aux_hi;  // GELU_tanh: binary32 nearest to 0.044715
    float aux_lo;  // GELU_tanh: 0.044715 - aux_hi
};

constexpr float kLn2f = 0.693147180559945309f;
// |base-2 exponent| beyond which 2^v leaves [2^-125, 2^125].
constexpr float kMaxExp = 125.0f;
// Base-2 exponent below which every rare-branch result rounds to zero:
// its other factors are below 2^(128 + 10) and 2^(138 - 300) < 2^-150.
constexpr float kZeroExp = -300.0f;
constexpr float kInvSqrt2f = 0.707106781186547524f;
constexpr float kInvSqrt2Pif = 0.398942280401432678f;
constexpr float kGeluTanhK = 1.59576912160573071f;  // 2 sqrt(2/pi)

__device__ __forceinline__ float exp2_hw(float v) { return __builtin_amdgcn_exp2f(v); }
__device__ __forceinline__ float rcp_hw(float v) { return __builtin_amdgcn_rcpf(v); }

// 2^(a C) for the activation's coefficient C.  v receives the binary32
// exponent a c_hi.  With P the rounding error of v and of c_hi is carried
// as w = (exact exponent - v) ln 2 and applied as 2^v (1 + w).
template <bool P>
__device__ __forceinline__ float exp2_lin(float a, const Coef& k, float& v)
{
    v = a * k.c_hi;
    float e = exp2_hw(v);
    if (P) {
        float err = fmaf(a, k.c_hi, -v);  // exact
        float w = fmaf(a, k.c_lo, err) * kLn2f;
        e = fmaf(e, w, e);
    }
    return e;
}

// Exponent v = vh + vl (vh the binary32 part) -> 2^v = ef * 2^kf, ef in [1, 2].
__device__ __forceinline__ void pow2_split(float vh, float vl, float& ef, int& kf)
{
    float f = floorf(vh);
    ef = exp2_hw(vh - f);
    ef = fmaf(ef, vl * kLn2f, ef);
    kf = (int)f;
}

// The exponent a C as a hi+lo pair.
__device__ __forceinline__ void lin_exponent(float a, const Coef& k, float& vh, float& vl)
{
    vh = a * k.c_hi;
    vl = fmaf(a, k.c_lo, fmaf(a, k.c_hi, -vh));
}

// m * g * 2^kf * ef rounded once: |frexp mantissa of m * g * ef| stays in the
// normal range for |g| in [2^-20, 2^10].
__device__ __forceinline__ float scale_pow2(float m, float g, float ef, int kf)
{
    int em;
    float mm = frexpf(m, &em);
    return ldexpf(mm * ef * g, em + kf);
}

// ---------------------------------------------------------------------------
// Swish: x Sigmoid(t), t = alpha x.  C = -alpha log2 e, so E = 2^(x C) = e^-t.
// kUnit: alpha is exactly 1 (t = x, one multiply less per element in the
// backward); the host selects it from the value of alpha.
// ---------------------------------------------------------------------------
template <bool kUnit>
struct SwishOpT {
    static constexpr bool kHasRare = true;

    template <bool P>
    __device__ static constexpr float rare_thr() { return kMaxExp; }

    template <bool P>
    __device__ static float fwd(float x, const Coef& k, float& rk)
    {
        float v;
        float e = exp2_lin<P>(x, k, v);
        float s = rcp_hw(1.0f + e);
        rk = fmaxf(rk, fabsf(v));
        return x * s;
    }

    template <bool P>
    __device__ static float bwd(float x, float dy, const Coef& k, float& rk)
    {
        float v;
        float e = exp2_lin<P>(x, k, v);
        float s = rcp_hw(1.0f + e);
        float c = e * s;  // 1 - s without cancellation
        float g = fmaf(kUnit ? x : k.p * x, c, 1.0f);
        rk = fmaxf(rk, fabsf(v));
        return dy * (s * g);
    }

    template <bool BWD, bool P>
    __device__ static bool is_rare(float x, const Coef& k)
    {
        return fabsf(x * k.c_hi) > kMaxExp;
    }

    // |t| > 86.6.  t > 0: Sigmoid(t) rounds to 1, y = x.  t < 0: y = x e^t.
    __device__ static float fwd_rare(float x, const Coef& k)
    {
        if (k.p * x >= 0.0f)
            return x;
        float vh, vl, ef;
        int kf;
        lin_exponent(x, k, vh, vl);  // = |t| log2 e
        if (-vh < kZeroExp)
            return copysignf(0.0f, x);  // also the limit at x = +-inf
        pow2_split(-vh, -vl, ef, kf);
        return scale_pow2(x, 1.0f, ef, kf);
    }

    // t > 0: dx = dy.  t < 0: 1 - s rounds to 1, dx = dy e^t (1 + t).
    __device__ static float bwd_rare(float x, float dy, const Coef& k)
    {
        float t = k.p * x;
        if (t >= 0.0f)
            return dy;
        float vh, vl, ef;
        int kf;
        lin_exponent(x, k, vh, vl);
        if (-vh < kZeroExp)
            return dy * -0.0f;
        pow2_split(-vh, -vl, ef, kf);
        return scale_pow2(dy, 1.0f + t, ef, kf);
    }
};
typedef SwishOpT<false> SwishOp;

// ---------------------------------------------------------------------------
// Sigmoid: C = -log2 e, E = e^-x, s = 1 / (1 + E), s' = s (E s).
// ---------------------------------------------------------------------------
struct SigmoidOp {
    static constexpr bool kHasRare = true;

    template <bool P>
    __device__ static constexpr float rare_thr() { return kMaxExp; }

    template <bool P>
    __device__ static float fwd(float x, const Coef& k, float& rk)
    {
        float v;
        float e = exp2_lin<P>(x, k, v);
        // x < -86.6: s is e^x, possibly subnormal.  x > 86.6: s rounds to 1
        // (and the exponent may have overflowed, which the P terms dislike).
        rk = fmaxf(rk, fabsf(v));
        return rcp_hw(1.0f + e);
    }

    template <bool P>
    __device__ static float bwd(float x, float dy, const Coef& k, float& rk)
    {
        float v;
        float e = exp2_lin<P>(x, k, v);
        float s = rcp_hw(1.0f + e);
        rk = fmaxf(rk, fabsf(v));
        return dy * (s * (e * s));
    }

    template <bool BWD, bool P>
    __device__ static bool is_rare(float x, const Coef& k)
    {
        return fabsf(x * k.c_hi) > kMaxExp;
    }

    __device__ static float fwd_rare(float x, const Coef& k)
    {
        if (x > 0.0f)
            return 1.0f;
        float vh, vl, ef;
        int kf;
        lin_exponent(x, k, vh, vl);  // = -x log2 e > 125
        if (-vh < kZeroExp)
            return 0.0f;
        pow2_split(-vh, -vl, ef, kf);
        return ldexpf(ef, kf);
    }

    // |x| > 86.6: s (1 - s) = e^-|x| (1 + O(e^-|x|)).
    __device__ static float bwd_rare(float x, float dy, const Coef& k)
    {
        float vh, vl, ef;
        int kf;
        lin_exponent(fabsf(x), k, vh, vl);  // = -|x| log2 e
        if (vh < kZeroExp)
            return dy * 0.0f;
        pow2_split(vh, vl, ef, kf);
        return scale_pow2(dy, 1.0f, ef, kf);
    }
};

// ---------------------------------------------------------------------------
// tanh: C = -2 log2 e, E = e^-2|x|.  tanh x = sign(x) (1 - E) / (1 + E) for
// |x| >= 1/8 (1 - E >= 0.22, no cancellation), the Maclaurin series
// x - x^3/3 + 2x^5/15 - 17x^7/315 below (truncation < 2e-9 relative); with
// bfloat16 I/O the switch is at 2^-8 and the series is just x.
// Derivative 1 - tanh^2 = 4 E / (1 + E)^2.
// ---------------------------------------------------------------------------
struct TanhOp {
    static constexpr bool kHasRare = true;

    template <bool P>
    __device__ static constexpr float rare_thr() { return kMaxExp; }

    template <bool P>
    __device__ static float fwd(float x, const Coef& k, float& /*rk: the forward has no rare case*/)
    {
        float a = fabsf(x);
        float v;
        float e = exp2_lin<false>(a, k, v);
        float big = (1.0f - e) * rcp_hw(1.0f + e);
        if (!P)  // bfloat16: tanh x = x to 2^-17 below 2^-8, and the
                 // cancellation of 1 - E costs under 2^-16 above it
            return a < 0.00390625f ? x : copysignf(big, x);
        float x2 = x * x;
        float poly = fmaf(x2, -17.0f / 315.0f, 2.0f / 15.0f);
        poly = fmaf(x2, poly, -1.0f / 3.0f);
        float small = fmaf(x * x2, poly, x);
        return a < 0.125f ? small : copysignf(big, x);
    }

    template <bool P>
    __device__ static float bwd(float x, float dy, const Coef& k, float& rk)
    {
        float v;
        float e = exp2_lin<P>(fabsf(x), k, v);
        float r = rcp_hw(1.0f + e);
        rk = fmaxf(rk, -v);  // v < -125, |x| > 43.3: 4E below the normal range
        return dy * (4.0f * e * r * r);
    }

    template <bool BWD, bool P>
    __device__ static bool is_rare(float x, const Coef& k)
    {
        return BWD && fabsf(x) * k.c_hi < -kMaxExp;
    }

    __device__ static float fwd_rare(float x, const Coef&) { return x; }  // never taken

    __device__ static float bwd_rare(float x, float dy, const Coef& k)
    {
        float vh, vl, ef;
        int kf;
        lin_exponent(fabsf(x), k, vh, vl);  // = -2|x| log2 e
        if (vh < kZeroExp)
            return dy * 0.0f;
        pow2_split(vh, vl, ef, kf);
        return scale_pow2(dy, 4.0f, ef, kf);
    }
};

// ---------------------------------------------------------------------------
// ReLU and LeakyReLU (slope a = k.p): compare and select; NaN propagates,
// and x = -inf gives the limits (0, and the slope a in the backward).
// ---------------------------------------------------------------------------
struct ReluOp {
    static constexpr bool kHasRare = false;

    template <bool P>
    __device__ static constexpr float rare_thr() { return INFINITY; }

    template <bool P>
    __device__ static float fwd(float x, const Coef&, float&)
    {
        return x > 0.0f ? x : (x <= 0.0f ? 0.0f : x);
    }

    template <bool P>
    __device__ static float bwd(float x, float dy, const Coef&, float&)
    {
        return dy * (x > 0.0f ? 1.0f : (x <= 0.0f ? 0.0f : x));
    }

    template <bool BWD, bool P>
    __device__ static bool is_rare(float, const Coef&) { return false; }
    __device__ static float fwd_rare(float x, const Coef&) { return x; }
    __device__ static float bwd_rare(float, float dy, const Coef&) { return dy; }
};

struct LeakyReluOp {
    static constexpr bool kHasRare = false;

    template <bool P>
    __device__ static constexpr float rare_thr() { return INFINITY; }

    template <bool P>
    __device__ static float fwd(float x, const Coef& k, float&)
    {
        return x > 0.0f ? x : k.p * x;
    }

    template <bool P>
    __device__ static float bwd(float x, float dy, const Coef& k, float&)
    {
        return dy * (x > 0.0f ? 1.0f : (x <= 0.0f ? k.p : x));
    }

    template <bool BWD, bool P>
    __device__ static bool is_rare(float, const Coef&) { return false; }
    __device__ static float fwd_rare(float x, const Coef&) { return x; }
    __device__ static float bwd_rare(float, float dy, const Coef&) { return dy; }
};

// ---------------------------------------------------------------------------
// GELU with erf.  Phi(x) = erfc(z) / 2 with z = -x / sqrt 2, evaluated by the
// Chebyshev-fitted form of Numerical Recipes in C (Press, Teukolsky,
// Vetterling, Flannery, 2nd ed., section 6.2, function erfcc):
//   erfc(|z|) = t exp(-z^2 + Q(t)),  t = 1 / (1 + |z| / 2),
// Q a degree-9 polynomial; fractional error below 1.2e-7 for every z >= 0,
// and erfc(-|z|) = 2 - erfc(|z|).  z^2 = x^2 / 2 is taken from the exact
// x^2 (hi+lo).  phi(x) = e^(-x^2/2) / sqrt(2 pi) with C = -log2(e) / 2.
// With bfloat16 I/O the tail erfc(|z|) / 2 is instead one exponential of a
// short polynomial (tail_short).  For x < -6 the rare branch applies
// e^(-x^2/2) by powers of two.
// ---------------------------------------------------------------------------
struct GeluErfOp {
    static constexpr bool kHasRare = true;
    static constexpr float kRareBelow = -6.0f;
    static constexpr float kLog2ef = 1.44269504088896341f;

    // Q(t) of the erfc form above (t in (0, 1]), degree 9.
    __device__ static float q_poly(float t)
    {
        float p = 0.17087277f;
        p = fmaf(t, p, -0.82215223f);
        p = fmaf(t, p, 1.48851587f);
        p = fmaf(t, p, -1.13520398f);
        p = fmaf(t, p, 0.27886807f);
        p = fmaf(t, p, -0.18628806f);
        p = fmaf(t, p, 0.09678418f);
        p = fmaf(t, p, 0.37409196f);
        p = fmaf(t, p, 1.00002368f);
        return fmaf(t, p, -1.26551223f);
    }

    // Binary32 I/O: erfc(|x| / sqrt 2) / 2 and, through e2, e^(-x^2/2).
    // Both are below 2^-2900 beyond |x| = 64: clamping keeps x^2 finite (a
    // NaN x still reaches the caller's result through its own factor x).
    __device__ static float half_erfc_abs(float x, const Coef& k, float* e2)
    {
        float a = fminf(fabsf(x), 64.0f);
        float t = rcp_hw(fmaf(0.5f * kInvSqrt2f, a, 1.0f));
        float q = q_poly(t);
        float x2 = a * a;
        float vh = x2 * k.c_hi;  // -x^2 log2(e) / 2
        float vl = fmaf(x2, k.c_lo, fmaf(x2, k.c_hi, -vh)) + fmaf(a, a, -x2) * k.c_hi;
        float eq = exp2_hw(fmaf(q, kLog2ef, vh + vl));  // e^(-z^2 + Q(t))
        if (e2) {
            float e = exp2_hw(vh);
            *e2 = fmaf(e, vl * kLn2f, e);
        }
        return 0.5f * t * eq;
    }

    // Bfloat16 I/O: the same tail as 2^L(s), s = a / 3 - 1, a = |x| clamped
    // to [0, 6] (beyond 6 the tail is below every binary32 ulp of 1 - h),
    // L the Chebyshev interpolant of log2 h on that range computed by
    // gen_gelu_bf16_poly.py: degree 6 for the forward (relative error
    // 5e-5), degree 9 for the backward (3.4e-6; Phi + x phi cancels near
    // x = -0.752).  One exponential and no reciprocal.
    template <bool BWD>
    __device__ static float tail_short(float x)
    {
        const float s = fmaf(fminf(fabsf(x), 6.0f), 1.0f / 3.0f, -1.0f);
        float p;
        if (BWD) {
            p = 0.0008011838f;
            p = fmaf(s, p, -0.0000443616f);
            p = fmaf(s, p, -0.005935571f);
            p = fmaf(s, p, 0.016855113f);
            p = fmaf(s, p, -0.03940879f);
            p = fmaf(s, p, 0.09169615f);
            p = fmaf(s, p, -0.2043446f);
            p = fmaf(s, p, -6.033987f);
            p = fmaf(s, p, -14.20953f);
            p = fmaf(s, p, -9.532935f);
        } else {
            p = 0.016779546f;
            p = fmaf(s, p, -0.048049062f);
            p = fmaf(s, p, 0.09174274f);
            p = fmaf(s, p, -0.20028456f);
            p = fmaf(s, p, -6.034002f);
            p = fmaf(s, p, -14.210027f);
            p = fmaf(s, p, -9.532934f);
        }
        return exp2_hw(p);
    }

    template <bool P>
    __device__ static constexpr float rare_thr() { return -kRareBelow; }

    // Key of the rare test x < -6: -x, canonicalised.  A plain negation
    // keeps a signaling NaN signaling, and a maximum that meets one returns
    // NaN, which would hide the rare elements of the same vector (the
    // keys of the other activations come out of arithmetic, which quiets).
    __device__ static float rare_key(float x) { return __builtin_canonicalizef(-x); }

    template <bool P>
    __device__ static float fwd(float x, const Coef& k, float& rk)
    {
        float h = P ? half_erfc_abs(x, k, nullptr) : tail_short<false>(x);
        float cdf = x < 0.0f ? h : 1.0f - h;
        rk = fmaxf(rk, rare_key(x));
        return x * cdf;
    }

    template <bool P>
    __device__ static float bwd(float x, float dy, const Coef& k, float& rk)
    {
        float e2, h;
        if (P) {
            h = half_erfc_abs(x, k, &e2);
        } else {
            h = tail_short<true>(x);
            const float a = fminf(fabsf(x), 64.0f);
            e2 = exp2_hw(a * a * k.c_hi);
        }
        float cdf = x < 0.0f ? h : 1.0f - h;
        rk = fmaxf(rk, rare_key(x));
        // x = +inf: the limit 1 (the product x phi would be inf * 0).
        return x == INFINITY ? dy : dy * fmaf(x, e2 * kInvSqrt2Pif, cdf);
    }

    template <bool BWD, bool P>
    __device__ static bool is_rare(float x, const Coef&)
    {
        return x < kRareBelow;
    }

    // x < -6.  Phi(x) = g e^(-x^2/2) with g = t e^Q(t) / 2 (the erfc form
    // without its Gaussian factor), which is applied by powers of two from
    // the exact x^2.
    __device__ static void split(float x, const Coef& k, float& g, float& ef, int& kf, bool& zero)
    {
        float a = fabsf(x);
        float t = rcp_hw(fmaf(0.5f * kInvSqrt2f, a, 1.0f));
        g = 0.5f * t * exp2_hw(q_poly(t) * kLog2ef);
        float x2 = a * a;
        float vh = x2 * k.c_hi;
        float vl = fmaf(x2, k.c_lo, fmaf(x2, k.c_hi, -vh)) + fmaf(a, a, -x2) * k.c_hi;
        zero = vh < kZeroExp;
        if (!zero)
            pow2_split(vh, vl, ef, kf);
    }

    __device__ static float fwd_rare(float x, const Coef& k)
    {
        float g, ef;
        int kf;
        bool zero;
        split(x, k, g, ef, kf, zero);
        return zero ? copysignf(0.0f, x) : scale_pow2(x, g, ef, kf);  // -0 at -inf
    }

    // dx = dy (Phi + x phi) = dy e^(-x^2/2) (g + x / sqrt(2 pi)).
    __device__ static float bwd_rare(float x, float dy, const Coef& k)
    {
        float g, ef;
        int kf;
        bool zero;
        split(x, k, g, ef, kf, zero);
        return zero ? dy * -0.0f : scale_pow2(dy, fmaf(x, kInvSqrt2Pif, g), ef, kf);
    }
};

// ---------------------------------------------------------------------------
// GELU with the tanh approximation, as x sigmoid(2u): C = -2 sqrt(2/pi) log2 e
// on a = x (1 + 0.044715 x^2), E = e^-2u.  The binary32 exponent carries
// about 2 ulps of rounding; with binary32 I/O the fast path is used only
// where that stays far inside the tolerance (|v| <= 20), and the rare branch
// carries the exponent as an exact-to-2^-44 hi+lo pair.
// ---------------------------------------------------------------------------
struct GeluTanhOp {
    static constexpr bool kHasRare = true;
    static constexpr float kPreciseMaxExp = 20.0f;

    // Binary32 I/O: rare outside |v| <= 20 (exponent precision).  bfloat16
    // I/O: rare outside |v| <= 125 (range; also keeps x (1 - s) 2u' from
    // forming 0 * inf for huge x).
    template <bool P>
    __device__ static bool flag(float v)
    {
        return fabsf(v) > (P ? kPreciseMaxExp : kMaxExp);
    }

    template <bool P>
    __device__ static constexpr float rare_thr() { return P ? kPreciseMaxExp : kMaxExp; }

    template <bool P>
    __device__ static float fwd(float x, const Coef& k, float& rk)
    {
        float a = x * fmaf(k.aux_hi * x, x, 1.0f);
        float v;
        float e = exp2_lin<false>(a, k, v);
        rk = fmaxf(rk, fabsf(v));
        return x * rcp_hw(1.0f + e);
    }

    template <bool P>
    __device__ static float bwd(float x, float dy, const Coef& k, float& rk)
    {
        float a = x * fmaf(k.aux_hi * x, x, 1.0f);
        float v;
        float e = exp2_lin<false>(a, k, v);
        float s = rcp_hw(1.0f + e);
        float c = e * s;                                               // 1 - s
        float du2 = kGeluTanhK * fmaf(3.0f * k.aux_hi * x, x, 1.0f);  // 2 u'
        float g = fmaf(x * c, du2, 1.0f);
        rk = fmaxf(rk, fabsf(v));
        return dy * (s * g);
    }

    template <bool BWD, bool P>
    __device__ static bool is_rare(float x, const Coef& k)
    {
        float a = x * fmaf(k.aux_hi * x, x, 1.0f);
        return flag<P>(a * k.c_hi);
    }

    // v = C (x + 0.044715 x^3) as vh + vl.
    __device__ static void exponent(float x, const Coef& k, float& vh, float& vl)
    {
        float x2 = x * x, x2e = fmaf(x, x, -x2);
        float p = k.aux_hi * x2;
        float pe = fmaf(k.aux_hi, x2, -p) + fmaf(k.aux_hi, x2e, k.aux_lo * x2);
        float q = 1.0f + p;  // two-sum of 1 and p
        float bb = q - 1.0f;
        float qe = ((1.0f - (q - bb)) + (p - bb)) + pe;
        float a = x * q;
        float ae = fmaf(x, q, -a) + x * qe;
        vh = k.c_hi * a;
        vl = fmaf(k.c_hi, a, -vh) + fmaf(k.c_hi, ae, k.c_lo * a);
    }

    __device__ static float fwd_rare(float x, const Coef& k)
    {
        float vh, vl;
        exponent(x, k, vh, vl);
        if (vh < -kMaxExp)
            return x;  // sigmoid(2u) rounds to 1
        if (vh > kMaxExp) {
            if (-vh < kZeroExp)
                return copysignf(0.0f, x);  // also the limit at x = -inf
            float ef;
            int kf;
            pow2_split(-vh, -vl, ef, kf);  // sigmoid(2u) = e^2u
            return scale_pow2(x, 1.0f, ef, kf);
        }
        float e = exp2_hw(vh);
        e = fmaf(e, vl * kLn2f, e);
        return x * rcp_hw(1.0f + e);
    }

    __device__ static float bwd_rare(float x, float dy, const Coef& k)
    {
        float vh, vl;
        exponent(x, k, vh, vl);
        float du2 = kGeluTanhK * fmaf(3.0f * k.aux_hi * x, x, 1.0f);
        if (vh < -kMaxExp)
            return dy;
        if (vh > kMaxExp) {
            if (-vh < kZeroExp)
                return dy * -0.0f;
            float ef;
            int kf;
            pow2_split(-vh, -vl, ef, kf);
            // s = e^2u, 1 - s rounds to 1: dx = dy e^2u (1 + x 2u').
            return scale_pow2(dy, fmaf(x, du2, 1.0f), ef, kf);
        }
        float e = exp2_hw(vh);
        e = fmaf(e, vl * kLn2f, e);
        float s = rcp_hw(1.0f + e);
        float g = fmaf(x * (e * s), du2, 1.0f);
        return dy * (s * g);
    }
};

template <int ACT> struct ActOp;
template <> struct ActOp<kSwish> : SwishOp {};
template <> struct ActOp<kRelu> : ReluOp {};
template <> struct ActOp<kLeakyRelu> : LeakyReluOp {};
template <> struct ActOp<kSigmoid> : SigmoidOp {};
template <> struct ActOp<kTanh> : TanhOp {};
template <> struct ActOp<kGeluErf> : GeluErfOp {};
template <> struct ActOp<kGeluTanh> : GeluTanhOp {};
template <> struct ActOp<kSwishUnit> : SwishOpT<true> {};

}  // namespace meswish
