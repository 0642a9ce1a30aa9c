/*
 * swish_oracle.c -- CPU oracle for the memory-efficient Swish activation.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously correct
 * definition that the GPU library is checked against.  Only the test suite,
 * the smoke check and the CPU-baseline leg of the benchmark may load it; the
 * product path (libmeswish and its Python binding) never does.  It shares no
 * code, header, table or constant with the GPU path.
 *
 * Everything is evaluated in IEEE binary64 (double) and rounded once, to
 * nearest-even, to the output type.  Build with gcc, no -ffast-math, with
 * -ffp-contract=off so that no fused multiply-add changes the rounding.
 *
 * Sources (the pages, cited by title and section):
 *   [P1] blog post "Memory efficient Swish" (adeeplearner.github.io,
 *        2021-05-17):
 *        - "What is a Swish activation function?": Swish(x) = x * Sigmoid(x),
 *          Sigmoid(x) = 1 / (1 + e^-x).
 *        - "How is Swish implemented?": the module multiplies the input by
 *          the sigmoid of alpha times the input (alpha defaults to 1.0).
 *        - "How is the memory efficient version Swish implemented?": forward
 *          saves only the input; backward recomputes the sigmoid s of the
 *          input and returns grad_output * s * (1 + input * (1 - s)).
 *        - "What makes this implementation save GPU memory?": that gradient
 *          is obtained by the product rule and depends on x alone.
 *   [P3] "What activations cost, in memory and in arithmetic", Step 1 and
 *        Step 2: element counts and bytes of one activation tensor.
 *
 * Readings where the pages leave a step open:
 *   - alpha in the backward: the memory-efficient code is written for
 *     alpha = 1.  For general alpha the product rule applied to
 *     x * Sigmoid(alpha x) gives s + alpha x s (1 - s) = s (1 + t (1 - s))
 *     with t = alpha x and s = Sigmoid(t); at alpha = 1 this is the printed
 *     expression term for term.
 *   - alpha is a binary32 value; the oracle uses it exactly, (double)alpha.
 *   - rounding of outputs: to nearest, ties to even, with gradual underflow,
 *     for binary32 and for bfloat16 alike.
 *   - bfloat16 is rounded directly from the binary64 value (never through
 *     binary32), so the oracle never rounds twice.
 *   - x = +-inf: the limits as x -> +-inf, with the parameter fixed (a
 *     zero alpha of Swish or zero slope of LeakyReLU keeps IEEE 0 * inf =
 *     NaN); see swish_limit below.
 *
 * Data layout: contiguous 1-D arrays.  dtype 0 = binary32 (float),
 * dtype 1 = bfloat16 stored as its 16-bit pattern (the upper half of the
 * binary32 pattern).  Multi-threading only splits the index range into
 * contiguous pieces; every element is computed by the same scalar code.
 */
#include <math.h>
#include <pthread.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#define ORACLE_F32 0
#define ORACLE_BF16 1

/* ------------------------------------------------------------------ */
/* Input widening: exact.                                              */
/* ------------------------------------------------------------------ */

static double widen_bf16(uint16_t bits)
{
    /* A bfloat16 pattern is the high half of a binary32 pattern. */
    uint32_t w = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return (double)f;
}

static double load(int dtype, const void *p, size_t i)
{
    if (dtype == ORACLE_F32)
        return (double)((const float *)p)[i];
    return widen_bf16(((const uint16_t *)p)[i]);
}

/* ------------------------------------------------------------------ */
/* Output rounding: round to nearest, ties to even.                   */
/* ------------------------------------------------------------------ */

float oracle_round_f32(double v)
{
    /* C's conversion from double to float rounds according to the current
     * rounding mode, which is left at its default (to nearest, ties to
     * even); it produces binary32 subnormals (gradual underflow) and
     * keeps the sign of zero. */
    return (float)v;
}

uint16_t oracle_round_bf16(double v)
{
    /* bfloat16: 8 exponent bits (same range as binary32) and 7 stored
     * fraction bits.  Its spacing at a value of exponent k is 2^(k-7); the
     * smallest exponent used for spacing is -126, which gives the
     * subnormals down to 2^-133. */
    uint16_t sign = signbit(v) ? 0x8000u : 0u;
    double a = fabs(v);
    if (isnan(v))
        return (uint16_t)(sign | 0x7FC0u);
    if (isinf(v))
        return (uint16_t)(sign | 0x7F80u);
    if (a == 0.0)
        return sign;
    int k = ilogb(a);
    if (k < -126)
        k = -126;
    double spacing = ldexp(1.0, k - 7);
    /* a / spacing is exact (division by a power of two within range);
     * nearbyint rounds it to the nearest integer, ties to even, in the
     * default rounding mode. */
    double r = nearbyint(a / spacing) * spacing;
    /* r is now a bfloat16 value, or 2^128 when the rounding carried past
     * the largest finite bfloat16; converting to binary32 is exact in the
     * first case and gives infinity in the second. */
    float f = (float)r;
    uint32_t w;
    memcpy(&w, &f, sizeof w);
    return (uint16_t)(sign | (uint16_t)(w >> 16));
}

static void store(int dtype, void *p, size_t i, double v)
{
    if (dtype == ORACLE_F32)
        ((float *)p)[i] = oracle_round_f32(v);
    else
        ((uint16_t *)p)[i] = oracle_round_bf16(v);
}

/* Round n binary64 values once to the output type (binary32 or bfloat16
 * bit patterns).  Used by the oracles whose arithmetic is written in numpy,
 * so that every oracle rounds through the same pinned routines. */
void oracle_round_n(int dtype, const double *v, void *out, size_t n)
{
    for (size_t i = 0; i < n; ++i)
        store(dtype, out, i, v[i]);
}

/* ------------------------------------------------------------------ */
/* The function and its derivative, in binary64.                      */
/* ------------------------------------------------------------------ */

/* Sigmoid(t) = 1 / (1 + e^-t)  ([P1] "What is a Swish activation
 * function?").  For t below about -709, e^-t overflows to +inf and the
 * quotient is +0, which is Sigmoid(t) rounded; no finite input gives NaN. */
double oracle_sigmoid(double t)
{
    return 1.0 / (1.0 + exp(-t));
}

/* Infinite inputs (reading of the pages, which define the functions on the
 * reals only): the value and dy times the derivative at x = +-inf are their
 * limits as x -> +-inf with the parameter held fixed.  Written out because
 * the finite formulas form 0 * inf there.  For Swish, with t = alpha x:
 *   t -> +inf: Sigmoid(t) -> 1, the value tends to x and the derivative
 *              s (1 + t (1 - s)) to 1 (t e^-t -> 0);
 *   t -> -inf: the value x e^t and the derivative e^t (1 + t) tend to 0,
 *              with the sign of x and a negative sign respectively.
 * alpha = 0 leaves t = 0 * inf, which stays NaN as in IEEE arithmetic. */
static double swish_limit(double x, double alpha)
{
    double t = alpha * x;
    if (isnan(t))
        return t;
    return t > 0.0 ? x : copysign(0.0, x);
}

static double swish_grad_limit(double x, double dy, double alpha)
{
    double t = alpha * x;
    if (isnan(t))
        return t;
    return t > 0.0 ? dy : dy * -0.0;
}

/* Swish with slope alpha: x * Sigmoid(alpha x)  ([P1] "How is Swish
 * implemented?"). */
double oracle_swish(double x, double alpha)
{
    if (isinf(x))
        return swish_limit(x, alpha);
    return x * oracle_sigmoid(alpha * x);
}

/* Gradient of the input for upstream gradient dy, recomputed from x alone
 * ([P1] "How is the memory efficient version Swish implemented?" and "What
 * makes this implementation save GPU memory?"):
 *     dx = dy * s * (1 + t * (1 - s)),   t = alpha x,  s = Sigmoid(t).
 * If scale is not NULL it receives the magnitude of the same expression
 * with every term taken positive,
 *     |dy| * s * (1 + |t| * (1 - s)),
 * which bounds the rounding error of any evaluation of the sum (used as the
 * error scale where 1 + t (1 - s) cancels). */
double oracle_swish_grad(double x, double dy, double alpha, double *scale)
{
    if (isinf(x)) {
        double g = swish_grad_limit(x, dy, alpha);
        if (scale)
            *scale = fabs(g);
        return g;
    }
    double t = alpha * x;
    double s = oracle_sigmoid(t);
    double one_minus_s = 1.0 - s;
    if (scale)
        *scale = fabs(dy) * s * (1.0 + fabs(t) * one_minus_s);
    return dy * s * (1.0 + t * one_minus_s);
}

/* ------------------------------------------------------------------ */
/* The activation family of [P3] "What activations cost, in memory and */
/* in arithmetic", Given: ReLU, LeakyReLU, sigmoid, tanh, GELU with    */
/* erf and GELU with the tanh approximation.  The page names them and  */
/* their flop counts; the definitions are the standard ones:           */
/*   ReLU(x)      = x if x > 0 else 0,  derivative 1 if x > 0 else 0   */
/*   LeakyReLU(x) = x if x > 0 else a x, derivative 1 if x > 0 else a  */
/*   sigmoid(x)   = 1 / (1 + e^-x),     derivative s (1 - s)           */
/*   tanh(x),                           derivative 1 / cosh(x)^2       */
/*   GELU(x)      = x Phi(x), Phi the standard normal CDF,             */
/*                  derivative Phi(x) + x phi(x), phi its density      */
/*   GELU_tanh(x) = x (1 + tanh(u)) / 2, u = sqrt(2/pi)(x + 0.044715x^3)*/
/* Where a textbook form would lose everything to cancellation in      */
/* binary64 it is replaced by an exact identity:                        */
/*   1 - sigmoid(x) = sigmoid(-x)  (the add-and-subtract-one step of   */
/*                                 [P1] "What makes this               */
/*                                 implementation save GPU memory?")   */
/*   Phi(x) = erfc(-x / sqrt 2) / 2                                    */
/*   (1 + tanh(u)) / 2 = sigmoid(2u)                                   */
/*   1 - tanh(x)^2 = 1 / cosh(x)^2                                     */
/* ------------------------------------------------------------------ */

#define ORACLE_ACT_SWISH 0
#define ORACLE_ACT_RELU 1
#define ORACLE_ACT_LEAKY_RELU 2
#define ORACLE_ACT_SIGMOID 3
#define ORACLE_ACT_TANH 4
#define ORACLE_ACT_GELU_ERF 5
#define ORACLE_ACT_GELU_TANH 6

static const double kInvSqrt2 = 0.70710678118654752440084436210484904;
static const double kInvSqrt2Pi = 0.39894228040143267793994605993438187;
static const double kSqrt2OverPi = 0.79788456080286535587989211986876374;
static const double kGeluTanhCubic = 0.044715;

static double std_normal_cdf(double x) { return 0.5 * erfc(-x * kInvSqrt2); }
static double std_normal_pdf(double x) { return kInvSqrt2Pi * exp(-0.5 * x * x); }

/* Value of activation `act` with parameter p (alpha of Swish, negative
 * slope of LeakyReLU; ignored by the others).  NaN in, NaN out. */
double oracle_act_f64(int act, double x, double p)
{
    if (isnan(x))
        return x;
    switch (act) {
    case ORACLE_ACT_SWISH:
        return oracle_swish(x, p);
    case ORACLE_ACT_RELU:
        return x > 0.0 ? x : 0.0;
    case ORACLE_ACT_LEAKY_RELU:
        return x > 0.0 ? x : p * x;
    case ORACLE_ACT_SIGMOID:
        return oracle_sigmoid(x);
    case ORACLE_ACT_TANH:
        return tanh(x);
    case ORACLE_ACT_GELU_ERF:
        if (isinf(x))  /* limits: x, and x Phi(x) -> -0 */
            return x > 0.0 ? x : -0.0;
        return x * std_normal_cdf(x);
    case ORACLE_ACT_GELU_TANH: {
        if (isinf(x))  /* limits: x, and x sigmoid(2u) -> -0 */
            return x > 0.0 ? x : -0.0;
        double u = kSqrt2OverPi * (x + kGeluTanhCubic * x * x * x);
        return x * oracle_sigmoid(2.0 * u);
    }
    default:
        return NAN;
    }
}

/* dy times the derivative of activation `act` at x, and (if scale is not
 * NULL) the same expression with every term of its sum taken positive --
 * the error scale for the sums that can cancel (Swish, GELU). */
double oracle_act_grad_f64(int act, double x, double dy, double p, double *scale)
{
    double g, m;
    if (isnan(x) || isnan(dy)) {
        if (scale)
            *scale = NAN;
        return NAN;
    }
    switch (act) {
    case ORACLE_ACT_SWISH:
        return oracle_swish_grad(x, dy, p, scale);
    case ORACLE_ACT_RELU:
        g = dy * (x > 0.0 ? 1.0 : 0.0);
        m = fabs(g);
        break;
    case ORACLE_ACT_LEAKY_RELU:
        g = dy * (x > 0.0 ? 1.0 : p);
        m = fabs(g);
        break;
    case ORACLE_ACT_SIGMOID:
        g = dy * oracle_sigmoid(x) * oracle_sigmoid(-x);
        m = fabs(g);
        break;
    case ORACLE_ACT_TANH: {
        double c = cosh(x);
        g = dy / (c * c);
        m = fabs(g);
        break;
    }
    case ORACLE_ACT_GELU_ERF: {
        if (isinf(x)) {  /* limits of Phi + x phi: 1 at +inf, -0 at -inf */
            g = x > 0.0 ? dy : dy * -0.0;
            m = fabs(g);
            break;
        }
        double cdf = std_normal_cdf(x), pdf = std_normal_pdf(x);
        g = dy * (cdf + x * pdf);
        m = fabs(dy) * (cdf + fabs(x) * pdf);
        break;
    }
    case ORACLE_ACT_GELU_TANH: {
        if (isinf(x)) {  /* limits of s (1 + x (1 - s) 2u'): 1 and -0 */
            g = x > 0.0 ? dy : dy * -0.0;
            m = fabs(g);
            break;
        }
        double u = kSqrt2OverPi * (x + kGeluTanhCubic * x * x * x);
        double du = kSqrt2OverPi * (1.0 + 3.0 * kGeluTanhCubic * x * x);
        double s = oracle_sigmoid(2.0 * u), c = oracle_sigmoid(-2.0 * u);
        g = dy * (s + x * s * c * 2.0 * du);
        m = fabs(dy) * (s + fabs(x) * s * c * 2.0 * du);
        break;
    }
    default:
        g = m = NAN;
    }
    if (scale)
        *scale = m;
    return g;
}

/* ------------------------------------------------------------------ */
/* Array drivers.                                                      */
/* ------------------------------------------------------------------ */

typedef struct {
    int act;
    int dtype;
    const void *x;
    const void *dy;
    void *out;
    double *scale;
    double alpha;
    size_t begin, end;
} oracle_job;

static void *fwd_range(void *arg)
{
    const oracle_job *j = (const oracle_job *)arg;
    for (size_t i = j->begin; i < j->end; ++i)
        store(j->dtype, j->out, i, oracle_act_f64(j->act, load(j->dtype, j->x, i), j->alpha));
    return NULL;
}

static void *bwd_range(void *arg)
{
    const oracle_job *j = (const oracle_job *)arg;
    for (size_t i = j->begin; i < j->end; ++i) {
        double m;
        double g = oracle_act_grad_f64(j->act, load(j->dtype, j->x, i),
                                       load(j->dtype, j->dy, i), j->alpha, &m);
        store(j->dtype, j->out, i, g);
        if (j->scale)
            j->scale[i] = m;
    }
    return NULL;
}

#define ORACLE_MAX_THREADS 256

/* Split [0, n) into `threads` contiguous pieces and run `fn` on each. */
static int run_split(void *(*fn)(void *), oracle_job base, size_t n, int threads)
{
    if (threads < 1)
        threads = 1;
    if (threads > ORACLE_MAX_THREADS)
        threads = ORACLE_MAX_THREADS;
    if ((size_t)threads > n)
        threads = n ? (int)n : 1;
    oracle_job jobs[ORACLE_MAX_THREADS];
    pthread_t tid[ORACLE_MAX_THREADS];
    int started[ORACLE_MAX_THREADS];
    for (int k = 0; k < threads; ++k) {
        jobs[k] = base;
        jobs[k].begin = n * (size_t)k / (size_t)threads;
        jobs[k].end = n * (size_t)(k + 1) / (size_t)threads;
        started[k] = 0;
    }
    for (int k = 1; k < threads; ++k)
        started[k] = pthread_create(&tid[k], NULL, fn, &jobs[k]) == 0;
    fn(&jobs[0]);
    int rc = 0;
    for (int k = 1; k < threads; ++k) {
        if (started[k])
            pthread_join(tid[k], NULL);
        else {
            fn(&jobs[k]); /* could not start a thread: do the piece here */
            rc = 1;
        }
    }
    return rc;
}

/* y[i] = round(x[i] * Sigmoid(alpha x[i])) for i in [0, n).
 * Returns 0, or -1 for an unknown dtype. */
int oracle_swish_fwd(int dtype, const void *x, void *y, size_t n, float alpha,
                     int threads)
{
    if (dtype != ORACLE_F32 && dtype != ORACLE_BF16)
        return -1;
    oracle_job j = {ORACLE_ACT_SWISH, dtype, x, NULL, y, NULL, (double)alpha, 0, 0};
    run_split(fwd_range, j, n, threads);
    return 0;
}

/* dx[i] = round(dy[i] * s (1 + t (1 - s))) with t = alpha x[i], s = Sigmoid(t).
 * scale (may be NULL) receives the binary64 error scale of each element.
 * Returns 0, or -1 for an unknown dtype. */
int oracle_swish_bwd(int dtype, const void *x, const void *dy, void *dx,
                     double *scale, size_t n, float alpha, int threads)
{
    if (dtype != ORACLE_F32 && dtype != ORACLE_BF16)
        return -1;
    oracle_job j = {ORACLE_ACT_SWISH, dtype, x, dy, dx, scale, (double)alpha, 0, 0};
    run_split(bwd_range, j, n, threads);
    return 0;
}

/* The same drivers for any activation of the family; p is the activation's
 * parameter as a binary32 value.  Returns -1 for an unknown act or dtype. */
int oracle_act_fwd(int act, int dtype, const void *x, void *y, size_t n, float p,
                   int threads)
{
    if (dtype != ORACLE_F32 && dtype != ORACLE_BF16)
        return -1;
    if (act < ORACLE_ACT_SWISH || act > ORACLE_ACT_GELU_TANH)
        return -1;
    oracle_job j = {act, dtype, x, NULL, y, NULL, (double)p, 0, 0};
    run_split(fwd_range, j, n, threads);
    return 0;
}

int oracle_act_bwd(int act, int dtype, const void *x, const void *dy, void *dx,
                   double *scale, size_t n, float p, int threads)
{
    if (dtype != ORACLE_F32 && dtype != ORACLE_BF16)
        return -1;
    if (act < ORACLE_ACT_SWISH || act > ORACLE_ACT_GELU_TANH)
        return -1;
    oracle_job j = {act, dtype, x, dy, dx, scale, (double)p, 0, 0};
    run_split(bwd_range, j, n, threads);
    return 0;
}

/* Binary64 results of the two drivers above, unrounded, for the checks that
 * pin the oracle (one element per call; slow on purpose). */
double oracle_swish_fwd_f64(double x, double alpha)
{
    return oracle_swish(x, alpha);
}

double oracle_swish_bwd_f64(double x, double dy, double alpha, double *scale)
{
    return oracle_swish_grad(x, dy, alpha, scale);
}
