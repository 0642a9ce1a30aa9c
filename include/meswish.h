/*
 * meswish.h -- C ABI of libmeswish, the memory-efficient Swish activation
 * for AMD Instinct MI355X (gfx950).
 *
 * The operation (cited by page title and section):
 *
 *   [P1] blog post "Memory efficient Swish" (adeeplearner.github.io,
 *        2021-05-17).
 *        - "What is a Swish activation function?" and "How is Swish
 *          implemented?": Swish(x) = x * Sigmoid(alpha x), with
 *          Sigmoid(t) = 1 / (1 + e^-t) and a slope alpha that defaults to 1.
 *        - "How is the memory efficient version Swish implemented?" and
 *          "What makes this implementation save GPU memory?": the forward
 *          keeps only the input; the backward recomputes s = Sigmoid(t) from
 *          it and returns dx = dy * s * (1 + t (1 - s)).  The page writes this
 *          for alpha = 1; with t = alpha x it is the product-rule derivative
 *          of x * Sigmoid(alpha x) for any alpha.
 *        - "Why simple Swish implementation is inefficient?": the plain
 *          module keeps three feature maps (input, sigmoid, product) for the
 *          backward; this library's callers keep one (the input).
 *   [P3] "What activations cost, in memory and in arithmetic", Conclusion:
 *        an activation reads and writes its tensor once and does a handful
 *        of flops per element, so it is bound by memory bandwidth.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Tensors are contiguous 1-D views of n elements (any logical shape,
 *   flattened).  All pointers are DEVICE pointers owned by the caller; the
 *   library allocates, frees and synchronises nothing.
 * - dtype is MESWISH_F32 (binary32) or MESWISH_BF16 (bfloat16).  Input and
 *   output share the dtype.  Arithmetic is binary32 in every case; outputs
 *   are rounded to nearest even, subnormals kept.
 * - alpha is a finite binary32 value (any sign) whose product with log2 e
 *   is finite in binary32: |alpha| <= about 2.3586e38 (larger values return
 *   MESWISH_EINVAL; the sigmoid is evaluated as 1 / (1 + 2^(x C)) with
 *   C = -alpha log2 e).
 * - Calls are asynchronous: they enqueue kernels on `stream` (a hipStream_t;
 *   NULL means the default stream) and return once the work is enqueued.
 *   Faults inside a kernel surface at the caller's next synchronisation.
 * - Any 16-byte alignment of the pointers gives the vectorised path when
 *   all pointers of a tensor share it; otherwise an element-wise path runs.
 *   Element alignment (4 bytes for binary32, 2 for bfloat16) is required.
 * - Aliasing: an output may coincide exactly with an input of the same
 *   tensor (in place); any other overlap of an output with an input or with
 *   another output returns MESWISH_EALIAS and launches nothing.
 * - n == 0 (or count == 0) is a no-op that returns MESWISH_OK.
 * - Errors are returned as status codes, never thrown; on any error
 *   nothing is launched.
 * - Stateless and reentrant: concurrent calls on different streams are safe
 *   as long as their buffers do not overlap.
 */
#ifndef MESWISH_H
#define MESWISH_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types. */
typedef enum { MESWISH_F32 = 0, MESWISH_BF16 = 1 } meswish_dtype;

/* Status codes. */
typedef enum {
    MESWISH_OK = 0,
    MESWISH_EINVAL = 1,   /* NULL pointer with n > 0, unknown dtype,
                             non-finite alpha (or, for Swish, |alpha| log2 e
                             beyond binary32), misaligned element pointer,
                             negative count, n too large */
    MESWISH_EALIAS = 2,   /* an output overlaps an input or another output
                             other than by exact, same-tensor coincidence */
    MESWISH_EHIP = 3,     /* the HIP runtime reported an error at launch */
    MESWISH_ETOOMANY = 4, /* grouped call with count > MESWISH_MAX_GROUP */
    MESWISH_ESCRATCH = 5  /* a call without a workspace needs more than the
                             library's static device array holds */
} meswish_status;

/* Largest number of tensors one grouped call accepts (one launch). */
#define MESWISH_MAX_GROUP 64

/*
 * Forward, [P1] "How is Swish implemented?":
 *     y[i] = x[i] * Sigmoid(alpha * x[i]),  i in [0, n).
 * x: n elements of dtype (read).  y: n elements of dtype (written);
 * y == x is allowed (in place -- then the caller must not need x for the
 * backward).  Nothing else is written: the caller keeps x for the backward.
 */
int swish_fwd(const void *x, void *y, size_t n, float alpha, int dtype,
              void *stream);

/*
 * Backward from the saved input alone, [P1] "How is the memory efficient
 * version Swish implemented?":
 *     t = alpha * x[i],  s = Sigmoid(t),
 *     dx[i] = dy[i] * s * (1 + t * (1 - s)).
 * x, dy: n elements of dtype (read; they may overlap each other freely).
 * dx: n elements of dtype (written); dx == x or dx == dy is allowed.
 * The gradient with respect to alpha is not produced (alpha is a fixed
 * hyper-parameter of the module).
 */
int swish_bwd(const void *x, const void *dy, void *dx, size_t n, float alpha,
              int dtype, void *stream);

/*
 * The activation family of "What activations cost, in memory and in
 * arithmetic" (Given), each with the save-the-input scheme of [P1] "How is
 * the memory efficient version Swish implemented?": the forward writes y
 * only; the backward recomputes what it needs from x and reads dy.
 * Definitions (param: alpha of Swish, negative slope of LeakyReLU; ignored
 * by the others but must be finite):
 */
typedef enum {
    MESWISH_ACT_SWISH = 0,      /* x sigmoid(param x)                        */
    MESWISH_ACT_RELU = 1,       /* x > 0 ? x : 0        (derivative 0 at 0)  */
    MESWISH_ACT_LEAKY_RELU = 2, /* x > 0 ? x : param x  (derivative param at 0) */
    MESWISH_ACT_SIGMOID = 3,    /* 1 / (1 + e^-x)                            */
    MESWISH_ACT_TANH = 4,       /* tanh x                                    */
    MESWISH_ACT_GELU_ERF = 5,   /* x Phi(x) = x (1 + erf(x / sqrt 2)) / 2    */
    MESWISH_ACT_GELU_TANH = 6   /* x (1 + tanh(sqrt(2/pi)(x + 0.044715 x^3))) / 2 */
} meswish_act;

/*
 * y[i] = f(x[i]) and dx[i] = dy[i] f'(x[i]) for the activation `act`, with
 * the conventions of swish_fwd / swish_bwd (which equal these calls with
 * MESWISH_ACT_SWISH).  Unknown act -> MESWISH_EINVAL.  NaN in x or dy gives
 * NaN out.
 */
int meswish_act_fwd(int act, const void *x, void *y, size_t n, float param,
                    int dtype, void *stream);
int meswish_act_bwd(int act, const void *x, const void *dy, void *dx,
                    size_t n, float param, int dtype, void *stream);

/* One tensor of a grouped forward. */
typedef struct {
    const void *x;
    void *y;
    size_t n;
} meswish_fwd_desc;

/* One tensor of a grouped backward. */
typedef struct {
    const void *x;
    const void *dy;
    void *dx;
    size_t n;
} meswish_bwd_desc;

/*
 * Grouped variants (Swish): the same operation on `count` tensors that share alpha
 * and dtype, in ONE kernel launch (for a network's many small activations,
 * e.g. the feature maps of an EfficientNet that the blog post measures in
 * "How much GPU memory is saved?").  `desc` is a HOST array of `count`
 * descriptors; it is read during the call only.  0 <= count <=
 * MESWISH_MAX_GROUP, else MESWISH_ETOOMANY (count > max) or MESWISH_EINVAL
 * (count < 0, desc NULL with count > 0).  Every element is computed exactly
 * as by swish_fwd / swish_bwd (results are bitwise identical).  Outputs of
 * different descriptors must not overlap any input or output of another
 * descriptor.
 */
int swish_fwd_grouped(const meswish_fwd_desc *desc, int count, float alpha,
                      int dtype, void *stream);
int swish_bwd_grouped(const meswish_bwd_desc *desc, int count, float alpha,
                      int dtype, void *stream);

/* Static, NUL-terminated description of a status code. */
const char *meswish_strerror(int status);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int meswish_version(void);

/* Kernel path a single-tensor call takes (see meswish_plan). */
typedef enum {
    MESWISH_PATH_NONE = -1,   /* nothing to launch (n == 0 or an error) */
    MESWISH_PATH_VECTOR = 0,  /* 16-byte vectors; scalar head and tail */
    MESWISH_PATH_ELEMENT = 1  /* pointers not congruent modulo 16 bytes */
} meswish_path;

/* Launch plan of a single-tensor call. */
typedef struct {
    int path;                   /* meswish_path */
    long long head;             /* elements before the first 16-byte boundary */
    long long nvec;             /* 16-byte vectors of the body */
    long long tail;             /* elements after the body (all n on the element path) */
    long long tiles;            /* work tiles (one block each) */
    long long grid;             /* blocks per launch (grid x block < 2^32) */
    long long block;            /* threads per block */
    long long elems_per_vector; /* 4 (binary32) or 8 (bfloat16) */
    long long vectors_per_tile; /* 16-byte vectors per tile */
    long long launches;         /* kernel launches (vector path: one per 2^30 tiles) */
} meswish_plan_t;

/*
 * Introspection of the host logic, for tests and tools: runs exactly the
 * argument checks of swish_fwd (bwd == 0; dy ignored) or swish_bwd
 * (bwd != 0) and, on success, fills *plan with the split those calls would
 * launch.  Launches nothing and never dereferences x, dy or out (it may
 * query the current device's compute-unit count).
 * Returns the status the call would return (MESWISH_EHIP excepted);
 * MESWISH_EINVAL if plan is NULL.  n == 0 gives MESWISH_OK with
 * path MESWISH_PATH_NONE.
 */
int meswish_plan(const void *x, const void *dy, const void *out, size_t n,
                 float alpha, int dtype, int bwd, meswish_plan_t *plan);

/*
 * Measurement helper (not part of the operation): a plain 16-byte-vector
 * device copy of `bytes` bytes from src to dst on `stream`, used to measure
 * the practical bandwidth ceiling of the same access pattern and to
 * calibrate hardware byte counters.  src and dst must be 16-byte aligned,
 * bytes a multiple of 16, and the ranges must not overlap.
 */
int meswish_copy(const void *src, void *dst, size_t bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MESWISH_H */
