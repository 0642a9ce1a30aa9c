/*
 * dense_bn.h -- C ABI of libmeswish's shared-buffer DenseNet layer stage
 * for AMD Instinct MI355X (gfx950).
 *
 * The operation (README of efficient_densenet_pytorch, "A memory-efficient
 * implementation of DenseNets", section Motivation): a DenseNet layer
 * concatenates every earlier feature map along the channel axis and applies
 * batch normalization and ReLU before its convolution.  Stored per layer,
 * these intermediate maps grow quadratically with depth; the efficient
 * implementation writes them into shared memory that every layer reuses and
 * re-populates them in the backward pass, so that only the (linear) layer
 * outputs are kept.
 *
 * Per layer, with sources x_j of shape [n, C_j, hw] (NCHW, hw = H * W)
 * placed at channels offset_j .. offset_j + C_j - 1 of the concatenation:
 *
 *     mean_c, var_c  batch statistics of channel c over (n, hw), biased
 *                    variance (training-mode batch normalization)
 *     xhat = (x - mean_c) / sqrt(var_c + eps)
 *     z    = ReLU(gamma_c xhat + beta_c)                         (forward)
 *
 *     g      = dz where gamma_c xhat + beta_c > 0, else 0
 *     dbeta  = sum g,  dgamma = sum g xhat   (over n and hw)
 *     dx     = gamma_c / sqrt(var_c + eps) (g - dbeta / M - xhat dgamma / M),
 *              M = n hw                                        (backward)
 *
 * The concatenation is never materialised: the forward reads the sources
 * in place and writes z, the one shared map of the forward; the backward
 * reads the sources and dz (the shared map of the backward) and writes
 * each source's gradient.  Channel statistics depend on one source only,
 * so they are computed once per feature map (dense_bn_stats) and reused by
 * every later layer.
 *
 * Conventions (as in meswish.h): device pointers owned by the caller, no
 * allocation or synchronisation, asynchronous on `stream` (a hipStream_t,
 * NULL = default stream), status codes from meswish_status, nothing
 * launched on an error.  dtype is MESWISH_F32 or MESWISH_BF16 for every
 * feature map of a call (x, z, dz, dx); gamma, beta, dgamma, dbeta are
 * binary32; statistics are binary64.  Arithmetic is binary32 per element
 * with binary64 statistics, reductions and ReLU thresholds.  Results are
 * deterministic: reductions have a fixed order.
 *
 * Limits: n * hw (elements per channel) in [1, 2^31); hw < 2^31; at most
 * DENSE_BN_MAX_SOURCES sources per call.  A layer with more sources is
 * computed by several calls over disjoint sources (channels are
 * independent).  Inputs must be finite.
 */
#ifndef DENSE_BN_H
#define DENSE_BN_H

#include <stddef.h>

#include "meswish.h"

#ifdef __cplusplus
extern "C" {
#endif

#define DENSE_BN_MAX_SOURCES 64

/* One source feature map of a layer. */
typedef struct {
    const void *x;        /* [n, channels, hw] of dtype (read) */
    void *dx;             /* [n, channels, hw] of dtype: its gradient
                             (written by dense_bn_relu_bwd; unused by the
                             forward, may be NULL there) */
    const double *stats;  /* [channels][2] = {mean, variance} of x, as
                             written by dense_bn_stats (read) */
    int channels;         /* C_j >= 1 */
    int offset;           /* first channel of this source in z, dz, gamma,
                             beta, dgamma, dbeta */
} dense_bn_source;

/* Bytes of workspace dense_bn_stats and dense_bn_relu_bwd need for
 * `channels` channels of n * hw elements each (channels of one source for
 * the statistics; the sum of the sources' channels for the backward).
 * 0 if the sizes are out of range. */
size_t dense_bn_workspace_bytes(size_t n, size_t channels, size_t hw);

/*
 * Batch statistics of one feature map x [n, channels, hw]:
 *     stats[2 c]     = mean of x[:, c, :]
 *     stats[2 c + 1] = mean of (x[:, c, :] - mean)^2
 * accumulated in binary64 about a per-channel pivot (the channel's first
 * element), in a fixed order.  workspace: device memory of at least
 * dense_bn_workspace_bytes(n, channels, hw) bytes, 8-byte aligned,
 * overwritten.  stats must not overlap x or the workspace.
 */
int dense_bn_stats(const void *x, size_t n, int channels, size_t hw, int dtype,
                   double *stats, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Forward of the layer stage, README "A memory-efficient implementation of
 * DenseNets", Motivation:
 *     z[:, offset_j + c, :] = ReLU(gamma (x_j[:, c, :] - mean) r + beta),
 *     r = 1 / sqrt(var + eps),
 * for every source j of src[0 .. count-1] and channel c of it, with
 * gamma, beta taken at channel offset_j + c.  z: [n, z_channels, hw] of
 * dtype, written only at the sources' channels.  The sources' channel
 * ranges in z must be disjoint and lie in [0, z_channels); z must not
 * overlap any source.  eps: finite, > 0.  count in [0, 64]; count == 0 is
 * a no-op.
 */
int dense_bn_relu_fwd(const dense_bn_source *src, int count, size_t n, size_t hw,
                      int z_channels, const float *gamma, const float *beta, float eps,
                      void *z, int dtype, void *stream);

/*
 * Backward of the layer stage, recomputed from the sources (nothing of the
 * forward is kept but the statistics): for every source j and channel c,
 * with k = offset_j + c,
 *     g  = dz[:, k, :] where gamma_k (x - mean) r + beta_k > 0, else 0
 *     dbeta[k]  = sum g,   dgamma[k] = sum g xhat
 *     dx_j[:, c, :] = gamma_k r (g - dbeta[k] / M - xhat dgamma[k] / M)
 * dz: [n, z_channels, hw] of dtype (read).  dgamma, dbeta: z_channels
 * binary32 values, written at the sources' channels.  workspace: at least
 * dense_bn_workspace_bytes(n, sum of the sources' channels, hw) bytes,
 * 8-byte aligned, overwritten.  Every dx_j must be non-NULL and must not
 * overlap any source, dz, another dx, the workspace or the parameter
 * arrays.
 */
int dense_bn_relu_bwd(const dense_bn_source *src, int count, size_t n, size_t hw,
                      int z_channels, const float *gamma, const float *beta, float eps,
                      const void *dz, float *dgamma, float *dbeta,
                      void *workspace, size_t workspace_bytes, int dtype, void *stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the
 * backward of dense_bn_relu_bwd without a workspace argument.  Its
 * per-block partial sums go to a static device array of
 * DENSE_BN_STATIC_WORKSPACE_BYTES bytes that the library holds on each GPU
 * it runs on, until the process ends; the call itself allocates, frees and
 * synchronises nothing.  Same arguments, checks and results (bit for bit)
 * as dense_bn_relu_bwd otherwise.  A call that needs more than the array
 * holds -- dense_bn_workspace_bytes(n, sum of the sources' channels, hw) >
 * DENSE_BN_STATIC_WORKSPACE_BYTES, e.g. more than 262,144 channel-chunks of
 * 4096 elements -- returns MESWISH_ESCRATCH and launches nothing.  Every
 * call on one GPU shares that GPU's array: calls that may run at the same
 * time on one GPU (on different streams) race and must be ordered by the
 * caller.  MESWISH_EHIP if the array's address cannot be looked up.
 */
#define DENSE_BN_STATIC_WORKSPACE_BYTES ((size_t)4 << 20)

int dense_bn_relu_bwd_noalloc(const dense_bn_source *src, int count, size_t n, size_t hw,
                              int z_channels, const float *gamma, const float *beta, float eps,
                              const void *dz, float *dgamma, float *dbeta, int dtype,
                              void *stream);

#ifdef __cplusplus
}
#endif

#endif /* DENSE_BN_H */
