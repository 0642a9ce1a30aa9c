/*
 * fft_conv.h -- C ABI of libmeswish's FFT convolution layers for AMD
 * Instinct MI355X (gfx950).
 *
 * The method ("Fast Training of Convolutional Networks through FFTs",
 * sections on backpropagation, the convolution theorem, the algorithm, the
 * GPU implementation and memory): a convolution layer with input maps
 * x[s, f] (n x n), kernels w[f', f] (k x k) and outputs y[s, f'] (n' x n',
 * n' = n - k + 1) computes
 *
 *   forward         y[s,f',i,j]  = sum_{f,a,b}  x[s,f,i+a,j+b] w[f',f,a,b]
 *   input gradient  gx[s,f,p,q]  = sum_{f',a,b} g[s,f',p-a,q-b] w[f',f,a,b]
 *   weight gradient gw[f',f,a,b] = sum_{s,i,j}  x[s,f,i+a,j+b] g[s,f',i,j]
 *
 * (g = dL/dy).  Every map is transformed once by a 2-D FFT on n x n, every
 * pairing of an f-indexed with an f'-indexed map becomes a product in the
 * frequency domain (a complex matrix product per frequency bin), and the
 * results are transformed back and cropped.  Transforms of real maps keep
 * the half spectrum, n (n/2 + 1) bins.  All three operations use one
 * caller-provided frequency buffer of fftconv_buffer_bytes() bytes, reused
 * by every layer (the page's memory-saving choice: nothing stays in the
 * frequency domain between calls, the backward recomputes its transforms).
 *
 * Layouts: real maps are binary32, contiguous, row-major: x [S][f][n][n],
 * w [f'][f][k][k], y and g [S][f'][n'][n'], gx [S][f][n][n],
 * gw [f'][f][k][k].  A spectrum array of B maps is bin-major: element
 * (bin p, map b) at index p * B + b, each a binary32 complex (re, im);
 * bin p = u (n/2 + 1) + v for frequencies u in [0, n), v in [0, n/2].
 *
 * Conventions (as in meswish.h): device pointers owned by the caller, no
 * allocation or synchronisation, asynchronous on `stream` (a hipStream_t,
 * NULL = default stream), status codes from meswish_status, nothing
 * launched on an error.  Outputs must not overlap inputs or the frequency
 * buffer.  Alignment (else MESWISH_EINVAL): real-map inputs 16 bytes, real
 * outputs 4 bytes, spectra and the frequency buffer 8 bytes.  n must be 8, 16, 32 or 64; 1 <= k <= n; S, f, f' >= 1 with
 * every map count below 2^31 and every spectrum array below 2^31
 * complex values.  Arithmetic is binary32.
 */
#ifndef FFT_CONV_H
#define FFT_CONV_H

#include <stddef.h>

#include "meswish.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Bytes of the frequency buffer for a layer: (S f + S f' + f f') half
 * spectra of n (n/2 + 1) complex binary32 values.  0 if out of range. */
size_t fftconv_buffer_bytes(int S, int f, int fo, int n);

/* Forward: y = sum_f x (*) w (valid cross-correlation), through
 * X = FFT(x), W = FFT(w padded), Y = sum_f X conj(W), y = crop(IFFT(Y)). */
int fftconv_fprop(const float *x, const float *w, float *y, int S, int f, int fo, int n, int k,
                  void *freq, size_t freq_bytes, void *stream);

/* Input gradient: gx = sum_f' g (x) w (full convolution), through
 * GX = sum_f' FFT(g padded) FFT(w padded), gx = IFFT(GX). */
int fftconv_bprop(const float *g, const float *w, float *gx, int S, int f, int fo, int n, int k,
                  void *freq, size_t freq_bytes, void *stream);

/* Weight gradient: gw = sum_s x (*) g, through
 * GW = sum_s FFT(x) conj(FFT(g padded)), gw = crop_k(IFFT(GW)). */
int fftconv_accgrad(const float *x, const float *g, float *gw, int S, int f, int fo, int n, int k,
                    void *freq, size_t freq_bytes, void *stream);

/* The stages, exposed for testing and measurement. */

/* Half spectra of `batch` real m x m maps zero-padded to n x n:
 * spec[p * batch + b] = sum_{r,c < m} x[b][r][c] e^{-2 pi i (u r + v c) / n}. */
int fftconv_r2c(const float *x, int batch, int m, int n, void *spec, void *stream);

/* Real maps from half spectra: y[b][r][c] = scale * Re(sum over the full
 * Hermitian spectrum of spec[., b] e^{+2 pi i (u r + v c) / n}) for
 * r, c < m (the top-left m x m of the n x n inverse). */
int fftconv_c2r(const void *spec, int batch, int n, int m, float scale, float *y, void *stream);

/* Per-bin products of the three operations, on spectra in the layouts
 * above (op: 0 forward C[s][f'] = sum_f A[s][f] conj(B[f'][f]);
 * 1 input gradient C[s][f] = sum_f' A[s][f'] B[f'][f];
 * 2 weight gradient C[f'][f] = sum_s conj(A[s][f']) B[s][f]),
 * for `bins` frequency bins; C is written bin-major like the inputs. */
int fftconv_cmul(int op, const void *a, const void *b, void *c, int S, int f, int fo, int bins,
                 void *stream);

#ifdef __cplusplus
}
#endif

#endif /* FFT_CONV_H */
