// fft_conv.hip -- FFT convolution layers of libmeswish for gfx950: batched
// small 2-D real FFTs, per-bin complex contractions, inverse FFTs with
// cropping, over one reused frequency buffer.
//
// The method ("Fast Training of Convolutional Networks through FFTs"):
// transform every input map, kernel and output gradient of a layer once,
// turn every pairwise convolution into a pointwise product in the
// frequency domain, transform back.  Formulas, layouts and contracts:
// include/fft_conv.h.
//
// Design for MI355X (CDNA4):
//   * Transforms.  The page's point is that a GPU FFT library parallelises
//     within one large transform, while this workload is many small ones.
//     Here one block transforms T maps of n x n at once, with T (n/2 + 1)
//     threads (one column transform each).  Every thread runs whole
//     length-n transforms in registers (radix-2 Cooley-Tukey, fully
//     unrolled: no data-dependent indexing, no scratch), first over rows,
//     then -- through LDS -- over the n/2 + 1 columns of the half spectrum.
//     Twiddles e^{-2 pi i j/n} are compile-time constants.  Zero rows of
//     padded maps (kernels, output gradients) skip their row transform.
//   * Spectra are stored bin-major (bin p, then map b), so the per-bin
//     matrices of the contraction are contiguous and the column pass writes
//     T consecutive maps of one bin together.
//   * Contraction.  For every bin, a complex matrix product (M x K) (K x N)
//     -- S x f by f x f' for the forward: a dense contraction, so it runs on
//     the matrix cores (v_mfma_f32_32x32x2f32, binary32 in and out), three
//     real products per pair of complex k (Gauss's form of the complex
//     product, its operand sums formed in registers after each LDS read).
//     Tiles of 64 x 64 (or 128 x 32 where that pads less) complex outputs,
//     K in steps of 8 through LDS, the next step's operands loaded as
//     16-byte pairs into registers while the current one is multiplied;
//     all tiles of one bin run on one XCD (shared operands stay in that
//     XCD's L2).
//   * Inverse.  Column transforms first, keeping only the rows that survive
//     the crop, then row transforms of the Hermitian half rows; only the
//     kept m x m corner is written, scaled by 1/n^2, and it goes out through
//     LDS as whole 16-byte vectors over the block's contiguous range of
//     maps (whole maps: each row's result over its own LDS row).
//   * Forward rows are assigned only to the m rows a map has, so no lane of
//     a wave idles on a zero row; the zero rows are filled in LDS.

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "fft_conv.h"

namespace fftconv {

// ---------------------------------------------------------------------------
// Complex helpers and the in-register transform.
// ---------------------------------------------------------------------------

__device__ __forceinline__ float2 cadd(float2 a, float2 b) { return make_float2(a.x + b.x, a.y + b.y); }
__device__ __forceinline__ float2 csub(float2 a, float2 b) { return make_float2(a.x - b.x, a.y - b.y); }
__device__ __forceinline__ float2 cmul(float2 a, float2 b)
{
    return make_float2(fmaf(a.x, b.x, -a.y * b.y), fmaf(a.x, b.y, a.y * b.x));
}
__device__ __forceinline__ float2 conjf2(float2 a) { return make_float2(a.x, -a.y); }

constexpr int ilog2(int n) { return n <= 1 ? 0 : 1 + ilog2(n / 2); }

constexpr int bitrev(int x, int bits)
{
    int r = 0;
    for (int i = 0; i < bits; ++i)
        r = (r << 1) | ((x >> i) & 1);
    return r;
}

// Twiddle factors e^{-2 pi i j / 64} = kCos64[j] - i kSin64[j], j < 32,
// rounded to binary32 (gen_fft_twiddles.py); a length-n transform uses
// entry j * 64 / n.  Indices are compile-time constants after unrolling, so
// the factors become instruction operands: no loads, no registers held.
constexpr float kCos64[32] = {
    1.000000000e+00f, 9.951847196e-01f, 9.807852507e-01f, 9.569403529e-01f,
    9.238795042e-01f, 8.819212914e-01f, 8.314695954e-01f, 7.730104327e-01f,
    7.071067691e-01f, 6.343932748e-01f, 5.555702448e-01f, 4.713967443e-01f,
    3.826834261e-01f, 2.902846634e-01f, 1.950903237e-01f, 9.801714122e-02f,
    0.000000000e+00f, -9.801714122e-02f, -1.950903237e-01f, -2.902846634e-01f,
    -3.826834261e-01f, -4.713967443e-01f, -5.555702448e-01f, -6.343932748e-01f,
    -7.071067691e-01f, -7.730104327e-01f, -8.314695954e-01f, -8.819212914e-01f,
    -9.238795042e-01f, -9.569403529e-01f, -9.807852507e-01f, -9.951847196e-01f};
constexpr float kSin64[32] = {
    0.000000000e+00f, 9.801714122e-02f, 1.950903237e-01f, 2.902846634e-01f,
    3.826834261e-01f, 4.713967443e-01f, 5.555702448e-01f, 6.343932748e-01f,
    7.071067691e-01f, 7.730104327e-01f, 8.314695954e-01f, 8.819212914e-01f,
    9.238795042e-01f, 9.569403529e-01f, 9.807852507e-01f, 9.951847196e-01f,
    1.000000000e+00f, 9.951847196e-01f, 9.807852507e-01f, 9.569403529e-01f,
    9.238795042e-01f, 8.819212914e-01f, 8.314695954e-01f, 7.730104327e-01f,
    7.071067691e-01f, 6.343932748e-01f, 5.555702448e-01f, 4.713967443e-01f,
    3.826834261e-01f, 2.902846634e-01f, 1.950903237e-01f, 9.801714122e-02f};

// In-place length-N DFT of a[] (N a power of two, N <= 64): forward with
// kernel e^{-2 pi i jk/N}, inverse (INV) with e^{+2 pi i jk/N}, unscaled.
// Iterative radix-2, decimation in time: bit-reversed input order, then
// log2 N stages.
template <int N, bool INV>
__device__ __forceinline__ void fft_reg(float2 (&a)[N])
{
    constexpr int L = ilog2(N);
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const int j = bitrev(i, L);
        if (i < j) {
            const float2 t = a[i];
            a[i] = a[j];
            a[j] = t;
        }
    }
#pragma unroll
    for (int len = 2; len <= N; len <<= 1) {
        const int half = len >> 1;
        const int step = N / len;
#pragma unroll
        for (int i = 0; i < N; i += len) {
#pragma unroll
            for (int j = 0; j < half; ++j) {
                const float2 u = a[i + j];
                float2 v = a[i + j + half];
                if (j != 0) {
                    const int t = j * step * (64 / N);
                    const float2 w = make_float2(kCos64[t], INV ? kSin64[t] : -kSin64[t]);
                    v = cmul(v, w);
                }
                a[i + j] = cadd(u, v);
                a[i + j + half] = csub(u, v);
            }
        }
    }
}

// Maps per block (a power of two: the T maps of one bin fill whole 128-byte
// lines) and threads per block: one column transform per thread, and the
// T N rows in two rounds.
// Maps per block for n = 32 and 16: longer runs per bin (256 and 512 bytes)
// measured faster than 128-byte runs (n = 32: transforms of the inputs and
// kernels 25 -> 22 and 39 -> 29 us on the measured layer).
#ifndef FFTCONV_MAPS_32
#define FFTCONV_MAPS_32 32
#endif
#ifndef FFTCONV_MAPS_16
#define FFTCONV_MAPS_16 64
#endif
#ifndef FFTCONV_C2R_MAPS_32
#define FFTCONV_C2R_MAPS_32 32
#endif
// Inverse transforms up to n = 32 can store their cropped maps through LDS
// as whole 16-byte vectors over the block's contiguous range of maps,
// instead of row by row from registers: 0 never, 1 for maps smaller than
// n x n (rows that are not whole 16-byte multiples), 2 always.  (The same
// staging of the forward transforms' loads measured slower on every map
// size.)  Whole maps (m = n) take FFTCONV_FULL_INPLACE instead: each row's
// result is written over its own LDS row, with no registers held across
// the block's barrier, then the block stores its range as 16-byte vectors
// (1), or each row is stored from registers (0).
#ifndef FFTCONV_STAGE_POLICY
#define FFTCONV_STAGE_POLICY 1
#endif
#ifndef FFTCONV_FULL_INPLACE
#define FFTCONV_FULL_INPLACE 1
#endif

static bool staged(int n, int m)
{
    return n <= 32 && (FFTCONV_STAGE_POLICY == 2 || (FFTCONV_STAGE_POLICY == 1 && m < n));
}

// Block-wide copy of `count` floats from LDS to global memory, in 16-byte
// vectors where the global side is 16-byte aligned (the LDS side always
// is), then the remainder element by element.
template <int NT>
__device__ __forceinline__ void global_from_lds(float* g, const float* lds, int count)
{
    int head = 0;
    if (((uintptr_t)g & 15u) == 0) {
        head = count & ~3;
        for (int i = 4 * (int)threadIdx.x; i < head; i += 4 * NT)
            *reinterpret_cast<float4*>(g + i) = *reinterpret_cast<const float4*>(lds + i);
    }
    for (int i = head + (int)threadIdx.x; i < count; i += NT)
        g[i] = lds[i];
}

template <int N, bool kInverse = false> struct Tile {
    static constexpr int T = N <= 8 ? 64 : N == 16 ? FFTCONV_MAPS_16
                           : N == 32 ? (kInverse ? FFTCONV_C2R_MAPS_32 : FFTCONV_MAPS_32) : 8;
    // n = 64 stays at 4 waves (its length-64 transforms need the register
    // file of a single wave per SIMD); its 264 column jobs take two rounds.
    static constexpr int kThreads = N == 64 ? 256 : T * (N / 2 + 1);
};
template <int N> using InvTile = Tile<N, true>;

// ---------------------------------------------------------------------------
// Forward transforms: `batch` real m x m maps (row-major, contiguous),
// zero-padded to N x N -> half spectra, bin-major.
// ---------------------------------------------------------------------------

// One set of maps to transform: `batch` maps of m x m at x -> spec.
struct R2cJob {
    const float* x;
    int batch, m;
    float2* spec;
};

// Blocks [0, blocks0) transform job a, the rest job b: the two inputs of a
// layer operation share one launch, so the smaller one fills the partial
// last round of the other.
template <int N>
__global__ __launch_bounds__(Tile<N>::kThreads) void r2c_kernel(R2cJob a, R2cJob b, int blocks0)
{
    constexpr int T = Tile<N>::T;
    constexpr int H = N / 2 + 1;
    constexpr int MS = N * H + 1;  // map stride in LDS, odd: no bank conflicts across maps
    __shared__ __align__(16) float2 buf[T * MS];
    const bool second = (int)blockIdx.x >= blocks0;
    const float* __restrict__ x = second ? b.x : a.x;
    float2* __restrict__ spec = second ? b.spec : a.spec;
    const int batch = second ? b.batch : a.batch;
    const int m = second ? b.m : a.m;
    const int64_t b0 = (int64_t)((int)blockIdx.x - (second ? blocks0 : 0)) * T;

    // Rows r < m: job = (map, r), so that no lane idles on a zero row while
    // the others of its wave transform (kernels and output gradients are
    // smaller than n x n).  Maps past the batch are zero.
    constexpr int NT = Tile<N>::kThreads;
    for (int job = threadIdx.x; job < T * m; job += NT) {
        const int map = job / m, r = job - map * m;
        const int64_t b = b0 + map;
        float2* out = buf + map * MS + r * H;
        if (b >= batch) {
#pragma unroll
            for (int v = 0; v < H; ++v)
                out[v] = make_float2(0.0f, 0.0f);
            continue;
        }
        const float* row = x + (b * m + r) * (int64_t)m;
        float2 a[N];
        if (m == N) {
#pragma unroll
            for (int c = 0; c < N; c += 4) {
                const float4 q = *reinterpret_cast<const float4*>(row + c);
                a[c] = make_float2(q.x, 0.0f);
                a[c + 1] = make_float2(q.y, 0.0f);
                a[c + 2] = make_float2(q.z, 0.0f);
                a[c + 3] = make_float2(q.w, 0.0f);
            }
        } else if ((m & 1) == 0 && ((uintptr_t)x & 7u) == 0) {
            // Even m: every row starts 8-byte aligned; load pairs.
#pragma unroll
            for (int c = 0; c < N; c += 2) {
                const float2 q = c < m ? *reinterpret_cast<const float2*>(row + c)
                                       : make_float2(0.0f, 0.0f);
                a[c] = make_float2(q.x, 0.0f);
                a[c + 1] = make_float2(q.y, 0.0f);
            }
        } else {
#pragma unroll
            for (int c = 0; c < N; ++c)
                a[c] = make_float2(c < m ? row[c] : 0.0f, 0.0f);
        }
        fft_reg<N, false>(a);
#pragma unroll
        for (int v = 0; v < H; ++v)
            out[v] = a[v];
    }
    // Rows m .. N - 1 (the zero padding): one contiguous run of (N - m) H
    // values per map, one whole wave per map (a partial last wave of the
    // block takes none).
    constexpr int kWholeWaves = NT / 64;
    if (m < N && (int)threadIdx.x < kWholeWaves * 64) {
        const int run = (N - m) * H;
        const int lane = (int)threadIdx.x & 63;
        for (int map = (int)threadIdx.x >> 6; map < T; map += kWholeWaves) {
            float2* z = buf + map * MS + m * H;
            for (int i = lane; i < run; i += 64)
                z[i] = make_float2(0.0f, 0.0f);
        }
    }
    __syncthreads();

    // Columns: job = (map, v), consecutive threads on consecutive maps.
    for (int job = threadIdx.x; job < T * H; job += NT) {
        const int map = job % T, v = job / T;
        const int64_t b = b0 + map;
        float2 a[N];
#pragma unroll
        for (int u = 0; u < N; ++u)
            a[u] = buf[map * MS + u * H + v];
        fft_reg<N, false>(a);
        if (b < batch) {
            // Bin (u, v) of map b: a per-thread base plus a block-uniform step.
            float2* col = spec + (int64_t)v * batch + b;
            const int64_t step = (int64_t)H * batch;
#pragma unroll
            for (int u = 0; u < N; ++u)
                col[u * step] = a[u];
        }
    }
}

// ---------------------------------------------------------------------------
// Inverse transforms: half spectra (bin-major) -> the top-left m x m of the
// real N x N maps, times scale.
// ---------------------------------------------------------------------------

template <int N, bool kStaged>
__global__ __launch_bounds__(InvTile<N>::kThreads) void c2r_kernel(const float2* __restrict__ spec,
                                                             int batch, int m, float scale,
                                                             float* __restrict__ y)
{
    constexpr int T = InvTile<N>::T;
    constexpr int H = N / 2 + 1;
    constexpr int MS = N * H + 1;
    __shared__ __align__(16) float2 buf[T * MS];
    const int64_t b0 = (int64_t)blockIdx.x * T;

    // Columns: inverse along u; keep rows p < m.
    constexpr int NT = InvTile<N>::kThreads;
    for (int job = threadIdx.x; job < T * H; job += NT) {
        const int map = job % T, v = job / T;
        const int64_t b = b0 + map;
        float2 a[N];
        if (b < batch) {
            const float2* col = spec + (int64_t)v * batch + b;
            const int64_t step = (int64_t)H * batch;
#pragma unroll
            for (int u = 0; u < N; ++u)
                a[u] = col[u * step];
        } else {
#pragma unroll
            for (int u = 0; u < N; ++u)
                a[u] = make_float2(0.0f, 0.0f);
        }
        fft_reg<N, true>(a);
#pragma unroll
        for (int p = 0; p < N; ++p)
            if (p < m)
                buf[map * MS + p * H + v] = a[p];
    }
    __syncthreads();

    // Rows p < m: the row is the half spectrum of a real signal.
    if constexpr (kStaged && N <= 32) {
        // The block's outputs (maps b0 .. b0 + T - 1, m x m each) are one
        // contiguous range of y: keep each row in registers, rebuild the
        // range in LDS once every row has been read, and store it with
        // whole 16-byte vectors.
        constexpr int R = (N + H - 1) / H;  // rows per thread: T m <= T N jobs over T H threads
        float keep[R][N];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int job = (int)threadIdx.x + r * NT;
            const int map = job / m;
            if (job >= T * m || b0 + map >= batch)
                continue;
            const float2* in = buf + map * MS + (job - map * m) * H;
            float2 a[N];
#pragma unroll
            for (int v = 0; v < H; ++v)
                a[v] = in[v];
#pragma unroll
            for (int v = H; v < N; ++v)
                a[v] = conjf2(in[N - v]);
            fft_reg<N, true>(a);
#pragma unroll
            for (int q = 0; q < N; ++q)
                keep[r][q] = a[q].x * scale;
        }
        __syncthreads();
        float* stage = reinterpret_cast<float*>(buf);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int job = (int)threadIdx.x + r * NT;
            const int map = job / m;
            if (job >= T * m || b0 + map >= batch)
                continue;
            float* row = stage + job * m;  // = map m^2 + p m
#pragma unroll
            for (int q = 0; q < N; ++q)
                if (q < m)
                    row[q] = keep[r][q];
        }
        __syncthreads();
        const int maps = (int)min<int64_t>(T, batch - b0);
        global_from_lds<NT>(y + b0 * m * m, stage, maps * m * m);
    } else if (FFTCONV_FULL_INPLACE && m == N && ((uintptr_t)y & 15u) == 0) {
        // Whole maps: each row job writes its N real outputs over the LDS
        // row it has just read (N floats fit in its H complex slots, and no
        // other thread touches that row), then the block stores its maps --
        // one contiguous range of y -- as whole 16-byte vectors, so that a
        // wave's store covers contiguous lines instead of one 16-byte piece
        // of 64 rows.
        for (int job = threadIdx.x; job < T * N; job += NT) {
            const int map = job / N, p = job - map * N;
            if (b0 + map >= batch)
                continue;
            float2* in = buf + map * MS + p * H;
            float2 a[N];
#pragma unroll
            for (int v = 0; v < H; ++v)
                a[v] = in[v];
#pragma unroll
            for (int v = H; v < N; ++v)
                a[v] = conjf2(in[N - v]);
            fft_reg<N, true>(a);
            float* o = reinterpret_cast<float*>(in);
#pragma unroll
            for (int q = 0; q < N; q += 2)
                *reinterpret_cast<float2*>(o + q) = make_float2(a[q].x * scale, a[q + 1].x * scale);
        }
        __syncthreads();
        const int maps = (int)min<int64_t>(T, batch - b0);
        float4* out = reinterpret_cast<float4*>(y + b0 * N * N);
        for (int e = threadIdx.x; e < maps * N * (N / 4); e += NT) {
            const int row = e / (N / 4), q4 = e - row * (N / 4);  // row = map N + p
            const int map = row / N, p = row - map * N;
            const float2* src = buf + map * MS + p * H + 2 * q4;
            const float2 lo = src[0], hi = src[1];
            out[e] = make_float4(lo.x, lo.y, hi.x, hi.y);
        }
    } else {
        for (int job = threadIdx.x; job < T * m; job += NT) {
            const int map = job / m, p = job - map * m;
            const int64_t b = b0 + map;
            if (b >= batch)
                continue;
            const float2* in = buf + map * MS + p * H;
            float2 a[N];
#pragma unroll
            for (int v = 0; v < H; ++v)
                a[v] = in[v];
#pragma unroll
            for (int v = H; v < N; ++v)
                a[v] = conjf2(in[N - v]);
            fft_reg<N, true>(a);
            float* out = y + (b * m + p) * (int64_t)m;
            if ((m & 3) == 0 && ((uintptr_t)y & 15u) == 0) {
                // m a multiple of 4: every row starts 16-byte aligned; store quads.
#pragma unroll
                for (int q = 0; q < N; q += 4)
                    if (q < m)
                        *reinterpret_cast<float4*>(out + q) =
                            make_float4(a[q].x * scale, a[q + 1].x * scale, a[q + 2].x * scale,
                                        a[q + 3].x * scale);
            } else if ((m & 1) == 0 && ((uintptr_t)y & 7u) == 0) {
                // Even m: every row starts 8-byte aligned; store pairs.
#pragma unroll
                for (int q = 0; q < N; q += 2)
                    if (q < m)
                        *reinterpret_cast<float2*>(out + q) =
                            make_float2(a[q].x * scale, a[q + 1].x * scale);
            } else {
#pragma unroll
                for (int q = 0; q < N; ++q)
                    if (q < m)
                        out[q] = a[q].x * scale;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Per-bin complex matrix products.
//   C[p][i][j] = sum_k A(p, i, k) B(p, k, j),  C row-major M x N per bin
//   A(p,i,k) = A[p sAp + i lda + k] (AK: k contiguous) or A[p sAp + k lda + i]
//   B(p,k,j) = B[p sBp + j ldb + k] (BK: k contiguous) or B[p sBp + k ldb + j]
// with optional conjugation of A or B.
// ---------------------------------------------------------------------------

typedef float f32x16 __attribute__((ext_vector_type(16)));

// The products run on the matrix cores, and one MFMA k-step takes two
// complex k: lane l supplies A[row l%32][k l/32] and B[k l/32][col l%32] of
// the pair.  Operands are staged into LDS as the complex values they are
// loaded as (re, im interleaved): one 8-byte LDS read gives a lane both
// parts, and the operand sums of the product (below) and the conjugations
// are formed in registers after the read.
// Block tile: 32 WR rows x 32 WC columns, WR WC waves of 32 x 32 each.  WC = 2
// in general; WC = 1 where 64-column tiles would pad the product (96
// columns take 3 tiles of 32 instead of 2 of 64, a quarter of them empty),
// and then WR = 4 where 128-row tiles pad no more than 64-row ones.
// (Two column subtiles per wave, reusing A, measured slower: 178 VGPRs.)
// Complex k per K-tile: 8 measured fastest on the measured layer (16: +2 %,
// 32: +6 %, registers 174-226).  Two LDS buffers per K-tile (one barrier
// instead of two) measured slower at 8 and 16.
#ifndef FFTCONV_KT
#define FFTCONV_KT 8
#endif
constexpr int kPK = FFTCONV_KT;
// Complex products with three real products per complex term instead of
// four (Gauss): with P = Re A + Im A, Q = Im B - Re B, R = Re B + Im B,
//   T1 = P Re B,  T2 = Re A Q,  T3 = Im A R,  Re C = T1 - T3,  Im C = T1 + T2.
// (0: the four products Re A Re B, Im A Im B, Re A Im B, Im A Re B.)
#ifndef FFTCONV_GAUSS
#define FFTCONV_GAUSS 1
#endif
// Least waves per SIMD the compiler must leave room for (register budget),
// per block tile; 1 sets no bound.  Unbounded, the 4-wave kernels keep
// their three accumulators in 48 AGPRs beside 54-58 VGPRs: 4 waves per
// SIMD.  Bounded, they keep them in VGPRs without spilling: 64 x 64 at 6
// waves (80 VGPRs; forward products 104 -> 98-99 us), 128 x 32 at 5 (80-92
// VGPRs; at 6 they spill).  The 2-wave 64 x 32 kernel: at most 4.
#ifndef FFTCONV_WPE_64X32
#define FFTCONV_WPE_64X32 (FFTCONV_GAUSS ? 4 : 5)
#endif
#ifndef FFTCONV_WPE_128X32
#define FFTCONV_WPE_128X32 5
#endif
#ifndef FFTCONV_WPE_64X64
#define FFTCONV_WPE_64X64 6
#endif
// 128 x 32 tiles (four waves of 32 x 32 in a column) for the 32-column
// products: 17 % fewer operand bytes per output than 64 x 32 tiles of two
// waves, 5-8 % faster input- and weight-gradient products.
// Operand loads in pairs of adjacent values, as 16-byte vectors where the
// tile is wholly inside the matrix and the pairs are aligned (1), or value
// by value (0).
#ifndef FFTCONV_PAIR_LOADS
#define FFTCONV_PAIR_LOADS 1
#endif
#ifndef FFTCONV_WR4
#define FFTCONV_WR4 1
#endif


template <bool AK, bool BK, bool CA, bool CB, int WC, int WR = 2>
__global__ __launch_bounds__(64 * WR * WC, WR * WC == 2 ? FFTCONV_WPE_64X32
                                          : WC == 2 ? FFTCONV_WPE_64X64 : FFTCONV_WPE_128X32)
void cgemm_kernel(const float2* __restrict__ A,
                                                               const float2* __restrict__ B,
                                                               float2* __restrict__ C, int M,
                                                               int N, int K, int64_t sAp,
                                                               int64_t sBp, int lda, int ldb,
                                                               int tiles_n, int tiles, int nbins)
{
    constexpr int NT = 64 * WR * WC;    // threads
    constexpr int BM = 32 * WR;         // block tile rows
    constexpr int BN = 32 * WC;         // block tile columns
    constexpr int LA = BM * kPK / NT;   // A values per thread per K-tile
    constexpr int LB = BN * kPK / NT;   // B values per thread per K-tile
    static_assert(LA * NT == BM * kPK && LB * NT == BN * kPK, "whole values per thread");
    constexpr bool kGauss = FFTCONV_GAUSS != 0;
    // Operands in LDS as complex values (re, im), one row of the tile per k.
    __shared__ __align__(16) float2 Al[kPK][BM + 2];
    __shared__ __align__(16) float2 Bl[kPK][BN + 2];
    const int xcd = (int)(blockIdx.x & 7u), q = (int)(blockIdx.x >> 3);
    const int p = (q / tiles) * 8 + xcd;
    if (p >= nbins)
        return;
    const int tile = q % tiles;
    const int i0 = (tile / tiles_n) * BM, j0 = (tile % tiles_n) * BN;
    const float2* Ap = A + p * sAp;
    const float2* Bp = B + p * sBp;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave / WC, wn = wave % WC;
    const int r = lane & 31, h = lane >> 5;
    f32x16 acc_re = f32x16{0}, acc_im = f32x16{0}, acc_t3 = f32x16{0};

    // Global -> register staging of one K-tile; the next tile's loads are
    // issued as soon as the current one is in LDS, before the barrier and
    // the current tile's products.  With kPairA (kPairB), each thread takes
    // pairs of values adjacent along the operand's contiguous dimension, and
    // a tile wholly inside the matrix with 16-byte aligned pairs loads each
    // pair as one 16-byte vector.
    constexpr bool kPairA = FFTCONV_PAIR_LOADS && LA % 2 == 0;
    constexpr bool kPairB = FFTCONV_PAIR_LOADS && LB % 2 == 0;
    // Paired slots are held as the 16-byte vectors they are loaded as, and
    // split only when stored to LDS: the loop then carries the load's own
    // registers (splitting at the load made the compiler copy them across
    // the loop's back edge, which waited for the loads at once).
    float2 ra[kPairA ? 1 : LA], rb[kPairB ? 1 : LB];
    float4 ra4[kPairA ? LA / 2 : 1], rb4[kPairB ? LB / 2 : 1];
    // Tiles wholly inside the matrices load without per-element checks.
    const bool a_inside = i0 + BM <= M, b_inside = j0 + BN <= N;
    const bool a_aligned = ((uintptr_t)A & 15u) == 0 && (sAp & 1) == 0 && (lda & 1) == 0;
    const bool b_aligned = ((uintptr_t)B & 15u) == 0 && (sBp & 1) == 0 && (ldb & 1) == 0;
    // Value slot s of this thread: its (k, row) in the tile.  Pairs: slots
    // 2q and 2q + 1 are adjacent along the contiguous dimension.
    auto a_slot = [&](int s2, int& k, int& i) {
        if constexpr (kPairA) {
            const int idx = threadIdx.x + (s2 >> 1) * NT;
            if (AK) { k = 2 * (idx % (kPK / 2)) + (s2 & 1); i = idx / (kPK / 2); }
            else { i = 2 * (idx % (BM / 2)) + (s2 & 1); k = idx / (BM / 2); }
        } else {
            const int idx = threadIdx.x + s2 * NT;
            k = AK ? idx % kPK : idx / BM;
            i = AK ? idx / kPK : idx % BM;
        }
    };
    auto b_slot = [&](int s2, int& k, int& j) {
        if constexpr (kPairB) {
            const int idx = threadIdx.x + (s2 >> 1) * NT;
            if (BK) { k = 2 * (idx % (kPK / 2)) + (s2 & 1); j = idx / (kPK / 2); }
            else { j = 2 * (idx % (BN / 2)) + (s2 & 1); k = idx / (BN / 2); }
        } else {
            const int idx = threadIdx.x + s2 * NT;
            k = BK ? idx % kPK : idx / BN;
            j = BK ? idx / kPK : idx % BN;
        }
    };
    // VEC: the block's tiles are wholly inside both matrices at every K-tile
    // and the pairs are 16-byte aligned, so the loads need no checks; the
    // two cases run separate copies of the loop (a branch per K-tile would
    // join the loaded registers and wait for the prefetch on the spot).
    auto fetch = [&](int k0, auto vec) {
        constexpr bool VEC = decltype(vec)::value;
        const bool k_inside = k0 + kPK <= K;
        auto a_get = [&](int s2) {
            int k, i;
            a_slot(s2, k, i);
            const int64_t off = AK ? (int64_t)(i0 + i) * lda + (k0 + k) : (int64_t)(k0 + k) * lda + (i0 + i);
            if (VEC)
                return Ap[off];
            return ((a_inside && k_inside) || (i0 + i < M && k0 + k < K)) ? Ap[off]
                                                                        : make_float2(0.0f, 0.0f);
        };
        auto b_get = [&](int s2) {
            int k, j;
            b_slot(s2, k, j);
            const int64_t off = BK ? (int64_t)(j0 + j) * ldb + (k0 + k) : (int64_t)(k0 + k) * ldb + (j0 + j);
            if (VEC)
                return Bp[off];
            return ((b_inside && k_inside) || (j0 + j < N && k0 + k < K)) ? Bp[off]
                                                                        : make_float2(0.0f, 0.0f);
        };
        if constexpr (kPairA) {
#pragma unroll
            for (int qq = 0; qq < LA; qq += 2) {
                if constexpr (VEC) {
                    int k, i;
                    a_slot(qq, k, i);
                    const int64_t off = AK ? (int64_t)(i0 + i) * lda + (k0 + k) : (int64_t)(k0 + k) * lda + (i0 + i);
                    ra4[qq / 2] = *reinterpret_cast<const float4*>(Ap + off);
                } else {
                    const float2 v0 = a_get(qq), v1 = a_get(qq + 1);
                    ra4[qq / 2] = make_float4(v0.x, v0.y, v1.x, v1.y);
                }
            }
        } else {
#pragma unroll
            for (int qq = 0; qq < LA; ++qq)
                ra[qq] = a_get(qq);
        }
        if constexpr (kPairB) {
#pragma unroll
            for (int qq = 0; qq < LB; qq += 2) {
                if constexpr (VEC) {
                    int k, j;
                    b_slot(qq, k, j);
                    const int64_t off = BK ? (int64_t)(j0 + j) * ldb + (k0 + k) : (int64_t)(k0 + k) * ldb + (j0 + j);
                    rb4[qq / 2] = *reinterpret_cast<const float4*>(Bp + off);
                } else {
                    const float2 w0 = b_get(qq), w1 = b_get(qq + 1);
                    rb4[qq / 2] = make_float4(w0.x, w0.y, w1.x, w1.y);
                }
            }
        } else {
#pragma unroll
            for (int qq = 0; qq < LB; ++qq)
                rb[qq] = b_get(qq);
        }
    };
    // Values go to LDS as loaded: a pair along k to two rows, a pair along
    // the rows or columns as one 16-byte store.
    auto stash = [&]() {
        if constexpr (kPairA) {
#pragma unroll
            for (int qq = 0; qq < LA; qq += 2) {
                int k, i;
                a_slot(qq, k, i);
                const float4 q4 = ra4[qq / 2];
                if (AK) {
                    Al[k][i] = make_float2(q4.x, q4.y);
                    Al[k + 1][i] = make_float2(q4.z, q4.w);
                } else {
                    *reinterpret_cast<float4*>(&Al[k][i]) = q4;
                }
            }
        } else {
#pragma unroll
            for (int qq = 0; qq < LA; ++qq) {
                int k, i;
                a_slot(qq, k, i);
                Al[k][i] = ra[qq];
            }
        }
        if constexpr (kPairB) {
#pragma unroll
            for (int qq = 0; qq < LB; qq += 2) {
                int k, j;
                b_slot(qq, k, j);
                const float4 q4 = rb4[qq / 2];
                if (BK) {
                    Bl[k][j] = make_float2(q4.x, q4.y);
                    Bl[k + 1][j] = make_float2(q4.z, q4.w);
                } else {
                    *reinterpret_cast<float4*>(&Bl[k][j]) = q4;
                }
            }
        } else {
#pragma unroll
            for (int qq = 0; qq < LB; ++qq) {
                int k, j;
                b_slot(qq, k, j);
                Bl[k][j] = rb[qq];
            }
        }
    };

    auto run = [&](auto vec) {
        fetch(0, vec);
        for (int k0 = 0; k0 < K; k0 += kPK) {
            stash();
            if (k0 + kPK < K)
                fetch(k0 + kPK, vec);  // the registers are free once stored
            __syncthreads();
#pragma unroll
            for (int kk = 0; kk < kPK; kk += 2) {
                const float2 a = Al[kk + h][wm * 32 + r];
                const float2 b = Bl[kk + h][wn * 32 + r];
                if constexpr (kGauss) {
                    // With a' = conj(a) under CA and b' = conj(b) under CB:
                    // acc_re: T1 = P Re b, P = Re a' + Im a'; acc_im: T2 =
                    // Re a Q, Q = Im b' - Re b; acc_t3: Im a R, R = Re b +
                    // Im b' (that is T3 = Im a' R up to the sign of CA).
                    const float pa = CA ? a.x - a.y : a.x + a.y;
                    const float qb = CB ? -(b.x + b.y) : b.y - b.x;
                    const float rb_ = CB ? b.x - b.y : b.x + b.y;
                    acc_re = __builtin_amdgcn_mfma_f32_32x32x2f32(pa, b.x, acc_re, 0, 0, 0);
                    acc_im = __builtin_amdgcn_mfma_f32_32x32x2f32(a.x, qb, acc_im, 0, 0, 0);
                    acc_t3 = __builtin_amdgcn_mfma_f32_32x32x2f32(a.y, rb_, acc_t3, 0, 0, 0);
                } else {
                    const float ai = CA ? -a.y : a.y, bi = CB ? -b.y : b.y;
                    acc_re = __builtin_amdgcn_mfma_f32_32x32x2f32(a.x, b.x, acc_re, 0, 0, 0);
                    acc_im = __builtin_amdgcn_mfma_f32_32x32x2f32(a.x, bi, acc_im, 0, 0, 0);
                    acc_re = __builtin_amdgcn_mfma_f32_32x32x2f32(-ai, bi, acc_re, 0, 0, 0);
                    acc_im = __builtin_amdgcn_mfma_f32_32x32x2f32(ai, b.x, acc_im, 0, 0, 0);
                }
            }
            __syncthreads();
        }
    };
    const bool fast = a_inside && b_inside && K % kPK == 0 && (!kPairA || a_aligned) &&
                      (!kPairB || b_aligned);
    if (fast)
        run(std::true_type{});
    else
        run(std::false_type{});
    float2* Cp = C + (int64_t)p * M * N;
    const int j = j0 + wn * 32 + r;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const int i = i0 + wm * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
        if (i < M && j < N) {
            if constexpr (kGauss)
                Cp[(int64_t)i * N + j] = make_float2(CA ? acc_re[v] + acc_t3[v] : acc_re[v] - acc_t3[v],
                                                     acc_re[v] + acc_im[v]);
            else
                Cp[(int64_t)i * N + j] = make_float2(acc_re[v], acc_im[v]);
        }
    }
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------


static bool n_ok(int n) { return n == 8 || n == 16 || n == 32 || n == 64; }

static int64_t bins(int n) { return (int64_t)n * (n / 2 + 1); }

static bool overlaps(const void* a, size_t na, const void* b, size_t nb)
{
    uintptr_t pa = (uintptr_t)a, pb = (uintptr_t)b;
    return na && nb && pa < pb + nb && pb < pa + na;
}

static int status_of(hipError_t e) { return e == hipSuccess ? MESWISH_OK : MESWISH_EHIP; }

template <int N>
static void r2c_launch(const R2cJob& a, const R2cJob& b, hipStream_t s)
{
    const int T = Tile<N>::T;
    const int blocks0 = (a.batch + T - 1) / T, blocks1 = (b.batch + T - 1) / T;
    hipLaunchKernelGGL(r2c_kernel<N>, dim3((unsigned)(blocks0 + blocks1)), dim3(Tile<N>::kThreads),
                       0, s, a, b, blocks0);
}

template <int N>
static void c2r_launch(const float2* spec, int batch, int m, float scale, float* y, hipStream_t s)
{
    using Tl = InvTile<N>;
    const unsigned grid = (unsigned)((batch + Tl::T - 1) / Tl::T);
    if (staged(N, m))
        hipLaunchKernelGGL((c2r_kernel<N, N <= 32>), dim3(grid), dim3(Tl::kThreads), 0, s, spec,
                           batch, m, scale, y);
    else
        hipLaunchKernelGGL((c2r_kernel<N, false>), dim3(grid), dim3(Tl::kThreads), 0, s, spec,
                           batch, m, scale, y);
}

// Transforms of one or two sets of maps (b.batch = 0 for one) in one launch.
static int launch_r2c(const R2cJob& a, const R2cJob& b, int n, hipStream_t s)
{
    switch (n) {
    case 8: r2c_launch<8>(a, b, s); break;
    case 16: r2c_launch<16>(a, b, s); break;
    case 32: r2c_launch<32>(a, b, s); break;
    default: r2c_launch<64>(a, b, s); break;
    }
    return status_of(hipGetLastError());
}

static int launch_c2r(const float2* spec, int batch, int n, int m, float scale, float* y, hipStream_t s)
{
    switch (n) {
    case 8: c2r_launch<8>(spec, batch, m, scale, y, s); break;
    case 16: c2r_launch<16>(spec, batch, m, scale, y, s); break;
    case 32: c2r_launch<32>(spec, batch, m, scale, y, s); break;
    default: c2r_launch<64>(spec, batch, m, scale, y, s); break;
    }
    return status_of(hipGetLastError());
}

// op 0: C[s][f'] = sum_f A[s][f] conj(B[f'][f]); 1: C[s][f] = sum_f' A[s][f'] B[f'][f];
// 2: C[f'][f] = sum_s conj(A[s][f']) B[s][f].
static int launch_cmul(int op, const float2* a, const float2* b, float2* c, int S, int f, int fo,
                       int nbins, hipStream_t s)
{
    int M, N, K;
    int64_t sAp, sBp;
    int lda, ldb;
    if (op == 0) {
        M = S; N = fo; K = f; sAp = (int64_t)S * f; sBp = (int64_t)fo * f; lda = f; ldb = f;
    } else if (op == 1) {
        M = S; N = f; K = fo; sAp = (int64_t)S * fo; sBp = (int64_t)fo * f; lda = fo; ldb = f;
    } else {
        M = fo; N = f; K = S; sAp = (int64_t)S * fo; sBp = (int64_t)S * f; lda = fo; ldb = f;
    }
    // 32-column block tiles where they pad less than 64-column ones.
#ifndef FFTCONV_WC
    const int wc = ((N + 63) / 64 * 64 - N > (N + 31) / 32 * 32 - N) ? 1 : 2;
#else
    const int wc = FFTCONV_WC;
#endif
    // 128-row tiles (four waves) for the 32-column kernel where they pad M
    // no more than 64-row ones.
    const int wr = (FFTCONV_WR4 && wc == 1 &&
                    (M + 127) / 128 * 128 - M <= (M + 63) / 64 * 64 - M) ? 4 : 2;
    const int ptm = (M + 32 * wr - 1) / (32 * wr);
    const int ptn = (N + 32 * wc - 1) / (32 * wc), ptiles = ptn * ptm;
    const int64_t pblocks = (int64_t)((nbins + 7) / 8) * 8 * ptiles;
    if (pblocks > 0x7FFFFFFF)
        return MESWISH_EINVAL;
    const dim3 pgrid((unsigned)pblocks), pthreads(64 * wr * wc);
#define FFTCONV_CGEMM(AK, BK, CA, CB)                                                            \
    do {                                                                                          \
        if (wc == 1 && wr == 4)                                                                   \
            hipLaunchKernelGGL((cgemm_kernel<AK, BK, CA, CB, 1, 4>), pgrid, pthreads, 0, s, \
                               a, b, c, M, N, K, sAp, sBp, lda, ldb, ptn, ptiles, nbins);         \
        else if (wc == 1)                                                                         \
            hipLaunchKernelGGL((cgemm_kernel<AK, BK, CA, CB, 1>), pgrid, pthreads, 0, s, a, \
                               b, c, M, N, K, sAp, sBp, lda, ldb, ptn, ptiles, nbins);            \
        else                                                                                      \
            hipLaunchKernelGGL((cgemm_kernel<AK, BK, CA, CB, 2>), pgrid, pthreads, 0, s, a, \
                               b, c, M, N, K, sAp, sBp, lda, ldb, ptn, ptiles, nbins);            \
    } while (0)
    if (op == 0)
        FFTCONV_CGEMM(true, true, false, true);
    else if (op == 1)
        FFTCONV_CGEMM(true, false, false, false);
    else
        FFTCONV_CGEMM(false, false, true, false);
#undef FFTCONV_CGEMM
    return status_of(hipGetLastError());
}

static bool sizes_ok(int S, int f, int fo, int n, int k)
{
    if (!n_ok(n) || S < 1 || f < 1 || fo < 1 || k < 1 || k > n)
        return false;
    const int64_t P = bins(n);
    const int64_t maps[3] = {(int64_t)S * f, (int64_t)S * fo, (int64_t)fo * f};
    for (int64_t b : maps)
        if (b >= (1ll << 31) || b * P >= (1ll << 31))
            return false;
    return true;
}

}  // namespace fftconv

using namespace fftconv;

extern "C" size_t fftconv_buffer_bytes(int S, int f, int fo, int n)
{
    if (!sizes_ok(S, f, fo, n, 1))
        return 0;
    const int64_t maps = (int64_t)S * f + (int64_t)S * fo + (int64_t)fo * f;
    return (size_t)(maps * bins(n)) * sizeof(float2);
}

extern "C" int fftconv_r2c(const float* x, int batch, int m, int n, void* spec, void* stream)
{
    if (!n_ok(n) || batch < 0 || m < 1 || m > n || (batch > 0 && (!x || !spec)))
        return MESWISH_EINVAL;
    if ((int64_t)batch * bins(n) >= (1ll << 31))
        return MESWISH_EINVAL;
    if (batch == 0)
        return MESWISH_OK;
    if (((uintptr_t)x & 15u) || ((uintptr_t)spec & 7u))
        return MESWISH_EINVAL;
    if (overlaps(x, (size_t)batch * m * m * 4, spec, (size_t)batch * bins(n) * 8))
        return MESWISH_EALIAS;
    const R2cJob a{x, batch, m, static_cast<float2*>(spec)}, none{x, 0, m, nullptr};
    return launch_r2c(a, none, n, static_cast<hipStream_t>(stream));
}

extern "C" int fftconv_c2r(const void* spec, int batch, int n, int m, float scale, float* y,
                           void* stream)
{
    if (!n_ok(n) || batch < 0 || m < 1 || m > n || !isfinite(scale) ||
        (batch > 0 && (!y || !spec)))
        return MESWISH_EINVAL;
    if ((int64_t)batch * bins(n) >= (1ll << 31))
        return MESWISH_EINVAL;
    if (batch == 0)
        return MESWISH_OK;
    if (((uintptr_t)y & 3u) || ((uintptr_t)spec & 7u))
        return MESWISH_EINVAL;
    if (overlaps(y, (size_t)batch * m * m * 4, spec, (size_t)batch * bins(n) * 8))
        return MESWISH_EALIAS;
    return launch_c2r(static_cast<const float2*>(spec), batch, n, m, scale, y,
                      static_cast<hipStream_t>(stream));
}

extern "C" int fftconv_cmul(int op, const void* a, const void* b, void* c, int S, int f, int fo,
                            int nbins, void* stream)
{
    if (op < 0 || op > 2 || S < 1 || f < 1 || fo < 1 || nbins < 1 || nbins > 65535 || !a || !b || !c)
        return MESWISH_EINVAL;
    if (((uintptr_t)a & 7u) || ((uintptr_t)b & 7u) || ((uintptr_t)c & 7u))
        return MESWISH_EINVAL;
    const int64_t sa = op == 0 ? (int64_t)S * f : (int64_t)S * fo;
    const int64_t sb = op == 2 ? (int64_t)S * f : (int64_t)fo * f;
    const int64_t sc = op == 0 ? (int64_t)S * fo : op == 1 ? (int64_t)S * f : (int64_t)fo * f;
    if (sa * nbins >= (1ll << 31) || sb * nbins >= (1ll << 31) || sc * nbins >= (1ll << 31))
        return MESWISH_EINVAL;
    const size_t cb = (size_t)(sc * nbins) * 8;
    if (overlaps(c, cb, a, (size_t)(sa * nbins) * 8) || overlaps(c, cb, b, (size_t)(sb * nbins) * 8))
        return MESWISH_EALIAS;
    return launch_cmul(op, static_cast<const float2*>(a), static_cast<const float2*>(b),
                       static_cast<float2*>(c), S, f, fo, nbins, static_cast<hipStream_t>(stream));
}

// The three operations.  The frequency buffer holds, in order, the spectra
// of the operation's two inputs and of its result.
static int run_op(int op, const float* in1, const float* in2, float* out, int S, int f, int fo,
                  int n, int k, void* freq, size_t freq_bytes, hipStream_t s)
{
    if (!sizes_ok(S, f, fo, n, k) || !in1 || !in2 || !out || !freq)
        return MESWISH_EINVAL;
    if (freq_bytes < fftconv_buffer_bytes(S, f, fo, n))
        return MESWISH_EINVAL;
    if (((uintptr_t)in1 & 15u) || ((uintptr_t)in2 & 15u) || ((uintptr_t)out & 3u) ||
        ((uintptr_t)freq & 7u))
        return MESWISH_EINVAL;
    const int m = n - k + 1;
    const int64_t P = bins(n);
    // Map counts and sizes of the two inputs and the output.
    int64_t b1, b2, bo;
    int m1, m2, mo;
    if (op == 0) {        // x, w -> y
        b1 = (int64_t)S * f; m1 = n; b2 = (int64_t)fo * f; m2 = k; bo = (int64_t)S * fo; mo = m;
    } else if (op == 1) { // g, w -> gx
        b1 = (int64_t)S * fo; m1 = m; b2 = (int64_t)fo * f; m2 = k; bo = (int64_t)S * f; mo = n;
    } else {              // g, x -> gw (A = G, B = X)
        b1 = (int64_t)S * fo; m1 = m; b2 = (int64_t)S * f; m2 = n; bo = (int64_t)fo * f; mo = k;
    }
    const size_t fb = fftconv_buffer_bytes(S, f, fo, n);
    const size_t ob = (size_t)bo * mo * mo * 4;
    if (overlaps(out, ob, in1, (size_t)b1 * m1 * m1 * 4) ||
        overlaps(out, ob, in2, (size_t)b2 * m2 * m2 * 4) || overlaps(out, ob, freq, fb) ||
        overlaps(freq, fb, in1, (size_t)b1 * m1 * m1 * 4) ||
        overlaps(freq, fb, in2, (size_t)b2 * m2 * m2 * 4))
        return MESWISH_EALIAS;
    float2* s1 = static_cast<float2*>(freq);
    float2* s2 = s1 + b1 * P;
    float2* so = s2 + b2 * P;
    int st = launch_r2c(R2cJob{in1, (int)b1, m1, s1}, R2cJob{in2, (int)b2, m2, s2}, n, s);
    if (st == MESWISH_OK)
        st = launch_cmul(op, s1, s2, so, S, f, fo, (int)P, s);
    if (st == MESWISH_OK)
        st = launch_c2r(so, (int)bo, n, mo, 1.0f / (float)(n * n), out, s);
    return st;
}

extern "C" int fftconv_fprop(const float* x, const float* w, float* y, int S, int f, int fo, int n,
                             int k, void* freq, size_t freq_bytes, void* stream)
{
    return run_op(0, x, w, y, S, f, fo, n, k, freq, freq_bytes, static_cast<hipStream_t>(stream));
}

extern "C" int fftconv_bprop(const float* g, const float* w, float* gx, int S, int f, int fo, int n,
                             int k, void* freq, size_t freq_bytes, void* stream)
{
    return run_op(1, g, w, gx, S, f, fo, n, k, freq, freq_bytes, static_cast<hipStream_t>(stream));
}

extern "C" int fftconv_accgrad(const float* x, const float* g, float* gw, int S, int f, int fo,
                               int n, int k, void* freq, size_t freq_bytes, void* stream)
{
    return run_op(2, g, x, gw, S, f, fo, n, k, freq, freq_bytes, static_cast<hipStream_t>(stream));
}
