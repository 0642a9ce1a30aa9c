// dense_bn.hip -- the shared-buffer DenseNet layer stage of libmeswish for
// gfx950: batch statistics, concatenation + batch normalization + ReLU
// (forward) and its backward, recomputed from the sources.
//
// The method (README of efficient_densenet_pytorch, "A memory-efficient
// implementation of DenseNets", Motivation): the concatenated input of a
// DenseNet layer and its batch-normalized form are kept only in memory that
// all layers share, and re-populated in the backward pass.  Here the
// concatenation is folded into the normalization kernel (the sources are
// read where they live), so the forward needs one shared map (z) and the
// backward one (dz).  Formulas and contracts: include/dense_bn.h.
//
// Design for MI355X (CDNA4):
//   * Every kernel streams feature maps once per pass at a few flops per
//     element: HBM-bound, so no LDS tiling and no MFMA.  LDS holds only the
//     per-wave partial sums of a block reduction.
//   * Work unit = (channel, chunk): one block handles 16 KiB of one channel
//     (4096 binary32 or 8192 bfloat16 elements).  The channel's parameters (mean, 1/sqrt(var + eps), the ReLU
//     threshold) are then uniform over the block and computed once per lane
//     in binary64 -- after the block's loads are issued, so their latency
//     hides the arithmetic.  A channel's n rows of hw elements sit at a
//     stride of C_j * hw (NCHW), and a lane moves 16-byte vectors along a
//     row whenever hw is a multiple of the vector width.
//   * The ReLU mask h > 0 (h = gamma (x - mean) r + beta) is decided as
//     x > t or x < t against the channel's threshold t = mean - beta / (gamma
//     r), computed in binary64 and rounded outward to binary32, so the
//     decision is the exact one for every binary32 input: forward and
//     backward agree with each other and with a binary64 evaluation.
//   * Reductions (statistics, dgamma, dbeta) accumulate in binary64 per
//     lane, then across the wave (shuffles) and the block (LDS), and write
//     one partial per block to the caller's workspace; a second pass sums
//     the partials of a channel in a fixed order.  No atomics: results are
//     bitwise reproducible.

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "dense_bn.h"

namespace dense_bn {

// Bytes of one channel per block (16 KiB: 4096 binary32 or 8192 bfloat16
// elements), and the non-temporal (streaming) cache policy as a bit mask:
// 1 = loads of the sources, 2 = loads of dz, 4 = stores of z and dx.  Both
// chosen by measurement on MI355X (streaming stores: +10 % on every pass).
#ifndef DENSE_BN_CHUNK_BYTES
#define DENSE_BN_CHUNK_BYTES 16384
#endif
#ifndef DENSE_BN_NT
#define DENSE_BN_NT 4
#endif
// The forward's vector path: threads per block and elements of one channel
// per block, per element type.  8 KiB blocks measured fastest in both:
// binary32 as one wave of 8 vectors per lane (5280 GB/s against 5018 for
// 256 threads over 32 KiB), bfloat16 as two waves of 4 vectors per lane
// (5237 against 5189); 1024- to 8192-element chunks of 64, 128 and 256
// threads were measured.
#ifndef DENSE_BN_FWD_BLOCK_F32
#define DENSE_BN_FWD_BLOCK_F32 64
#endif
#ifndef DENSE_BN_FWD_CHUNK_F32
#define DENSE_BN_FWD_CHUNK_F32 2048
#endif
#ifndef DENSE_BN_FWD_BLOCK_BF16
#define DENSE_BN_FWD_BLOCK_BF16 128
#endif
#ifndef DENSE_BN_FWD_CHUNK_BF16
#define DENSE_BN_FWD_CHUNK_BF16 4096
#endif

constexpr int kBlock = 256;             // threads per block
constexpr int kWaves = kBlock / 64;
constexpr int kMaxSources = DENSE_BN_MAX_SOURCES;
// The workspace is sized for the smallest chunk (binary32).
constexpr int kMinChunk = DENSE_BN_CHUNK_BYTES / 4;
static_assert(kMinChunk % (kBlock * 8) == 0, "a chunk must give every lane whole vectors");
static_assert(DENSE_BN_FWD_CHUNK_F32 % (DENSE_BN_FWD_BLOCK_F32 * 4) == 0 &&
                  DENSE_BN_FWD_CHUNK_BF16 % (DENSE_BN_FWD_BLOCK_BF16 * 8) == 0,
              "whole 16-byte vectors per lane");
constexpr bool kNtX = (DENSE_BN_NT & 1) != 0;
constexpr bool kNtDz = (DENSE_BN_NT & 2) != 0;
constexpr bool kNtOut = (DENSE_BN_NT & 4) != 0;

// ---------------------------------------------------------------------------
// Element types and vector access.
// ---------------------------------------------------------------------------

struct bf16_t {
    uint16_t bits;
};

typedef float float2_v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));

// Two binary32 values -> two bfloat16 (round to nearest even; gfx950
// v_cvt_pk_bf16_f32), packed low | high << 16.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    float2_v f = {lo, hi};
    bf16x2_v b = __builtin_convertvector(f, bf16x2_v);
    uint32_t u;
    __builtin_memcpy(&u, &b, sizeof u);
    return u;
}

template <typename IO> struct Elem;

typedef uint32_t u32x4_v __attribute__((ext_vector_type(4)));

// 16-byte global load / store; kNT selects the non-temporal policy.
template <bool kNT>
__device__ __forceinline__ uint4 ld16(const void* p)
{
    if (kNT) {
        u32x4_v v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_v*>(p));
        return make_uint4(v.x, v.y, v.z, v.w);
    }
    return *reinterpret_cast<const uint4*>(p);
}

template <bool kNT>
__device__ __forceinline__ void st16(void* p, const uint4& v)
{
    if (kNT) {
        u32x4_v w = {v.x, v.y, v.z, v.w};
        __builtin_nontemporal_store(w, reinterpret_cast<u32x4_v*>(p));
    } else {
        *reinterpret_cast<uint4*>(p) = v;
    }
}

template <> struct Elem<float> {
    static constexpr int kVec = 4;  // elements per 16-byte vector
    __device__ static void unpack(const uint4& v, float (&f)[4])
    {
        f[0] = __uint_as_float(v.x);
        f[1] = __uint_as_float(v.y);
        f[2] = __uint_as_float(v.z);
        f[3] = __uint_as_float(v.w);
    }
    template <bool kNT>
    __device__ static void load(const float* p, int64_t i, float (&f)[4])
    {
        unpack(ld16<kNT>(p + i), f);
    }
    template <bool kNT>
    __device__ static void store(float* p, int64_t i, const float (&f)[4])
    {
        st16<kNT>(p + i, make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]),
                                    __float_as_uint(f[2]), __float_as_uint(f[3])));
    }
    template <bool kNT>
    __device__ static void load(const float* p, int64_t i, float (&f)[1]) { f[0] = p[i]; }
    template <bool kNT>
    __device__ static void store(float* p, int64_t i, const float (&f)[1]) { p[i] = f[0]; }
};

template <> struct Elem<bf16_t> {
    static constexpr int kVec = 8;
    __device__ static void unpack(const uint4& v, float (&f)[8])
    {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            f[2 * k] = __uint_as_float(w[k] << 16);
            f[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
        }
    }
    template <bool kNT>
    __device__ static void load(const bf16_t* p, int64_t i, float (&f)[8])
    {
        unpack(ld16<kNT>(p + i), f);
    }
    template <bool kNT>
    __device__ static void store(bf16_t* p, int64_t i, const float (&f)[8])
    {
        st16<kNT>(p + i, make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]),
                                    pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7])));
    }
    template <bool kNT>
    __device__ static void load(const bf16_t* p, int64_t i, float (&f)[1])
    {
        f[0] = __uint_as_float((uint32_t)p[i].bits << 16);
    }
    template <bool kNT>
    __device__ static void store(bf16_t* p, int64_t i, const float (&f)[1])
    {
        p[i].bits = (uint16_t)(pack_bf16x2(f[0], 0.0f) & 0xFFFFu);
    }
};

// One vector's registers as loaded: the 16 bytes as they arrive, unpacked to
// binary32 only where used (bfloat16 doubles in size when unpacked, so this
// keeps fewer registers live across the loads); the element-wise path keeps
// its one element.
template <typename IO, int V> struct Raw {
    uint4 u;
    template <bool kNT> __device__ void fetch(const IO* p, int64_t i) { u = ld16<kNT>(p + i); }
    __device__ void unpack(float (&f)[V]) const { Elem<IO>::unpack(u, f); }
};

template <typename IO> struct Raw<IO, 1> {
    float f0;
    template <bool kNT> __device__ void fetch(const IO* p, int64_t i)
    {
        float f[1];
        Elem<IO>::template load<kNT>(p, i, f);
        f0 = f[0];
    }
    __device__ void unpack(float (&f)[1]) const { f[0] = f0; }
};

// ---------------------------------------------------------------------------
// Geometry: a channel is n rows of hw elements; in units of V-element
// vectors, rows of pv = hw / V vectors.  Vector v of a channel lies in row
// v / pv at position v % pv.  The quotient uses the round-up multiply-shift
// method of Granlund and Montgomery ("Division by invariant integers using
// multiplication", 1994): q = (umulhi(v, m) + v) >> s with s = ceil(log2 d)
// and m = floor(2^32 (2^s - d) / d) + 1, exact for v < 2^31.
// ---------------------------------------------------------------------------

// Elements of one channel per block for element type IO.
template <typename IO, int kBytes = DENSE_BN_CHUNK_BYTES>
constexpr int chunk_elems() { return kBytes / (int)sizeof(IO); }

// The forward's vector path takes its own chunk and block: it keeps no
// partials (the element-wise path keeps the common chunk and block, which
// bound its registers).
template <typename IO, int V>
constexpr int fwd_chunk_bytes()
{
    return V == 1 ? DENSE_BN_CHUNK_BYTES
                  : (sizeof(IO) == 4 ? DENSE_BN_FWD_CHUNK_F32 : DENSE_BN_FWD_CHUNK_BF16) *
                        (int)sizeof(IO);
}

template <typename IO, int V> constexpr int fwd_block()
{
    return V == 1 ? kBlock : sizeof(IO) == 4 ? DENSE_BN_FWD_BLOCK_F32 : DENSE_BN_FWD_BLOCK_BF16;
}

struct FastDiv {
    uint32_t d, m, s;
};

__device__ __forceinline__ uint32_t fdiv(uint32_t v, const FastDiv& f)
{
    return (__umulhi(v, f.m) + v) >> f.s;
}

struct Geom {
    FastDiv pv;        // divisor: vectors per row
    uint32_t mv;       // vectors per channel (n * pv)
    int chunks;        // blocks per channel
    double m;          // elements per channel (n * hw)
};

// ---------------------------------------------------------------------------
// Source table of a call (kernel argument; at most 64 sources).
// ---------------------------------------------------------------------------

// Structure of arrays, so that `first` is one contiguous block of the
// kernel arguments that a block reads with a few wide scalar loads.
struct Table {
    const void* x[kMaxSources];
    void* dx[kMaxSources];
    const double* stats[kMaxSources];
    int channels[kMaxSources];   // C_j
    int offset[kMaxSources];     // first channel in z / gamma / beta / dz / dgamma / dbeta
    int first[kMaxSources];      // first channel of source j in the call's channel order;
                                 // INT_MAX past the last source
};

// Source and channel of this block: blocks are (channel, chunk) pairs in the
// call's channel order (sources in table order, channels within each).
struct Where {
    int j, cl, zc, chunk, g;
};

__device__ __forceinline__ Where locate(const Table& t, int chunks)
{
    Where w;
    w.g = (int)blockIdx.x / chunks;
    w.chunk = (int)blockIdx.x - w.g * chunks;
    // j = number of sources after the first whose first channel is <= g:
    // independent compares, no chain of dependent loads.
    int j = 0;
#pragma unroll
    for (int k = 1; k < kMaxSources; ++k)
        j += (w.g >= t.first[k]) ? 1 : 0;
    w.j = j;
    w.cl = w.g - t.first[j];
    w.zc = t.offset[j] + w.cl;
    return w;
}

// ---------------------------------------------------------------------------
// Per-channel parameters of the normalization and the ReLU mask.
// ---------------------------------------------------------------------------

// Largest binary32 <= t, and smallest binary32 >= t (t finite or infinite).
__device__ __forceinline__ float next_down(float f)
{
    if (f == 0.0f)
        return -1.40129846e-45f;
    uint32_t u = __float_as_uint(f);
    return __uint_as_float(f > 0.0f ? u - 1u : u + 1u);
}

__device__ __forceinline__ float next_up(float f)
{
    if (f == 0.0f)
        return 1.40129846e-45f;
    uint32_t u = __float_as_uint(f);
    return __uint_as_float(f > 0.0f ? u + 1u : u - 1u);
}

__device__ __forceinline__ float f32_down(double t)
{
    float f = (float)t;
    if ((double)f > t)
        f = (f == INFINITY) ? 3.40282347e38f : next_down(f);
    return f;
}

__device__ __forceinline__ float f32_up(double t)
{
    float f = (float)t;
    if ((double)f < t)
        f = (f == -INFINITY) ? -3.40282347e38f : next_up(f);
    return f;
}

struct Chan {
    float mu;     // mean, rounded to binary32
    float r;      // 1 / sqrt(var + eps), rounded
    float a;      // gamma r, rounded
    float beta;
    float lo, hi; // h > 0  <=>  lo < x < hi
};

__device__ __forceinline__ Chan chan_params(const double* stats, int cl, float gamma, float beta,
                                            float eps)
{
    const double mean = stats[2 * cl], var = stats[2 * cl + 1];
    const double sd = sqrt(var + (double)eps);
    const double rr = 1.0 / sd;
    Chan c;
    c.mu = (float)mean;
    c.r = (float)rr;
    c.a = (float)((double)gamma * rr);
    c.beta = beta;
    // gamma (x - mean) / sd + beta > 0  <=>  x > t (gamma > 0) or x < t
    // (gamma < 0), t = mean - beta sd / gamma; for gamma = 0 it is beta > 0.
    if (gamma > 0.0f) {
        c.lo = f32_down(mean - (double)beta * sd / (double)gamma);
        c.hi = INFINITY;
    } else if (gamma < 0.0f) {
        c.lo = -INFINITY;
        c.hi = f32_up(mean - (double)beta * sd / (double)gamma);
    } else {
        c.lo = beta > 0.0f ? -INFINITY : INFINITY;
        c.hi = INFINITY;
    }
    return c;
}

__device__ __forceinline__ bool passes(float x, const Chan& c) { return x > c.lo && x < c.hi; }

// ---------------------------------------------------------------------------
// Block reduction of two binary64 sums; every thread receives the totals.
// The order of additions is fixed, so every block (and every call) that
// reduces the same values gets the same bits.
// ---------------------------------------------------------------------------

__device__ __forceinline__ void block_sum2(double& a, double& b)
{
    __shared__ double part[2 * kWaves];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        a += __shfl_xor(a, o);
        b += __shfl_xor(b, o);
    }
    const int w = (int)threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        part[2 * w] = a;
        part[2 * w + 1] = b;
    }
    __syncthreads();
    a = 0.0;
    b = 0.0;
#pragma unroll
    for (int k = 0; k < kWaves; ++k) {
        a += part[2 * k];
        b += part[2 * k + 1];
    }
}

// Offsets (in elements) of vector v of channel (cl of a C-channel map).
__device__ __forceinline__ int64_t elem_offset(uint32_t v, const FastDiv& pv, int64_t channels,
                                               int64_t cl, int V)
{
    const uint32_t row = fdiv(v, pv);
    const uint32_t pos = v - row * pv.d;
    return (((int64_t)row * channels + cl) * (int64_t)pv.d + pos) * V;
}

// ---------------------------------------------------------------------------
// Kernels.  V is the vector width in elements (Elem<IO>::kVec, or 1 for the
// element-wise path); each lane handles kPer vectors of its block's chunk.
// ---------------------------------------------------------------------------

template <typename IO, int V>
__global__ __launch_bounds__(kBlock) void stats_partial_kernel(const IO* __restrict__ x,
                                                               int channels, Geom geo,
                                                               double* __restrict__ ws)
{
    constexpr int kChunk = chunk_elems<IO>();
    constexpr int kPer = kChunk / (kBlock * V);
    const int c = (int)blockIdx.x / geo.chunks;
    const int chunk = (int)blockIdx.x - c * geo.chunks;
    Raw<IO, V> rx[kPer];
    bool ok[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const uint32_t v = (uint32_t)chunk * (uint32_t)(kChunk / V) + (uint32_t)(i * kBlock) +
                           threadIdx.x;
        ok[i] = v < geo.mv;
        if (ok[i])
            rx[i].template fetch<kNtX>(x, elem_offset(v, geo.pv, channels, c, V));
    }
    float pivot[1];
    Elem<IO>::template load<false>(x, (int64_t)c * geo.pv.d * V, pivot);
    const double k = (double)pivot[0];
    double s1 = 0.0, s2 = 0.0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        if (!ok[i])
            continue;
        float f[V];
        rx[i].unpack(f);
#pragma unroll
        for (int e = 0; e < V; ++e) {
            const double d = (double)f[e] - k;
            s1 += d;
            s2 = fma(d, d, s2);
        }
    }
    block_sum2(s1, s2);
    if (threadIdx.x == 0) {
        ws[2 * (int64_t)blockIdx.x] = s1;
        ws[2 * (int64_t)blockIdx.x + 1] = s2;
    }
}

// One block per channel: sum the channel's partials (lane-strided, then the
// block reduction), then mean = pivot + S1 / M, var = S2 / M - (S1 / M)^2.
template <typename IO>
__global__ __launch_bounds__(kBlock) void stats_final_kernel(const IO* __restrict__ x, Geom geo,
                                                             int vec, const double* __restrict__ ws,
                                                             double* __restrict__ stats)
{
    const int c = (int)blockIdx.x;
    double s1 = 0.0, s2 = 0.0;
    for (int k = (int)threadIdx.x; k < geo.chunks; k += kBlock) {
        s1 += ws[2 * ((int64_t)c * geo.chunks + k)];
        s2 += ws[2 * ((int64_t)c * geo.chunks + k) + 1];
    }
    block_sum2(s1, s2);
    if (threadIdx.x == 0) {
        float pivot[1];
        Elem<IO>::template load<false>(x, (int64_t)c * geo.pv.d * vec, pivot);
        const double m1 = s1 / geo.m;
        double var = s2 / geo.m - m1 * m1;
        if (!(var > 0.0))
            var = 0.0;
        stats[2 * c] = (double)pivot[0] + m1;
        stats[2 * c + 1] = var;
    }
}

template <typename IO, int V>
__global__ __launch_bounds__((fwd_block<IO, V>())) void fwd_kernel(
    Table t, Geom geo, int z_channels, const float* __restrict__ gamma,
    const float* __restrict__ beta, float eps, IO* __restrict__ z)
{
    constexpr int kChunk = chunk_elems<IO, fwd_chunk_bytes<IO, V>()>();
    constexpr int kB = fwd_block<IO, V>();
    constexpr int kPer = kChunk / (kB * V);
    const Where w = locate(t, geo.chunks);
    const IO* x = static_cast<const IO*>(t.x[w.j]);
    const int cj = t.channels[w.j];
    Raw<IO, V> rx[kPer];
    uint32_t vv[kPer];
    bool ok[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        vv[i] = (uint32_t)w.chunk * (uint32_t)(kChunk / V) + (uint32_t)(i * kB) + threadIdx.x;
        ok[i] = vv[i] < geo.mv;
        if (ok[i])
            rx[i].template fetch<kNtX>(x, elem_offset(vv[i], geo.pv, cj, w.cl, V));
    }
    const Chan ch = chan_params(t.stats[w.j], w.cl, gamma[w.zc], beta[w.zc], eps);
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        if (!ok[i])
            continue;
        float f[V], y[V];
        rx[i].unpack(f);
#pragma unroll
        for (int e = 0; e < V; ++e) {
            const float h = fmaf(f[e] - ch.mu, ch.a, ch.beta);
            y[e] = passes(f[e], ch) ? fmaxf(h, 0.0f) : 0.0f;
        }
        Elem<IO>::template store<kNtOut>(z, elem_offset(vv[i], geo.pv, z_channels, w.zc, V), y);
    }
}

template <typename IO, int V>
__global__ __launch_bounds__(kBlock) void bwd_reduce_kernel(Table t, Geom geo, int z_channels,
                                                            const float* __restrict__ gamma,
                                                            const float* __restrict__ beta,
                                                            float eps, const IO* __restrict__ dz,
                                                            double* __restrict__ ws)
{
    constexpr int kChunk = chunk_elems<IO>();
    constexpr int kPer = kChunk / (kBlock * V);
    const Where w = locate(t, geo.chunks);
    const IO* x = static_cast<const IO*>(t.x[w.j]);
    const int cj = t.channels[w.j];
    Raw<IO, V> rx[kPer], rd[kPer];
    bool ok[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const uint32_t v =
            (uint32_t)w.chunk * (uint32_t)(kChunk / V) + (uint32_t)(i * kBlock) + threadIdx.x;
        ok[i] = v < geo.mv;
        if (ok[i]) {
            rx[i].template fetch<kNtX>(x, elem_offset(v, geo.pv, cj, w.cl, V));
            rd[i].template fetch<kNtDz>(dz, elem_offset(v, geo.pv, z_channels, w.zc, V));
        }
    }
    const Chan ch = chan_params(t.stats[w.j], w.cl, gamma[w.zc], beta[w.zc], eps);
    double sg = 0.0, sgx = 0.0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        if (!ok[i])
            continue;
        float f[V], d[V];
        rx[i].unpack(f);
        rd[i].unpack(d);
#pragma unroll
        for (int e = 0; e < V; ++e) {
            const float g = passes(f[e], ch) ? d[e] : 0.0f;
            const float xh = (f[e] - ch.mu) * ch.r;
            sg += (double)g;
            sgx = fma((double)g, (double)xh, sgx);
        }
    }
    block_sum2(sg, sgx);
    if (threadIdx.x == 0) {
        ws[2 * (int64_t)blockIdx.x] = sg;
        ws[2 * (int64_t)blockIdx.x + 1] = sgx;
    }
}

template <typename IO, int V>
__global__ __launch_bounds__(kBlock) void bwd_apply_kernel(Table t, Geom geo, int z_channels,
                                                           const float* __restrict__ gamma,
                                                           const float* __restrict__ beta,
                                                           float eps, const IO* __restrict__ dz,
                                                           const double* __restrict__ ws,
                                                           float* __restrict__ dgamma,
                                                           float* __restrict__ dbeta)
{
    constexpr int kChunk = chunk_elems<IO>();
    constexpr int kPer = kChunk / (kBlock * V);
    const Where w = locate(t, geo.chunks);
    const IO* x = static_cast<const IO*>(t.x[w.j]);
    IO* dx = static_cast<IO*>(t.dx[w.j]);
    const int cj = t.channels[w.j];
    Raw<IO, V> rx[kPer], rd[kPer];
    int64_t off[kPer];
    bool ok[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const uint32_t v =
            (uint32_t)w.chunk * (uint32_t)(kChunk / V) + (uint32_t)(i * kBlock) + threadIdx.x;
        ok[i] = v < geo.mv;
        if (ok[i]) {
            off[i] = elem_offset(v, geo.pv, cj, w.cl, V);
            rx[i].template fetch<kNtX>(x, off[i]);
            rd[i].template fetch<kNtDz>(dz, elem_offset(v, geo.pv, z_channels, w.zc, V));
        }
    }
    // This channel's sums over all its blocks' partials.
    double sg = 0.0, sgx = 0.0;
    const int64_t base = (int64_t)w.g * geo.chunks;
    for (int k = (int)threadIdx.x; k < geo.chunks; k += kBlock) {
        sg += ws[2 * (base + k)];
        sgx += ws[2 * (base + k) + 1];
    }
    block_sum2(sg, sgx);
    if (w.chunk == 0 && threadIdx.x == 0) {
        dbeta[w.zc] = (float)sg;
        dgamma[w.zc] = (float)sgx;
    }
    const Chan ch = chan_params(t.stats[w.j], w.cl, gamma[w.zc], beta[w.zc], eps);
    const float k1 = (float)(sg / geo.m);
    const float k2 = (float)(sgx / geo.m);
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        if (!ok[i])
            continue;
        float f[V], d[V], out[V];
        rx[i].unpack(f);
        rd[i].unpack(d);
#pragma unroll
        for (int e = 0; e < V; ++e) {
            const float g = passes(f[e], ch) ? d[e] : 0.0f;
            const float xh = (f[e] - ch.mu) * ch.r;
            out[e] = ch.a * (g - fmaf(xh, k2, k1));
        }
        Elem<IO>::template store<kNtOut>(dx, off[i], out);
    }
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------

static FastDiv make_fastdiv(uint32_t d)
{
    uint32_t s = 0;
    while ((1ull << s) < d)
        ++s;
    const uint64_t m = ((1ull << 32) * ((1ull << s) - d)) / d + 1;
    return FastDiv{d, (uint32_t)m, s};
}

static size_t esize(int dtype) { return dtype == MESWISH_F32 ? 4 : 2; }

static bool dtype_ok(int dtype) { return dtype == MESWISH_F32 || dtype == MESWISH_BF16; }

static bool overlaps(const void* a, size_t na, const void* b, size_t nb)
{
    uintptr_t pa = (uintptr_t)a, pb = (uintptr_t)b;
    return na && nb && pa < pb + nb && pb < pa + na;
}

// Elements per channel within the limits, else 0.
static uint64_t channel_elems(size_t n, size_t hw)
{
    if (n == 0 || hw == 0 || hw >= (1ull << 31) || n >= (1ull << 31))
        return 0;
    const uint64_t m = (uint64_t)n * (uint64_t)hw;
    return m < (1ull << 31) ? m : 0;
}

static int chunks_of(uint64_t m, int chunk) { return (int)((m + chunk - 1) / chunk); }

template <typename IO, int kBytes = DENSE_BN_CHUNK_BYTES>
static Geom make_geom(size_t n, size_t hw, int V)
{
    Geom g;
    g.pv = make_fastdiv((uint32_t)(hw / V));
    g.mv = (uint32_t)(n * (hw / V));
    g.m = (double)((uint64_t)n * hw);
    g.chunks = chunks_of((uint64_t)n * hw, chunk_elems<IO, kBytes>());
    return g;
}

static int launch(const void* fn, int64_t grid, void** args, hipStream_t stream,
                  int block = kBlock)
{
    if (grid <= 0 || grid > 0x7FFFFFFF)
        return MESWISH_EINVAL;
    hipError_t e = hipLaunchKernel(fn, dim3((unsigned)grid), dim3(block), args, 0, stream);
    return e == hipSuccess ? MESWISH_OK : MESWISH_EHIP;
}

// A set of device ranges, each an input or an output, checked pairwise:
// no output may overlap any other range.
struct Regions {
    struct R {
        const void* p;
        size_t bytes;
        bool out;
    };
    R r[4 * kMaxSources + 16];
    int count = 0;
    void add(const void* p, size_t bytes, bool out) { r[count++] = R{p, bytes, out}; }
    bool disjoint() const
    {
        for (int i = 0; i < count; ++i)
            for (int k = i + 1; k < count; ++k)
                if ((r[i].out || r[k].out) && overlaps(r[i].p, r[i].bytes, r[k].p, r[k].bytes))
                    return false;
        return true;
    }
};

static bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Validate a call's sources and build its table.  Returns a status; on
// success *vec tells whether every tensor allows 16-byte vectors.
static int build_table(const dense_bn_source* src, int count, size_t n, size_t hw, int z_channels,
                       int dtype, bool bwd, Table& t, int& total, bool& vec, Regions& reg)
{
    if (count < 0)
        return MESWISH_EINVAL;
    if (count > kMaxSources)
        return MESWISH_ETOOMANY;
    if (count > 0 && !src)
        return MESWISH_EINVAL;
    const size_t es = esize(dtype);
    const size_t vec_bytes = 16;
    vec = (hw * es) % vec_bytes == 0;
    total = 0;
    for (int j = 0; j < kMaxSources; ++j) {
        t.x[j] = nullptr;
        t.dx[j] = nullptr;
        t.stats[j] = nullptr;
        t.channels[j] = 0;
        t.offset[j] = 0;
        t.first[j] = 0x7FFFFFFF;
    }
    for (int j = 0; j < count; ++j) {
        const dense_bn_source& s = src[j];
        if (!s.x || !s.stats || s.channels < 1 || s.offset < 0 ||
            (int64_t)s.offset + s.channels > (int64_t)z_channels)
            return MESWISH_EINVAL;
        if (bwd && !s.dx)
            return MESWISH_EINVAL;
        if (!aligned(s.x, es) || !aligned(s.stats, 8) || (bwd && !aligned(s.dx, es)))
            return MESWISH_EINVAL;
        vec = vec && aligned(s.x, vec_bytes) && (!bwd || aligned(s.dx, vec_bytes));
        for (int k = 0; k < j; ++k)
            if (s.offset < src[k].offset + src[k].channels && src[k].offset < s.offset + s.channels)
                return MESWISH_EINVAL;  // two sources claim the same channel
        if ((int64_t)total + s.channels > 0x7FFFFFFF)
            return MESWISH_EINVAL;
        t.x[j] = s.x;
        t.dx[j] = s.dx;
        t.stats[j] = s.stats;
        t.channels[j] = s.channels;
        t.offset[j] = s.offset;
        t.first[j] = total;
        total += s.channels;
        const size_t bytes = n * (size_t)s.channels * hw * es;
        reg.add(s.x, bytes, false);
        reg.add(s.stats, (size_t)s.channels * 2 * sizeof(double), false);
        if (bwd)
            reg.add(s.dx, bytes, true);
    }
    return MESWISH_OK;
}

template <typename IO, int V>
static int run_stats(const void* x, size_t n, int channels, size_t hw, double* stats, double* ws,
                     hipStream_t stream)
{
    Geom geo = make_geom<IO>(n, hw, V);
    const IO* xp = static_cast<const IO*>(x);
    void* a1[] = {&xp, &channels, &geo, &ws};
    int st = launch(reinterpret_cast<const void*>(&stats_partial_kernel<IO, V>),
                    (int64_t)channels * geo.chunks, a1, stream);
    if (st != MESWISH_OK)
        return st;
    int vec = V;
    void* a2[] = {&xp, &geo, &vec, &ws, &stats};
    return launch(reinterpret_cast<const void*>(&stats_final_kernel<IO>), channels, a2, stream);
}

template <typename IO, int V>
static int run_fwd(Table& t, int total, size_t n, size_t hw, int z_channels, const float* gamma,
                   const float* beta, float eps, void* z, hipStream_t stream)
{
    Geom geo = make_geom<IO, fwd_chunk_bytes<IO, V>()>(n, hw, V);
    IO* zp = static_cast<IO*>(z);
    void* a[] = {&t, &geo, &z_channels, &gamma, &beta, &eps, &zp};
    return launch(reinterpret_cast<const void*>(&fwd_kernel<IO, V>),
                  (int64_t)total * geo.chunks, a, stream, fwd_block<IO, V>());
}

template <typename IO, int V>
static int run_bwd(Table& t, int total, size_t n, size_t hw, int z_channels, const float* gamma,
                   const float* beta, float eps, const void* dz, float* dgamma, float* dbeta,
                   double* ws, hipStream_t stream)
{
    Geom geo = make_geom<IO>(n, hw, V);
    const IO* dzp = static_cast<const IO*>(dz);
    const int64_t grid = (int64_t)total * geo.chunks;
    void* a1[] = {&t, &geo, &z_channels, &gamma, &beta, &eps, &dzp, &ws};
    int st = launch(reinterpret_cast<const void*>(&bwd_reduce_kernel<IO, V>), grid, a1, stream);
    if (st != MESWISH_OK)
        return st;
    const double* wsc = ws;
    void* a2[] = {&t, &geo, &z_channels, &gamma, &beta, &eps, &dzp, &wsc, &dgamma, &dbeta};
    return launch(reinterpret_cast<const void*>(&bwd_apply_kernel<IO, V>), grid, a2, stream);
}

}  // namespace dense_bn

using namespace dense_bn;

extern "C" size_t dense_bn_workspace_bytes(size_t n, size_t channels, size_t hw)
{
    const uint64_t m = channel_elems(n, hw);
    if (m == 0 || channels == 0 || channels >= (1ull << 31))
        return 0;
    return channels * (size_t)chunks_of(m, kMinChunk) * 2 * sizeof(double);
}

extern "C" int dense_bn_stats(const void* x, size_t n, int channels, size_t hw, int dtype,
                              double* stats, void* workspace, size_t workspace_bytes, void* stream)
{
    if (!dtype_ok(dtype) || channels < 1 || !x || !stats || !workspace)
        return MESWISH_EINVAL;
    const size_t need = dense_bn_workspace_bytes(n, (size_t)channels, hw);
    if (need == 0 || workspace_bytes < need)
        return MESWISH_EINVAL;
    const size_t es = esize(dtype);
    if (!aligned(x, es) || !aligned(stats, 8) || !aligned(workspace, 8))
        return MESWISH_EINVAL;
    Regions reg;
    reg.add(x, n * (size_t)channels * hw * es, false);
    reg.add(stats, (size_t)channels * 2 * sizeof(double), true);
    reg.add(workspace, need, true);
    if (!reg.disjoint())
        return MESWISH_EALIAS;
    const bool vec = aligned(x, 16) && (hw * es) % 16 == 0;
    double* ws = static_cast<double*>(workspace);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (dtype == MESWISH_F32)
        return vec ? run_stats<float, 4>(x, n, channels, hw, stats, ws, s)
                   : run_stats<float, 1>(x, n, channels, hw, stats, ws, s);
    return vec ? run_stats<bf16_t, 8>(x, n, channels, hw, stats, ws, s)
               : run_stats<bf16_t, 1>(x, n, channels, hw, stats, ws, s);
}

static bool params_ok(int z_channels, const float* gamma, const float* beta, float eps)
{
    return z_channels >= 1 && gamma && beta && aligned(gamma, 4) && aligned(beta, 4) &&
           isfinite(eps) && eps > 0.0f;
}

extern "C" int dense_bn_relu_fwd(const dense_bn_source* src, int count, size_t n, size_t hw,
                                 int z_channels, const float* gamma, const float* beta, float eps,
                                 void* z, int dtype, void* stream)
{
    if (!dtype_ok(dtype) || !params_ok(z_channels, gamma, beta, eps) || !z ||
        channel_elems(n, hw) == 0)
        return MESWISH_EINVAL;
    if (!aligned(z, esize(dtype)))
        return MESWISH_EINVAL;
    Table t;
    int total = 0;
    bool vec = false;
    Regions reg;
    int st = build_table(src, count, n, hw, z_channels, dtype, false, t, total, vec, reg);
    if (st != MESWISH_OK)
        return st;
    if (count == 0)
        return MESWISH_OK;
    reg.add(z, n * (size_t)z_channels * hw * esize(dtype), true);
    reg.add(gamma, (size_t)z_channels * 4, false);
    reg.add(beta, (size_t)z_channels * 4, false);
    if (!reg.disjoint())
        return MESWISH_EALIAS;
    vec = vec && aligned(z, 16);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (dtype == MESWISH_F32)
        return vec ? run_fwd<float, 4>(t, total, n, hw, z_channels, gamma, beta, eps, z, s)
                   : run_fwd<float, 1>(t, total, n, hw, z_channels, gamma, beta, eps, z, s);
    return vec ? run_fwd<bf16_t, 8>(t, total, n, hw, z_channels, gamma, beta, eps, z, s)
               : run_fwd<bf16_t, 1>(t, total, n, hw, z_channels, gamma, beta, eps, z, s);
}

namespace dense_bn {

// The backward of both entry points; `workspace` is the caller's memory or
// the library's static scratch.  too_big: status when the workspace is
// smaller than the call needs.
static int relu_bwd(const dense_bn_source* src, int count, size_t n, size_t hw, int z_channels,
                    const float* gamma, const float* beta, float eps, const void* dz,
                    float* dgamma, float* dbeta, void* workspace, size_t workspace_bytes,
                    int dtype, hipStream_t s, int too_big)
{
    if (!dtype_ok(dtype) || !params_ok(z_channels, gamma, beta, eps) || !dz || !dgamma ||
        !dbeta || !workspace || channel_elems(n, hw) == 0)
        return MESWISH_EINVAL;
    if (!aligned(dz, esize(dtype)) || !aligned(dgamma, 4) || !aligned(dbeta, 4) ||
        !aligned(workspace, 8))
        return MESWISH_EINVAL;
    Table t;
    int total = 0;
    bool vec = false;
    Regions reg;
    int st = build_table(src, count, n, hw, z_channels, dtype, true, t, total, vec, reg);
    if (st != MESWISH_OK)
        return st;
    if (count == 0)
        return MESWISH_OK;
    const size_t need = dense_bn_workspace_bytes(n, (size_t)total, hw);
    if (need == 0)
        return MESWISH_EINVAL;
    if (workspace_bytes < need)
        return too_big;
    reg.add(dz, n * (size_t)z_channels * hw * esize(dtype), false);
    reg.add(gamma, (size_t)z_channels * 4, false);
    reg.add(beta, (size_t)z_channels * 4, false);
    reg.add(dgamma, (size_t)z_channels * 4, true);
    reg.add(dbeta, (size_t)z_channels * 4, true);
    reg.add(workspace, need, true);
    if (!reg.disjoint())
        return MESWISH_EALIAS;
    vec = vec && aligned(dz, 16);
    double* ws = static_cast<double*>(workspace);
    if (dtype == MESWISH_F32)
        return vec ? run_bwd<float, 4>(t, total, n, hw, z_channels, gamma, beta, eps, dz, dgamma,
                                       dbeta, ws, s)
                   : run_bwd<float, 1>(t, total, n, hw, z_channels, gamma, beta, eps, dz, dgamma,
                                       dbeta, ws, s);
    return vec ? run_bwd<bf16_t, 8>(t, total, n, hw, z_channels, gamma, beta, eps, dz, dgamma,
                                    dbeta, ws, s)
               : run_bwd<bf16_t, 1>(t, total, n, hw, z_channels, gamma, beta, eps, dz, dgamma,
                                    dbeta, ws, s);
}

}  // namespace dense_bn

extern "C" int dense_bn_relu_bwd(const dense_bn_source* src, int count, size_t n, size_t hw,
                                 int z_channels, const float* gamma, const float* beta, float eps,
                                 const void* dz, float* dgamma, float* dbeta, void* workspace,
                                 size_t workspace_bytes, int dtype, void* stream)
{
    return relu_bwd(src, count, n, hw, z_channels, gamma, beta, eps, dz, dgamma, dbeta, workspace,
                    workspace_bytes, dtype, static_cast<hipStream_t>(stream), MESWISH_EINVAL);
}

// ---------------------------------------------------------------------------
// The backward without a caller workspace: its per-block partial sums go to
// `scratch`, a fixed array in device memory that every GPU the library runs
// on holds until the process ends.  Host code never passes the array's name
// to a kernel (on the host it is a stand-in symbol, not a device address):
// its address on each device is looked up once, with that device current,
// and kept per device.  Every partial slot a call reads is written by the
// same call first, so the array needs no clearing; calls that overlap on
// one GPU share the array and race.
// ---------------------------------------------------------------------------

static __device__ __align__(256) double scratch[DENSE_BN_STATIC_WORKSPACE_BYTES / sizeof(double)];

namespace dense_bn {

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mutex;
static void* g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on the current device, or nullptr.
static void* scratch_on_current_device()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess)
            return nullptr;
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}

}  // namespace dense_bn

extern "C" int dense_bn_relu_bwd_noalloc(const dense_bn_source* src, int count, size_t n,
                                         size_t hw, int z_channels, const float* gamma,
                                         const float* beta, float eps, const void* dz,
                                         float* dgamma, float* dbeta, int dtype, void* stream)
{
    void* ws = scratch_on_current_device();
    if (!ws)
        return MESWISH_EHIP;
    return relu_bwd(src, count, n, hw, z_channels, gamma, beta, eps, dz, dgamma, dbeta, ws,
                    DENSE_BN_STATIC_WORKSPACE_BYTES, dtype, static_cast<hipStream_t>(stream),
                    MESWISH_ESCRATCH);
}
