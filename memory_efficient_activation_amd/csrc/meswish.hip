// meswish.hip -- HIP kernels and C-ABI launchers of libmeswish for gfx950.
//
// The operation (blog post "Memory efficient Swish", adeeplearner.github.io,
// 2021-05-17):
//   forward  ("How is Swish implemented?")               y  = x * Sigmoid(t)
//   backward ("How is the memory efficient version Swish implemented?")
//                                                          dx = dy * s * (1 + t (1 - s))
// with t = alpha x and s = Sigmoid(t) = 1 / (1 + e^-t) ("What is a Swish
// activation function?").  The backward reads only x and dy: the input is
// the one tensor kept between the passes.  The same save-the-input skeleton
// serves the activation family of "What activations cost, in memory and in
// arithmetic" (Given); the per-element math of each is in act_math.h.
//
// Design for MI355X (CDNA4):
//   * The work is element-wise with an arithmetic intensity of about one to
//     two flops per byte ("What activations cost, in memory and in
//     arithmetic", Conclusion), far below the ~20 flop/byte ridge of the
//     chip's vector ALUs, so HBM bandwidth is the bound: no LDS, no MFMA, no
//     atomics, no barriers.  Each lane moves 16-byte vectors (4 binary32 or
//     8 bfloat16), a wave touches 1 KiB contiguous per access, and a thread
//     issues all its loads of a tile before any arithmetic.
//   * One tile of kBlock x kUnroll vectors per block, one block
//     per tile (the dispatcher keeps all 256 CUs of the 8 XCDs busy and
//     balances the tail); the loop over tiles only matters when the grid
//     is capped.  Tile shape and cache policy (non-temporal loads/stores
//     per stream) were chosen by measurement on MI355X.
//   * Arithmetic is binary32 with the hardware exp2 and reciprocal
//     (v_exp_f32, v_rcp_f32).  For Swish: E = e^-t = 2^(-t log2 e),
//     s = 1 / (1 + E), 1 - s = E s.  Both s and 1 - s come out with small
//     relative error for every t (no cancellation); the forward costs one
//     exp, one reciprocal and three multiply/adds per element.
//   * binary32 I/O: exponents are carried as hi+lo pairs where the result's
//     accuracy depends on them.
//   * Results whose exponential leaves [2^-125, 2^125] take a rare branch,
//     per wave, that applies small factors by powers of two (frexp/ldexp)
//     so that subnormal results round once and keep gradual underflow (the
//     hardware transcendentals flush subnormals).
//   * bfloat16 I/O: widening is a 16-bit shift; narrowing is the gfx950
//     v_cvt_pk_bf16_f32 (round to nearest even), two elements per op.

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <string.h>

#include <atomic>

#include "meswish.h"
#include "act_math.h"

// Threads per block, per element type and direction (one wave: measured
// against 128, 256 and 512, and against other sizes per direction, on the
// bf16 [8, 2048, 4096] Swish: the fastest step and the fastest kernels
// alone).
#ifndef MESWISH_BLOCK_BF16
#define MESWISH_BLOCK_BF16 64
#endif
#ifndef MESWISH_BLOCK_BF16_FWD
#define MESWISH_BLOCK_BF16_FWD MESWISH_BLOCK_BF16
#endif
#ifndef MESWISH_BLOCK_BF16_BWD
#define MESWISH_BLOCK_BF16_BWD MESWISH_BLOCK_BF16
#endif
#ifndef MESWISH_BLOCK_F32
#define MESWISH_BLOCK_F32 64
#endif
// Threads per block of the grouped kernel (bf16): one wave, as for single
// tensors (measured against 128 and 256 with 1, 2 and 4 tiles per block:
// 6583 GB/s for the EfficientNet-shaped group against 6253-6313 with 256
// threads).
#ifndef MESWISH_GROUP_BLOCK_BF16
#define MESWISH_GROUP_BLOCK_BF16 64
#endif
// 16-byte vectors per thread and stream, per element type.
#ifndef MESWISH_UNROLL_BF16
#define MESWISH_UNROLL_BF16 1
#endif
#ifndef MESWISH_UNROLL_F32
#define MESWISH_UNROLL_F32 1
#endif
// Consecutive tiles per block of the grouped kernel.  A grouped block finds
// its tensor through dependent scalar loads before its first vector load;
// with one-wave blocks two tiles per block share that cost best in both
// directions (one: 6344-6359 GB/s, four: 6229-6304).
#ifndef MESWISH_GROUP_TILES_FWD
#define MESWISH_GROUP_TILES_FWD 2
#endif
#ifndef MESWISH_GROUP_TILES_BWD
#define MESWISH_GROUP_TILES_BWD 2
#endif
#ifndef MESWISH_BLOCKS_PER_CU
#define MESWISH_BLOCKS_PER_CU 100000
#endif
// Minimum waves per SIMD the compiler must allow (caps VGPRs); 0 = no cap.
#ifndef MESWISH_MIN_WAVES
#define MESWISH_MIN_WAVES 0
#endif
#if MESWISH_MIN_WAVES > 0
#define MESWISH_BOUNDS __launch_bounds__((Shape<IO, kBwd>::kBlock), MESWISH_MIN_WAVES)
#define MESWISH_GROUP_BOUNDS __launch_bounds__((GroupShape<IO, kBwd>::kBlock), MESWISH_MIN_WAVES)
#else
#define MESWISH_BOUNDS __launch_bounds__((Shape<IO, kBwd>::kBlock))
#define MESWISH_GROUP_BOUNDS __launch_bounds__((GroupShape<IO, kBwd>::kBlock))
#endif
#define MESWISH_COPY_BOUNDS __launch_bounds__(MESWISH_COPY_BLOCK)
// Non-temporal (streaming) cache policy per stream, as bit masks:
// 1 = loads of x, 2 = loads of dy, 4 = stores of the result; chosen per
// direction and element type by measurement.
#ifndef MESWISH_NT_FWD_BF16
#define MESWISH_NT_FWD_BF16 5
#endif
#ifndef MESWISH_NT_BWD_BF16
#define MESWISH_NT_BWD_BF16 6
#endif
#ifndef MESWISH_NT_FWD_F32
#define MESWISH_NT_FWD_F32 5
#endif
#ifndef MESWISH_NT_BWD_F32
#define MESWISH_NT_BWD_F32 7
#endif
#ifndef MESWISH_NT_COPY
#define MESWISH_NT_COPY 5
#endif
#ifndef MESWISH_COPY_BLOCK
#define MESWISH_COPY_BLOCK 64
#endif
#ifndef MESWISH_COPY_UNROLL
#define MESWISH_COPY_UNROLL 1
#endif

namespace meswish {

constexpr int kCopyBlock = MESWISH_COPY_BLOCK;
constexpr int kCopyUnroll = MESWISH_COPY_UNROLL;
constexpr int kCopyTileVecs = kCopyBlock * kCopyUnroll;

// ---------------------------------------------------------------------------
// Element types.
// ---------------------------------------------------------------------------

struct bf16_t {
    uint16_t bits;
};

typedef float float2_v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    float2_v f = {lo, hi};
    bf16x2_v b = __builtin_convertvector(f, bf16x2_v);
    uint32_t u;
    __builtin_memcpy(&u, &b, sizeof u);
    return u;
}

template <typename IO> struct Io;

template <> struct Io<float> {
    static constexpr int kPerVec = 4;
    static constexpr bool kPrecise = true;
    __device__ static void unpack(const uint4& v, float (&f)[4])
    {
        f[0] = __uint_as_float(v.x);
        f[1] = __uint_as_float(v.y);
        f[2] = __uint_as_float(v.z);
        f[3] = __uint_as_float(v.w);
    }
    __device__ static uint4 pack(const float (&f)[4])
    {
        return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]),
                          __float_as_uint(f[2]), __float_as_uint(f[3]));
    }
    __device__ static float load1(const float* p, int64_t i) { return p[i]; }
    __device__ static void store1(float* p, int64_t i, float v) { p[i] = v; }
};

template <> struct Io<bf16_t> {
    static constexpr int kPerVec = 8;
    static constexpr bool kPrecise = false;
    __device__ static void unpack(const uint4& v, float (&f)[8])
    {
        f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
        f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
        f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
        f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
    }
    __device__ static uint4 pack(const float (&f)[8])
    {
        return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]),
                          pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7]));
    }
    __device__ static float load1(const bf16_t* p, int64_t i)
    {
        return __uint_as_float((uint32_t)p[i].bits << 16);
    }
    __device__ static void store1(bf16_t* p, int64_t i, float v)
    {
        p[i].bits = (uint16_t)(pack_bf16x2(v, 0.0f) & 0xFFFFu);
    }
};

template <typename IO, bool kBwd> struct NtPolicy;
template <> struct NtPolicy<float, false> { static constexpr int kMask = MESWISH_NT_FWD_F32; };
template <> struct NtPolicy<float, true> { static constexpr int kMask = MESWISH_NT_BWD_F32; };
template <> struct NtPolicy<bf16_t, false> { static constexpr int kMask = MESWISH_NT_FWD_BF16; };
template <> struct NtPolicy<bf16_t, true> { static constexpr int kMask = MESWISH_NT_BWD_BF16; };

// Launch shape per element type and direction: threads per block and
// 16-byte vectors per thread and stream.
template <typename IO, bool kBwd> struct Shape;
template <bool kBwd> struct Shape<float, kBwd> {
    static constexpr int kBlock = MESWISH_BLOCK_F32;
    static constexpr int kUnroll = MESWISH_UNROLL_F32;
};
template <bool kBwd> struct Shape<bf16_t, kBwd> {
    static constexpr int kBlock = kBwd ? MESWISH_BLOCK_BF16_BWD : MESWISH_BLOCK_BF16_FWD;
    static constexpr int kUnroll = MESWISH_UNROLL_BF16;
};

// The grouped kernel's shape.
template <typename IO, bool kBwd> struct GroupShape : Shape<IO, kBwd> {};
template <bool kBwd> struct GroupShape<bf16_t, kBwd> : Shape<bf16_t, kBwd> {
    static constexpr int kBlock = MESWISH_GROUP_BLOCK_BF16;
};

// 16-byte vectors per tile (one block's share of work).
template <typename IO, bool kBwd, typename SH = Shape<IO, kBwd>>
constexpr int tile_vecs() { return SH::kBlock * SH::kUnroll; }

typedef uint32_t u32x4_v __attribute__((ext_vector_type(4)));

// 16-byte global load / store; kNT selects the non-temporal (streaming)
// cache policy.
template <bool kNT>
__device__ __forceinline__ uint4 ld16(const uint4* p)
{
    if (kNT) {
        u32x4_v v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_v*>(p));
        return make_uint4(v.x, v.y, v.z, v.w);
    }
    return *p;
}

template <bool kNT>
__device__ __forceinline__ void st16(uint4* p, const uint4& v)
{
    if (kNT) {
        u32x4_v w = {v.x, v.y, v.z, v.w};
        __builtin_nontemporal_store(w, reinterpret_cast<u32x4_v*>(p));
    } else {
        *p = v;
    }
}

constexpr int kNtCopy = MESWISH_NT_COPY;

// One 16-byte vector of the forward / backward of activation ACT.
template <typename IO, int ACT>
__device__ __forceinline__ uint4 fwd_vec(const uint4& xv, const Coef& k)
{
    using Op = ActOp<ACT>;
    constexpr int E = Io<IO>::kPerVec;
    constexpr bool P = Io<IO>::kPrecise;
    float xf[E], yf[E];
    Io<IO>::unpack(xv, xf);
    float rk = 0.0f;
#pragma unroll
    for (int j = 0; j < E; ++j)
        yf[j] = Op::template fwd<P>(xf[j], k, rk);
    if (Op::kHasRare && __builtin_expect(rk > Op::template rare_thr<P>(), 0)) {
#pragma unroll
        for (int j = 0; j < E; ++j)
            if (Op::template is_rare<false, P>(xf[j], k))
                yf[j] = Op::fwd_rare(xf[j], k);
    }
    return Io<IO>::pack(yf);
}

template <typename IO, int ACT>
__device__ __forceinline__ uint4 bwd_vec(const uint4& xv, const uint4& dv, const Coef& k)
{
    using Op = ActOp<ACT>;
    constexpr int E = Io<IO>::kPerVec;
    constexpr bool P = Io<IO>::kPrecise;
    float xf[E], df[E], gf[E];
    Io<IO>::unpack(xv, xf);
    Io<IO>::unpack(dv, df);
    float rk = 0.0f;
#pragma unroll
    for (int j = 0; j < E; ++j)
        gf[j] = Op::template bwd<P>(xf[j], df[j], k, rk);
    if (Op::kHasRare && __builtin_expect(rk > Op::template rare_thr<P>(), 0)) {
#pragma unroll
        for (int j = 0; j < E; ++j)
            if (Op::template is_rare<true, P>(xf[j], k))
                gf[j] = Op::bwd_rare(xf[j], df[j], k);
    }
    return Io<IO>::pack(gf);
}

// One element (head, tail and unaligned paths).
template <typename IO, bool kBwd, int ACT>
__device__ __forceinline__ void one_element(const IO* x, const IO* dy, IO* out, int64_t i,
                                            const Coef& k)
{
    using Op = ActOp<ACT>;
    constexpr bool P = Io<IO>::kPrecise;
    float xv = Io<IO>::load1(x, i);
    float rk = 0.0f;
    float r;
    if (kBwd) {
        float dv = Io<IO>::load1(dy, i);
        r = Op::template bwd<P>(xv, dv, k, rk);
        if (Op::kHasRare && rk > Op::template rare_thr<P>())
            r = Op::bwd_rare(xv, dv, k);
    } else {
        r = Op::template fwd<P>(xv, k, rk);
        if (Op::kHasRare && rk > Op::template rare_thr<P>())
            r = Op::fwd_rare(xv, k);
    }
    Io<IO>::store1(out, i, r);
}

// One tile: the nv <= tile_vecs<IO, kBwd>() 16-byte vectors that start at xb, db,
// ob.  The base pointers and nv are uniform over the block and lane offsets
// are 32-bit, so every load and store addresses as a scalar base plus a
// vector offset, with no 64-bit address arithmetic per lane.
template <typename IO, bool kBwd, int ACT, typename SH = Shape<IO, kBwd>,
          int kNt = NtPolicy<IO, kBwd>::kMask>
__device__ __forceinline__ void body_tile(const uint4* xb, const uint4* db, uint4* ob,
                                          uint32_t nv, const Coef& k)
{
    constexpr int kUnroll = SH::kUnroll;
    constexpr int kBlock = SH::kBlock;
    const uint32_t i = threadIdx.x;
    if (nv == (uint32_t)tile_vecs<IO, kBwd, SH>()) {
        uint4 a[kUnroll], b[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            a[u] = ld16<(kNt & 1) != 0>(xb + (i + u * kBlock));
        if (kBwd) {
#pragma unroll
            for (int u = 0; u < kUnroll; ++u)
                b[u] = ld16<(kNt & 2) != 0>(db + (i + u * kBlock));
        }
        // Keep every load of the tile ahead of the first use of its data, so
        // that a thread has all of them in flight at once.
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            st16<(kNt & 4) != 0>(ob + (i + u * kBlock),
                                  kBwd ? bwd_vec<IO, ACT>(a[u], b[u], k) : fwd_vec<IO, ACT>(a[u], k));
    } else {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint32_t j = i + u * kBlock;
            if (j < nv) {
                uint4 a = ld16<(kNt & 1) != 0>(xb + j);
                uint4 r;
                if (kBwd)
                    r = bwd_vec<IO, ACT>(a, ld16<(kNt & 2) != 0>(db + j), k);
                else
                    r = fwd_vec<IO, ACT>(a, k);
                st16<(kNt & 4) != 0>(ob + j, r);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Kernels.
// ---------------------------------------------------------------------------

// Single tensor, all pointers congruent modulo 16 bytes: `head` scalar
// elements, then a body of 16-byte vectors in `tiles` tiles (all full but
// the last, which holds last_vecs vectors), then `tail` scalar elements.
// Tile indices are 32-bit (the host splits larger tensors into several
// launches); the loop over tiles only runs more than once when the grid is
// capped.
template <typename IO, bool kBwd, int ACT>
__global__ MESWISH_BOUNDS void act_vec_kernel(const IO* x, const IO* dy, IO* out,
                                              uint32_t head, uint32_t tiles,
                                              uint32_t last_vecs, uint32_t tail, Coef k)
{
    constexpr int E = Io<IO>::kPerVec;
    constexpr uint32_t kTileVecs = tile_vecs<IO, kBwd>();
    const uint4* xv = reinterpret_cast<const uint4*>(x + head);
    const uint4* dv = kBwd ? reinterpret_cast<const uint4*>(dy + head) : nullptr;
    uint4* ov = reinterpret_cast<uint4*>(out + head);
    for (uint32_t t = blockIdx.x; t < tiles; t += gridDim.x) {
        const size_t v0 = (size_t)t * kTileVecs;
        body_tile<IO, kBwd, ACT>(xv + v0, kBwd ? dv + v0 : nullptr, ov + v0,
                                 t + 1 < tiles ? kTileVecs : last_vecs, k);
    }
    if (blockIdx.x == 0 && threadIdx.x < head + tail) {
        const size_t nvec = tiles ? (size_t)(tiles - 1) * kTileVecs + last_vecs : 0;
        const size_t i = threadIdx.x < head ? (size_t)threadIdx.x
                                            : head + nvec * E + (threadIdx.x - head);
        one_element<IO, kBwd, ACT>(x, dy, out, (int64_t)i, k);
    }
}

// Single tensor, element by element (pointers not congruent modulo 16).
template <typename IO, bool kBwd, int ACT>
__global__ MESWISH_BOUNDS void act_elem_kernel(const IO* x, const IO* dy, IO* out,
                                                            int64_t n, Coef k)
{
    constexpr int kBlock = Shape<IO, kBwd>::kBlock;
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n; i += stride)
        one_element<IO, kBwd, ACT>(x, dy, out, i, k);
}

// Grouped: up to MESWISH_MAX_GROUP tensors in one launch.  Tensor j covers
// tiles [tile_begin[j], tile_begin[j+1]) of the concatenated tile space; a
// block takes G consecutive tiles at a time (G b .. G b + G - 1, then G
// (b + gridDim) ..) and finds each tile's tensor by a forward scan (tiles of
// one block are increasing, so the scan is amortised O(1)).  The first tile of a tensor also does its scalar head and
// tail.  A tensor whose pointers are not congruent modulo 16 bytes (flag 0)
// is processed element by element, tile_vecs<IO, kBwd>() elements per tile.
struct GroupArgs {
    const void* x[MESWISH_MAX_GROUP];
    const void* dy[MESWISH_MAX_GROUP];
    void* out[MESWISH_MAX_GROUP];
    int64_t n[MESWISH_MAX_GROUP];
    int64_t tile_begin[MESWISH_MAX_GROUP + 1];
    int32_t head[MESWISH_MAX_GROUP];  // -1: element-wise tensor
    int32_t count;
};

template <typename IO, bool kBwd, int ACT>
__global__ MESWISH_GROUP_BOUNDS void act_group_kernel(GroupArgs g, Coef k)
{
    constexpr int E = Io<IO>::kPerVec;
    using SH = GroupShape<IO, kBwd>;
    constexpr int kUnroll = SH::kUnroll;
    constexpr int64_t kTileVecs = tile_vecs<IO, kBwd, SH>();
    constexpr int G = kBwd ? MESWISH_GROUP_TILES_BWD : MESWISH_GROUP_TILES_FWD;
    const int64_t total = g.tile_begin[g.count];
    int j = 0;
    for (int64_t tile = blockIdx.x * (int64_t)G; tile < total;
         tile += (tile % G == G - 1) ? (int64_t)gridDim.x * G - (G - 1) : 1) {
        while (tile >= g.tile_begin[j + 1])
            ++j;
        const IO* x = static_cast<const IO*>(g.x[j]);
        const IO* dy = static_cast<const IO*>(g.dy[j]);
        IO* out = static_cast<IO*>(g.out[j]);
        const int64_t n = g.n[j];
        const int64_t local = tile - g.tile_begin[j];
        const int32_t head = g.head[j];
        if (head < 0) {
            int64_t e0 = local * kTileVecs;
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                int64_t i = e0 + u * SH::kBlock + threadIdx.x;
                if (i < n)
                    one_element<IO, kBwd, ACT>(x, dy, out, i, k);
            }
            continue;
        }
        const int64_t nvec = (n - head) / E;
        const int64_t tail = n - head - nvec * E;
        const int64_t v0 = local * kTileVecs;
        const int64_t left = nvec - v0;
        const uint32_t nv = left >= kTileVecs ? (uint32_t)kTileVecs : (uint32_t)(left > 0 ? left : 0);
        body_tile<IO, kBwd, ACT, SH>(reinterpret_cast<const uint4*>(x + head) + v0,
                                 kBwd ? reinterpret_cast<const uint4*>(dy + head) + v0 : nullptr,
                                 reinterpret_cast<uint4*>(out + head) + v0, nv, k);
        const int64_t t = threadIdx.x;  // head >= 0 here
        if (local == 0 && t < head + tail) {
            int64_t i = t < head ? t : head + nvec * E + (t - head);
            one_element<IO, kBwd, ACT>(x, dy, out, i, k);
        }
    }
}

// Plain 16-byte copy (measurement helper).
__global__ MESWISH_COPY_BOUNDS void copy16_kernel(const uint4* src, uint4* dst, int64_t nvec)
{
    const int64_t stride = (int64_t)gridDim.x * kCopyTileVecs;
    for (int64_t t0 = (int64_t)blockIdx.x * kCopyTileVecs; t0 < nvec; t0 += stride) {
        int64_t i = t0 + threadIdx.x;
        if (t0 + kCopyTileVecs <= nvec) {
            uint4 a[kCopyUnroll];
#pragma unroll
            for (int u = 0; u < kCopyUnroll; ++u)
                a[u] = ld16<(kNtCopy & 1) != 0>(src + i + u * kCopyBlock);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int u = 0; u < kCopyUnroll; ++u)
                st16<(kNtCopy & 4) != 0>(dst + i + u * kCopyBlock, a[u]);
        } else {
#pragma unroll
            for (int u = 0; u < kCopyUnroll; ++u)
                if (i + u * kCopyBlock < nvec)
                    st16<(kNtCopy & 4) != 0>(dst + i + u * kCopyBlock,
                                               ld16<(kNtCopy & 1) != 0>(src + i + u * kCopyBlock));
        }
    }
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------

constexpr int kMaxDevices = 64;
static std::atomic<int> g_cu_count[kMaxDevices];

// Compute units of the current device (cached per device).
static int cu_count()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0)
        return 256;
    if (dev < kMaxDevices) {
        int c = g_cu_count[dev].load(std::memory_order_relaxed);
        if (c > 0)
            return c;
    }
    int c = 0;
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        c <= 0)
        c = 256;
    if (dev < kMaxDevices)
        g_cu_count[dev].store(c, std::memory_order_relaxed);
    return c;
}

// Blocks for `tiles` tiles of `block` threads: one block per tile, capped
// at MESWISH_BLOCKS_PER_CU per compute unit and so that grid x block stays
// below 2^32 threads, the launch limit (the kernels loop over the tiles a
// capped grid leaves).
static int64_t grid_for_tiles(int64_t tiles, int block)
{
    int64_t cap = (int64_t)cu_count() * MESWISH_BLOCKS_PER_CU;
    const int64_t thread_cap = (int64_t)(UINT32_MAX / (uint32_t)block);
    if (cap > thread_cap)
        cap = thread_cap;
    if (tiles < 1)
        tiles = 1;
    return tiles < cap ? tiles : cap;
}

// Tiles per launch of the vector kernel: tile indices stay 32-bit, and a
// tile index plus the grid never wraps.  Longer tensors take several
// launches of this many tiles each.  (A test build sets a small value so
// that the multi-launch split runs on tensors that fit a GPU.)
#ifndef MESWISH_MAX_LAUNCH_TILES
#define MESWISH_MAX_LAUNCH_TILES (1 << 30)
#endif
constexpr int64_t kMaxLaunchTiles = (int64_t)(MESWISH_MAX_LAUNCH_TILES);
static_assert(kMaxLaunchTiles >= 1 && kMaxLaunchTiles <= ((int64_t)1 << 30),
              "tile indices and tile + grid must stay below 2^32");

static size_t elem_size(int dtype) { return dtype == MESWISH_F32 ? 4 : 2; }

static bool dtype_ok(int dtype) { return dtype == MESWISH_F32 || dtype == MESWISH_BF16; }

// Ranges [a, a+na) and [b, b+nb) overlap.
static bool overlaps(const void* a, size_t na, const void* b, size_t nb)
{
    uintptr_t pa = (uintptr_t)a, pb = (uintptr_t)b;
    return na && nb && pa < pb + nb && pb < pa + na;
}

// An output range may coincide exactly with an input range of the same
// tensor, or be disjoint from it.
static bool alias_ok(const void* out, const void* in, size_t bytes)
{
    return out == in || !overlaps(out, bytes, in, bytes);
}

static int launch(const void* fn, int64_t grid, void** args, hipStream_t stream, int block)
{
    hipError_t e = hipLaunchKernel(fn, dim3((unsigned)grid), dim3(block), args, 0, stream);
    return e == hipSuccess ? MESWISH_OK : MESWISH_EHIP;
}

// Elements before the first 16-byte boundary of p (p element-aligned).
static int64_t head_elems(const void* p, size_t esize)
{
    uintptr_t mis = (uintptr_t)p & 15u;
    return mis ? (int64_t)((16u - mis) / esize) : 0;
}

// Per-activation coefficients (see Coef in act_math.h).
static Coef make_coef(int act, float p)
{
    const double log2e = 1.44269504088896340735992468100189214;
    const double sqrt_2_over_pi = 0.797884560802865355879892119868763737;
    double c = 0.0;
    switch (act) {
    case kSwish:
        c = -(double)p * log2e;  // e^-(p x)
        break;
    case kSigmoid:
        c = -log2e;  // e^-x
        break;
    case kTanh:
        c = -2.0 * log2e;  // e^-2|x|
        break;
    case kGeluErf:
        c = -0.5 * log2e;  // e^-(x^2 / 2)
        break;
    case kGeluTanh:
        c = -2.0 * sqrt_2_over_pi * log2e;  // e^-2u over x (1 + 0.044715 x^2)
        break;
    default:
        break;
    }
    const double cubic = 0.044715;
    Coef k;
    k.p = p;
    k.c_hi = (float)c;
    k.c_lo = (float)(c - (double)k.c_hi);
    k.aux_hi = (float)cubic;
    k.aux_lo = (float)(cubic - (double)k.aux_hi);
    return k;
}

// How one tensor is split between the kernels' paths (see meswish_plan_t).
template <typename IO, bool kBwd, typename SH = Shape<IO, kBwd>>
static meswish_plan_t make_plan(const void* x, const void* dy, const void* out, size_t n)
{
    constexpr int E = Io<IO>::kPerVec;
    constexpr int64_t kTileVecs = tile_vecs<IO, kBwd, SH>();
    meswish_plan_t p;
    memset(&p, 0, sizeof p);
    uintptr_t mx = (uintptr_t)x & 15u, mo = (uintptr_t)out & 15u;
    uintptr_t md = kBwd ? ((uintptr_t)dy & 15u) : mx;
    const int64_t nn = (int64_t)n;
    if (mx == mo && mx == md) {
        int64_t head = head_elems(x, sizeof(IO));
        if (head > nn)
            head = nn;
        p.path = MESWISH_PATH_VECTOR;
        p.head = head;
        p.nvec = (nn - head) / E;
        p.tail = nn - head - p.nvec * E;
        p.tiles = (p.nvec + kTileVecs - 1) / kTileVecs;
    } else {
        p.path = MESWISH_PATH_ELEMENT;
        p.tail = nn;
        p.tiles = (nn + kTileVecs - 1) / kTileVecs;
    }
    p.block = SH::kBlock;
    if (p.path == MESWISH_PATH_VECTOR) {
        p.launches = p.tiles > kMaxLaunchTiles ? (p.tiles + kMaxLaunchTiles - 1) / kMaxLaunchTiles : 1;
        p.grid = grid_for_tiles(p.tiles < kMaxLaunchTiles ? p.tiles : kMaxLaunchTiles, (int)p.block);
    } else {
        p.launches = 1;
        p.grid = grid_for_tiles(p.tiles, (int)p.block);
    }
    p.elems_per_vector = E;
    p.vectors_per_tile = kTileVecs;
    return p;
}

template <typename IO, bool kBwd, int ACT>
static int run_single(const void* x, const void* dy, void* out, size_t n, Coef k,
                      hipStream_t stream)
{
    constexpr int E = Io<IO>::kPerVec;
    constexpr int64_t kTileVecs = tile_vecs<IO, kBwd>();
    const meswish_plan_t p = make_plan<IO, kBwd>(x, dy, out, n);
    const IO* xp = static_cast<const IO*>(x);
    const IO* dp = static_cast<const IO*>(dy);
    IO* op = static_cast<IO*>(out);
    if (p.path == MESWISH_PATH_VECTOR) {
        // Launch c covers tiles [c L, min((c + 1) L, tiles)) of the body, L =
        // kMaxLaunchTiles; the first also does the head, the last the tail.
        int64_t done = 0;  // elements of the body before launch c
        for (int64_t c = 0; c < p.launches; ++c) {
            const int64_t t0 = c * kMaxLaunchTiles;
            const int64_t nt = p.tiles - t0 < kMaxLaunchTiles ? p.tiles - t0 : kMaxLaunchTiles;
            const int64_t vecs = (t0 + nt) * kTileVecs <= p.nvec ? nt * kTileVecs : p.nvec - t0 * kTileVecs;
            const bool first = c == 0, last = c + 1 == p.launches;
            uint32_t head = first ? (uint32_t)p.head : 0;
            uint32_t tail = last ? (uint32_t)p.tail : 0;
            uint32_t tiles = (uint32_t)nt;
            uint32_t last_vecs = nt ? (uint32_t)(vecs - (nt - 1) * kTileVecs) : 0;
            const int64_t off = first ? 0 : p.head + done;
            const IO* xc = xp + off;
            const IO* dc = kBwd ? dp + off : dp;
            IO* oc = op + off;
            void* args[] = {&xc, &dc, &oc, &head, &tiles, &last_vecs, &tail, &k};
            int rc = launch(reinterpret_cast<const void*>(&act_vec_kernel<IO, kBwd, ACT>), p.grid,
                            args, stream, (int)p.block);
            if (rc != MESWISH_OK)
                return rc;
            done += vecs * E;
        }
        return MESWISH_OK;
    }
    int64_t nn = (int64_t)n;
    void* args[] = {&xp, &dp, &op, &nn, &k};
    return launch(reinterpret_cast<const void*>(&act_elem_kernel<IO, kBwd, ACT>), p.grid, args,
                  stream, (int)p.block);
}

template <bool kBwd, int ACT>
static int run_dtype(int dtype, const void* x, const void* dy, void* out, size_t n, Coef k,
                     hipStream_t s)
{
    if (dtype == MESWISH_F32)
        return run_single<float, kBwd, ACT>(x, dy, out, n, k, s);
    return run_single<bf16_t, kBwd, ACT>(x, dy, out, n, k, s);
}

template <bool kBwd>
static int run_act(int act, int dtype, const void* x, const void* dy, void* out, size_t n,
                   float p, hipStream_t s)
{
    const Coef k = make_coef(act, p);
    switch (act) {
    case kSwish:
        // alpha == 1: the backward without the multiply by alpha (the same
        // results bit for bit, as alpha x = x exactly).
        if (kBwd && p == 1.0f)
            return run_dtype<kBwd, kSwishUnit>(dtype, x, dy, out, n, k, s);
        return run_dtype<kBwd, kSwish>(dtype, x, dy, out, n, k, s);
    case kRelu:
        return run_dtype<kBwd, kRelu>(dtype, x, dy, out, n, k, s);
    case kLeakyRelu:
        return run_dtype<kBwd, kLeakyRelu>(dtype, x, dy, out, n, k, s);
    case kSigmoid:
        return run_dtype<kBwd, kSigmoid>(dtype, x, dy, out, n, k, s);
    case kTanh:
        return run_dtype<kBwd, kTanh>(dtype, x, dy, out, n, k, s);
    case kGeluErf:
        return run_dtype<kBwd, kGeluErf>(dtype, x, dy, out, n, k, s);
    case kGeluTanh:
        return run_dtype<kBwd, kGeluTanh>(dtype, x, dy, out, n, k, s);
    default:
        return MESWISH_EINVAL;
    }
}

template <typename IO, bool kBwd>
static int run_group(GroupArgs& g, Coef k, hipStream_t stream)
{
    int64_t tiles = 0;
    for (int j = 0; j < g.count; ++j) {
        g.tile_begin[j] = tiles;
        int64_t t = 0;
        g.head[j] = 0;
        if (g.n[j] > 0) {
            const meswish_plan_t p =
                make_plan<IO, kBwd, GroupShape<IO, kBwd>>(g.x[j], g.dy[j], g.out[j], (size_t)g.n[j]);
            if (p.path == MESWISH_PATH_VECTOR) {
                g.head[j] = (int32_t)p.head;
                // A tensor shorter than one vector still needs its scalar tile.
                t = p.tiles > 0 ? p.tiles : 1;
            } else {
                g.head[j] = -1;
                t = p.tiles;
            }
        }
        tiles += t;
    }
    g.tile_begin[g.count] = tiles;
    if (tiles == 0)
        return MESWISH_OK;
    constexpr int G = kBwd ? MESWISH_GROUP_TILES_BWD : MESWISH_GROUP_TILES_FWD;
    int64_t grid = grid_for_tiles((tiles + G - 1) / G, GroupShape<IO, kBwd>::kBlock);
    void* args[] = {&g, &k};
    const void* fn = kBwd && k.p == 1.0f
                         ? reinterpret_cast<const void*>(&act_group_kernel<IO, kBwd, kSwishUnit>)
                         : reinterpret_cast<const void*>(&act_group_kernel<IO, kBwd, kSwish>);
    return launch(fn, grid, args, stream, GroupShape<IO, kBwd>::kBlock);
}

// Common argument checks.  Returns MESWISH_OK or an error code.
static int check_common(float alpha, int dtype)
{
    if (!dtype_ok(dtype))
        return MESWISH_EINVAL;
    if (!isfinite(alpha))
        return MESWISH_EINVAL;
    return MESWISH_OK;
}

// Swish's exponent coefficient -alpha log2 e must be a finite binary32
// value (|alpha| <= about 2.36e38); beyond that the kernels' e^-t = 2^(x C)
// would take C = -inf.
static int check_swish_alpha(float alpha)
{
    const double c = -(double)alpha * 1.44269504088896340735992468100189214;
    return isfinite((float)c) ? MESWISH_OK : MESWISH_EINVAL;
}

static int check_tensor(const void* p, size_t n, size_t esize)
{
    if (p == nullptr)
        return MESWISH_EINVAL;
    if ((uintptr_t)p % esize)
        return MESWISH_EINVAL;
    if (n > (size_t)INT64_MAX / 16)
        return MESWISH_EINVAL;
    return MESWISH_OK;
}

}  // namespace meswish

using namespace meswish;

namespace meswish {

// Argument checks of one single-tensor call (dy is NULL for the forward).
static int check_single(int act, const void* x, const void* dy, const void* out, size_t n,
                        float alpha, int dtype, bool bwd)
{
    int rc = check_common(alpha, dtype);
    if (rc == MESWISH_OK && act == kSwish)
        rc = check_swish_alpha(alpha);
    if (rc != MESWISH_OK || n == 0)
        return rc;
    size_t es = elem_size(dtype);
    if ((rc = check_tensor(x, n, es)) != MESWISH_OK || (rc = check_tensor(out, n, es)) != MESWISH_OK)
        return rc;
    if (bwd && (rc = check_tensor(dy, n, es)) != MESWISH_OK)
        return rc;
    if (!alias_ok(out, x, n * es) || (bwd && !alias_ok(out, dy, n * es)))
        return MESWISH_EALIAS;
    return MESWISH_OK;
}

}  // namespace meswish

extern "C" int meswish_act_fwd(int act, const void* x, void* y, size_t n, float param, int dtype,
                               void* stream)
{
    if (act < 0 || act >= kActCount)
        return MESWISH_EINVAL;
    int rc = check_single(act, x, nullptr, y, n, param, dtype, false);
    if (rc != MESWISH_OK || n == 0)
        return rc;
    return run_act<false>(act, dtype, x, nullptr, y, n, param, static_cast<hipStream_t>(stream));
}

extern "C" int meswish_act_bwd(int act, const void* x, const void* dy, void* dx, size_t n,
                               float param, int dtype, void* stream)
{
    if (act < 0 || act >= kActCount)
        return MESWISH_EINVAL;
    int rc = check_single(act, x, dy, dx, n, param, dtype, true);
    if (rc != MESWISH_OK || n == 0)
        return rc;
    return run_act<true>(act, dtype, x, dy, dx, n, param, static_cast<hipStream_t>(stream));
}

extern "C" int swish_fwd(const void* x, void* y, size_t n, float alpha, int dtype, void* stream)
{
    return meswish_act_fwd(kSwish, x, y, n, alpha, dtype, stream);
}

extern "C" int swish_bwd(const void* x, const void* dy, void* dx, size_t n, float alpha, int dtype,
                         void* stream)
{
    return meswish_act_bwd(kSwish, x, dy, dx, n, alpha, dtype, stream);
}

extern "C" int meswish_plan(const void* x, const void* dy, const void* out, size_t n, float alpha,
                            int dtype, int bwd, meswish_plan_t* plan)
{
    if (plan == nullptr)
        return MESWISH_EINVAL;
    memset(plan, 0, sizeof *plan);
    plan->path = MESWISH_PATH_NONE;
    int rc = check_single(kSwish, x, dy, out, n, alpha, dtype, bwd != 0);
    if (rc != MESWISH_OK || n == 0)
        return rc;
    if (dtype == MESWISH_F32)
        *plan = bwd ? make_plan<float, true>(x, dy, out, n) : make_plan<float, false>(x, dy, out, n);
    else
        *plan = bwd ? make_plan<bf16_t, true>(x, dy, out, n) : make_plan<bf16_t, false>(x, dy, out, n);
    return MESWISH_OK;
}

namespace meswish {

// Validates a group and fills the kernel arguments.  in2 is NULL for the
// forward.  Outputs may coincide exactly with their own tensor's inputs;
// every other overlap involving an output is rejected.
static int fill_group(GroupArgs& g, int count, const void* const* in1, const void* const* in2,
                      void* const* out, const size_t* n, int dtype)
{
    size_t es = elem_size(dtype);
    g.count = count;
    for (int j = 0; j < count; ++j) {
        int rc;
        if (n[j] == 0) {
            g.x[j] = in1[j];
            g.dy[j] = in2 ? in2[j] : nullptr;
            g.out[j] = out[j];
            g.n[j] = 0;
            continue;
        }
        if ((rc = check_tensor(in1[j], n[j], es)) != MESWISH_OK ||
            (rc = check_tensor(out[j], n[j], es)) != MESWISH_OK)
            return rc;
        if (in2 && (rc = check_tensor(in2[j], n[j], es)) != MESWISH_OK)
            return rc;
        g.x[j] = in1[j];
        g.dy[j] = in2 ? in2[j] : nullptr;
        g.out[j] = out[j];
        g.n[j] = (int64_t)n[j];
    }
    for (int j = 0; j < count; ++j) {
        size_t bj = n[j] * es;
        if (!bj)
            continue;
        if (!alias_ok(out[j], in1[j], bj) || (in2 && !alias_ok(out[j], in2[j], bj)))
            return MESWISH_EALIAS;
        for (int i = 0; i < count; ++i) {
            size_t bi = n[i] * es;
            if (i == j || !bi)
                continue;
            if (overlaps(out[j], bj, out[i], bi) || overlaps(out[j], bj, in1[i], bi) ||
                (in2 && overlaps(out[j], bj, in2[i], bi)))
                return MESWISH_EALIAS;
        }
    }
    return MESWISH_OK;
}

}  // namespace meswish

extern "C" int swish_fwd_grouped(const meswish_fwd_desc* desc, int count, float alpha, int dtype,
                                 void* stream)
{
    int rc = check_common(alpha, dtype);
    if (rc == MESWISH_OK)
        rc = check_swish_alpha(alpha);
    if (rc != MESWISH_OK)
        return rc;
    if (count < 0 || (count > 0 && desc == nullptr))
        return MESWISH_EINVAL;
    if (count > MESWISH_MAX_GROUP)
        return MESWISH_ETOOMANY;
    if (count == 0)
        return MESWISH_OK;
    const void* in1[MESWISH_MAX_GROUP];
    void* out[MESWISH_MAX_GROUP];
    size_t n[MESWISH_MAX_GROUP];
    for (int j = 0; j < count; ++j) {
        in1[j] = desc[j].x;
        out[j] = desc[j].y;
        n[j] = desc[j].n;
    }
    GroupArgs g;
    memset(&g, 0, sizeof g);
    if ((rc = fill_group(g, count, in1, nullptr, out, n, dtype)) != MESWISH_OK)
        return rc;
    Coef k = make_coef(kSwish, alpha);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (dtype == MESWISH_F32)
        return run_group<float, false>(g, k, s);
    return run_group<bf16_t, false>(g, k, s);
}

extern "C" int swish_bwd_grouped(const meswish_bwd_desc* desc, int count, float alpha, int dtype,
                                 void* stream)
{
    int rc = check_common(alpha, dtype);
    if (rc == MESWISH_OK)
        rc = check_swish_alpha(alpha);
    if (rc != MESWISH_OK)
        return rc;
    if (count < 0 || (count > 0 && desc == nullptr))
        return MESWISH_EINVAL;
    if (count > MESWISH_MAX_GROUP)
        return MESWISH_ETOOMANY;
    if (count == 0)
        return MESWISH_OK;
    const void* in1[MESWISH_MAX_GROUP];
    const void* in2[MESWISH_MAX_GROUP];
    void* out[MESWISH_MAX_GROUP];
    size_t n[MESWISH_MAX_GROUP];
    for (int j = 0; j < count; ++j) {
        in1[j] = desc[j].x;
        in2[j] = desc[j].dy;
        out[j] = desc[j].dx;
        n[j] = desc[j].n;
    }
    GroupArgs g;
    memset(&g, 0, sizeof g);
    if ((rc = fill_group(g, count, in1, in2, out, n, dtype)) != MESWISH_OK)
        return rc;
    Coef k = make_coef(kSwish, alpha);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (dtype == MESWISH_F32)
        return run_group<float, true>(g, k, s);
    return run_group<bf16_t, true>(g, k, s);
}

extern "C" int meswish_copy(const void* src, void* dst, size_t bytes, void* stream)
{
    if (bytes == 0)
        return MESWISH_OK;
    if (!src || !dst || ((uintptr_t)src & 15u) || ((uintptr_t)dst & 15u) || (bytes & 15u))
        return MESWISH_EINVAL;
    if (overlaps(src, bytes, dst, bytes))
        return MESWISH_EALIAS;
    const uint4* s = static_cast<const uint4*>(src);
    uint4* d = static_cast<uint4*>(dst);
    int64_t nvec = (int64_t)(bytes / 16);
    int64_t grid = grid_for_tiles((nvec + kCopyTileVecs - 1) / kCopyTileVecs, kCopyBlock);
    void* args[] = {&s, &d, &nvec};
    return launch(reinterpret_cast<const void*>(&copy16_kernel), grid, args,
                  static_cast<hipStream_t>(stream), kCopyBlock);
}

extern "C" const char* meswish_strerror(int status)
{
    switch (status) {
    case MESWISH_OK:
        return "success";
    case MESWISH_EINVAL:
        return "invalid argument (null or misaligned pointer, unknown dtype, non-finite alpha "
               "or Swish alpha beyond 2.3586e38, bad count or size)";
    case MESWISH_EALIAS:
        return "an output partially overlaps an input or another output";
    case MESWISH_EHIP:
        return "the HIP runtime reported an error at kernel launch";
    case MESWISH_ETOOMANY:
        return "grouped call with more tensors than MESWISH_MAX_GROUP";
    case MESWISH_ESCRATCH:
        return "the call needs more scratch than the library's static device array holds "
               "(use the entry point that takes a workspace)";
    default:
        return "unknown status";
    }
}

extern "C" int meswish_version(void) { return 100; }
