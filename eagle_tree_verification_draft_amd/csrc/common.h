// common.h -- device helpers shared by the libeagle kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/eagle.h"

namespace eagle {

constexpr int kWave = 64;
constexpr int kMaxChildren = 16;
constexpr int kMaxMMax = 64;
constexpr int kMaxHeads = 1024;           // query heads per call
constexpr long long kMaxQueryRows = 1ll << 26;   // batch x num_q_heads x m_max
constexpr int kMaxVocab = 1 << 17;

// ---------------------------------------------------------------------------
// softmax weights: w = floor(exp_s(x) * 2^35), x = (l - M) / T clamped at -32.
// exp_s: y = x * RN32(1/ln2); n = rint(y); f = y - n; p = sum_j RN32(ln2^j/j!) f^j
// by Horner with fused multiply-adds; exp_s = p * 2^n.  All fp32, no
// contraction (the library is built with -ffp-contract=off).
// ---------------------------------------------------------------------------
constexpr float kL2E = 0x1.715476p+0f;
constexpr float kE0 = 0x1.000000p+0f;
constexpr float kE1 = 0x1.62e430p-1f;
constexpr float kE2 = 0x1.ebfbe0p-3f;
constexpr float kE3 = 0x1.c6b08ep-5f;
constexpr float kE4 = 0x1.3b2ab6p-7f;
constexpr float kE5 = 0x1.5d87fep-10f;
constexpr float kE6 = 0x1.430912p-13f;
// adding 1.5 * 2^23 rounds any |y| < 2^22 to an integer (ties to even) and
// leaves that integer in the low mantissa bits
constexpr float kRoundMagic = 0x1.8p+23f;
constexpr int kRoundMagicBits = 0x4B400000;

// Weight of an already-formed x (NaN in -> NaN out; no undefined conversions).
__device__ __forceinline__ float weight_from_x(float x)
{
    x = __builtin_elementwise_maximum(x, -32.0f);   // clamp below at -32; NaN stays NaN
    const float y = x * kL2E;
    const float t = y + kRoundMagic;
    const float n = t - kRoundMagic;
    const int ni = __float_as_int(t) - kRoundMagicBits;
    const float f = y - n;
    float p = kE6;
    p = __builtin_fmaf(p, f, kE5);
    p = __builtin_fmaf(p, f, kE4);
    p = __builtin_fmaf(p, f, kE3);
    p = __builtin_fmaf(p, f, kE2);
    p = __builtin_fmaf(p, f, kE1);
    p = __builtin_fmaf(p, f, kE0);
    return __builtin_floorf(__builtin_ldexpf(p, ni + 35));
}

__device__ __forceinline__ float weight_of(float l, float M) { return weight_from_x(l - M); }

__device__ __forceinline__ float weight_of_t(float l, float M, float T, bool unit_t)
{
    const float d = l - M;
    return weight_from_x(unit_t ? d : d / T);
}

// ---------------------------------------------------------------------------
// 16-byte loads; the streaming variant marks the lines non-temporal (data read
// once, e.g. logit rows) so they do not displace reused data in the caches
// ---------------------------------------------------------------------------
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 ld16_stream(const void *p)
{
    const u32x4 v = __builtin_nontemporal_load(static_cast<const u32x4 *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// Hides a value's origin from the optimiser so that expressions derived from
// it are recomputed instead of being kept live across loops (register pressure).
__device__ __forceinline__ uint4 opaque(uint4 v)
{
    asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w));
    return v;
}

// ---------------------------------------------------------------------------
// element conversions
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// round-to-nearest-even fp32 -> bf16 bits (NaN kept quiet)
__device__ __forceinline__ uint16_t f32_to_bf16(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// (value desc, id asc): does (va, ia) come before (vb, ib)?
__device__ __forceinline__ bool before(float va, int ia, float vb, int ib)
{
    return va > vb || (va == vb && ia < ib);
}

// ---------------------------------------------------------------------------
// wave / block reductions (blockDim.x a multiple of 64, <= 1024)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

__device__ __forceinline__ double wave_sum_d(double v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

__device__ __forceinline__ int wave_sum_i(int v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// argmax by (value desc, id asc) over the wave
__device__ __forceinline__ void wave_best(float &v, int &id)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float ov = __shfl_xor(v, o);
        const int oi = __shfl_xor(id, o);
        if (before(ov, oi, v, id)) { v = ov; id = oi; }
    }
}

// Scratch for the block reductions: 16 slots per kind.
struct BlockScratch {
    float f[16];
    int i[16];
    double d[16];
};

__device__ __forceinline__ float block_max(float v, BlockScratch &s)
{
    const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
    v = wave_max(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) s.f[w] = v;
    __syncthreads();
    float r = s.f[0];
    for (int j = 1; j < nw; ++j) r = fmaxf(r, s.f[j]);
    return r;
}

__device__ __forceinline__ double block_sum_d(double v, BlockScratch &s)
{
    const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
    v = wave_sum_d(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) s.d[w] = v;
    __syncthreads();
    double r = 0.0;
    for (int j = 0; j < nw; ++j) r += s.d[j];
    return r;
}

__device__ __forceinline__ void block_best(float &v, int &id, BlockScratch &s)
{
    const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
    wave_best(v, id);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) { s.f[w] = v; s.i[w] = id; }
    __syncthreads();
    v = s.f[0];
    id = s.i[0];
    for (int j = 1; j < nw; ++j)
        if (before(s.f[j], s.i[j], v, id)) { v = s.f[j]; id = s.i[j]; }
}

// exclusive prefix sum over the block; returns the block total in *total
__device__ __forceinline__ int block_exclusive_scan(int v, int *total, BlockScratch &s)
{
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
    int incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(incl, o);
        if (lane >= o) incl += t;
    }
    __syncthreads();
    if (lane == 63) s.i[w] = incl;
    __syncthreads();
    int base = 0, tot = 0;
    for (int j = 0; j < nw; ++j) {
        if (j < w) base += s.i[j];
        tot += s.i[j];
    }
    *total = tot;
    return base + incl - v;
}

// ---------------------------------------------------------------------------
// workspace header: the first 256 bytes of every workspace
// ---------------------------------------------------------------------------
struct WsHeader {
    uint32_t err;
    uint32_t pad[63];
};
constexpr size_t kWsHeader = 256;

__device__ __forceinline__ void raise_error(uint32_t *err, uint32_t bits)
{
    if (err) atomicOr(err, bits);
}

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace eagle
