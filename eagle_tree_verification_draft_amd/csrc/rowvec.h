// rowvec.h -- 16-byte vector access to one logit row (fp32, or bf16 held as
// uint16 bits), shared by the row-statistics and acceptance kernels.
#pragma once
#include "common.h"

namespace eagle {

template <typename T> struct Vec;
template <> struct Vec<float> { static constexpr int n = 4; };
template <> struct Vec<uint16_t> { static constexpr int n = 8; };

template <typename T>
__device__ __forceinline__ void unpack(const uint4 &u, float *out);
template <>
__device__ __forceinline__ void unpack<float>(const uint4 &u, float *o)
{
    o[0] = __uint_as_float(u.x); o[1] = __uint_as_float(u.y);
    o[2] = __uint_as_float(u.z); o[3] = __uint_as_float(u.w);
}
template <>
__device__ __forceinline__ void unpack<uint16_t>(const uint4 &u, float *o)
{
    o[0] = bf16_lo(u.x); o[1] = bf16_hi(u.x); o[2] = bf16_lo(u.y); o[3] = bf16_hi(u.y);
    o[4] = bf16_lo(u.z); o[5] = bf16_hi(u.z); o[6] = bf16_lo(u.w); o[7] = bf16_hi(u.w);
}

template <typename T>
__device__ __forceinline__ float load_scalar(const T *p);
template <> __device__ __forceinline__ float load_scalar<float>(const float *p) { return *p; }
template <> __device__ __forceinline__ float load_scalar<uint16_t>(const uint16_t *p) { return bf16_to_f32(*p); }

// One 16-byte vector of a row starting at element `base`; missing elements
// read as -inf (never a candidate, weight 0).  Logit rows are read with the
// default cache policy: they are usually written just before, and a
// non-temporal read does not benefit from lines still held in the caches.
template <typename T>
__device__ __forceinline__ uint4 load_vec(const T *row, int base, int V, bool vec_ok)
{
    constexpr int VEC = Vec<T>::n;
    if (vec_ok && base + VEC <= V) return *reinterpret_cast<const uint4 *>(row + base);
    float f[8];
#pragma unroll
    for (int e = 0; e < VEC; ++e) f[e] = (base + e < V) ? load_scalar<T>(row + base + e) : -__builtin_inff();
    if constexpr (VEC == 4) {
        return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3]));
    } else {
        // re-pack to bf16 pairs (values came from bf16, so truncation is exact)
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            w[e] = (__float_as_uint(f[2 * e]) >> 16) | (__float_as_uint(f[2 * e + 1]) & 0xffff0000u);
        return make_uint4(w[0], w[1], w[2], w[3]);
    }
}

// Branch-free row load for rows whose 16-byte vectors are aligned and that hold
// at least one full vector: vector gi is loaded from min(gi, nfull - 1) (nfull =
// V / VEC full vectors) so every load issues back to back; a vector at or past
// the ragged end is then rebuilt from scalar loads, -inf past the end.
template <typename T>
__device__ __forceinline__ uint4 load_vec_clamped(const T *row, int gi, int nfull)
{
    constexpr int VEC = Vec<T>::n;
    return *reinterpret_cast<const uint4 *>(row + (size_t)min(gi, nfull - 1) * VEC);
}
template <typename T>
__device__ __forceinline__ void fix_tail(uint4 &v, const T *row, int gi, int nfull, int V)
{
    if (gi >= nfull) v = load_vec<T>(row, gi * Vec<T>::n, V, false);
}

}  // namespace eagle
