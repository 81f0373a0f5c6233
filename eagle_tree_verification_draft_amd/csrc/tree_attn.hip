// tree_attn.hip -- tree-masked attention of the draft queries over the KV
// prefix plus the draft tokens (EAGLE-1 explainer, "Role of Tree Attention";
// EAGLE-2 explainer, "Attention mask adjustment").
//
// bf16 path (head_dim 128).  Work unit = (sequence, kv head, row group,
// key split).  The G query heads of a kv head are folded into the query rows
// (row = node * G + g), so every K/V byte is read from HBM once per kv head.
// Each wave owns 32 query rows.  Per 64-key tile the workgroup stages K
// [64][128] and V^T [128][64] in LDS with 16-byte coalesced loads; each wave
// computes S^T = K Q^T and O^T += V^T P^T with v_mfma_f32_32x32x16_bf16 (fp32
// accumulation), with an online softmax in fp32 between them.  K rows are
// stored in LDS with bits 2 and 3 of the key index swapped, which makes the
// S^T accumulator registers of a lane exactly the P^T operand that lane needs
// (8 consecutive keys), so no shuffles are needed between the two products.
// The draft tokens form one extra tile (at most 64 keys) masked by the
// ancestor bits.  With several key splits, each writes an unnormalised
// partial (O, max, sum); the last split to finish (device-scope counter)
// merges them.
#include "common.h"
#include "internal.h"

namespace eagle {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kTK = 64;            // keys per tile
constexpr int kHD = 128;           // head dim of the bf16 path
constexpr int kKS = kHD + 8;       // LDS row of the K tile, bf16 elements (272 B)
constexpr int kVS = kTK + 8;       // LDS row of the V^T tile, bf16 elements (144 B)
constexpr int kMaxWaves = 8;

struct AttnArgs {
    const void *q, *kd, *vd, *kc, *vc;
    const int32_t *block_table, *prefix_len, *num_nodes;
    const uint64_t *anc;
    void *out;
    float *part_o;
    float2 *part_ml;
    uint32_t *cnt, *err;
    int Hq, Hkv, G, d, m_max, block_size, max_blocks, cap, chunk, nsplit, RG, rows_pg, units0;
    float scale_log2;
    bool v_vec;   // contiguous V^T rows are 16-byte aligned
};

__device__ __forceinline__ int swap23(int t) { return (t & ~12) | ((t & 4) << 1) | ((t & 8) >> 1); }

// address of key `key`'s K row (head_dim elements) for (b, kvh)
template <typename T>
__device__ __forceinline__ const T *k_row(const AttnArgs &a, int b, int kvh, int key)
{
    const T *kc = static_cast<const T *>(a.kc);
    if (a.block_size == 0)
        return kc + (((size_t)b * a.Hkv + kvh) * a.cap + key) * (size_t)a.d;
    const int blk = a.block_table[(size_t)b * a.max_blocks + key / a.block_size];
    return kc + (((size_t)blk * a.Hkv + kvh) * a.block_size + key % a.block_size) * (size_t)a.d;
}

// address of V^T element (e, key); consecutive keys are contiguous within a
// row of the contiguous cache and within a page of the paged cache
template <typename T>
__device__ __forceinline__ const T *v_elem(const AttnArgs &a, int b, int kvh, int e, int key)
{
    const T *vc = static_cast<const T *>(a.vc);
    if (a.block_size == 0)
        return vc + (((size_t)b * a.Hkv + kvh) * a.d + e) * (size_t)a.cap + key;
    const int blk = a.block_table[(size_t)b * a.max_blocks + key / a.block_size];
    return vc + (((size_t)blk * a.Hkv + kvh) * a.d + e) * (size_t)a.block_size + key % a.block_size;
}

struct AttnSmem {
    uint16_t K[kTK * kKS];
    uint16_t Vt[kHD * kVS];
    int last;
};

__global__ __launch_bounds__(512) void k_tree_attn_bf16(AttnArgs a)
{
    __shared__ AttnSmem sm;
    const int tid = threadIdx.x, NT = blockDim.x, lane = tid & 63, wv = tid >> 6;
    const int ln = lane & 31, hh = lane >> 5;
    // block -> (split, row group, sequence/kv head); all splits and row groups
    // of one (sequence, kv head) share blockIdx mod 8 when units0 % 8 == 0,
    // which keeps them on one XCD and its L2
    const int x = blockIdx.x;
    const int u0 = x % a.units0;
    const int rest = x / a.units0;
    const int rg = rest % a.RG, s = rest / a.RG;
    const int b = u0 / a.Hkv, kvh = u0 % a.Hkv;
    const int G = a.G, m_max = a.m_max;

    int L = a.prefix_len[b];
    if (L < 0 || L > a.cap) {
        if (tid == 0 && s == 0 && rg == 0) raise_error(a.err, EAGLE_DEVERR_PREFIX);
        L = L < 0 ? 0 : a.cap;
    }
    int n = a.num_nodes[b];
    n = n < 0 ? 0 : (n > m_max ? m_max : n);
    const int nsplit_b = L > 0 ? (L + a.chunk - 1) / a.chunk : 1;
    if (s >= nsplit_b) return;
    const int key_lo = s * a.chunk, key_hi = min(L, key_lo + a.chunk);
    const bool has_draft = (s == nsplit_b - 1);

    const int row0 = rg * a.rows_pg + wv * 32;          // first row of this wave
    const int rows_valid = n * G;                        // rows with a real node
    const bool wave_active = row0 < rows_valid && wv * 32 < a.rows_pg;
    const int my_row = row0 + ln;
    const int my_node = my_row / G;
    const bool row_ok = my_row < rows_valid;

    // Q fragments (B operand of S^T = K Q^T): lane holds q[my_row][16ks + 8hh .. +7]
    bf16x8 qf[8];
    {
        const uint16_t *qb = static_cast<const uint16_t *>(a.q);
        const int h = kvh * G + (my_row % G);
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            uint4 v = make_uint4(0, 0, 0, 0);
            if (wave_active && my_node < m_max)
                v = *reinterpret_cast<const uint4 *>(qb + (((size_t)b * m_max + my_node) * a.Hq + h) * kHD +
                                                     16 * ks + 8 * hh);
            qf[ks] = __builtin_bit_cast(bf16x8, v);
        }
    }
    uint64_t my_anc = 0;
    if (row_ok) my_anc = a.anc[(size_t)b * m_max + my_node];

    f32x16 oacc[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.0f;
    float m_run = -__builtin_inff(), l_run = 0.0f;

    const int ntiles = (key_hi - key_lo + kTK - 1) / kTK + (has_draft ? 1 : 0);
    for (int tile = 0; tile < ntiles; ++tile) {
        const bool draft = has_draft && tile == ntiles - 1;
        const int k0 = key_lo + tile * kTK;
        // ---- stage K and V^T in LDS ----
        if (!draft) {
            for (int c = tid; c < kTK * 16; c += NT) {
                const int t = c >> 4, col = (c & 15) * 8;
                uint4 v = make_uint4(0, 0, 0, 0);
                if (k0 + t < key_hi) v = *reinterpret_cast<const uint4 *>(k_row<uint16_t>(a, b, kvh, k0 + t) + col);
                *reinterpret_cast<uint4 *>(&sm.K[swap23(t) * kKS + col]) = v;
            }
            for (int c = tid; c < kHD * 8; c += NT) {
                const int e = c >> 3, kk = (c & 7) * 8;
                const int key = k0 + kk;
                uint4 v = make_uint4(0, 0, 0, 0);
                if (key + 8 <= key_hi && (a.block_size != 0 || a.v_vec)) {
                    v = *reinterpret_cast<const uint4 *>(v_elem<uint16_t>(a, b, kvh, e, key));
                } else if (key < key_hi) {
                    uint16_t h8[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) h8[j] = (key + j < key_hi) ? *v_elem<uint16_t>(a, b, kvh, e, key + j) : 0;
                    v = make_uint4(h8[0] | ((uint32_t)h8[1] << 16), h8[2] | ((uint32_t)h8[3] << 16),
                                   h8[4] | ((uint32_t)h8[5] << 16), h8[6] | ((uint32_t)h8[7] << 16));
                }
                *reinterpret_cast<uint4 *>(&sm.Vt[e * kVS + kk]) = v;
            }
        } else {
            const uint16_t *kd = static_cast<const uint16_t *>(a.kd);
            const uint16_t *vd = static_cast<const uint16_t *>(a.vd);
            for (int c = tid; c < kTK * 16; c += NT) {
                const int j = c >> 4, col = (c & 15) * 8;
                uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
                if (j < n) {
                    const size_t o = (((size_t)b * m_max + j) * a.Hkv + kvh) * kHD + col;
                    kv = *reinterpret_cast<const uint4 *>(kd + o);
                    vv = *reinterpret_cast<const uint4 *>(vd + o);
                }
                *reinterpret_cast<uint4 *>(&sm.K[swap23(j) * kKS + col]) = kv;
                const uint32_t w4[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    sm.Vt[(col + 2 * q) * kVS + j] = (uint16_t)(w4[q] & 0xffffu);
                    sm.Vt[(col + 2 * q + 1) * kVS + j] = (uint16_t)(w4[q] >> 16);
                }
            }
        }
        __syncthreads();

        if (wave_active) {
            // ---- S^T = K Q^T for the two 32-key halves ----
            f32x16 sacc[2];
#pragma unroll
            for (int sh = 0; sh < 2; ++sh) {
#pragma unroll
                for (int r = 0; r < 16; ++r) sacc[sh][r] = 0.0f;
#pragma unroll
                for (int ks = 0; ks < 8; ++ks) {
                    const bf16x8 av = *reinterpret_cast<const bf16x8 *>(&sm.K[(32 * sh + ln) * kKS + 16 * ks + 8 * hh]);
                    sacc[sh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qf[ks], sacc[sh], 0, 0, 0);
                }
            }
            // sacc[sh][8t + q] is the score of tile key 32sh + 16t + 8hh + q for row my_row
            float tmax = -__builtin_inff();
#pragma unroll
            for (int sh = 0; sh < 2; ++sh) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = 32 * sh + 16 * (r >> 3) + 8 * hh + (r & 7);
                    bool ok = row_ok;
                    if (draft) ok = ok && key < n && ((my_anc >> key) & 1ull);
                    else ok = ok && (k0 + key < key_hi);
                    const float v = ok ? sacc[sh][r] * a.scale_log2 : -__builtin_inff();
                    sacc[sh][r] = v;
                    tmax = fmaxf(tmax, v);
                }
            }
            tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
            const float m_new = fmaxf(m_run, tmax);
            const float m_use = m_new == -__builtin_inff() ? 0.0f : m_new;
            const float corr = __builtin_amdgcn_exp2f(m_run - m_use);
            float lsum = 0.0f;
            bf16x8 pf[2][2];
#pragma unroll
            for (int sh = 0; sh < 2; ++sh) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float p = __builtin_amdgcn_exp2f(sacc[sh][r] - m_use);
                    lsum += p;
                    pf[sh][r >> 3][r & 7] = (__bf16)p;
                }
            }
            lsum += __shfl_xor(lsum, 32);
            l_run = l_run * corr + lsum;
            m_run = m_new;
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[dt][r] *= corr;
            // ---- O^T += V^T P^T ----
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
                for (int sh = 0; sh < 2; ++sh) {
#pragma unroll
                    for (int t = 0; t < 2; ++t) {
                        const bf16x8 av = *reinterpret_cast<const bf16x8 *>(
                            &sm.Vt[(32 * dt + ln) * kVS + 32 * sh + 16 * t + 8 * hh]);
                        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pf[sh][t], oacc[dt], 0, 0, 0);
                    }
                }
            }
        }
        __syncthreads();
    }

    // ---- epilogue ----
    // oacc[dt][r] is O^T[d = 32dt + 8(r>>2) + 4hh + (r&3)][my_row]
    const int h_out = kvh * G + (my_row % G);
    const bool row_exists = wv * 32 + ln < a.rows_pg && my_node < m_max;
    uint16_t *out = static_cast<uint16_t *>(a.out);
    if (nsplit_b == 1) {
        if (row_exists) {
            const float inv = (row_ok && l_run > 0.0f) ? 1.0f / l_run : 0.0f;
            uint16_t *o = out + (((size_t)b * m_max + my_node) * a.Hq + h_out) * kHD;
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int d0 = 32 * dt + 8 * j + 4 * hh;
                    uint2 w;
                    w.x = f32_to_bf16(oacc[dt][4 * j] * inv) | ((uint32_t)f32_to_bf16(oacc[dt][4 * j + 1] * inv) << 16);
                    w.y = f32_to_bf16(oacc[dt][4 * j + 2] * inv) | ((uint32_t)f32_to_bf16(oacc[dt][4 * j + 3] * inv) << 16);
                    *reinterpret_cast<uint2 *>(o + d0) = w;
                }
        }
        return;
    }
    const int unit = u0 * a.RG + rg;
    const size_t pbase = ((size_t)unit * a.nsplit + s) * a.rows_pg;
    const int row_local = wv * 32 + ln;
    if (row_local < a.rows_pg) {
        float *po = a.part_o + (pbase + row_local) * kHD;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int d0 = 32 * dt + 8 * j + 4 * hh;
                *reinterpret_cast<float4 *>(po + d0) =
                    make_float4(oacc[dt][4 * j], oacc[dt][4 * j + 1], oacc[dt][4 * j + 2], oacc[dt][4 * j + 3]);
            }
        if (hh == 0) a.part_ml[pbase + row_local] = make_float2(row_ok ? m_run : -__builtin_inff(), row_ok ? l_run : 0.0f);
    }
    __threadfence();
    __syncthreads();
    if (tid == 0) {
        const unsigned prev = atomicAdd(&a.cnt[unit], 1u);
        sm.last = prev == (unsigned)(nsplit_b - 1);
    }
    __syncthreads();
    if (!sm.last) return;
    __threadfence();
    for (int idx = tid; idx < a.rows_pg * 32; idx += NT) {
        const int rl = idx >> 5, d4 = (idx & 31) * 4;
        const int row = rg * a.rows_pg + rl, node = row / G;
        if (node >= m_max) continue;
        const int h = kvh * G + (row % G);
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        if (node < n) {
            float M = -__builtin_inff();
            for (int sp = 0; sp < nsplit_b; ++sp)
                M = fmaxf(M, a.part_ml[((size_t)unit * a.nsplit + sp) * a.rows_pg + rl].x);
            const float Mu = M == -__builtin_inff() ? 0.0f : M;
            float den = 0.0f;
            for (int sp = 0; sp < nsplit_b; ++sp) {
                const size_t pr = ((size_t)unit * a.nsplit + sp) * a.rows_pg + rl;
                const float2 ml = a.part_ml[pr];
                const float wgt = __builtin_amdgcn_exp2f(ml.x - Mu);
                den += wgt * ml.y;
                const float4 o4 = *reinterpret_cast<const float4 *>(a.part_o + pr * kHD + d4);
                acc.x += wgt * o4.x; acc.y += wgt * o4.y; acc.z += wgt * o4.z; acc.w += wgt * o4.w;
            }
            const float inv = den > 0.0f ? 1.0f / den : 0.0f;
            acc.x *= inv; acc.y *= inv; acc.z *= inv; acc.w *= inv;
        }
        uint2 w;
        w.x = f32_to_bf16(acc.x) | ((uint32_t)f32_to_bf16(acc.y) << 16);
        w.y = f32_to_bf16(acc.z) | ((uint32_t)f32_to_bf16(acc.w) << 16);
        *reinterpret_cast<uint2 *>(out + (((size_t)b * m_max + node) * a.Hq + h) * kHD + d4) = w;
    }
    if (tid == 0) a.cnt[unit] = 0;
}

// ---------------------------------------------------------------------------
// fp32 path: one wave per output row (sequence, node, q head), exact fp32
// arithmetic on the vector ALUs, 64 keys per step with an online softmax.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void k_tree_attn_f32(AttnArgs a)
{
    __shared__ float s_q[kHD];
    __shared__ float s_p[64];
    const int lane = threadIdx.x;
    const int h = blockIdx.x % a.Hq;
    const int i = (blockIdx.x / a.Hq) % a.m_max;
    const int b = blockIdx.x / (a.Hq * a.m_max);
    const int kvh = h / a.G, d = a.d, m_max = a.m_max;
    float *out = static_cast<float *>(a.out) + (((size_t)b * m_max + i) * a.Hq + h) * d;
    int n = a.num_nodes[b];
    n = n < 0 ? 0 : (n > m_max ? m_max : n);
    if (i >= n) {
        for (int e = lane; e < d; e += 64) out[e] = 0.0f;
        return;
    }
    int L = a.prefix_len[b];
    if (L < 0 || L > a.cap) {
        if (lane == 0 && i == 0 && h == 0) raise_error(a.err, EAGLE_DEVERR_PREFIX);
        L = L < 0 ? 0 : a.cap;
    }
    const float *q = static_cast<const float *>(a.q) + (((size_t)b * m_max + i) * a.Hq + h) * d;
    for (int e = lane; e < d; e += 64) s_q[e] = q[e];
    const uint64_t bits = a.anc[(size_t)b * m_max + i];
    __syncthreads();
    float m_run = -__builtin_inff(), l_run = 0.0f, acc0 = 0.0f, acc1 = 0.0f;
    const int nchunks = (L + 63) / 64 + 1;
    for (int c = 0; c < nchunks; ++c) {
        const bool draft = c == nchunks - 1;
        const int key = draft ? lane : c * 64 + lane;
        bool ok;
        const float *kp;
        if (draft) {
            ok = key < n && ((bits >> key) & 1ull);
            kp = static_cast<const float *>(a.kd) + (((size_t)b * m_max + (ok ? key : 0)) * a.Hkv + kvh) * d;
        } else {
            ok = key < L;
            kp = k_row<float>(a, b, kvh, ok ? key : 0);
        }
        float sc = -__builtin_inff();
        if (ok) {
            float dot = 0.0f;
            for (int e = 0; e < d; ++e) dot = __builtin_fmaf(s_q[e], kp[e], dot);
            sc = dot * a.scale_log2;
        }
        const float cm = wave_max(sc);
        const float m_new = fmaxf(m_run, cm);
        const float m_use = m_new == -__builtin_inff() ? 0.0f : m_new;
        const float corr = __builtin_amdgcn_exp2f(m_run - m_use);
        const float p = __builtin_amdgcn_exp2f(sc - m_use);
        float ps = p;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) ps += __shfl_xor(ps, o);
        l_run = l_run * corr + ps;
        m_run = m_new;
        __syncthreads();
        s_p[lane] = p;
        __syncthreads();
        acc0 *= corr;
        acc1 *= corr;
        const int kmax = draft ? n : min(64, L - c * 64);
        for (int t = 0; t < kmax; ++t) {
            const float pt = s_p[t];
            if (pt == 0.0f) continue;
            if (draft) {
                const float *vp = static_cast<const float *>(a.vd) + (((size_t)b * m_max + t) * a.Hkv + kvh) * d;
                acc0 = __builtin_fmaf(pt, vp[lane], acc0);
                if (d > 64) acc1 = __builtin_fmaf(pt, vp[lane + 64], acc1);
            } else {
                acc0 = __builtin_fmaf(pt, *v_elem<float>(a, b, kvh, lane, c * 64 + t), acc0);
                if (d > 64) acc1 = __builtin_fmaf(pt, *v_elem<float>(a, b, kvh, lane + 64, c * 64 + t), acc1);
            }
        }
    }
    const float inv = l_run > 0.0f ? 1.0f / l_run : 0.0f;
    out[lane] = acc0 * inv;
    if (d > 64) out[lane + 64] = acc1 * inv;
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
AttnPlan attn_plan(const eagle_attn_params *a, int32_t batch)
{
    AttnPlan P;
    P.G = a->num_q_heads / a->num_kv_heads;
    P.rows = a->m_max * P.G;
    // capacity: every prefix_len is clamped to it, so it bounds every split count
    if (a->block_size > 0) {
        const long long pc = (long long)a->max_blocks * a->block_size;
        P.max_prefix = (a->max_prefix > 0 && a->max_prefix < pc) ? a->max_prefix : (int)pc;
    } else {
        P.max_prefix = a->max_prefix;
    }
    if (a->dtype == EAGLE_F32) {
        P.row_groups = 1; P.waves = 1; P.chunk = 0; P.nsplit = 1;
        P.off_part = P.off_ml = P.off_cnt = kWsHeader;
        P.total = kWsHeader;
        return P;
    }
    P.row_groups = (P.rows + 32 * kMaxWaves - 1) / (32 * kMaxWaves);
    const int rows_pg = (P.rows + P.row_groups - 1) / P.row_groups;
    P.waves = (rows_pg + 31) / 32;
    if (P.waves < 4) P.waves = 4;   // extra waves only help stage K/V
    const int units = batch * a->num_kv_heads * P.row_groups;
    const int Lb = P.max_prefix > 0 ? P.max_prefix : 1;
    const int target = units > 0 ? (512 + units - 1) / units : 1;
    int chunk = (Lb + target - 1) / target;
    chunk = (chunk + kTK - 1) / kTK * kTK;
    if (chunk < 256) chunk = 256;
    if (chunk > 4096) chunk = 4096;
    P.chunk = chunk;
    P.nsplit = (Lb + chunk - 1) / chunk;
    const size_t rows_alloc = (size_t)units * P.nsplit * (size_t)(32 * ((rows_pg + 31) / 32));
    size_t o = kWsHeader;
    P.off_part = o; o = align_up(o + (P.nsplit > 1 ? rows_alloc * kHD * sizeof(float) : 0), 256);
    P.off_ml = o;   o = align_up(o + (P.nsplit > 1 ? rows_alloc * sizeof(float2) : 0), 256);
    P.off_cnt = o;  o = align_up(o + (size_t)units * sizeof(uint32_t), 256);
    P.total = o;
    return P;
}

hipError_t launch_tree_attn(const eagle_attn_params *p, const AttnPlan &P, int32_t batch,
                            const void *q, const void *k_draft, const void *v_draft,
                            const void *k_cache, const void *v_cache, const int32_t *block_table,
                            const int32_t *prefix_len, const uint64_t *anc, const int32_t *num_nodes,
                            void *out, void *ws, hipStream_t st)
{
    if (batch <= 0) return hipSuccess;
    char *base = static_cast<char *>(ws);
    AttnArgs a;
    a.q = q; a.kd = k_draft; a.vd = v_draft; a.kc = k_cache; a.vc = v_cache;
    a.block_table = block_table; a.prefix_len = prefix_len; a.num_nodes = num_nodes; a.anc = anc;
    a.out = out;
    a.part_o = reinterpret_cast<float *>(base + P.off_part);
    a.part_ml = reinterpret_cast<float2 *>(base + P.off_ml);
    a.cnt = reinterpret_cast<uint32_t *>(base + P.off_cnt);
    a.err = reinterpret_cast<uint32_t *>(base);
    a.Hq = p->num_q_heads; a.Hkv = p->num_kv_heads; a.G = P.G; a.d = p->head_dim;
    a.m_max = p->m_max; a.block_size = p->block_size; a.max_blocks = p->max_blocks;
    a.cap = P.max_prefix;
    a.chunk = P.chunk; a.nsplit = P.nsplit; a.RG = P.row_groups;
    a.rows_pg = (P.rows + P.row_groups - 1) / P.row_groups;
    a.rows_pg = 32 * ((a.rows_pg + 31) / 32);
    a.units0 = batch * p->num_kv_heads;
    const float scale = p->scale > 0.0f ? p->scale : 1.0f / sqrtf((float)p->head_dim);
    a.scale_log2 = scale * 1.4426950408889634f;
    a.v_vec = (p->block_size > 0) || (p->max_prefix % 8 == 0);
    if (p->dtype == EAGLE_F32) {
        const dim3 g((unsigned)(batch * p->m_max * p->num_q_heads));
        hipLaunchKernelGGL(k_tree_attn_f32, g, dim3(64), 0, st, a);
    } else {
        const dim3 g((unsigned)(a.units0 * P.row_groups * P.nsplit));
        hipLaunchKernelGGL(k_tree_attn_bf16, g, dim3(64 * P.waves), 0, st, a);
    }
    return hipGetLastError();
}

}  // namespace eagle
