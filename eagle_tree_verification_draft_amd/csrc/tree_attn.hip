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
// partial (O, max, sum) and a second kernel merges them.
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
    uint32_t *err;
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

constexpr int kTileChunks = kTK * kHD * 2 / 16;   // 16-byte chunks per K (or V^T) tile: 1024
constexpr int kMaxPages = 4096 / 8 + 2;             // pages of one split (chunk <= 4096, page >= 8)

typedef unsigned int u32x4a __attribute__((ext_vector_type(4)));

// One LDS buffer: K tile [64 keys][128 dims] and V^T tile [128 dims][64 keys],
// bf16, rows unpadded.  Row r of K holds key swap23(r); its 16-byte chunk J
// (dims 8J..8J+7) sits at position J ^ (r & 15).  Row e of V^T holds keys
// chunk J (keys 8J..8J+7) at position J ^ ((e >> 1) & 7).  With these XOR
// swizzles the MFMA operand reads (32 rows, one chunk each) hit distinct banks
// in every group of 8 lanes, and every wave's direct global->LDS load writes
// 1 KB contiguously.
struct AttnBuf {
    u32x4a K[kTK * 16];
    u32x4a Vt[kHD * 8];
};

struct AttnSmem {
    union {
        AttnBuf buf[2];
    } u;
    int bt[kMaxPages];
};

__device__ __forceinline__ int kpos(int r, int J) { return r * 16 + (J ^ (r & 15)); }
__device__ __forceinline__ int vpos(int e, int J) { return e * 8 + (J ^ ((e >> 1) & 7)); }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4a v) { return __builtin_bit_cast(bf16x8, v); }

// 16 bytes per lane from global memory straight into LDS at dst + 16 * lane
// (dst must be the same for the whole wave)
__device__ __forceinline__ void load_lds16(const void *src, void *dst_wave)
{
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)src,
                                     (__attribute__((address_space(3))) void *)dst_wave, 16, 0, 0);
}

__global__ __launch_bounds__(512) void k_tree_attn_bf16(AttnArgs a)
{
    __shared__ AttnSmem sm;
    const int tid = threadIdx.x, NT = blockDim.x, lane = tid & 63, wv = tid >> 6, NW = NT >> 6;
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
    const bool paged = a.block_size != 0;
    const int bs = a.block_size;
    const int page0 = paged ? key_lo / bs : 0;

    // pages of this split -> LDS
    if (paged && key_hi > key_lo) {
        const int np = (key_hi - 1) / bs - page0 + 1;
        for (int i = tid; i < np; i += NT) sm.bt[i] = a.block_table[(size_t)b * a.max_blocks + page0 + i];
    }

    const int row0 = rg * a.rows_pg + wv * 32;          // first row of this wave
    const int rows_valid = n * G;                        // rows with a real node
    const bool wave_active = row0 < rows_valid && wv * 32 < a.rows_pg;
    const bool wave_full = row0 + 32 <= rows_valid;
    const int my_row = row0 + ln;
    const int my_node = my_row / G;
    const bool row_ok = my_row < rows_valid;

    // Q fragments (B operand of S^T = K Q^T): lane holds q[my_row][16ks + 8hh .. +7]
    bf16x8 qf[8];
    {
        const u32x4a *qrow = reinterpret_cast<const u32x4a *>(
            static_cast<const uint16_t *>(a.q) +
            (((size_t)b * m_max + (my_node < m_max ? my_node : 0)) * a.Hq + kvh * G + (my_row % G)) * kHD);
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            u32x4a v = {0, 0, 0, 0};
            if (wave_active && my_node < m_max) v = qrow[2 * ks + hh];
            qf[ks] = as_bf16x8(v);
        }
    }
    uint64_t my_anc = 0;
    if (row_ok) my_anc = a.anc[(size_t)b * m_max + my_node];
    __syncthreads();   // sm.bt visible

    const uint16_t *kc = static_cast<const uint16_t *>(a.kc);
    const uint16_t *vc = static_cast<const uint16_t *>(a.vc);
    const size_t kvbase = (size_t)b * a.Hkv + kvh;      // contiguous cache: (b, kvh) slab
    const uint16_t *kslab = paged ? kc : kc + kvbase * (size_t)a.cap * kHD;
    const uint16_t *vslab = paged ? vc : vc + kvbase * (size_t)kHD * a.cap;

    const int nprefix = (key_hi - key_lo + kTK - 1) / kTK;
    const int ntiles = nprefix + (has_draft ? 1 : 0);
    // a tile goes global->LDS directly when all 64 keys are valid (and, for a
    // contiguous cache, V^T rows are 16-byte aligned); otherwise it is staged
    // through registers with explicit zeros
    auto direct = [&](int tile) {
        return tile < nprefix && key_lo + (tile + 1) * kTK <= key_hi && (paged || a.v_vec);
    };
    auto k_src = [&](int key, int J) -> const uint16_t * {
        if (!paged) return kslab + (size_t)key * kHD + J * 8;
        const int blk = sm.bt[key / bs - page0];
        return kc + (((size_t)blk * a.Hkv + kvh) * bs + key % bs) * kHD + J * 8;
    };
    auto v_src = [&](int e, int key) -> const uint16_t * {
        if (!paged) return vslab + (size_t)e * a.cap + key;
        const int blk = sm.bt[key / bs - page0];
        return vc + (((size_t)blk * a.Hkv + kvh) * kHD + e) * bs + key % bs;
    };
    // direct loads of a full tile into buffer `bi`: slot = 64 * it + lane
    auto issue_direct = [&](int tile, int bi) {
        const int k0 = key_lo + tile * kTK;
        AttnBuf &B = sm.u.buf[bi];
        for (int it = wv; it < kTileChunks / 64; it += NW) {
            const int slot = it * 64 + lane;
            const int r = slot >> 4, P = slot & 15;
            load_lds16(k_src(k0 + swap23(r), P ^ (r & 15)), &B.K[it * 64]);
            const int e = slot >> 3, Q = slot & 7;
            load_lds16(v_src(e, k0 + 8 * (Q ^ ((e >> 1) & 7))), &B.Vt[it * 64]);
        }
    };
    // register-staged load and store of a tail or draft tile into buffer `bi`
    auto stage_regs = [&](int tile, int bi) {
        AttnBuf &B = sm.u.buf[bi];
        const bool draft = has_draft && tile == ntiles - 1;
        const int k0 = key_lo + tile * kTK;
        uint16_t *vt16 = reinterpret_cast<uint16_t *>(B.Vt);
        for (int c = tid; c < kTileChunks; c += NT) {
            const int t = c >> 4, J = c & 15;
            u32x4a kv = {0, 0, 0, 0};
            if (draft) {
                u32x4a vv = {0, 0, 0, 0};
                if (t < n) {
                    const size_t o = (((size_t)b * m_max + t) * a.Hkv + kvh) * kHD + J * 8;
                    kv = *reinterpret_cast<const u32x4a *>(static_cast<const uint16_t *>(a.kd) + o);
                    vv = *reinterpret_cast<const u32x4a *>(static_cast<const uint16_t *>(a.vd) + o);
                }
                // draft V arrives key-major: transpose into V^T (dims 8J..8J+7 of key t)
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    const int e = 8 * J + q;
                    const uint16_t h = (uint16_t)((vv[q >> 1] >> (16 * (q & 1))) & 0xffffu);
                    vt16[vpos(e, t >> 3) * 8 + (t & 7)] = h;
                }
            } else {
                if (k0 + t < key_hi) kv = *reinterpret_cast<const u32x4a *>(k_src(k0 + t, J));
                const int e = c >> 3, Jv = c & 7, key = k0 + 8 * Jv;
                u32x4a vv = {0, 0, 0, 0};
                if (key < key_hi) {
                    const uint16_t *vp = v_src(e, key);
                    uint32_t w[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const uint32_t lo = (key + 2 * q < key_hi) ? vp[2 * q] : 0u;
                        const uint32_t hi = (key + 2 * q + 1 < key_hi) ? vp[2 * q + 1] : 0u;
                        w[q] = lo | (hi << 16);
                    }
                    vv = u32x4a{w[0], w[1], w[2], w[3]};
                }
                B.Vt[vpos(e, Jv)] = vv;
            }
            const int r = swap23(t);
            B.K[kpos(r, J)] = kv;
        }
    };

    f32x16 oacc[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.0f;
    // running max in raw score units and running sum; scores enter exp2 as
    // fma(s, c, -m c) with c = scale * log2(e) > 0
    const float c2 = a.scale_log2;
    float m_run = -__builtin_inff(), l_run = 0.0f;

    if (ntiles > 0 && direct(0)) issue_direct(0, 0);
    for (int tile = 0; tile < ntiles; ++tile) {
        const int bi = tile & 1;
        const bool draft = has_draft && tile == ntiles - 1;
        const int k0 = key_lo + tile * kTK;
        if (!direct(tile)) stage_regs(tile, bi);
        __builtin_amdgcn_s_waitcnt(0);        // this wave's loads into buffer bi have landed
        __syncthreads();                      // ... and everyone's; tile - 1 is fully consumed
        if (tile + 1 < ntiles && direct(tile + 1)) issue_direct(tile + 1, bi ^ 1);
        const AttnBuf &B = sm.u.buf[bi];

        if (wave_active) {
            // ---- S^T = K Q^T: two independent 32-key accumulators ----
            f32x16 s0, s1;
#pragma unroll
            for (int r = 0; r < 16; ++r) { s0[r] = 0.0f; s1[r] = 0.0f; }
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                const bf16x8 a0 = as_bf16x8(B.K[kpos(ln, 2 * ks + hh)]);
                const bf16x8 a1 = as_bf16x8(B.K[kpos(32 + ln, 2 * ks + hh)]);
                s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[ks], s0, 0, 0, 0);
                s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf[ks], s1, 0, 0, 0);
            }
            // s0/s1[8t + q] is the raw score of tile key 32sh + 16t + 8hh + q for row my_row
            const bool fast = !draft && k0 + kTK <= key_hi && wave_full;
            if (!fast) {
                if (draft) {
                    const uint32_t m0 = (uint32_t)my_anc >> (8 * hh), m1 = (uint32_t)(my_anc >> 32) >> (8 * hh);
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int bit = 16 * (r >> 3) + (r & 7);
                        s0[r] = (row_ok && ((m0 >> bit) & 1u)) ? s0[r] : -__builtin_inff();
                        s1[r] = (row_ok && ((m1 >> bit) & 1u)) ? s1[r] : -__builtin_inff();
                    }
                } else {
                    const int lim = key_hi - k0 - 8 * hh;    // tile keys below lim + 8hh are valid
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int kq = 16 * (r >> 3) + (r & 7);
                        s0[r] = (row_ok && kq < lim) ? s0[r] : -__builtin_inff();
                        s1[r] = (row_ok && 32 + kq < lim) ? s1[r] : -__builtin_inff();
                    }
                }
            }
            float tmax = -__builtin_inff();
#pragma unroll
            for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, fmaxf(s0[r], s1[r]));
            tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
            const float m_new = fmaxf(m_run, tmax);
            const float m_use = m_new == -__builtin_inff() ? 0.0f : m_new;
            const float mc = m_use * c2;
            const float corr = __builtin_amdgcn_exp2f(m_run * c2 - mc);
            float lsum = 0.0f;
            bf16x8 pf[2][2];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[r], c2, -mc));
                const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[r], c2, -mc));
                lsum += p0 + p1;
                pf[0][r >> 3][r & 7] = (__bf16)p0;
                pf[1][r >> 3][r & 7] = (__bf16)p1;
            }
            lsum += __shfl_xor(lsum, 32);
            l_run = l_run * corr + lsum;
            m_run = m_new;
            if (__any(corr != 1.0f)) {
#pragma unroll
                for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) oacc[dt][r] *= corr;
            }
            // ---- O^T += V^T P^T: four independent accumulators per k-step ----
#pragma unroll
            for (int sh = 0; sh < 2; ++sh) {
#pragma unroll
                for (int t = 0; t < 2; ++t) {
#pragma unroll
                    for (int dt = 0; dt < 4; ++dt) {
                        const bf16x8 av = as_bf16x8(B.Vt[vpos(32 * dt + ln, 4 * sh + 2 * t + hh)]);
                        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pf[sh][t], oacc[dt], 0, 0, 0);
                    }
                }
            }
        }
    }
    __syncthreads();

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
        // partial max in log2 units (raw max times c), as the merge expects
        if (hh == 0) a.part_ml[pbase + row_local] = make_float2(row_ok ? m_run * c2 : -__builtin_inff(), row_ok ? l_run : 0.0f);
    }
}

// ---------------------------------------------------------------------------
// Merge of the key splits (launched right after the main kernel on the same
// stream, so the kernel boundary makes every partial visible): for each row,
// O = sum_s w_s O_s with w_s = exp2(m_s - M) / sum_s exp2(m_s - M) l_s.
// One workgroup per (unit, 16 rows); thread = (row, 8 dims).
// ---------------------------------------------------------------------------
constexpr int kMergeRows = 16;

__global__ __launch_bounds__(256) void k_tree_attn_merge(AttnArgs a)
{
    const int tid = threadIdx.x;
    const int blocks_per_unit = (a.rows_pg + kMergeRows - 1) / kMergeRows;
    const int unit = blockIdx.x / blocks_per_unit;
    const int rl = (blockIdx.x % blocks_per_unit) * kMergeRows + (tid >> 4);
    const int d8 = (tid & 15) * 8;
    const int rg = unit % a.RG, u0 = unit / a.RG;
    const int b = u0 / a.Hkv, kvh = u0 % a.Hkv;
    const int G = a.G, m_max = a.m_max;
    int L = a.prefix_len[b];
    L = L < 0 ? 0 : (L > a.cap ? a.cap : L);
    const int nsplit_b = L > 0 ? (L + a.chunk - 1) / a.chunk : 1;
    if (nsplit_b == 1 || rl >= a.rows_pg) return;          // written by the main kernel
    const int row = rg * a.rows_pg + rl, node = row / G;
    if (node >= m_max) return;
    int n = a.num_nodes[b];
    n = n < 0 ? 0 : (n > m_max ? m_max : n);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (node < n) {
        const size_t base = (size_t)unit * a.nsplit * a.rows_pg + rl;
        float M = -__builtin_inff(), den = 0.0f;
        // batches of 4 splits: all loads of a batch are issued before use
        for (int s0 = 0; s0 < nsplit_b; s0 += 4) {
            float2 ml[4];
            float4 o0[4], o1[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const size_t pr = base + (size_t)min(s0 + q, nsplit_b - 1) * a.rows_pg;
                ml[q] = a.part_ml[pr];
                o0[q] = *reinterpret_cast<const float4 *>(a.part_o + pr * kHD + d8);
                o1[q] = *reinterpret_cast<const float4 *>(a.part_o + pr * kHD + d8 + 4);
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (s0 + q >= nsplit_b) break;
                // online merge in log2 units
                const float Mn = fmaxf(M, ml[q].x);
                const float Mu = Mn == -__builtin_inff() ? 0.0f : Mn;
                const float sc = __builtin_amdgcn_exp2f(M - Mu), w = __builtin_amdgcn_exp2f(ml[q].x - Mu);
                den = den * sc + w * ml[q].y;
                acc[0] = acc[0] * sc + w * o0[q].x; acc[1] = acc[1] * sc + w * o0[q].y;
                acc[2] = acc[2] * sc + w * o0[q].z; acc[3] = acc[3] * sc + w * o0[q].w;
                acc[4] = acc[4] * sc + w * o1[q].x; acc[5] = acc[5] * sc + w * o1[q].y;
                acc[6] = acc[6] * sc + w * o1[q].z; acc[7] = acc[7] * sc + w * o1[q].w;
                M = Mn;
            }
        }
        const float inv = den > 0.0f ? 1.0f / den : 0.0f;
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] *= inv;
    }
    uint4 w4;
    w4.x = f32_to_bf16(acc[0]) | ((uint32_t)f32_to_bf16(acc[1]) << 16);
    w4.y = f32_to_bf16(acc[2]) | ((uint32_t)f32_to_bf16(acc[3]) << 16);
    w4.z = f32_to_bf16(acc[4]) | ((uint32_t)f32_to_bf16(acc[5]) << 16);
    w4.w = f32_to_bf16(acc[6]) | ((uint32_t)f32_to_bf16(acc[7]) << 16);
    const int h = kvh * G + (row % G);
    *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(a.out) + (((size_t)b * m_max + node) * a.Hq + h) * kHD + d8) = w4;
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
    P.off_cnt = o;
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
        if (P.nsplit > 1) {
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
            const int bpu = (a.rows_pg + kMergeRows - 1) / kMergeRows;
            hipLaunchKernelGGL(k_tree_attn_merge, dim3((unsigned)(a.units0 * P.row_groups * bpu)), dim3(256), 0, st, a);
        }
    }
    return hipGetLastError();
}

}  // namespace eagle
