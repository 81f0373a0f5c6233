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
#include <algorithm>

#include "common.h"
#include "internal.h"

namespace eagle {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kTK = 64;            // keys per tile
constexpr int kHD = 128;           // head dim of the bf16 path
constexpr int kMaxWaves = 8;

struct AttnArgs {
    const void *q, *kd, *vd, *kc, *vc;
    const int32_t *block_table, *prefix_len, *num_nodes;
    const uint64_t *anc;
    void *out;
    float *part_o;
    float2 *part_ml;
    int2 *sched_tab;   // sched != 0: (sequence, split) of each block group, or (-1, -1)
    uint32_t *err;
    int Hq, Hkv, G, d, m_max, block_size, max_blocks, cap, chunk, nsplit, RG, rows_pg, units0, sched;
    float scale_log2;
};

// a key half as a type, so that code for one half is compiled with h fixed
template <int H> struct HalfC { static constexpr int value = H; };

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
constexpr int kMaxPages = 4096 / 8 + 2;             // pages of one split (at most 513 pages of keys, + 1 unaligned)

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

// LDS of one workgroup: a ring of kRing tile buffers (kRing - 1 tiles in flight
// ahead of the one in use).  A paged cache needs the split's page list and a
// staging area for the draft V rows, so its ring has 4 buffers; a contiguous
// cache stages the draft V rows in the draft buffer's own V^T area, and its
// ring of 5 buffers fills the 160 KB of LDS.
template <int kRing> struct AttnSmem;
template <> struct AttnSmem<4> {
    AttnBuf buf[4];
    u32x4a dv[kTK * 16];   // draft V rows as they arrive (key-major, swizzled like K)
    // element offset of each page of the split within the cache, kv head
    // included: page p's (kv head, key, dim) K element sits at pb[p] +
    // key * head_dim + dim, its V^T element at pb[p] + dim * page + key
    unsigned long long pb[kMaxPages];
};
template <> struct AttnSmem<5> {
    AttnBuf buf[5];
};
static_assert(sizeof(AttnSmem<5>) <= 160 * 1024, "LDS");

__device__ __forceinline__ unsigned long long *page_list(AttnSmem<4> &sm) { return sm.pb; }
__device__ __forceinline__ unsigned long long *page_list(AttnSmem<5> &) { return nullptr; }   // contiguous only
// where the draft V rows land (key-major) before the transpose into V^T
__device__ __forceinline__ u32x4a *draft_rows(AttnSmem<4> &sm, AttnBuf &) { return sm.dv; }
__device__ __forceinline__ u32x4a *draft_rows(AttnSmem<5> &, AttnBuf &B) { return B.Vt; }


__device__ __forceinline__ int kpos(int r, int J) { return r * 16 + (J ^ (r & 15)); }
__device__ __forceinline__ int vpos(int e, int J) { return e * 8 + (J ^ ((e >> 1) & 7)); }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4a v) { return __builtin_bit_cast(bf16x8, v); }

// a value the optimiser must treat as new at this point (keeps expressions
// built from it from being hoisted out of loops and held in registers)
__device__ __forceinline__ int opaque_i(int v)
{
    asm volatile("" : "+v"(v));
    return v;
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// acc + the sum of the eight bf16 values of v (dot products with ones: the
// sum of exactly the weights the PV product multiplies).  The pairs are taken
// with vector shuffles: a bit cast of one 32-bit element of the vector to
// bf16x2 was compiled as element 0 every time.
__device__ __forceinline__ float add_bf16x8(bf16x8 v, float acc)
{
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 0, 1), one, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 2, 3), one, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 4, 5), one, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 6, 7), one, acc, false);
    return acc;
}

// v combined with the value of lane ^ 32 through one lane-half swap (a VALU
// instruction, no LDS round trip); the result is the same in both lanes
__device__ __forceinline__ float max_xor32(float v)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float v)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// 16 bytes per lane from global memory straight into LDS at dst + 16 * lane
// (dst must be the same for the whole wave).  The loads carry the non-temporal
// cache policy (bit 1 of the policy operand): K/V lines are streamed once, and
// streaming reads marked so run measurably closer to the HBM peak.
constexpr int kCachePolicyNT = 2;

__device__ __forceinline__ void load_lds16(const void *src, void *dst_wave)
{
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)src,
                                     (__attribute__((address_space(3))) void *)dst_wave, 16, 0, kCachePolicyNT);
}

// s_waitcnt with vmcnt = n and the other counters left free (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
template <int n>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(n >= 0 && n < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

// waits until this wave's loads of the current item have landed, the loads of
// `later` later items (at most kMaxLater) still outstanding
template <int kLw, int kMaxLater>
__device__ __forceinline__ void wait_item(int later)
{
    if (kMaxLater >= 3 && later >= 3) wait_vmcnt<(kMaxLater >= 3 ? 3 : 0) * kLw>();
    else if (kMaxLater >= 2 && later >= 2) wait_vmcnt<(kMaxLater >= 2 ? 2 : 0) * kLw>();
    else if (later >= 1) wait_vmcnt<kLw>();
    else wait_vmcnt<0>();
}

// Work items of one workgroup, in processing order: the prefix tiles of the
// split, then the draft tile (last key split only, when the sequence has
// nodes).  With a contiguous cache the first prefix tiles are requested
// before prefix_len is read (every key below the capacity is addressable);
// requests that turn out to lie past it are drained, never used.  Every item
// reaches LDS by direct global->LDS loads, kAhead items
// ahead of the one being computed, so every wave issues the same number of
// loads per item and a partial wait (vmcnt) separates the items in flight:
//   - prefix tile: K rows and V^T chunks; keys at or past prefix_len read the
//     last valid key (finite data; the scores of those keys are masked), and
//     V^T entries of those keys are zeroed in LDS before use, since the chunk
//     that straddles prefix_len may carry anything past it;
//   - draft tile: K rows of the draft tokens, and their V rows key-major into a
//     staging area (the 4-buffer ring's own, or the draft buffer's V^T area),
//     transposed to V^T in LDS (zeros for keys >= num_nodes) before use.
//
// kKS = 2 (few query rows): the waves form kNW / 2 row waves x 2 key halves;
// a wave computes its 32 rows against one 32-key half of every tile with its
// own online-softmax state, and the two halves' states are combined through
// LDS at the end, so every SIMD works on every tile.
// which waves issue the tile loads (see the kernel)
constexpr int kLoadAll = 0, kLoadProducers = 1;

template <int kNW, int kKS, int kLoad, int kRing>
__device__ __forceinline__ void tree_attn_body(const AttnArgs &a, AttnSmem<kRing> &sm)
{
    constexpr int kAhead = kRing - 1;                   // tiles in flight ahead of the one in use
    constexpr bool kProd = kLoad == kLoadProducers;
    constexpr int kPer = kTileChunks / 64 / kNW;        // 16-byte slots per loading wave per operand per tile
    constexpr int kLw = 2 * kPer;                       // loads per loading wave per item
    constexpr int kRW = kNW / kKS;                 // row waves
    unsigned long long *const pb = page_list(sm);
    const int tid = threadIdx.x, NT = kNW * 64, lane = tid & 63, wv = tid >> 6;
    constexpr int kThreads = kNW * 64 * (kProd ? 2 : 1);
    // kLoadProducers: waves kNW.. only issue the tile loads (producers), so
    // their issue stalls never hold up the compute waves that share their
    // SIMDs (kLoadAll: every wave issues its share and computes)
    const bool producer = kProd && wv >= kNW;
    const bool loader = !kProd || producer;
    const int lw = kProd ? wv - kNW : wv;               // loader wave index
    const int ln = lane & 31, hh = lane >> 5;
    int rw = wv % kRW;                                  // row wave (32 query rows)
    const int kh = wv / kRW;                            // key half (kKS = 2)
    // 8-wave form with 5 to 7 row blocks: the waves past the first
    // nb - (8 - nb) take the last 8 - nb blocks by key halves, so that every
    // SIMD computes the same share of a tile (6 blocks: four SIMDs with one
    // whole block and one half each, instead of two with two whole blocks).
    // hsplit: 0 = both key halves, 1 = keys 0..31 only, 2 = keys 32..63 only.
    int hsplit = 0, nsplit_rb = 0, nfull_rb = 0;
    if (kNW == 8 && kKS == 1) {
        const int nb = a.rows_pg / 32;
        if (nb >= 5 && nb <= 7) {
            nsplit_rb = 8 - nb;
            nfull_rb = nb - nsplit_rb;
            if (wv >= nfull_rb) {
                const int j = wv - nfull_rb;
                rw = nfull_rb + (j >> 1);
                hsplit = 1 + (j & 1);
            }
        }
    }
    // block -> (split, row group, sequence/kv head).  In split-major order
    // all splits and row groups of one (sequence, kv head) share blockIdx
    // mod 8 when units0 % 8 == 0, which keeps them on one XCD and its L2.
    // With a schedule table, consecutive groups of Hkv * RG blocks take one
    // (sequence, split) each, in the table's order, kv head fastest: when
    // Hkv % 8 == 0 a (sequence, kv head) keeps blockIdx mod 8 = kv head mod 8
    // from split to split, which is also the XCD of its merge blocks.  A
    // group without an entry has nothing to do.
    const int x = blockIdx.x;
    int u0, rg, s;
    if (a.sched) {
        const int g = a.Hkv * a.RG, qg = x / g, wi = x - qg * g;
        const int2 e = a.sched_tab[qg];
        if (e.x < 0) return;                            // nothing requested yet
        u0 = e.x * a.Hkv + wi % a.Hkv;
        rg = wi / a.Hkv;
        s = e.y;
    } else {
        u0 = x % a.units0;
        const int rest = x / a.units0;
        rg = rest % a.RG;
        s = rest / a.RG;
    }
    const int b = u0 / a.Hkv, kvh = u0 % a.Hkv;
    const int G = a.G, m_max = a.m_max;

    const bool paged = kRing == 4 && a.block_size != 0;   // the 5-buffer ring serves contiguous caches
    const int bs = a.block_size;
    const int key_lo = s * a.chunk;
    const int row0 = rg * a.rows_pg + rw * 32;          // first row of this wave
    const int my_row = row0 + ln;
    const int my_node = my_row / G;
    const bool row_exists = rw * 32 + ln < a.rows_pg && my_node < m_max;

    const uint16_t *kc = static_cast<const uint16_t *>(a.kc);
    const uint16_t *vc = static_cast<const uint16_t *>(a.vc);
    const uint16_t *kd = static_cast<const uint16_t *>(a.kd);
    const uint16_t *vd = static_cast<const uint16_t *>(a.vd);
    const size_t kvbase = (size_t)b * a.Hkv + kvh;      // contiguous cache: (b, kvh) slab
    const uint16_t *kslab = paged ? kc : kc + kvbase * (size_t)a.cap * kHD;
    const uint16_t *vslab = paged ? vc : vc + kvbase * (size_t)kHD * a.cap;

    // Items of the split: its prefix tiles, then (last split, nodes present)
    // the draft tile.  Until the prefix length is known, key_hi and nprefix
    // describe the keys below the cache capacity, which are all addressable
    // in a contiguous cache: its first tiles are requested before the length
    // arrives (a paged cache needs the block table first).
    int key_hi = paged ? key_lo : min(a.cap, key_lo + a.chunk);
    int nprefix = key_hi > key_lo ? (key_hi - key_lo + kTK - 1) / kTK : 0;
    int n = 0, page0 = 0;

    auto k_src = [&](int key, int J) -> const uint16_t * {
        if (!paged) return kslab + (size_t)key * kHD + J * 8;
        return kc + pb[key / bs - page0] + (key % bs) * kHD + J * 8;
    };
    auto v_src = [&](int e, int key) -> const uint16_t * {
        if (!paged) return vslab + (size_t)e * a.cap + key;
        return vc + pb[key / bs - page0] + e * bs + key % bs;
    };
    const size_t drow = (size_t)b * m_max;               // draft rows of this sequence
    // pages of 8, 16, 32 or 64 keys tile a 64-key tile exactly (power-of-two
    // page index arithmetic); other page sizes take the general path
    const bool fast_pages = !paged || (kTK % bs == 0);
    const int bshift = paged ? __builtin_ctz(bs) : 0;
    const size_t pstride = (size_t)a.Hkv * bs * kHD;     // elements per page (K and V^T alike)
    const size_t kvh_off = (size_t)kvh * bs * kHD;
    // Per-lane parts of a full tile's addresses, the same for every tile (in
    // elements): the K row chunk and the V^T chunk of each load slot, within
    // the tile (contiguous cache) or within their page, with the page's slot
    // in the tile (paged cache; one K load covers 4 keys of one page).
    // (paged: the page slot sits in bits 16.. above the offset, which is
    // below 2^13 for pages of at most 64 keys: one register per operand)
    int kofs[kPer], vofs[kPer];
#pragma unroll
    for (int q = 0; q < kPer; ++q) {
        const int it = lw * kPer + q, slot = it * 64 + lane;
        const int r = slot >> 4, P = slot & 15, e = slot >> 3, Q = slot & 7;
        const int ko = swap23(r), kj = (P ^ (r & 15)) << 3, vj = (Q ^ ((e >> 1) & 7)) << 3;
        if (!paged) {
            kofs[q] = ko * kHD + kj;
            vofs[q] = e * a.cap + vj;           // below 2^31: capacity <= 2^24
        } else {
            kofs[q] = ((ko & (bs - 1)) * kHD + kj) | ((ko >> bshift) << 16);
            vofs[q] = (e * bs + (vj & (bs - 1))) | ((vj >> bshift) << 16);
        }
    }
    auto issue = [&](int item) {
        AttnBuf &B = sm.buf[item % kRing];
        if (item >= nprefix) {
#pragma unroll
            for (int q = 0; q < kPer; ++q) {
                const int it = lw * kPer + q, slot = it * 64 + lane;
                const int r = slot >> 4, P = slot & 15;
                const int t = swap23(r);
                load_lds16(kd + ((drow + (t < n ? t : 0)) * a.Hkv + kvh) * kHD + (P ^ (r & 15)) * 8, &B.K[it * 64]);
                load_lds16(vd + ((drow + (r < n ? r : 0)) * a.Hkv + kvh) * kHD + (P ^ (r & 15)) * 8, &draft_rows(sm, B)[it * 64]);
            }
        } else if (key_lo + (item + 1) * kTK <= key_hi && fast_pages) {
            // full tile: lane offsets from shifts and masks only
            const int k0 = key_lo + item * kTK;
            if (!paged) {
                const uint16_t *kt = kslab + (size_t)k0 * kHD, *vt = vslab + k0;
#pragma unroll
                for (int q = 0; q < kPer; ++q) {
                    const int it = lw * kPer + q;
                    load_lds16(kt + kofs[q], &B.K[it * 64]);
                    load_lds16(vt + vofs[q], &B.Vt[it * 64]);
                }
            } else {
                const unsigned long long *pt = pb + ((k0 >> bshift) - page0);
                unsigned long long pk[kPer], pv[kPer];
#pragma unroll
                for (int q = 0; q < kPer; ++q) {
                    pk[q] = pt[kofs[q] >> 16];
                    pv[q] = pt[vofs[q] >> 16];
                }
#pragma unroll
                for (int q = 0; q < kPer; ++q) {
                    const int it = lw * kPer + q;
                    // (offsets re-read each tile: hoisted 64-bit bases cost registers)
                    load_lds16(kc + pk[q] + (opaque_i(kofs[q]) & 0xffff), &B.K[it * 64]);
                    load_lds16(vc + pv[q] + (opaque_i(vofs[q]) & 0xffff), &B.Vt[it * 64]);
                }
            }
        } else {
            const int k0 = key_lo + item * kTK, klast = key_hi - 1;
            const int vlast = k0 + ((klast - k0) & ~7);   // first key of the chunk holding klast
#pragma unroll
            for (int q = 0; q < kPer; ++q) {
                const int it = lw * kPer + q, slot = it * 64 + lane;
                const int r = slot >> 4, P = slot & 15;
                const int key = min(k0 + swap23(r), klast);
                load_lds16(k_src(key, P ^ (r & 15)), &B.K[it * 64]);
                const int e = slot >> 3, Q = slot & 7;
                const int vk = min(k0 + 8 * (Q ^ ((e >> 1) & 7)), vlast);
                load_lds16(v_src(e, vk), &B.Vt[it * 64]);
            }
        }
    };

    const int nspec = paged ? 0 : min(kAhead, nprefix);
    if (loader)
        for (int i = 0; i < nspec; ++i) issue(i);
    // Q fragments (B operand of S^T = K Q^T): lane holds q[my_row][16ks + 8hh .. +7]
    // (rows below m_max are addressable whatever num_nodes says; rows without
    // a node are zeroed below), the ancestor bits, and the sequence's lengths
    bf16x8 qf[8];
    {
        const u32x4a *qrow = reinterpret_cast<const u32x4a *>(
            static_cast<const uint16_t *>(a.q) +
            (((size_t)b * m_max + (my_node < m_max ? my_node : 0)) * a.Hq + kvh * G + (my_row % G)) * kHD);
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            u32x4a v = {0, 0, 0, 0};
            if (row_exists && !producer) v = qrow[2 * ks + hh];
            qf[ks] = as_bf16x8(v);
        }
    }
    uint64_t my_anc = (row_exists && !producer) ? a.anc[(size_t)b * m_max + my_node] : 0;
    int L = a.prefix_len[b];
    n = a.num_nodes[b];
    if (L < 0 || L > a.cap) {
        if (tid == 0 && s == 0 && rg == 0) raise_error(a.err, EAGLE_DEVERR_PREFIX);
        L = L < 0 ? 0 : a.cap;
    }
    n = n < 0 ? 0 : (n > m_max ? m_max : n);
    const int nsplit_b = L > 0 ? (L + a.chunk - 1) / a.chunk : 1;
    if (s >= nsplit_b) {
        wait_vmcnt<0>();   // no LDS write may land after the workgroup has left
        return;
    }
    key_hi = min(L, key_lo + a.chunk);
    nprefix = key_hi > key_lo ? (key_hi - key_lo + kTK - 1) / kTK : 0;
    const bool last_split = (s == nsplit_b - 1);
    const int ndraft = (last_split && n > 0) ? 1 : 0;
    const int nitems = nprefix + ndraft;
    // requested tiles past the prefix are not items: drain them before their
    // buffers are reused
    if (nspec > nprefix) wait_vmcnt<0>();

    if (paged) {
        // pages of this split -> LDS
        page0 = key_lo / bs;
        if (key_hi > key_lo) {
            const int np = (key_hi - 1) / bs - page0 + 1;
            for (int i = tid; i < np; i += kThreads)
                pb[i] = (unsigned long long)a.block_table[(size_t)b * a.max_blocks + page0 + i] * pstride + kvh_off;
        }
        __syncthreads();   // page list visible
    }

    const int rows_valid = n * G;                        // rows with a real node
    const bool wave_active = !producer && row0 < rows_valid && rw * 32 < a.rows_pg;
    const bool row_ok = !producer && my_row < rows_valid && rw * 32 + ln < a.rows_pg;
    if (!row_ok) {
        my_anc = 0;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) qf[ks] = as_bf16x8(u32x4a{0, 0, 0, 0});
    }

    f32x16 oacc[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.0f;
    // exponent reference in raw score units (finite: 0 until a tile moves it)
    // and running sum; scores enter exp2 as fma(s, c, -m c) with
    // c = scale * log2(e) > 0
    const float c2 = a.scale_log2;
    float m_run = 0.0f, l_run = 0.0f;

    // the remaining first items (from the first one not requested as a
    // prefix tile: a sequence shorter than the capacity has its draft tile
    // among the speculative requests, which were drained above); one full
    // wait then covers them, the Q fragments and the ancestor bits (the
    // compiler cannot count loads across the data-dependent issue loops, so a
    // later wait for the Q registers would be a full wait inside the pipeline)
    if (loader)
        for (int i = min(nspec, nprefix); i < kAhead && i < nitems; ++i) issue(i);
    // (producers wait for their first tiles here too: letting them run ahead
    // of the first barrier measured slower)
    wait_vmcnt<0>();
    if (producer) {
        // the same barriers as the compute waves: one per item, one more for
        // items the compute waves fix up in LDS (draft tile, tail tile), and
        // the two of the key-half combine
        for (int item = 0; item < nitems; ++item) {
            wait_item<kLw, kAhead - 1>(min(kAhead - 1, nitems - 1 - item));
            __syncthreads();
            const int k0 = key_lo + item * kTK;
            if (item >= nprefix || k0 + kTK > key_hi) __syncthreads();
            if (item + kAhead < nitems) issue(item + kAhead);
        }
        wait_vmcnt<0>();
        if constexpr (kKS == 2) {
            __syncthreads();
            __syncthreads();
        }
        return;
    }
    // The tile loop, compiled once per kind of wave: hs = 0 for waves that
    // compute both key halves, 1 or 2 for the waves of a split row block
    // (separate loops keep the one-half code from crowding the registers of
    // the pipelined loop).  Every copy meets the same barriers.
    auto tile_loop = [&](auto hsc) {
        constexpr int hs = decltype(hsc)::value;
        for (int item = 0; item < nitems; ++item) {
            // this wave's loads of `item` have landed once at most the loads of
            // the (up to kAhead - 1) later items issued so far are outstanding
            wait_item<kLw, kAhead - 1>(min(kAhead - 1, nitems - 1 - item));
            __syncthreads();                      // ... and every wave's; item - 1 is fully consumed
            AttnBuf &B = sm.buf[item % kRing];
            const bool draft = item >= nprefix;
            // V^T of this item: with the 5-buffer ring the draft's V rows are staged
            // in its own buffer's V^T area and transposed into the previous item's
            // buffer (fully consumed, and the draft is the last item, so nothing is
            // requested into it again)
            u32x4a *const Vt = (kRing == 5 && draft) ? sm.buf[(item + kRing - 1) % kRing].Vt : B.Vt;
            const int k0 = key_lo + item * kTK;
            if (draft) {
                // draft V rows (key-major) -> V^T, zeros for keys >= n; thread =
                // (8 dims, 8 keys): an 8x8 block of bf16 transposed in registers
                const u32x4a *dv = draft_rows(sm, B);
                if (tid < 128) {
                    const int e8 = tid & 15, kg = tid >> 4;
                    u32x4a rows[8];
    #pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        const int t = 8 * kg + u;
                        rows[u] = t < n ? dv[t * 16 + (e8 ^ (t & 15))] : u32x4a{0, 0, 0, 0};
                    }
    #pragma unroll
                    for (int q = 0; q < 8; ++q) {
                        const int sh = 16 * (q & 1), w = q >> 1;
                        u32x4a o;
    #pragma unroll
                        for (int p = 0; p < 4; ++p) {
                            const uint32_t lo = (rows[2 * p][w] >> sh) & 0xffffu;
                            const uint32_t hi = (rows[2 * p + 1][w] >> sh) & 0xffffu;
                            o[p] = lo | (hi << 16);
                        }
                        Vt[vpos(8 * e8 + q, kg)] = o;
                    }
                }
                __syncthreads();
            } else if (k0 + kTK > key_hi) {
                // tail tile: zero V^T entries of keys >= key_hi in every chunk from
                // the one holding key_hi on (those chunks were loaded from it)
                const int lim = key_hi - k0, J0 = lim >> 3, nJ = 8 - J0;
                for (int c = tid; c < kHD * nJ; c += NT) {
                    const int e = c / nJ, J = J0 + c % nJ;
                    u32x4a v = B.Vt[vpos(e, J)];
    #pragma unroll
                    for (int p = 0; p < 4; ++p) {
                        const int key = 8 * J + 2 * p;
                        const uint32_t keep = (key < lim ? 0xffffu : 0u) | (key + 1 < lim ? 0xffff0000u : 0u);
                        v[p] &= keep;
                    }
                    B.Vt[vpos(e, J)] = v;
                }
                __syncthreads();
            }
            if (!kProd && item + kAhead < nitems) issue(item + kAhead);

            if (kNW == 8 && wave_active) {
                // Two compute waves per SIMD: the tile goes by key halves h = 0, 1
                // (keys 32h..32h+31), software-pipelined so that the products of
                // one half are interleaved with the softmax of the other:
                //   QK(0); QK(1) with weights(0); PV(0) with weights(1); PV(1).
                // A half's weights are formed against the reference in force
                // when they are formed (the lazy rule below, per half); a
                // reference moved by half 1 applies to O as it stands after
                // PV(0), whose weights were formed against the old one.  A wave
                // of a split row block (hsplit) computes its one half only.
                f32x16 sh[2];
    #pragma unroll
                for (int h = 0; h < 2; ++h)
    #pragma unroll
                    for (int r = 0; r < 16; ++r) sh[h][r] = 0.0f;
                u32x4a kb[8];
                // sh[h][8t + q] is the raw score of tile key 32h + 16t + 8hh + q for
                // row my_row; masking as in the other forms
                auto mask_half = [&](int h) {
                    if (draft) {
                        const uint32_t mk = (uint32_t)(my_anc >> (32 * h)) >> (8 * hh);
    #pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int bit = 16 * (r >> 3) + (r & 7);
                            sh[h][r] = ((mk >> bit) & 1u) ? sh[h][r] : -__builtin_inff();
                        }
                    } else if (k0 + kTK > key_hi) {
                        const int lim = key_hi - k0 - 8 * hh;
    #pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int kq = 32 * h + 16 * (r >> 3) + (r & 7);
                            sh[h][r] = kq < lim ? sh[h][r] : -__builtin_inff();
                        }
                    }
                };
                bf16x8 ph[2][2];
                // half h's weights against the current reference; returns their row sum
                auto weigh_half = [&](int h) -> float {
                    const float mc = m_run * c2;
    #pragma unroll
                    for (int r = 0; r < 16; ++r)
                        ph[h][r >> 3][r & 7] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(sh[h][r], c2, -mc));
                    return sum_xor32(add_bf16x8(ph[h][0], 0.0f) + add_bf16x8(ph[h][1], 0.0f));
                };
                // the lazy rule of the other forms, for one half
                auto settle_half = [&](int h, float lsum) {
                    if (__any(!(lsum <= 256.0f) || l_run + lsum == 0.0f)) {
                        float tmax = -__builtin_inff();
    #pragma unroll
                        for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, sh[h][r]);
                        tmax = max_xor32(tmax);
                        const bool empty = l_run == 0.0f;
                        const float m_new = empty ? (tmax == -__builtin_inff() ? m_run : tmax) : fmaxf(m_run, tmax);
                        const float corr = empty ? 1.0f : __builtin_amdgcn_exp2f((m_run - m_new) * c2);
                        l_run *= corr;
    #pragma unroll
                        for (int dt = 0; dt < 4; ++dt)
    #pragma unroll
                            for (int r = 0; r < 16; ++r) oacc[dt][r] *= corr;
                        m_run = m_new;
                        lsum = weigh_half(h);
                    }
                    l_run += lsum;
                };
                // one key half of the tile, QK, weights, PV (split row blocks)
                auto one_half = [&](auto hc) {
                    constexpr int h = decltype(hc)::value;
    #pragma unroll
                    for (int j = 0; j < 8; ++j) kb[j] = B.K[kpos(32 * h + ln, 2 * j + hh)];
                    __builtin_amdgcn_sched_barrier(0);
    #pragma unroll
                    for (int j = 0; j < 8; ++j) sh[h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kb[j]), qf[j], sh[h], 0, 0, 0);
                    __builtin_amdgcn_sched_barrier(0);
    #pragma unroll
                    for (int j = 0; j < 8; ++j) kb[j] = Vt[vpos(32 * (j & 3) + ln, 4 * h + 2 * (j >> 2) + hh)];
                    mask_half(h);
                    settle_half(h, weigh_half(h));
                    __builtin_amdgcn_sched_barrier(0);
    #pragma unroll
                    for (int j = 0; j < 8; ++j)
                        oacc[j & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kb[j]), ph[h][j >> 2], oacc[j & 3], 0, 0, 0);
                    __builtin_amdgcn_sched_barrier(0);
                };
                if constexpr (hs == 1) {
                    one_half(HalfC<0>{});
                } else if constexpr (hs == 2) {
                    one_half(HalfC<1>{});
                } else {
    #pragma unroll
                for (int j = 0; j < 8; ++j) kb[j] = B.K[kpos(ln, 2 * j + hh)];
                __builtin_amdgcn_sched_barrier(0);
    #pragma unroll
                for (int j = 0; j < 8; ++j) sh[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kb[j]), qf[j], sh[0], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
    #pragma unroll
                for (int j = 0; j < 8; ++j) kb[j] = B.K[kpos(32 + ln, 2 * j + hh)];
                mask_half(0);
                // ---- QK(1) with weights(0) ----
    #pragma unroll
                for (int j = 0; j < 8; ++j) sh[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kb[j]), qf[j], sh[1], 0, 0, 0);
                float ls = weigh_half(0);
    #pragma unroll
                for (int i = 0; i < 8; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
                settle_half(0, ls);
                // V^T operands of half 0 (keys 0..31: chunks 2t + hh)
    #pragma unroll
                for (int j = 0; j < 8; ++j) kb[j] = Vt[vpos(32 * (j & 3) + ln, 2 * (j >> 2) + hh)];
                mask_half(1);
                __builtin_amdgcn_sched_barrier(0);
                // ---- PV(0) with weights(1) ----
    #pragma unroll
                for (int j = 0; j < 8; ++j)
                    oacc[j & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kb[j]), ph[0][j >> 2], oacc[j & 3], 0, 0, 0);
                ls = weigh_half(1);
    #pragma unroll
                for (int i = 0; i < 8; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
                settle_half(1, ls);
                // ---- PV(1) ----
    #pragma unroll
                for (int j = 0; j < 8; ++j) kb[j] = Vt[vpos(32 * (j & 3) + ln, 4 + 2 * (j >> 2) + hh)];
                __builtin_amdgcn_sched_barrier(0);
    #pragma unroll
                for (int j = 0; j < 8; ++j)
                    oacc[j & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kb[j]), ph[1][j >> 2], oacc[j & 3], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
                }
            } else if (wave_active) {
                // ---- S^T = K Q^T: two independent 32-key accumulators ----
                // the K operands are read from LDS ahead of the products (all of
                // them with 4 waves; in two halves with 8 waves, two per SIMD,
                // whose registers hold only half), so the products issue back to
                // back behind one LDS round trip per group
                constexpr int kGroup = kNW == 8 ? 4 : 8;
                // key halves this wave covers: sh = 0, 1 (kKS = 1) or sh = kh
                constexpr int kNH = 2 / kKS;
                const int sh0 = kKS == 2 ? kh : 0;
                f32x16 sacc[kNH];
    #pragma unroll
                for (int u = 0; u < kNH; ++u)
    #pragma unroll
                    for (int r = 0; r < 16; ++r) sacc[u][r] = 0.0f;
    #pragma unroll
                for (int g0 = 0; g0 < 8; g0 += kGroup) {
                    u32x4a ka[kNH][kGroup];
    #pragma unroll
                    for (int j = 0; j < kGroup; ++j)
    #pragma unroll
                        for (int u = 0; u < kNH; ++u) ka[u][j] = B.K[kpos(32 * (sh0 + u) + ln, 2 * (g0 + j) + hh)];
                    __builtin_amdgcn_sched_barrier(0);
    #pragma unroll
                    for (int j = 0; j < kGroup; ++j)
    #pragma unroll
                        for (int u = 0; u < kNH; ++u)
                            sacc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ka[u][j]), qf[g0 + j], sacc[u], 0, 0, 0);
                    __builtin_amdgcn_sched_barrier(0);
                }
                // the V^T operands of this tile, in flight during the softmax (with
                // 8 waves, two per SIMD, the registers hold them only after it)
                constexpr int kNV = 8 * kNH;                  // V^T operands per tile
                constexpr int kEarly = kNW == 8 ? 0 : kNV;
                u32x4a va[kNV];
    #pragma unroll
                for (int j = 0; j < kEarly; ++j) {
                    const int sh = sh0 + (j >> 3), t = (j >> 2) & 1, dt = j & 3;
                    va[j] = Vt[vpos(32 * dt + ln, 4 * sh + 2 * t + hh)];
                }
                __builtin_amdgcn_sched_barrier(0);
                // sacc[u][8t + q] is the raw score of tile key 32(sh0 + u) + 16t + 8hh + q
                // for row my_row.  Rows without a node have zero Q (finite scores, never
                // written out), so only keys need masking: past prefix_len in the
                // tail tile, and non-ancestors in the draft tile.
                if (draft) {
    #pragma unroll
                    for (int u = 0; u < kNH; ++u) {
                        const uint32_t mk = (uint32_t)(my_anc >> (32 * (sh0 + u))) >> (8 * hh);
    #pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int bit = 16 * (r >> 3) + (r & 7);
                            sacc[u][r] = ((mk >> bit) & 1u) ? sacc[u][r] : -__builtin_inff();
                        }
                    }
                } else if (k0 + kTK > key_hi) {
                    const int lim = key_hi - k0 - 8 * hh;    // tile keys below lim + 8hh are valid
    #pragma unroll
                    for (int u = 0; u < kNH; ++u)
    #pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int kq = 32 * (sh0 + u) + 16 * (r >> 3) + (r & 7);
                            sacc[u][r] = kq < lim ? sacc[u][r] : -__builtin_inff();
                        }
                }
                // Weights against the current reference, and their row sum (of
                // the bf16 weights themselves, as the PV product uses them)
                bf16x8 pf[kNH][2];
                auto weigh = [&]() -> float {
                    const float mc = m_run * c2;
    #pragma unroll
                    for (int u = 0; u < kNH; ++u)
    #pragma unroll
                        for (int r = 0; r < 16; ++r)
                            pf[u][r >> 3][r & 7] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(sacc[u][r], c2, -mc));
                    float s0 = 0.0f, s1 = 0.0f;
    #pragma unroll
                    for (int u = 0; u < kNH; ++u) {
                        s0 = add_bf16x8(pf[u][0], s0);
                        s1 = add_bf16x8(pf[u][1], s1);
                    }
                    return sum_xor32(s0 + s1);
                };
                float lsum = weigh();
                // Lazy rescaling: the reference m_run moves only when some weight
                // exceeds 2^8 (then so does the row sum), or while nothing has
                // been accumulated (reference 0 may lie far above every score,
                // where all weights underflow).  Otherwise every weight is at
                // most 2^8, which fp32 sums and bf16 products carry as well as
                // weights below 1, and O / l is unchanged.  When it moves, it goes
                // to the row max (only up once something is accumulated), O and l
                // are rescaled and the weights formed again; the row max is not
                // computed otherwise.
                if (__any(!(lsum <= 256.0f) || l_run + lsum == 0.0f)) {
                    float tmax = -__builtin_inff();
    #pragma unroll
                    for (int u = 0; u < kNH; ++u)
    #pragma unroll
                        for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, sacc[u][r]);
                    tmax = max_xor32(tmax);
                    const bool empty = l_run == 0.0f;
                    const float m_new = empty ? (tmax == -__builtin_inff() ? m_run : tmax) : fmaxf(m_run, tmax);
                    const float corr = empty ? 1.0f : __builtin_amdgcn_exp2f((m_run - m_new) * c2);
                    l_run *= corr;
    #pragma unroll
                    for (int dt = 0; dt < 4; ++dt)
    #pragma unroll
                        for (int r = 0; r < 16; ++r) oacc[dt][r] *= corr;
                    m_run = m_new;
                    lsum = weigh();
                }
                l_run += lsum;
                // ---- O^T += V^T P^T: four independent accumulators per k-step ----
                if constexpr (kEarly == kNV) {
    #pragma unroll
                    for (int j = 0; j < kNV; ++j) {
                        const int u = j >> 3, t = (j >> 2) & 1, dt = j & 3;
                        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(va[j]), pf[u][t], oacc[dt], 0, 0, 0);
                    }
                } else {
    #pragma unroll
                    for (int g0 = 0; g0 < kNV; g0 += 8) {
    #pragma unroll
                        for (int j = g0; j < g0 + 8; ++j) {
                            const int sh = sh0 + (j >> 3), t = (j >> 2) & 1, dt = j & 3;
                            va[j] = Vt[vpos(32 * dt + ln, 4 * sh + 2 * t + hh)];
                        }
                        __builtin_amdgcn_sched_barrier(0);
    #pragma unroll
                        for (int j = g0; j < g0 + 8; ++j) {
                            const int u = j >> 3, t = (j >> 2) & 1, dt = j & 3;
                            oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(va[j]), pf[u][t], oacc[dt], 0, 0, 0);
                        }
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
            }
        }
    };
    if (kNW == 8 && hsplit == 1) tile_loop(HalfC<1>{});
    else if (kNW == 8 && hsplit == 2) tile_loop(HalfC<2>{});
    else tile_loop(HalfC<0>{});

    if (kNW == 8 && kKS == 1 && nsplit_rb > 0) {
        // split row blocks: the key-1 half's state goes through LDS to the
        // key-0 half's wave, which combines and writes the rows (the tile
        // ring is free once every wave has left the loop)
        __syncthreads();
        const int slot = rw - nfull_rb;                 // split block of this wave
        float *xo = reinterpret_cast<float *>(sm.buf) + (size_t)slot * 64 * 64;   // [64 regs][64 lanes]
        float2 *xml = reinterpret_cast<float2 *>(reinterpret_cast<float *>(sm.buf) + (size_t)3 * 64 * 64) + slot * 64;
        if (hsplit == 2 && wave_active) {
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) xo[(16 * dt + r) * 64 + lane] = oacc[dt][r];
            xml[lane] = make_float2(m_run, l_run);
        }
        __syncthreads();
        if (hsplit == 2) return;
        if (hsplit == 1 && wave_active) {
            // a half with nothing accumulated (every key masked) has no max
            const float2 o = xml[lane];
            const float ma = l_run > 0.0f ? m_run : -__builtin_inff(), mb = o.y > 0.0f ? o.x : -__builtin_inff();
            const float mn = fmaxf(ma, mb);
            const float mu = mn == -__builtin_inff() ? 0.0f : mn;
            const float e0 = __builtin_amdgcn_exp2f((ma - mu) * c2), e1 = __builtin_amdgcn_exp2f((mb - mu) * c2);
            l_run = l_run * e0 + o.y * e1;
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[dt][r] = oacc[dt][r] * e0 + xo[(16 * dt + r) * 64 + lane] * e1;
            m_run = mn;
        }
    }
    if constexpr (kKS == 2) {
        // combine the key halves: the second half's state goes through LDS
        // (the tile ring is free once every wave has left the loop)
        __syncthreads();
        float *xo = reinterpret_cast<float *>(sm.buf) + (size_t)rw * 64 * 64;   // [64 regs][64 lanes]
        float2 *xml = reinterpret_cast<float2 *>(reinterpret_cast<float *>(sm.buf) + (size_t)kRW * 64 * 64) + rw * 64;
        if (kh == 1 && wave_active) {
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) xo[(16 * dt + r) * 64 + lane] = oacc[dt][r];
            xml[lane] = make_float2(m_run, l_run);
        }
        __syncthreads();
        if (kh == 1) return;
        if (wave_active) {
            // a half with nothing accumulated (every key masked) has no max
            const float2 o = xml[lane];
            const float ma = l_run > 0.0f ? m_run : -__builtin_inff(), mb = o.y > 0.0f ? o.x : -__builtin_inff();
            const float mn = fmaxf(ma, mb);
            const float mu = mn == -__builtin_inff() ? 0.0f : mn;
            const float e0 = __builtin_amdgcn_exp2f((ma - mu) * c2), e1 = __builtin_amdgcn_exp2f((mb - mu) * c2);
            l_run = l_run * e0 + o.y * e1;
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[dt][r] = oacc[dt][r] * e0 + xo[(16 * dt + r) * 64 + lane] * e1;
            m_run = mn;
        }
    }

    // ---- epilogue ----
    // oacc[dt][r] is O^T[d = 32dt + 8(r>>2) + 4hh + (r&3)][my_row]
    const int h_out = kvh * G + (my_row % G);
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
    // partials of the rows with a real node only (the merge reads no others)
    if (row_ok) {
        const int unit = u0 * a.RG + rg;
        const size_t pbase = ((size_t)unit * a.nsplit + s) * a.rows_pg;
        const int row_local = rw * 32 + ln;
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
        // (a row with nothing accumulated has no max: -inf, as the merge expects)
        if (hh == 0) a.part_ml[pbase + row_local] = make_float2(l_run > 0.0f ? m_run * c2 : -__builtin_inff(), l_run);
    }
}

template <int kNW, int kKS, int kLoad, int kRing>
__global__ __launch_bounds__(kNW * 64 * (kLoad == kLoadProducers ? 2 : 1)) void k_tree_attn_bf16(AttnArgs a)
{
    __shared__ AttnSmem<kRing> sm;
    tree_attn_body<kNW, kKS, kLoad, kRing>(a, sm);
}

// One launch for batches that mix sequences with many and with few query
// rows (trees and chains): a workgroup whose row group holds at most 64 rows
// with a real node takes the 4-wave key-half form with 4 load waves (two
// SIMDs compute every tile instead of one), the others the 8-wave form.  The
// key-half form writes the first 64 rows of its row group; with a single
// split the group's other rows (no real node) are zeroed here.
template <int kRing>
__global__ __launch_bounds__(512) void k_tree_attn_bf16_mixed(AttnArgs a)
{
    __shared__ AttnSmem<kRing> sm;
    const int x = blockIdx.x;
    int u0, rg, s;
    if (a.sched) {
        const int g = a.Hkv * a.RG, qg = x / g, wi = x - qg * g;
        const int2 e = a.sched_tab[qg];
        if (e.x < 0) return;
        u0 = e.x * a.Hkv + wi % a.Hkv;
        rg = wi / a.Hkv;
        s = e.y;
    } else {
        u0 = x % a.units0;
        const int rest = x / a.units0;
        rg = rest % a.RG;
        s = rest / a.RG;
    }
    const int b = u0 / a.Hkv, kvh = u0 % a.Hkv;
    int n = a.num_nodes[b];
    n = n < 0 ? 0 : (n > a.m_max ? a.m_max : n);
    if (n * a.G - rg * a.rows_pg > 64) {
        tree_attn_body<8, 1, kLoadAll, kRing>(a, sm);
        return;
    }
    tree_attn_body<4, 2, kLoadProducers, kRing>(a, sm);
    int L = a.prefix_len[b];
    L = L < 0 ? 0 : (L > a.cap ? a.cap : L);
    if (s != 0 || (L > 0 && (L + a.chunk - 1) / a.chunk > 1)) return;
    // rows 64 .. rows_pg - 1 of the row group, 16 bytes per thread
    uint4 *out = static_cast<uint4 *>(a.out);
    const int per_row = kHD * 2 / 16;
    for (int t = threadIdx.x; t < (a.rows_pg - 64) * per_row; t += blockDim.x) {
        const int row = rg * a.rows_pg + 64 + t / per_row, node = row / a.G;
        if (node >= a.m_max) continue;
        const int h = kvh * a.G + row % a.G;
        out[(((size_t)b * a.m_max + node) * a.Hq + h) * per_row + t % per_row] = make_uint4(0u, 0u, 0u, 0u);
    }
}

// ---------------------------------------------------------------------------
// Dispatch order of the key splits (one workgroup, before the main kernel):
// workgroups start in blockIdx order as compute units free up, so the order
// decides how well the last round fills the chip.  Split-major order ends
// with the late splits of the longest sequences; this order is the longest-
// first rule in two parts, which is exact here because every split but a
// sequence's last covers a full chunk:
//   1. every split but the last of every sequence (full chunks), sequence by
//      sequence;
//   2. the last split of every sequence, longest first (ties: lower sequence
//      first), weighing a tile by the form that computes it: with the mixed
//      launch a tile of a sequence with at most 64 query rows (key-half
//      form) costs about half one of the 8-wave form (1.5 against 2.8 us
//      per CU on this chip), so a split weighs (prefix tiles + draft tile)
//      x 10 or x 19.
// Entry q holds (sequence, split) for blocks q * Hkv * RG .. + Hkv * RG - 1;
// entries past the last item hold (-1, -1).
// ---------------------------------------------------------------------------
constexpr int kSchedMaxBatch = 1024;

__global__ __launch_bounds__(1024) void k_attn_schedule(AttnArgs a)
{
    __shared__ int s_ns[kSchedMaxBatch], s_lt[kSchedMaxBatch];
    const int B = a.units0 / a.Hkv, ct = a.chunk / kTK, tid = threadIdx.x, NT = blockDim.x;
    for (int b = tid; b < B; b += NT) {
        int L = a.prefix_len[b];
        L = L < 0 ? 0 : (L > a.cap ? a.cap : L);       // as the main kernel clamps it
        int n = a.num_nodes[b];
        n = n < 0 ? 0 : (n > a.m_max ? a.m_max : n);
        const int ns = L > 0 ? (L + a.chunk - 1) / a.chunk : 1;
        s_ns[b] = ns;
        s_lt[b] = ((L + kTK - 1) / kTK - (ns - 1) * ct + (n > 0 ? 1 : 0)) * (n * a.G > 64 ? 19 : 10);
    }
    __syncthreads();
    // (the loops over the batch are unrolled so that their LDS reads go out
    // in groups instead of one round trip per sequence)
    int n1 = 0;                                         // full-chunk splits in all
#pragma unroll 16
    for (int c = 0; c < B; ++c) n1 += s_ns[c] - 1;
    for (int b = tid; b < B; b += NT) {
        const int lt = s_lt[b], ns = s_ns[b];
        int before = 0, rank = 0;
#pragma unroll 16
        for (int c = 0; c < B; ++c) {
            const int l2 = s_lt[c];
            before += c < b ? s_ns[c] - 1 : 0;
            rank += (l2 > lt || (l2 == lt && c < b)) ? 1 : 0;
        }
        for (int j = 0; j < ns - 1; ++j) a.sched_tab[before + j] = make_int2(b, j);
        a.sched_tab[n1 + rank] = make_int2(b, ns - 1);
    }
    for (int q = n1 + B + tid; q < B * a.nsplit; q += NT) a.sched_tab[q] = make_int2(-1, -1);
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
    // block -> (sequence/kv head, row group, row block) in the main kernel's
    // order, so each unit's partials are merged on the XCD whose L2 holds them
    const int x = blockIdx.x;
    const int u0 = x % a.units0;
    const int rest = x / a.units0;
    const int rg = rest % a.RG, j = rest / a.RG;
    const int unit = u0 * a.RG + rg;
    const int rl = j * kMergeRows + (tid >> 4);
    const int d8 = (tid & 15) * 8;
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
        // batches of 8 splits: all loads of a batch are issued before use
        for (int s0 = 0; s0 < nsplit_b; s0 += 8) {
            float2 ml[8];
            float4 o0[8], o1[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const size_t pr = base + (size_t)min(s0 + q, nsplit_b - 1) * a.rows_pg;
                ml[q] = a.part_ml[pr];
                o0[q] = *reinterpret_cast<const float4 *>(a.part_o + pr * kHD + d8);
                o1[q] = *reinterpret_cast<const float4 *>(a.part_o + pr * kHD + d8 + 4);
            }
#pragma unroll
            for (int q = 0; q < 8; ++q) {
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
// fp32 path: exact fp32 arithmetic on the vector ALUs.  A workgroup serves
// four rows (node, q head) of one (sequence, kv head) with KG key groups of
// four waves.  The keys go by in chunks of 64 (the prefix, then the draft
// nodes); group g takes chunks g, g + KG, ..., stages each chunk's K and V^T
// once in its own LDS buffer with coalesced loads (the next chunk's loads are
// issued before the current chunk's products), and keeps an online softmax
// per row.  The groups' partial (max, sum, output) are merged in LDS at the
// end.  QK: lane = key; PV: lane = dimension (two at D = 128).  Padded LDS
// rows (D + 4, 68 floats) keep the 16-byte reads of both products free of
// bank conflicts.
// ---------------------------------------------------------------------------
constexpr int kF32Rows = 4;

template <int D, int KG>
struct F32Smem {
    float k[KG][64][D + 4];      // K chunk, key-major
    float v[KG][D][68];          // V^T chunk, dimension-major
    float q[kF32Rows][D];
    float p[KG * kF32Rows][64];
    float mo[KG][kF32Rows][D];   // partial outputs
    float2 ml[KG][kF32Rows];     // partial (max, sum)
};

template <int D, int KG, bool kPaged>
__global__ __launch_bounds__(64 * kF32Rows * KG) void k_tree_attn_f32(AttnArgs a)
{
    constexpr int kT = 64 * kF32Rows;           // threads of one key group
    constexpr int kPer = 64 * D / kT;           // K (and V) elements per thread per chunk
    __shared__ F32Smem<D, KG> sm;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int w = wv % kF32Rows, g = wv / kF32Rows, gt = tid % kT;
    const int m_max = a.m_max, G = a.G;
    const int nrb = (m_max * G + kF32Rows - 1) / kF32Rows;
    const int rb = blockIdx.x % nrb;
    const int kvh = (blockIdx.x / nrb) % a.Hkv;
    const int b = blockIdx.x / (nrb * a.Hkv);
    const int r = rb * kF32Rows + w;           // row = node * G + q head within the kv head
    const int i = r / G, h = kvh * G + r % G;
    int n = a.num_nodes[b];
    n = n < 0 ? 0 : (n > m_max ? m_max : n);
    int L = a.prefix_len[b];
    if (L < 0 || L > a.cap) {
        if (tid == 0 && rb == 0 && kvh == 0) raise_error(a.err, EAGLE_DEVERR_PREFIX);
        L = L < 0 ? 0 : a.cap;
    }
    const bool live = i < m_max && i < n;      // wave-uniform
    if (live && g == 0) {
        const float *q = static_cast<const float *>(a.q) + (((size_t)b * m_max + i) * a.Hq + h) * D;
        for (int e = lane; e < D; e += 64) sm.q[w][e] = q[e];
    }
    const uint64_t bits = live ? a.anc[(size_t)b * m_max + i] : 0;
    const int npc = (L + 63) / 64, nchunks = npc + 1;
    float kr[kPer], vr[kPer];
    const float *kd0 = static_cast<const float *>(a.kd) + ((size_t)b * m_max * a.Hkv + kvh) * D;
    const float *vd0 = static_cast<const float *>(a.vd) + ((size_t)b * m_max * a.Hkv + kvh) * D;
    // contiguous cache slice of (b, kvh); unused by the paged kernel
    const float *kc0 = static_cast<const float *>(a.kc) + (kPaged ? 0 : ((size_t)b * a.Hkv + kvh) * (size_t)a.cap * D);
    const float *vc0 = static_cast<const float *>(a.vc) + (kPaged ? 0 : ((size_t)b * a.Hkv + kvh) * (size_t)D * a.cap);
    float m_run = -__builtin_inff(), l_run = 0.0f, acc0 = 0.0f, acc1 = 0.0f;
    const int rounds = (nchunks + KG - 1) / KG;
    // Round j stages chunk (j - 1) * KG + g (held in registers) in LDS, issues
    // the loads of chunk j * KG + g, then computes the staged chunk.
    for (int j = 0; j <= rounds; ++j) {
        const int c = (j - 1) * KG + g;
        if (j > 0) {
            __syncthreads();             // the previous chunk's LDS reads are done
            if (c < nchunks) {
#pragma unroll
                for (int u = 0; u < kPer; ++u) {
                    const int idx = u * kT + gt;
                    if constexpr (kPaged) sm.k[g][gt % 64][gt / 64 + u * (kT / 64)] = kr[u];
                    else sm.k[g][idx / D][idx % D] = kr[u];
                    sm.v[g][idx / 64][idx % 64] = vr[u];
                }
            }
            __syncthreads();
        }
        const int cn = j * KG + g;
        if (cn < nchunks) {
            // K element (key, e) with e fastest, V^T element (e, key) with key
            // fastest; keys past the chunk's end read as zero
            const bool draft = cn == npc;
            const int kmax = draft ? n : min(64, L - cn * 64);
            // Per-thread element pointers advanced by a fixed stride per step
            // u.  Contiguous kernel: K element (key, e) = idx / D, idx % D.
            // Paged kernel: K element (gt % 64, gt / 64 + u * kT / 64), so
            // that each thread looks up one page per chunk.  V^T element
            // (e, key) = idx / 64, idx % 64 in both.
            const float *kp, *vp;
            size_t ks, vs;
            if (draft) {
                if constexpr (kPaged) {
                    kp = kd0 + (size_t)(gt % 64) * a.Hkv * D + gt / 64;
                    ks = kT / 64;
                } else {
                    kp = kd0 + (size_t)(gt / D) * a.Hkv * D + gt % D;
                    ks = (size_t)(kT / D) * a.Hkv * D;
                }
                vp = vd0 + (size_t)(gt % 64) * a.Hkv * D + gt / 64;
                vs = kT / 64;
            } else if constexpr (kPaged) {
                const int key = cn * 64 + (gt % 64 < kmax ? gt % 64 : 0);
                kp = k_row<float>(a, b, kvh, key) + gt / 64;
                ks = kT / 64;
                vp = v_elem<float>(a, b, kvh, gt / 64, key);
                vs = (size_t)(kT / 64) * a.block_size;
            } else {
                kp = kc0 + (size_t)cn * 64 * D + gt;
                ks = kT;
                vp = vc0 + (size_t)(gt / 64) * a.cap + cn * 64 + gt % 64;
                vs = (size_t)(kT / 64) * a.cap;
            }
            const bool vok = gt % 64 < kmax;
#pragma unroll
            for (int u = 0; u < kPer; ++u) {
                const bool kok = kPaged ? vok : (u * kT + gt) / D < kmax;
                kr[u] = kok ? *kp : 0.0f;
                vr[u] = vok ? *vp : 0.0f;
                kp += ks;
                vp += vs;
            }
        }
        if (j == 0 || !live || c >= nchunks) continue;
        const bool draft = c == npc;
        const bool ok = draft ? (lane < n && ((bits >> lane) & 1ull)) : (c * 64 + lane < L);
        float dot = 0.0f;
#pragma unroll 4
        for (int e = 0; e < D; e += 4) {
            const float4 kq = *reinterpret_cast<const float4 *>(&sm.k[g][lane][e]);
            const float4 qq = *reinterpret_cast<const float4 *>(&sm.q[w][e]);
            dot = __builtin_fmaf(qq.x, kq.x, dot);
            dot = __builtin_fmaf(qq.y, kq.y, dot);
            dot = __builtin_fmaf(qq.z, kq.z, dot);
            dot = __builtin_fmaf(qq.w, kq.w, dot);
        }
        const float sc = ok ? dot * a.scale_log2 : -__builtin_inff();
        const float m_new = fmaxf(m_run, wave_max(sc));
        const float m_use = m_new == -__builtin_inff() ? 0.0f : m_new;
        const float corr = __builtin_amdgcn_exp2f(m_run - m_use);
        const float p = __builtin_amdgcn_exp2f(sc - m_use);
        float ps = p;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) ps += __shfl_xor(ps, o);
        l_run = l_run * corr + ps;
        m_run = m_new;
        sm.p[wv][lane] = p;              // read back by this wave only
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        acc0 *= corr;
        acc1 *= corr;
#pragma unroll 4
        for (int t = 0; t < 64; t += 4) {
            const float4 pp = *reinterpret_cast<const float4 *>(&sm.p[wv][t]);
            const float4 v0 = *reinterpret_cast<const float4 *>(&sm.v[g][lane][t]);
            acc0 = __builtin_fmaf(pp.x, v0.x, acc0);
            acc0 = __builtin_fmaf(pp.y, v0.y, acc0);
            acc0 = __builtin_fmaf(pp.z, v0.z, acc0);
            acc0 = __builtin_fmaf(pp.w, v0.w, acc0);
            if constexpr (D > 64) {
                const float4 v1 = *reinterpret_cast<const float4 *>(&sm.v[g][lane + 64][t]);
                acc1 = __builtin_fmaf(pp.x, v1.x, acc1);
                acc1 = __builtin_fmaf(pp.y, v1.y, acc1);
                acc1 = __builtin_fmaf(pp.z, v1.z, acc1);
                acc1 = __builtin_fmaf(pp.w, v1.w, acc1);
            }
        }
    }
    // merge the key groups: rescale each to the common maximum
    if (lane == 0) sm.ml[g][w] = make_float2(m_run, l_run);
    sm.mo[g][w][lane] = acc0;
    if constexpr (D > 64) sm.mo[g][w][lane + 64] = acc1;
    __syncthreads();
    if (g != 0 || i >= m_max) return;
    float M = -__builtin_inff();
#pragma unroll
    for (int u = 0; u < KG; ++u) M = fmaxf(M, sm.ml[u][w].x);
    float l = 0.0f, o0 = 0.0f, o1 = 0.0f;
#pragma unroll
    for (int u = 0; u < KG; ++u) {
        const float2 ml = sm.ml[u][w];
        const float s = ml.x == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(ml.x - M);
        l = __builtin_fmaf(ml.y, s, l);
        o0 = __builtin_fmaf(sm.mo[u][w][lane], s, o0);
        if constexpr (D > 64) o1 = __builtin_fmaf(sm.mo[u][w][lane + 64], s, o1);
    }
    float *out = static_cast<float *>(a.out) + (((size_t)b * m_max + i) * a.Hq + h) * D;
    const float inv = live && l > 0.0f ? 1.0f / l : 0.0f;
    out[lane] = live ? o0 * inv : 0.0f;
    if constexpr (D > 64) out[lane + 64] = live ? o1 * inv : 0.0f;
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
        P.row_groups = 1; P.waves = 1; P.chunk = 0; P.nsplit = 1; P.sched = 0;
        P.off_part = P.off_ml = P.off_cnt = kWsHeader;
        P.total = kWsHeader;
        return P;
    }
    P.row_groups = (P.rows + 32 * kMaxWaves - 1) / (32 * kMaxWaves);
    const int rows_pg = (P.rows + P.row_groups - 1) / P.row_groups;
    // 4 or 8 waves (the load slots of a tile divide evenly); waves past the
    // rows only help load
    P.waves = rows_pg <= 128 ? 4 : 8;
    const int units = batch * a->num_kv_heads * P.row_groups;
    // Key splits: one workgroup per CU (the LDS ring fills most of it), so a
    // launch runs in rounds of kCUs workgroups.  Pick the split count that
    // minimises rounds x tiles per split (ties: fewer splits), with at most
    // 128 tiles (8192 keys; a paged split's page list must fit its LDS
    // array) and, when the prefix allows, at least 6 tiles per split (a split
    // costs a merge share and a workgroup's fixed cost: workload 2's call ran
    // 18.2 us with 5 to 7 tiles per split, 20.1 us with 4).
    constexpr long long kCUs = 256;
    const int tiles = P.max_prefix > 0 ? (P.max_prefix + kTK - 1) / kTK : 1;
    int max_per = 128;
    if (a->block_size > 0) max_per = std::min(max_per, (kMaxPages - 1) * a->block_size / kTK);
    const int ns_lo = (tiles + max_per - 1) / max_per;
    const int ns_hi = tiles >= 6 * ns_lo ? tiles / 6 : ns_lo;
    int best = ns_lo;
    long long best_cost = -1;
    for (int ns = ns_lo; ns <= ns_hi; ++ns) {
        const long long per = (tiles + ns - 1) / ns;
        const long long rounds = ((long long)units * ns + kCUs - 1) / kCUs;
        const long long cost = rounds * per;
        if (best_cost < 0 || cost < best_cost) { best_cost = cost; best = ns; }
    }
    const int per = (tiles + best - 1) / best;
    P.chunk = per * kTK;
    P.nsplit = (tiles + per - 1) / per;
    if ((long long)units * P.nsplit > INT32_MAX) { P.total = 0; return P; }   // rejected by the caller
    // Longest-first dispatch (k_attn_schedule) when the launch takes more
    // than one round of long workgroups: with prefixes of different lengths
    // the split-major order leaves CUs idle in the last round.
    P.sched = (per >= 32 && (long long)units * P.nsplit > kCUs && batch <= kSchedMaxBatch) ? 1 : 0;
    const size_t rows_alloc = (size_t)units * P.nsplit * (size_t)(32 * ((rows_pg + 31) / 32));
    size_t o = kWsHeader;
    P.off_part = o; o = align_up(o + (P.nsplit > 1 ? rows_alloc * kHD * sizeof(float) : 0), 256);
    P.off_ml = o;   o = align_up(o + (P.nsplit > 1 ? rows_alloc * sizeof(float2) : 0), 256);
    P.off_cnt = o;  o = align_up(o + (P.sched ? (size_t)batch * P.nsplit * sizeof(int2) : 0), 256);
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
    a.sched_tab = reinterpret_cast<int2 *>(base + P.off_cnt);
    a.sched = P.sched;
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
    if (p->dtype == EAGLE_F32) {
        // key groups: four at D = 64, two at D = 128 (the LDS buffers of one workgroup)
        const int nrb = (P.rows + kF32Rows - 1) / kF32Rows;
        const dim3 g((unsigned)(batch * p->num_kv_heads * nrb));
        const bool paged = p->block_size > 0;
        if (p->head_dim == 64) {
            if (paged) hipLaunchKernelGGL((k_tree_attn_f32<64, 4, true>), g, dim3(64 * kF32Rows * 4), 0, st, a);
            else hipLaunchKernelGGL((k_tree_attn_f32<64, 4, false>), g, dim3(64 * kF32Rows * 4), 0, st, a);
        } else {
            if (paged) hipLaunchKernelGGL((k_tree_attn_f32<128, 2, true>), g, dim3(64 * kF32Rows * 2), 0, st, a);
            else hipLaunchKernelGGL((k_tree_attn_f32<128, 2, false>), g, dim3(64 * kF32Rows * 2), 0, st, a);
        }
    } else {
        const dim3 g((unsigned)(a.units0 * P.row_groups * P.nsplit));
        const bool contiguous = p->block_size == 0;
        if (P.sched) {
            hipLaunchKernelGGL(k_attn_schedule, dim3(1), dim3(1024), 0, st, a);
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
        if (P.waves == 4 && a.rows_pg <= 64) {
            if (contiguous) hipLaunchKernelGGL((k_tree_attn_bf16<4, 2, kLoadProducers, 5>), g, dim3(512), 0, st, a);
            else hipLaunchKernelGGL((k_tree_attn_bf16<4, 2, kLoadProducers, 4>), g, dim3(512), 0, st, a);
        } else if (P.waves == 4) {
            if (contiguous) hipLaunchKernelGGL((k_tree_attn_bf16<4, 1, kLoadAll, 5>), g, dim3(256), 0, st, a);
            else hipLaunchKernelGGL((k_tree_attn_bf16<4, 1, kLoadAll, 4>), g, dim3(256), 0, st, a);
        } else {
            if (contiguous) hipLaunchKernelGGL((k_tree_attn_bf16_mixed<5>), g, dim3(512), 0, st, a);
            else hipLaunchKernelGGL((k_tree_attn_bf16_mixed<4>), g, dim3(512), 0, st, a);
        }
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
