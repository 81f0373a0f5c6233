// build_tree.hip -- dynamic draft tree construction (EAGLE-2 explainer,
// "Dynamic draft tree construction"): per-row softmax statistics and top-C
// children (kernel 1), then per-sequence expansion, rerank and compaction
// (kernel 2).
#include "common.h"
#include "internal.h"
#include "rowvec.h"

namespace eagle {

// ---------------------------------------------------------------------------
// Kernel 1: draft-row statistics, one workgroup per draft row r: M = row max;
// the exact integer weights w = W35(l - M) summed in fp64 (exact in any
// order); and the top-C by (logit desc, id asc), written in rank order with
// their logits (the tree kernel forms c = w / W from them).
//
// Two forms:
//   - k_row_stats (few rows, where latency matters): the row is read once with
//     16-byte coalesced loads and kept in registers across up to 1024 threads;
//   - k_row_stats_stream (many rows or long rows): a streaming max pass, then a
//     streaming weight pass over the same lines (second read from the caches,
//     non-temporal), with few registers, so two workgroups share a compute
//     unit and overlap.
//
// Candidates: every element >= T, with T such that at least C elements are
// >= T: with at least C waves, the C-th largest wave maximum (C waves hold
// such an element); otherwise the largest over waves of the C-th largest lane
// maximum of the wave.  They are appended to an LDS list during the weight
// pass and ranked there; if more than kCandCap qualify (heavy ties) or
// T = -inf, C rounds of block argmax over the row select exactly.
// ---------------------------------------------------------------------------
constexpr int kCandCap = 2048;

struct RowStatsSmem {
    BlockScratch red;
    float cand_v[kCandCap + 16];   // +16: segment reads may run past the count
    int cand_i[kCandCap + 16];
    int rank[kCandCap];
    int sel[kMaxChildren];
    float thr[16];
    int count;
};

// Candidate threshold: needs sm.red.f = the wave maxima (left there by
// block_max) when C <= waves, else the per-lane maxima.
__device__ __forceinline__ float row_threshold(float lmax, int C, RowStatsSmem &sm)
{
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, nw = blockDim.x >> 6;
    if (C <= nw) {
        if (tid < nw) {
            const float fj = sm.red.f[tid];
            int gt = 0, ge = 0;
            for (int i = 0; i < nw; ++i) {
                const float fi = sm.red.f[i];
                gt += fi > fj ? 1 : 0;
                ge += fi >= fj ? 1 : 0;
            }
            if (gt < C && C <= ge) sm.thr[0] = fj;
        }
        if (tid == 0) sm.count = 0;
        __syncthreads();
        return sm.thr[0];
    }
    float sv = lmax;
#pragma unroll
    for (int k = 2; k <= 64; k <<= 1) {
#pragma unroll
        for (int j = k >> 1; j > 0; j >>= 1) {
            const float o = __shfl_xor(sv, j);
            const bool keep_max = ((lane & j) == 0) == ((lane & k) == 0);
            sv = keep_max ? fmaxf(sv, o) : fminf(sv, o);
        }
    }
    const float tw = __shfl(sv, C - 1);
    if (lane == 0) sm.thr[wv] = tw;
    if (tid == 0) sm.count = 0;
    __syncthreads();
    float thr = sm.thr[0];
    for (int j = 1; j < nw; ++j) thr = fmaxf(thr, sm.thr[j]);
    return thr;
}

// Ranks the candidate list (complete: called after a barrier) and writes the
// row's top-C; returns false if the list overflowed (caller falls back).
__device__ __forceinline__ bool rank_candidates(int C, int total, RowStatsSmem &sm, int32_t *out_id,
                                                float *out_v)
{
    const int tid = threadIdx.x, NT = blockDim.x;
    if (total > kCandCap) return false;
    // rank of every candidate: comparisons split into segments of 16, one
    // (segment, candidate) pair per thread; the lanes of a wave share a
    // segment, so their LDS reads broadcast; partial counts meet in LDS atomics
    for (int i = tid; i < total; i += NT) sm.rank[i] = 0;
    __syncthreads();
    const int nseg = (total + 15) / 16;
    for (int t = tid; t < total * nseg; t += NT) {
        const int g = t / total, i = t % total;
        const float vi = sm.cand_v[i];
        const int ii = sm.cand_i[i];
        int cnt = 0;
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int j = 16 * g + q;
            cnt += (j < total && before(sm.cand_v[j], sm.cand_i[j], vi, ii)) ? 1 : 0;
        }
        if (cnt) atomicAdd(&sm.rank[i], cnt);
    }
    __syncthreads();
    for (int i = tid; i < total; i += NT)
        if (sm.rank[i] < C) sm.sel[sm.rank[i]] = i;
    __syncthreads();
    if (tid < C) {
        const int i = sm.sel[tid];   // total >= C: T leaves at least C candidates
        out_id[tid] = sm.cand_i[i];
        out_v[tid] = sm.cand_v[i];
    }
    return true;
}

// bf16 weight histogram.  A weight depends only on the logit's value and the
// row maximum, a bf16 logit takes one of 2^16 values, and the weight sum is an
// exact integer (every partial sum below 2^53), so the sum may be formed as
// the sum over values of count x weight.  Logits of magnitude in [2^-9, 2^7)
// (16 binades of both signs, 4096 bins) are counted in LDS during the weight
// pass and each bin's weight is formed once per row; any other logit (tiny,
// zero, huge, inf, NaN, the -inf padding) takes its weight directly.  Same
// integers, same sum: W is bit-identical to the element-by-element form, at
// about a third of its VALU work per element.
constexpr uint32_t kHistE0 = 127 - 9;             // biased exponent of the lowest binade
constexpr uint32_t kHistSide = 16 * 128;          // bins per sign
constexpr int kHistBins = 2 * kHistSide;
constexpr int kHistMinVocab = 4 * kHistBins;      // shorter rows: element by element

// adds one element's weight: to its bin, or directly to wsum
__device__ __forceinline__ void hist_add(unsigned *hist, float f, float M, double &wsum)
{
    const uint32_t fb = __float_as_uint(f);
    const uint32_t rel = (fb & 0x7FFF0000u) - (kHistE0 << 23);
    if (rel < (kHistSide << 16)) atomicAdd(&hist[(rel >> 16) + (fb >> 31) * kHistSide], 1u);
    else wsum += (double)weight_of(f, M);
}

// the bins' share of the weight sum (after a barrier that follows the counts);
// count <= 2^17 and weight <= 2^36, so each product is exact in fp64
__device__ __forceinline__ void hist_sum(const unsigned *hist, float M, double &wsum)
{
    for (int i = threadIdx.x; i < kHistBins; i += blockDim.x) {
        const unsigned c = hist[i];
        if (c) {
            const uint32_t sgn = (uint32_t)i / kHistSide, rel = (uint32_t)i % kHistSide;
            const float v = __uint_as_float(((sgn << 15) | ((kHistE0 << 7) + rel)) << 16);
            wsum += (double)c * (double)weight_of(v, M);
        }
    }
}

// Rows held in registers: vector j of a thread holds elements
// [(j * NT + tid) * VEC, + VEC).
template <typename T, int kNV, bool kHist>
__global__ __launch_bounds__(1024) void k_row_stats(RowStatsArgs a)
{
    constexpr int VEC = Vec<T>::n;
    __shared__ RowStatsSmem sm;
    __shared__ unsigned hist[kHist ? kHistBins : 1];
    const int g = blockIdx.x;   // input row; its statistics go to slot r_all
    const int b = g / a.rows_in, r = a.row_base + g % a.rows_in;
    const size_t r_all = (size_t)b * a.r_max + r;
    const int kind = a.kind ? a.kind[b] : EAGLE_TREE_DYNAMIC;
    const int rows_needed = kind == EAGLE_TREE_CHAIN ? a.chain_k : a.rows_dyn;
    if (r >= rows_needed) return;
    const int C = kind == EAGLE_TREE_CHAIN ? 1 : a.children;
    const int V = a.vocab, NT = blockDim.x, tid = threadIdx.x;
    const T *row = static_cast<const T *>(a.logits) + (size_t)g * (size_t)a.row_stride;

    uint4 x[kNV];
#pragma unroll
    for (int j = 0; j < kNV; ++j) x[j] = load_vec<T>(row, (j * NT + tid) * VEC, V, a.vec_ok);
    if constexpr (kHist)
        for (int i = tid; i < kHistBins; i += NT) hist[i] = 0;   // ordered by block_max's barriers

    float lmax = -__builtin_inff();
#pragma unroll
    for (int j = 0; j < kNV; ++j) {
        float f[VEC];
        unpack<T>(x[j], f);
#pragma unroll
        for (int e = 0; e < VEC; ++e) lmax = fmaxf(lmax, f[e]);
    }
    if (tid == 0) sm.thr[0] = -__builtin_inff();   // stays -inf (exact fallback) if no maximum qualifies
    const float M = block_max(lmax, sm.red);       // wave maxima stay in sm.red.f
    const float thr = row_threshold(lmax, C, sm);

    const bool use_list = thr != -__builtin_inff();
    double wsum = 0.0;
#pragma unroll
    for (int j = 0; j < kNV; ++j) {
        float f[VEC];
        unpack<T>(x[j], f);
        const int base = (j * NT + tid) * VEC;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            if constexpr (kHist) hist_add(hist, f[e], M, wsum);
            else wsum += (double)weight_of(f[e], M);
            // padding reads -inf, below any finite T; with T = -inf the list
            // is not used (exact selection instead), so nothing is appended
            if (use_list && f[e] >= thr) {
                const int o = atomicAdd(&sm.count, 1);
                if (o < kCandCap) { sm.cand_v[o] = f[e]; sm.cand_i[o] = base + e; }
            }
        }
    }
    if constexpr (kHist) {
        __syncthreads();
        hist_sum(hist, M, wsum);
    }
    const double W = block_sum_d(wsum, sm.red);   // contains barriers: the list is complete
    int32_t *out_id = a.top_id + (size_t)r_all * a.children;
    float *out_v = a.top_v + (size_t)r_all * a.children;
    if (!(use_list && rank_candidates(C, sm.count, sm, out_id, out_v))) {
        // heavy ties or T = -inf: C rounds of "best element after the previous
        // pick" over the registers (rare; exact for any input)
        float pv = __builtin_inff();
        int pi = -1;
        for (int c = 0; c < C; ++c) {
            float bv = -__builtin_inff();
            int bi = 0x7fffffff;
#pragma unroll
            for (int j = 0; j < kNV; ++j) {
                float f[VEC];
                unpack<T>(x[j], f);
                const int base = (j * NT + tid) * VEC;
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    const int id = base + e;
                    if (id < V && before(pv, pi, f[e], id) && before(f[e], id, bv, bi)) { bv = f[e]; bi = id; }
                }
            }
            block_best(bv, bi, sm.red);
            if (tid == 0) { out_id[c] = bi; out_v[c] = bv; }
            pv = bv;
            pi = bi;
        }
    }
    if (tid == 0) {
        a.W[r_all] = W;
        a.M[r_all] = M;
    }
}

// Streaming form: a max pass, then a weight pass over the same lines.
template <typename T, bool kHist>
__global__ __launch_bounds__(1024) void k_row_stats_stream(RowStatsArgs a)
{
    constexpr int VEC = Vec<T>::n;
    __shared__ RowStatsSmem sm;
    __shared__ unsigned hist[kHist ? kHistBins : 1];
    const int g = blockIdx.x;   // input row; its statistics go to slot r_all
    const int b = g / a.rows_in, r = a.row_base + g % a.rows_in;
    const size_t r_all = (size_t)b * a.r_max + r;
    const int kind = a.kind ? a.kind[b] : EAGLE_TREE_DYNAMIC;
    const int rows_needed = kind == EAGLE_TREE_CHAIN ? a.chain_k : a.rows_dyn;
    if (r >= rows_needed) return;
    const int C = kind == EAGLE_TREE_CHAIN ? 1 : a.children;
    const int V = a.vocab, NT = blockDim.x, tid = threadIdx.x;
    const T *row = static_cast<const T *>(a.logits) + (size_t)g * (size_t)a.row_stride;
    const int nvec = (V + VEC - 1) / VEC;
    if constexpr (kHist)
        for (int i = tid; i < kHistBins; i += NT) hist[i] = 0;   // ordered by block_max's barriers

    float lmax = -__builtin_inff();
    for (int v0 = tid; v0 < nvec; v0 += 4 * NT) {
        uint4 x[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int v = v0 + u * NT;
            x[u] = v < nvec ? load_vec<T>(row, v * VEC, V, a.vec_ok) : make_uint4(0u, 0u, 0u, 0u);   // (skipped below)
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (v0 + u * NT >= nvec) continue;
            float f[VEC];
            unpack<T>(x[u], f);
#pragma unroll
            for (int e = 0; e < VEC; ++e) lmax = fmaxf(lmax, f[e]);
        }
    }
    if (tid == 0) sm.thr[0] = -__builtin_inff();
    const float M = block_max(lmax, sm.red);   // wave maxima stay in sm.red.f
    const float thr = row_threshold(lmax, C, sm);

    const bool use_list = thr != -__builtin_inff();
    double wsum = 0.0;
    // the weight pass is the lines' last use: non-temporal reads (the max
    // pass reads them with the default policy, so they are still cached)
    for (int v0 = tid; v0 < nvec; v0 += 4 * NT) {
        uint4 x[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int v = v0 + u * NT;
            x[u] = v >= nvec ? make_uint4(0u, 0u, 0u, 0u)   // (skipped below)
                 : (a.vec_ok && v * VEC + VEC <= V) ? ld16_stream(row + v * VEC) : load_vec<T>(row, v * VEC, V, a.vec_ok);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int v = v0 + u * NT;
            if (v >= nvec) continue;
            float f[VEC];
            unpack<T>(x[u], f);
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                if constexpr (kHist) hist_add(hist, f[e], M, wsum);
                else wsum += (double)weight_of(f[e], M);
                const int id = v * VEC + e;
                if (use_list && f[e] >= thr) {   // as in the register form
                    const int o = atomicAdd(&sm.count, 1);
                    if (o < kCandCap) { sm.cand_v[o] = f[e]; sm.cand_i[o] = id; }
                }
            }
        }
    }
    if constexpr (kHist) {
        __syncthreads();
        hist_sum(hist, M, wsum);
    }
    const double W = block_sum_d(wsum, sm.red);
    int32_t *out_id = a.top_id + (size_t)r_all * a.children;
    float *out_v = a.top_v + (size_t)r_all * a.children;
    if (!(use_list && rank_candidates(C, sm.count, sm, out_id, out_v))) {
        float pv = __builtin_inff();
        int pi = -1;
        for (int c = 0; c < C; ++c) {
            float bv = -__builtin_inff();
            int bi = 0x7fffffff;
            for (int id = tid; id < V; id += NT) {
                const float f = load_scalar<T>(row + id);
                if (before(pv, pi, f, id) && before(f, id, bv, bi)) { bv = f; bi = id; }
            }
            block_best(bv, bi, sm.red);
            if (tid == 0) { out_id[c] = bi; out_v[c] = bv; }
            pv = bv;
            pi = bi;
        }
    }
    if (tid == 0) {
        a.W[r_all] = W;
        a.M[r_all] = M;
    }
}

// ---------------------------------------------------------------------------
// Children drawn from the draft (sampled build), one workgroup per draft row:
// M and the exact weight sum W as above, then `children` draws without
// replacement by the inverse CDF of the integer weights.  With R the weight
// left and word r, the target is s = floor(r R / 2^32) and the drawn token is
// the first, in id order, of the tokens not yet drawn whose inclusive
// cumulative weight exceeds s (the first token not yet drawn when no weight
// is left).  Each thread owns a contiguous chunk of the row and keeps its
// chunk's undrawn weight, so a draw is one block scan of those sums plus one
// thread's walk through its chunk.  The drawn ids, in draw order, and their
// logits take the place of the top-C lists.
// ---------------------------------------------------------------------------
struct DrawSmem {
    unsigned long long part[16];
    float fmax[16];
    int drawn[kMaxChildren];
    float drawn_w[kMaxChildren];
    float drawn_l[kMaxChildren];
    int first_free[16];
    int walk_lo, walk_hi;              // the chunk holding the draw
    unsigned long long walk_excl;      // undrawn weight before it
};

__device__ __forceinline__ unsigned long long block_sum_u64(unsigned long long v, DrawSmem &sm)
{
    const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) sm.part[w] = v;
    __syncthreads();
    unsigned long long r = 0;
    for (int j = 0; j < nw; ++j) r += sm.part[j];
    return r;
}

// exclusive prefix sum over the block's threads
__device__ __forceinline__ unsigned long long block_exclusive_u64(unsigned long long v, DrawSmem &sm)
{
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    unsigned long long incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const unsigned long long t = __shfl_up(incl, o);
        if (lane >= o) incl += t;
    }
    __syncthreads();
    if (lane == 63) sm.part[w] = incl;
    __syncthreads();
    unsigned long long base = 0;
    for (int j = 0; j < w; ++j) base += sm.part[j];
    return base + incl - v;
}

template <typename T>
__global__ __launch_bounds__(1024) void k_row_draws(RowStatsArgs a, const uint32_t *words)
{
    __shared__ DrawSmem sm;
    const int g = blockIdx.x;
    const int b = g / a.rows_in, r = a.row_base + g % a.rows_in;
    const size_t r_all = (size_t)b * a.r_max + r;
    if (r >= a.rows_dyn) return;
    const int C = a.children, V = a.vocab, NT = blockDim.x, tid = threadIdx.x;
    constexpr int VEC = Vec<T>::n;
    const T *row = static_cast<const T *>(a.logits) + (size_t)g * (size_t)a.row_stride;
    // this thread's chunk [lo, hi): whole 16-byte vectors
    const int per = ((V + NT - 1) / NT + VEC - 1) / VEC * VEC;
    const int lo = min(V, tid * per), hi = min(V, lo + per);
    float lmax = -__builtin_inff();
    for (int j = tid; j * VEC < V; j += NT) {   // coalesced
        float f[VEC];
        unpack<T>(load_vec<T>(row, j * VEC, V, a.vec_ok), f);
#pragma unroll
        for (int e = 0; e < VEC; ++e) lmax = fmaxf(lmax, f[e]);
    }
    lmax = wave_max(lmax);
    if ((tid & 63) == 0) sm.fmax[tid >> 6] = lmax;
    __syncthreads();
    float M = sm.fmax[0];
    for (int j = 1; j < (NT >> 6); ++j) M = fmaxf(M, sm.fmax[j]);
    unsigned long long own = 0;
    for (int v0 = lo; v0 < hi; v0 += VEC) {
        float f[VEC];
        unpack<T>(load_vec<T>(row, v0, V, a.vec_ok), f);
#pragma unroll
        for (int e = 0; e < VEC; ++e) own += (unsigned long long)weight_of(f[e], M);   // -inf past V: 0
    }
    int32_t *out_id = a.top_id + r_all * a.children;
    float *out_v = a.top_v + r_all * a.children;
    if (!__builtin_isfinite(M)) {
        // a NaN or infinite logit: reported, no draws (every thread leaves here)
        if (tid == 0) {
            raise_error(a.err, EAGLE_DEVERR_NONFINITE_ROW);
            a.W[r_all] = 0.0;
            a.M[r_all] = M;
        }
        for (int t = tid; t < C; t += NT) { out_id[t] = -1; out_v[t] = -__builtin_inff(); }
        return;
    }
    if (tid == 0) {
        // an empty walk until a chunk claims the draw (one always does: s < R)
        sm.walk_lo = sm.walk_hi = 0;
        sm.walk_excl = 0;
    }
    const unsigned long long W = block_sum_u64(own, sm);
    unsigned long long R = W;
    for (int t = 0; t < C; ++t) {
        if (tid == 0) {
            sm.drawn[t] = -1;
            sm.drawn_w[t] = 0.0f;
            sm.drawn_l[t] = -__builtin_inff();
        }
        const uint32_t word = words[r_all * C + t];
        // s = floor(word * R / 2^32), R < 2^53
        const unsigned long long s = (unsigned long long)word * (R >> 32) +
                                     (((unsigned long long)word * (R & 0xffffffffull)) >> 32);
        const unsigned long long excl = block_exclusive_u64(own, sm);
        int first = 0x7fffffff;
        if (R > 0 && excl <= s && s < excl + own) {
            // the target falls in this chunk: wave 0 walks it below
            sm.walk_lo = lo;
            sm.walk_hi = hi;
            sm.walk_excl = excl;
        } else if (R == 0) {
            // no weight left: the first token not yet drawn
            for (int v = lo; v < hi && first == 0x7fffffff; ++v) {
                bool taken = false;
                for (int q = 0; q < t; ++q) taken |= sm.drawn[q] == v;
                if (!taken) first = v;
            }
        }
        if (R == 0) {
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) first = min(first, __shfl_xor(first, o));
            if ((tid & 63) == 0) sm.first_free[tid >> 6] = first;
        }
        __syncthreads();
        if (R > 0 && tid < 64) {
            // wave 0 walks the chunk 64 tokens at a time: the draw is the
            // first undrawn token whose running weight passes s
            const int wlo = sm.walk_lo, whi = sm.walk_hi;
            unsigned long long cum = sm.walk_excl;
            for (int v0 = wlo; v0 < whi; v0 += 64) {
                const int v = v0 + tid;
                float l = -__builtin_inff(), w = 0.0f;
                if (v < whi) {
                    bool taken = false;
                    for (int q = 0; q < t; ++q) taken |= sm.drawn[q] == v;
                    l = load_scalar<T>(row + v);
                    if (!taken) w = weight_of(l, M);
                }
                unsigned long long incl = (unsigned long long)w;
#pragma unroll
                for (int o = 1; o < 64; o <<= 1) {
                    const unsigned long long u = __shfl_up(incl, o);
                    if (tid >= o) incl += u;
                }
                const unsigned long long hit = __ballot(cum + incl > s);
                if (hit) {
                    const int f = __ffsll((long long)hit) - 1;
                    const float lf = __shfl(l, f), wf = __shfl(w, f);
                    if (tid == 0) {
                        sm.drawn[t] = v0 + f;
                        sm.drawn_w[t] = wf;
                        sm.drawn_l[t] = lf;
                    }
                    break;
                }
                cum += __shfl(incl, 63);
            }
        }
        if (R == 0 && tid == 0) {
            int f = sm.first_free[0];
            for (int j = 1; j < (NT >> 6); ++j) f = min(f, sm.first_free[j]);
            if (f < V) {   // (C <= V: a token is always left)
                sm.drawn[t] = f;
                sm.drawn_l[t] = load_scalar<T>(row + f);
                sm.drawn_w[t] = weight_of(sm.drawn_l[t], M);
            }
        }
        __syncthreads();
        const int x = sm.drawn[t];
        const unsigned long long wx = (unsigned long long)sm.drawn_w[t];
        if (x >= lo && x < hi) own -= wx;
        R -= wx;
        if (tid == 0) {
            out_id[t] = x;
            out_v[t] = sm.drawn_l[t];
        }
    }
    if (tid == 0) {
        a.W[r_all] = (double)W;
        a.M[r_all] = M;
    }
}

// ---------------------------------------------------------------------------
// Kernel 2: one workgroup per sequence, everything in LDS.  Candidates are
// numbered in creation order; the candidates of one depth form lists of C
// (the children of one expanded node, or of the root), and every entry of a
// list precedes every entry of a later list in creation order.  Per depth:
//   - the rank of each candidate within its depth, by (V desc, creation asc),
//     is the number of entries of every list of the depth that come first: one
//     (candidate, list) pair per thread, partial counts added with LDS atomics
//     (no ordering inside a list is assumed);
//   - the candidates are scattered to rank order; the first k are expanded.
// The rerank then merges the depths' rank-ordered lists: a candidate's overall
// rank is its rank within its depth plus, for every other depth, how many of
// that depth's first m entries come first (binary search: earlier depths win
// ties, later depths lose them).  Ranks below m are the selected nodes.
// ---------------------------------------------------------------------------
struct TreeSmem {
    double conf[kMaxRows * kMaxChildren];   // c of every (row, child)
    int cid[kMaxRows * kMaxChildren];       // token of every (row, child)
    double V[kMaxCand + kMaxChildren];      // by creation index (+ slack: whole-list reads)
    double key[kMaxCand + kMaxChildren];    // ranking key by creation index: V, or c (confidence policies)
    double sV[kMaxCand];                    // keys in rank order, each depth at its offset
    int ord[kMaxCand];                      // creation index in rank order, each depth at its offset
    int tok[kMaxCand];
    int par[kMaxCand];
    int dep[kMaxCand];
    int row[kMaxCand];
    int rank_d[kMaxCand];                   // rank within the depth
    int ahead[kMaxCand];                    // entries of other depths that come first
    int rank_of[kMaxCand];                  // overall rank, -1 if not selected
    int sel[kMaxMMax];                      // creation index by overall rank
    int prank[kMaxMMax];                    // parent's rank by rank (ancestor masks)
    int gord[kMaxCand];                     // creation index by overall key order (policy 2)
    int chain[kMaxDepth];                   // missing ancestors of one candidate (policy 2)
    int m_out;                              // nodes selected
    int lvl_off[kMaxDepth + 1];             // first creation index of each depth, then N
};

// next double below v, for a key v >= 0 (0 -> the negative denormal closest
// to 0): for finite x, x >= v exactly when x > below(v)
__device__ __forceinline__ double below(double v)
{
    return v > 0.0 ? __longlong_as_double(__double_as_longlong(v) - 1) : -__longlong_as_double(1ll);
}

// kC: the children per list when fixed at compile time (10, the common case),
// or 0 for any C up to kMaxChildren
template <int kC>
__global__ __launch_bounds__(1024) void k_tree_select(TreeSelectArgs a)
{
    __shared__ TreeSmem sm;
    const int b = blockIdx.x, tid = threadIdx.x, NT = blockDim.x;
    const int kind = a.kind ? a.kind[b] : EAGLE_TREE_DYNAMIC;
    const int m_max = a.m_max, Cw = a.children;
    const size_t rb = (size_t)b * a.r_max;
    int32_t *tokens = a.tokens + (size_t)b * m_max, *parent = a.parent + (size_t)b * m_max;
    int32_t *depth = a.depth + (size_t)b * m_max, *src_row = a.src_row + (size_t)b * m_max;
    double *score = a.score + (size_t)b * m_max;

    if (a.levels && a.levels[b] != a.depth_max) {
        // incremental build with levels missing: an empty tree
        if (tid == 0) {
            raise_error(a.err, EAGLE_DEVERR_TREE);
            a.num_nodes[b] = 0;
        }
        for (int i = tid; i < m_max; i += NT) {
            tokens[i] = -1; parent[i] = -1; depth[i] = -1; score[i] = 0.0; src_row[i] = -1;
        }
        return;
    }

    if (kind == EAGLE_TREE_CHAIN) {
        const int K = a.chain_k;
        if (tid == 0) {
            double Vp = 1.0;
            for (int i = 0; i < K; ++i) {
                // the row's argmax and its confidence
                const float bv = a.top_v[(rb + i) * Cw];
                const int bi = a.top_id[(rb + i) * Cw];
                const double W = a.W[rb + i];
                const float M = a.M[rb + i];
                if (!__builtin_isfinite(M) || !__builtin_isfinite(W)) raise_error(a.err, EAGLE_DEVERR_NONFINITE_ROW);
                Vp = Vp * ((double)weight_of(bv, M) / W);
                tokens[i] = bi;
                parent[i] = i - 1;
                depth[i] = i + 1;
                score[i] = Vp;
                src_row[i] = (i + 1 < K) ? i + 1 : -1;
            }
            a.num_nodes[b] = K;
        }
        for (int i = K + tid; i < m_max; i += NT) {
            tokens[i] = -1; parent[i] = -1; depth[i] = -1; score[i] = 0.0; src_row[i] = -1;
        }
        if (a.anc) {
            // a chain's node i sees nodes 0..i and sits at depth i + 1
            const int L = a.prefix_len[b];
            for (int i = tid; i < m_max; i += NT) {
                a.anc[(size_t)b * m_max + i] = i < K ? (i == 63 ? ~0ull : (2ull << i) - 1) : 0ull;
                a.pos[(size_t)b * m_max + i] = i < K ? L + i : -1;
            }
        }
        return;
    }

    const int D = a.depth_max, k = a.topk, C = kC ? kC : a.children, m = a.m;
    constexpr int kSlots = kC ? kC : kMaxChildren;   // list entries read per list
    const bool conf_key = a.policy == EAGLE_POLICY_CONF || a.policy == EAGLE_POLICY_CONF_NO_RERANK;
    const int R = 1 + (D - 1) * k;
    // the rows' children in rank order, c = W35(l - M) / W
    for (int i = tid; i < R * C; i += NT) {
        const int r = i / C, j = i - r * C;
        const size_t o = (rb + r) * Cw + j;
        const float M = a.M[rb + r];
        const double W = a.W[rb + r];
        sm.cid[i] = a.top_id[o];
        sm.conf[i] = (double)weight_of(a.top_v[o], M) / W;
        if (j == 0 && (!__builtin_isfinite(M) || !__builtin_isfinite(W))) raise_error(a.err, EAGLE_DEVERR_NONFINITE_ROW);
    }
    for (int i = tid; i < kMaxCand; i += NT) {
        sm.rank_d[i] = 0;
        sm.ahead[i] = 0;
        sm.rank_of[i] = -1;
    }
    __syncthreads();
    // depth 1: the children of the root's row 0, one list
    for (int j = tid; j < C; j += NT) {
        sm.V[j] = sm.conf[j];
        sm.key[j] = sm.conf[j];
        sm.tok[j] = sm.cid[j];
        sm.par[j] = -1;
        sm.dep[j] = 1;
        sm.row[j] = -1;
    }
    if (tid == 0) sm.lvl_off[0] = 0;
    __syncthreads();

    int off = 0, n = C, nl = 1;   // this depth: first creation index, candidates, lists
    for (int lv = 0; lv < D; ++lv) {
        // ---- rank within the depth: pairs (candidate x, list q) ----
        // consecutive threads take consecutive x of one list q, so the reads
        // of q's entries are broadcasts; a thread keeps its x and steps q
        {
            const int lanes_x = n < NT ? n : NT;
            const int qstep = NT / lanes_x;
            const int x0 = tid % lanes_x, q0 = tid / lanes_x;
            for (int x = x0; q0 < qstep && x < n; x += lanes_x) {
                const int p = x / C, j = x - p * C;
                const double vx = sm.key[off + x];
                int c = 0;
                for (int q = q0; q < nl; q += qstep) {
                    // the whole list is read first (one LDS round trip); slots
                    // past C are read but not counted
                    const double *L = sm.key + off + q * C;
                    double vl[kSlots];
#pragma unroll
                    for (int i = 0; i < kSlots; ++i) vl[i] = L[i];
                    if (q != p) {
                        // an earlier list's entries precede x when their key is
                        // at least x's (ties: created first), a later list's
                        // when it is greater: one compare against t each
                        const double t = q < p ? below(vx) : vx;
#pragma unroll
                        for (int i = 0; i < kSlots; ++i) c += ((kC || i < C) && vl[i] > t) ? 1 : 0;
                    } else {
                        // x's own list: entries created before x win ties
#pragma unroll
                        for (int i = 0; i < kSlots; ++i)
                            c += ((kC || i < C) && (vl[i] > vx || (vl[i] == vx && i < j))) ? 1 : 0;
                    }
                }
                if (c) atomicAdd(&sm.rank_d[off + x], c);
            }
        }
        __syncthreads();
        for (int x = tid; x < n; x += NT) {
            const int r = sm.rank_d[off + x];
            sm.ord[off + r] = off + x;
            sm.sV[off + r] = sm.key[off + x];
        }
        __syncthreads();
        if (lv + 1 == D) break;
        // ---- expansion: the first k in rank order own rows 1 + lv k + p ----
        const int ne = min(k, n), noff = off + n;
        for (int t = tid; t < ne * C; t += NT) {
            const int p = t / C, j = t - p * C;
            const int e = sm.ord[off + p], r = 1 + lv * k + p, g = noff + t;
            sm.V[g] = sm.V[e] * sm.conf[r * C + j];
            sm.key[g] = conf_key ? sm.conf[r * C + j] : sm.V[g];
            sm.tok[g] = sm.cid[r * C + j];
            sm.par[g] = e;
            sm.dep[g] = lv + 2;
            sm.row[g] = -1;
            if (j == 0) sm.row[e] = r;
        }
        if (tid == 0) sm.lvl_off[lv + 1] = noff;
        __syncthreads();
        off = noff;
        n = ne * C;
        nl = ne;
    }
    const int N = off + n;

    if (tid == 0) sm.lvl_off[D] = N;
    __syncthreads();
    if (a.policy == kPolicyAllCandidates) {
        // sampled children: the tree is every candidate, in creation order
        for (int g = tid; g < N; g += NT) {
            sm.sel[g] = g;
            sm.rank_of[g] = g;
        }
        if (tid == 0) sm.m_out = N;
        __syncthreads();
    } else if (a.policy == EAGLE_POLICY_EAGLE2) {
        // ---- rerank: merge the depths' rank-ordered lists (first m of each) ----
        // item = (entry i < m of depth lv, other depth od); the depth sizes follow
        // from (C, k) alone, so items are located without reading LDS
        int items = 0;
        if (D > 1) {
            int nn = C;
            for (int lv = 0; lv < D; ++lv) {
                items += min(nn, m) * (D - 1);
                nn = min(k, nn) * C;
            }
        }
        for (int t = tid; t < items; t += NT) {
            int lv = 0, nn = C, base = 0, o = 0;
            while (base + min(nn, m) * (D - 1) <= t) {
                base += min(nn, m) * (D - 1);
                o += nn;
                nn = min(k, nn) * C;
                ++lv;
            }
            const int u = t - base, i = u / (D - 1);
            int od = u - i * (D - 1);
            od += od >= lv ? 1 : 0;
            const double v = sm.sV[o + i];
            const int so = sm.lvl_off[od];
            const double *s = sm.sV + so;
            const bool win_ties = od < lv;   // earlier depth: smaller creation indices
            // the entries of od that come first are a prefix of its rank order
            int lo = 0, hi = min(sm.lvl_off[od + 1] - so, m);
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                const double y = s[mid];
                if (y > v || (win_ties && y == v)) lo = mid + 1;
                else hi = mid;
            }
            if (lo) atomicAdd(&sm.ahead[sm.ord[o + i]], lo);
        }
        __syncthreads();
        for (int g = tid; g < N; g += NT) {
            const int rd = sm.rank_d[g];
            if (rd < m) {
                const int r = rd + sm.ahead[g];
                if (r < m) {
                    sm.sel[r] = g;
                    sm.rank_of[g] = r;
                }
            }
        }
        if (tid == 0) sm.m_out = m;
        __syncthreads();
    } else if (a.policy == EAGLE_POLICY_NO_RERANK || a.policy == EAGLE_POLICY_CONF_NO_RERANK) {
        // no rerank: every depth's first k by the key, depth by depth
        for (int g = tid; g < N; g += NT) {
            const int lv = sm.dep[g] - 1, rd = sm.rank_d[g];
            if (rd < k) {
                int base = 0, nn = C;
                for (int d = 0; d < lv; ++d) {
                    base += min(k, nn);
                    nn = min(k, nn) * C;
                }
                sm.sel[base + rd] = g;
                sm.rank_of[g] = base + rd;
            }
        }
        if (tid == 0) {
            int tot = 0, nn = C;
            for (int d = 0; d < D; ++d) {
                tot += min(k, nn);
                nn = min(k, nn) * C;
            }
            sm.m_out = tot;
        }
        __syncthreads();
    } else {
        // confidence rerank: every candidate's place in the overall key order
        // (its rank in its depth plus, for every other depth, the entries that
        // come first), then one thread takes the candidates in that order,
        // each with its missing ancestors (root first), while the tree stays
        // within m nodes
        for (int t = tid; t < N * (D - 1); t += NT) {
            const int g = t / (D - 1), lv = sm.dep[g] - 1;
            int od = t - g * (D - 1);
            od += od >= lv ? 1 : 0;
            const double v = sm.key[g];
            const int so = sm.lvl_off[od];
            const double *sv = sm.sV + so;
            const bool win_ties = od < lv;
            int lo = 0, hi = sm.lvl_off[od + 1] - so;
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                const double y = sv[mid];
                if (y > v || (win_ties && y == v)) lo = mid + 1;
                else hi = mid;
            }
            if (lo) atomicAdd(&sm.ahead[g], lo);
        }
        __syncthreads();
        for (int g = tid; g < N; g += NT) {
            const int r = sm.rank_d[g] + sm.ahead[g];
            if (r < N) sm.gord[r] = g;
        }
        __syncthreads();
        if (tid == 0) {
            int n_sel = 0;
            for (int t = 0; t < N && n_sel < m; ++t) {
                int nc = 0;
                for (int q = sm.gord[t]; q >= 0 && q < N && sm.rank_of[q] < 0 && nc < kMaxDepth; q = sm.par[q])
                    sm.chain[nc++] = q;
                if (nc == 0 || n_sel + nc > m) continue;
                for (int c = nc - 1; c >= 0; --c) {
                    sm.rank_of[sm.chain[c]] = n_sel;
                    sm.sel[n_sel++] = sm.chain[c];
                }
            }
            sm.m_out = n_sel;
        }
        __syncthreads();
    }
    const int m_out = sm.m_out;
    // connected tree check: every selected node's parent is selected (then,
    // by induction, every ancestor is).  It holds by construction: c <= 1, so
    // V never grows along a path, and parents are created before children.
    for (int r = tid; r < m_out; r += NT) {
        const int i = sm.sel[r];
        const int q = sm.par[i];
        const int pr = q < 0 ? -1 : sm.rank_of[q];
        if (q >= 0 && pr < 0) raise_error(a.err, EAGLE_DEVERR_CLOSURE);
        tokens[r] = sm.tok[i];
        parent[r] = pr;
        depth[r] = sm.dep[i];
        score[r] = sm.V[i];
        src_row[r] = sm.row[i];
        sm.prank[r] = pr;
    }
    for (int r = m_out + tid; r < m_max; r += NT) {
        tokens[r] = -1; parent[r] = -1; depth[r] = -1; score[r] = 0.0; src_row[r] = -1;
    }
    if (tid == 0) a.num_nodes[b] = m_out;
    if (a.anc) {
        // ancestor masks: node r and the nodes on its path to the root (rank
        // order is topological, so parents have smaller ranks); position =
        // prefix_len + depth - 1
        const int L = a.prefix_len[b];
        __syncthreads();
        for (int r = tid; r < m_max; r += NT) {
            uint64_t acc = 0;
            int pos = -1;
            if (r < m_out) {
                acc = 1ull << r;
                // (bounded: a tree with non-finite scores, already reported,
                // may leave ranks unassigned)
                int q = sm.prank[r];
                for (int it = 0; it < kMaxMMax && q >= 0 && q < m_out; ++it, q = sm.prank[q]) acc |= 1ull << q;
                pos = L + __popcll(acc) - 1;
            }
            a.anc[(size_t)b * m_max + r] = acc;
            a.pos[(size_t)b * m_max + r] = pos;
        }
    }
}

// ---------------------------------------------------------------------------
// Incremental build (the draft runs one forward per depth): level 0 brings
// the root's row, level l >= 1 the rows of the k nodes expanded at depth l, in
// expansion order (rows 1 + (l - 1) k + p).  After the level's row
// statistics, k_tree_frontier forms the V of the level's children (depth
// l + 1) exactly as k_tree_select does, ranks them by (V desc, creation asc)
// and writes the first k: the nodes whose rows the next level brings.  Once
// every level is in, k_tree_select builds the tree from the statistics of all
// levels, so the tree equals the one-shot build's over the same rows.
// ---------------------------------------------------------------------------
constexpr int kFrontierThreads = 256;

__global__ __launch_bounds__(kFrontierThreads) void k_tree_frontier(FrontierArgs a)
{
    __shared__ double V[kMaxTopk * kMaxChildren];
    __shared__ double key[kMaxTopk * kMaxChildren];   // ranking key: V, or c (confidence policies)
    __shared__ int in_order;
    const int b = blockIdx.x, tid = threadIdx.x, NT = blockDim.x;
    const int C = a.children, k = a.topk, lv = a.level;
    const size_t rb = (size_t)b * a.r_max;
    int32_t *f_tok = a.f_tok + (size_t)b * k, *f_par = a.f_par + (size_t)b * k;
    double *f_score = a.f_score + (size_t)b * k;
    double *fV = a.fV + (size_t)b * kMaxTopk;
    if (tid == 0) {
        in_order = lv == 0 || a.levels[b] == lv;
        if (!in_order) raise_error(a.err, EAGLE_DEVERR_TREE);
    }
    for (int i = tid; i < k; i += NT) {
        f_tok[i] = -1; f_par[i] = -1; f_score[i] = 0.0;
    }
    __syncthreads();
    if (!in_order) return;
    // the level's children in creation order: (parent p, child j)
    const int n = (lv == 0 ? 1 : a.fn[b]) * C;
    for (int x = tid; x < n; x += NT) {
        const int p = x / C, j = x - p * C;
        const size_t r = rb + (lv == 0 ? 0 : 1 + (size_t)(lv - 1) * k + p);
        const float M = a.M[r];
        const double W = a.W[r];
        const double c = (double)weight_of(a.top_v[r * C + j], M) / W;
        V[x] = lv == 0 ? c : fV[p] * c;
        key[x] = (a.policy == EAGLE_POLICY_CONF || a.policy == EAGLE_POLICY_CONF_NO_RERANK) ? c : V[x];
        if (j == 0 && (!__builtin_isfinite(M) || !__builtin_isfinite(W))) raise_error(a.err, EAGLE_DEVERR_NONFINITE_ROW);
    }
    __syncthreads();   // fV is read: it may now be overwritten
    const int ne = lv + 1 < a.depth_max ? min(k, n) : 0;   // depth D is not expanded
    for (int x = tid; x < n; x += NT) {
        const double kx = key[x];
        int rk = 0;
        for (int y = 0; y < n; ++y) rk += (key[y] > kx || (key[y] == kx && y < x)) ? 1 : 0;
        if (rk < ne) {
            const int p = x / C, j = x - p * C;
            const size_t r = rb + (lv == 0 ? 0 : 1 + (size_t)(lv - 1) * k + p);
            f_tok[rk] = a.top_id[r * C + j];
            f_par[rk] = lv == 0 ? -1 : p;
            f_score[rk] = V[x];
            fV[rk] = V[x];
        }
    }
    if (tid == 0) {
        a.fn[b] = ne;
        a.levels[b] = lv + 1;
    }
}

// ---------------------------------------------------------------------------
// EAGLE-1's static tree: template node i (parents first) is the tchild[i]-th
// top token of its parent's row; the root owns row 0 and the q-th template
// node with children owns row 1 + q.  One wave per sequence, lane i = node i
// (templates of up to 64 nodes); V is formed root first by one lane, as the
// dynamic build forms it.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void k_tree_template(TemplateArgs a)
{
    __shared__ double sV[kMaxMMax];
    __shared__ double sc[kMaxMMax];
    __shared__ int sdep[kMaxMMax];
    __shared__ int spar[kMaxMMax];
    const int b = blockIdx.x, i = threadIdx.x, n = a.n_t, C = a.children;
    const size_t rb = (size_t)b * a.r_max;
    int32_t *tokens = a.tokens + (size_t)b * a.m_max, *parent = a.parent + (size_t)b * a.m_max;
    int32_t *depth = a.depth + (size_t)b * a.m_max, *src_row = a.src_row + (size_t)b * a.m_max;
    double *score = a.score + (size_t)b * a.m_max;
    const int p = i < n ? a.tparent[i] : -1, j = i < n ? a.tchild[i] : 0;
    const bool bad_node = i < n && (p < -1 || p >= i || j < 0 || j >= C);
    // rows: node q owns one iff some node names it as parent
    bool has_child = false;
    for (int q = 0; q < n; ++q) has_child |= __shfl(p, q) == i;
    const unsigned long long owners = __ballot(i < n && has_child);
    const int row = has_child ? 1 + __popcll(owners & ((1ull << i) - 1)) : -1;
    const bool bad = __ballot(bad_node) != 0 || 1 + __popcll(owners) > a.r_max;
    if (bad) {
        // an invalid template: an empty tree
        if (i == 0) {
            raise_error(a.err, EAGLE_DEVERR_TREE);
            a.num_nodes[b] = 0;
        }
        if (i < a.m_max) { tokens[i] = -1; parent[i] = -1; depth[i] = -1; score[i] = 0.0; src_row[i] = -1; }
        return;
    }
    // the parent's row and this node's token and confidence
    const int prow_any = __shfl(row, p < 0 ? 0 : p);   // every lane takes part in the shuffle
    const int prow = p < 0 ? 0 : prow_any;
    int tok = -1;
    spar[i] = p;
    if (i < n) {
        const size_t o = (rb + prow) * C + j;
        const float M = a.M[rb + prow];
        const double W = a.W[rb + prow];
        tok = a.top_id[o];
        sc[i] = (double)weight_of(a.top_v[o], M) / W;
        if (!__builtin_isfinite(M) || !__builtin_isfinite(W)) raise_error(a.err, EAGLE_DEVERR_NONFINITE_ROW);
    }
    __syncthreads();
    if (i == 0) {
        for (int q = 0; q < n; ++q) {
            const int pq = spar[q];
            sV[q] = (pq < 0 ? 1.0 : sV[pq]) * sc[q];
            sdep[q] = pq < 0 ? 1 : sdep[pq] + 1;
        }
    }
    __syncthreads();
    if (i < a.m_max) {
        tokens[i] = i < n ? tok : -1;
        parent[i] = i < n ? p : -1;
        depth[i] = i < n ? sdep[i] : -1;
        score[i] = i < n ? sV[i] : 0.0;
        src_row[i] = i < n ? row : -1;
    }
    if (i == 0) a.num_nodes[b] = n;
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
BuildLayout build_layout(const eagle_tree_params *p, int32_t batch)
{
    BuildLayout L;
    const size_t rows = (size_t)batch * p->r_max;
    size_t o = kWsHeader;
    L.off_M = o;      o = align_up(o + rows * sizeof(float), 256);
    L.off_W = o;      o = align_up(o + rows * sizeof(double), 256);
    L.off_id = o;     o = align_up(o + rows * p->children * sizeof(int32_t), 256);
    L.off_v = o;      o = align_up(o + rows * p->children * sizeof(float), 256);
    L.off_fV = o;     o = align_up(o + (size_t)batch * kMaxTopk * sizeof(double), 256);
    L.off_fn = o;     o = align_up(o + (size_t)batch * sizeof(int32_t), 256);
    L.off_lv = o;     o = align_up(o + (size_t)batch * sizeof(int32_t), 256);
    L.total = o;
    return L;
}

// Register path: vectors per thread (1, 2, 4 or 8) for a row of `vocab`
// elements read by up to 1024 threads; 0: the row needs the streaming kernel.
constexpr int kRegisterRowsMax = 256;

int row_vectors(int vocab, int vec)
{
    const long long per = 1024LL * vec;
    for (int nv = 1; nv <= 8; nv *= 2)
        if (vocab <= per * nv) return nv;
    return 0;
}

// threads of the register path: enough for the row, a multiple of 64
int row_threads(int vocab, int vec)
{
    const int nv = row_vectors(vocab, vec);
    const long long per = (long long)(nv ? nv : 8) * vec;
    long long nt = (vocab + per - 1) / per;
    nt = (nt + 63) / 64 * 64;
    return (int)(nt < 64 ? 64 : (nt > 1024 ? 1024 : nt));
}

// row statistics of ra.rows input rows (register or streaming form)
static hipError_t launch_row_stats(const RowStatsArgs &ra, eagle_dtype dt, hipStream_t st)
{
    if (ra.rows <= 0) return hipSuccess;
    const int vec = dt == EAGLE_F32 ? 4 : 8;
    const int nv = row_vectors(ra.vocab, vec);
    const int nt = row_threads(ra.vocab, vec);
    // registers for few rows (each row's latency is the step's), streaming
    // for many rows (workgroups overlap) and for rows too long for registers
    if (nv == 0 || ra.rows > kRegisterRowsMax) {
#define EAGLE_STREAM(T, H) hipLaunchKernelGGL((k_row_stats_stream<T, H>), dim3((unsigned)ra.rows), dim3(1024), 0, st, ra)
        if (dt == EAGLE_F32) EAGLE_STREAM(float, false);
        else if (ra.vocab >= kHistMinVocab) EAGLE_STREAM(uint16_t, true);
        else EAGLE_STREAM(uint16_t, false);
#undef EAGLE_STREAM
    } else {
        const dim3 g1((unsigned)ra.rows);
#define EAGLE_ROWS(T, NV, H) hipLaunchKernelGGL((k_row_stats<T, NV, H>), g1, dim3(nt), 0, st, ra)
        if (dt == EAGLE_F32) {
            if (nv == 1) EAGLE_ROWS(float, 1, false);
            else if (nv == 2) EAGLE_ROWS(float, 2, false);
            else if (nv == 4) EAGLE_ROWS(float, 4, false);
            else EAGLE_ROWS(float, 8, false);
        } else if (ra.vocab >= kHistMinVocab) {   // (nv >= 2 here)
            if (nv == 2) EAGLE_ROWS(uint16_t, 2, true);
            else if (nv == 4) EAGLE_ROWS(uint16_t, 4, true);
            else EAGLE_ROWS(uint16_t, 8, true);
        } else {
            if (nv == 1) EAGLE_ROWS(uint16_t, 1, false);
            else if (nv == 2) EAGLE_ROWS(uint16_t, 2, false);
            else if (nv == 4) EAGLE_ROWS(uint16_t, 4, false);
            else EAGLE_ROWS(uint16_t, 8, false);
        }
#undef EAGLE_ROWS
    }
    return hipGetLastError();
}

static RowStatsArgs row_stats_args(const eagle_tree_params *p, int32_t batch, const BuildLayout &L, void *ws,
                                   const void *logits, eagle_dtype dt, int64_t row_stride, const int32_t *kind,
                                   int rows_in, int row_base)
{
    char *base = static_cast<char *>(ws);
    RowStatsArgs ra;
    ra.logits = logits;
    ra.row_stride = row_stride;
    ra.rows = batch * rows_in;
    ra.r_max = p->r_max;
    ra.vocab = p->vocab;
    ra.children = p->children;
    ra.chain_k = p->chain_k;
    ra.rows_dyn = 1 + (p->depth - 1) * p->topk;
    ra.rows_in = rows_in;
    ra.row_base = row_base;
    ra.kind = kind;
    ra.M = reinterpret_cast<float *>(base + L.off_M);
    ra.W = reinterpret_cast<double *>(base + L.off_W);
    ra.top_id = reinterpret_cast<int32_t *>(base + L.off_id);
    ra.top_v = reinterpret_cast<float *>(base + L.off_v);
    ra.err = reinterpret_cast<uint32_t *>(base);
    const size_t esz = dt == EAGLE_F32 ? 4 : 2;
    ra.vec_ok = ((uintptr_t)logits % 16 == 0) && ((size_t)row_stride * esz % 16 == 0);
    return ra;
}

static hipError_t launch_select(const eagle_tree_params *p, int32_t batch, const RowStatsArgs &ra,
                                const int32_t *kind, const int32_t *levels, int32_t *tokens, int32_t *parent,
                                int32_t *depth, double *score, int32_t *src_row, int32_t *num_nodes,
                                hipStream_t st, const int32_t *prefix_len, uint64_t *anc, int32_t *pos,
                                int policy);

static hipError_t launch_select(const eagle_tree_params *p, int32_t batch, const RowStatsArgs &ra,
                                const int32_t *kind, const int32_t *levels, int32_t *tokens, int32_t *parent,
                                int32_t *depth, double *score, int32_t *src_row, int32_t *num_nodes,
                                hipStream_t st, const int32_t *prefix_len = nullptr, uint64_t *anc = nullptr,
                                int32_t *pos = nullptr)
{
    return launch_select(p, batch, ra, kind, levels, tokens, parent, depth, score, src_row, num_nodes, st, prefix_len,
                         anc, pos, p->policy);
}

static hipError_t launch_select(const eagle_tree_params *p, int32_t batch, const RowStatsArgs &ra,
                                const int32_t *kind, const int32_t *levels, int32_t *tokens, int32_t *parent,
                                int32_t *depth, double *score, int32_t *src_row, int32_t *num_nodes,
                                hipStream_t st, const int32_t *prefix_len, uint64_t *anc, int32_t *pos,
                                int policy)
{
    TreeSelectArgs ta;
    ta.kind = kind;
    ta.depth_max = p->depth;
    ta.topk = p->topk;
    ta.children = p->children;
    ta.m = p->m;
    ta.chain_k = p->chain_k;
    ta.m_max = p->m_max;
    ta.r_max = p->r_max;
    ta.policy = policy;
    ta.top_id = ra.top_id;
    ta.top_v = ra.top_v;
    ta.M = ra.M;
    ta.W = ra.W;
    ta.tokens = tokens;
    ta.parent = parent;
    ta.depth = depth;
    ta.score = score;
    ta.src_row = src_row;
    ta.num_nodes = num_nodes;
    ta.levels = levels;
    ta.prefix_len = prefix_len;
    ta.anc = anc;
    ta.pos = pos;
    ta.err = ra.err;
    if (batch <= 0) return hipSuccess;
    if (p->children == 10) hipLaunchKernelGGL(k_tree_select<10>, dim3(batch), dim3(1024), 0, st, ta);
    else hipLaunchKernelGGL(k_tree_select<0>, dim3(batch), dim3(1024), 0, st, ta);
    return hipGetLastError();
}

hipError_t launch_build_tree(const eagle_tree_params *p, int32_t batch, const void *logits,
                             eagle_dtype dt, int64_t row_stride, const int32_t *kind,
                             int32_t *tokens, int32_t *parent, int32_t *depth, double *score,
                             int32_t *src_row, int32_t *num_nodes, void *ws, hipStream_t st)
{
    const BuildLayout L = build_layout(p, batch);
    const RowStatsArgs ra = row_stats_args(p, batch, L, ws, logits, dt, row_stride, kind, p->r_max, 0);
    hipError_t e = launch_row_stats(ra, dt, st);
    if (e != hipSuccess) return e;
    return launch_select(p, batch, ra, kind, nullptr, tokens, parent, depth, score, src_row, num_nodes, st);
}

hipError_t launch_build_tree_mask(const eagle_tree_params *p, int32_t batch, const void *logits,
                                  eagle_dtype dt, int64_t row_stride, const int32_t *kind,
                                  const int32_t *prefix_len, int32_t *tokens, int32_t *parent, int32_t *depth,
                                  double *score, int32_t *src_row, int32_t *num_nodes, uint64_t *anc,
                                  int32_t *pos, void *ws, hipStream_t st)
{
    const BuildLayout L = build_layout(p, batch);
    const RowStatsArgs ra = row_stats_args(p, batch, L, ws, logits, dt, row_stride, kind, p->r_max, 0);
    hipError_t e = launch_row_stats(ra, dt, st);
    if (e != hipSuccess) return e;
    return launch_select(p, batch, ra, kind, nullptr, tokens, parent, depth, score, src_row, num_nodes, st,
                         prefix_len, anc, pos);
}

hipError_t launch_build_tree_sampled(const eagle_tree_params *p, int32_t batch, const void *logits,
                                    eagle_dtype dt, int64_t row_stride, const uint32_t *child_words,
                                    int32_t *tokens, int32_t *parent, int32_t *depth, double *score,
                                    int32_t *src_row, int32_t *num_nodes, void *ws, hipStream_t st)
{
    const BuildLayout L = build_layout(p, batch);
    const RowStatsArgs ra = row_stats_args(p, batch, L, ws, logits, dt, row_stride, nullptr, p->r_max, 0);
    if (ra.rows > 0) {
        int nt = ((p->vocab + 7) / 8 + 63) / 64 * 64;
        nt = nt < 64 ? 64 : (nt > 1024 ? 1024 : nt);
        if (dt == EAGLE_F32)
            hipLaunchKernelGGL(k_row_draws<float>, dim3((unsigned)ra.rows), dim3(nt), 0, st, ra, child_words);
        else
            hipLaunchKernelGGL(k_row_draws<uint16_t>, dim3((unsigned)ra.rows), dim3(nt), 0, st, ra, child_words);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return launch_select(p, batch, ra, nullptr, nullptr, tokens, parent, depth, score, src_row, num_nodes, st,
                         nullptr, nullptr, nullptr, kPolicyAllCandidates);
}

hipError_t launch_build_tree_template(const eagle_tree_params *p, int32_t batch, const void *logits,
                                     eagle_dtype dt, int64_t row_stride, int32_t n_tmpl, const int32_t *tparent,
                                     const int32_t *tchild, int32_t *tokens, int32_t *parent, int32_t *depth,
                                     double *score, int32_t *src_row, int32_t *num_nodes, void *ws, hipStream_t st)
{
    const BuildLayout L = build_layout(p, batch);
    RowStatsArgs ra = row_stats_args(p, batch, L, ws, logits, dt, row_stride, nullptr, p->r_max, 0);
    ra.rows_dyn = p->r_max;   // every row of the template's layout
    hipError_t e = launch_row_stats(ra, dt, st);
    if (e != hipSuccess) return e;
    TemplateArgs ta;
    ta.n_t = n_tmpl;
    ta.children = p->children;
    ta.r_max = p->r_max;
    ta.m_max = p->m_max;
    ta.tparent = tparent;
    ta.tchild = tchild;
    ta.M = ra.M;
    ta.W = ra.W;
    ta.top_id = ra.top_id;
    ta.top_v = ra.top_v;
    ta.tokens = tokens;
    ta.parent = parent;
    ta.depth = depth;
    ta.score = score;
    ta.src_row = src_row;
    ta.num_nodes = num_nodes;
    ta.err = ra.err;
    hipLaunchKernelGGL(k_tree_template, dim3((unsigned)batch), dim3(64), 0, st, ta);
    return hipGetLastError();
}

hipError_t launch_tree_expand(const eagle_tree_params *p, int32_t batch, int32_t level, const void *logits,
                              eagle_dtype dt, int64_t row_stride, int32_t *f_tok, int32_t *f_par,
                              double *f_score, void *ws, hipStream_t st)
{
    const BuildLayout L = build_layout(p, batch);
    const int rows_in = level == 0 ? 1 : p->topk;
    const int row_base = level == 0 ? 0 : 1 + (level - 1) * p->topk;
    const RowStatsArgs ra = row_stats_args(p, batch, L, ws, logits, dt, row_stride, nullptr, rows_in, row_base);
    hipError_t e = launch_row_stats(ra, dt, st);
    if (e != hipSuccess) return e;
    char *base = static_cast<char *>(ws);
    FrontierArgs fa;
    fa.level = level;
    fa.depth_max = p->depth;
    fa.topk = p->topk;
    fa.children = p->children;
    fa.r_max = p->r_max;
    fa.policy = p->policy;
    fa.M = ra.M;
    fa.W = ra.W;
    fa.top_id = ra.top_id;
    fa.top_v = ra.top_v;
    fa.fV = reinterpret_cast<double *>(base + L.off_fV);
    fa.fn = reinterpret_cast<int32_t *>(base + L.off_fn);
    fa.levels = reinterpret_cast<int32_t *>(base + L.off_lv);
    fa.f_tok = f_tok;
    fa.f_par = f_par;
    fa.f_score = f_score;
    fa.err = ra.err;
    hipLaunchKernelGGL(k_tree_frontier, dim3((unsigned)batch), dim3(kFrontierThreads), 0, st, fa);
    return hipGetLastError();
}

hipError_t launch_tree_finish(const eagle_tree_params *p, int32_t batch, int32_t *tokens, int32_t *parent,
                              int32_t *depth, double *score, int32_t *src_row, int32_t *num_nodes, void *ws,
                              hipStream_t st)
{
    const BuildLayout L = build_layout(p, batch);
    const RowStatsArgs ra = row_stats_args(p, batch, L, ws, nullptr, EAGLE_BF16, p->vocab, nullptr, 0, 0);
    const int32_t *levels = reinterpret_cast<const int32_t *>(static_cast<char *>(ws) + L.off_lv);
    return launch_select(p, batch, ra, nullptr, levels, tokens, parent, depth, score, src_row, num_nodes, st);
}

}  // namespace eagle
