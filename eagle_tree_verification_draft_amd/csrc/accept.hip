// accept.hip -- acceptance walk over the verified tree (EAGLE-1 explainer,
// "Verification"; EAGLE-2 explainer, "Key contributions": lossless by
// rejection sampling).  One workgroup per sequence walks from the root; each
// step reads one target row (the current node's) once from HBM into registers.
#include "common.h"
#include "internal.h"
#include "rowvec.h"

namespace eagle {

constexpr int kAcceptThreads = 1024;

struct AcceptArgs {
    const void *target;
    int64_t row_stride;
    int m_max, vocab, max_accept, mode;
    float temperature;
    bool unit_t, vec_ok;
    const int32_t *tokens, *parent, *num_nodes;
    const uint32_t *words;
    int32_t *accepted, *accept_len, *bonus;
    uint32_t *err;
};

struct AcceptSmem {
    BlockScratch red;
    int tok[kMaxMMax];
    int par[kMaxMMax];
    double wchild[kMaxMMax];
    int removed[kMaxMMax];
    double part[1024 / 64];
    int next;
    int nrem;
    unsigned long long R;
    int bonus;
};

// exclusive scan of exact integer-valued doubles over the block
__device__ __forceinline__ double block_exclusive_scan_d(double v, double *part)
{
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
    double incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const double t = __shfl_up(incl, o);
        if (lane >= o) incl += t;
    }
    __syncthreads();
    if (lane == 63) part[w] = incl;
    __syncthreads();
    double base = 0.0;
    for (int j = 0; j < w; ++j) base += part[j];
    (void)nw;
    return base + incl - v;
}

// Visits this thread's elements of a row as (value, index): 16-byte vector
// loads in a rolled loop (coalesced across the workgroup), scalar loads for a
// ragged tail or an unaligned row.
template <typename T, typename F>
__device__ __forceinline__ void for_each_elem(const T *row, int V, bool vec_ok, F &&fn)
{
    constexpr int VEC = Vec<T>::n;
    const int NT = blockDim.x, tid = threadIdx.x;
    const int nvec = vec_ok ? V / VEC : 0;
    // batches of 4 independent 16-byte loads per thread
    for (int j0 = tid; j0 < nvec; j0 += 4 * NT) {
        uint4 u[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int j = j0 + q * NT;
            u[q] = j < nvec ? *reinterpret_cast<const uint4 *>(row + (size_t)j * VEC) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int j = j0 + q * NT;
            if (j < nvec) {
                float f[VEC];
                unpack<T>(u[q], f);
#pragma unroll
                for (int e = 0; e < VEC; ++e) fn(f[e], j * VEC + e);
            }
        }
    }
    for (int v = nvec * VEC + tid; v < V; v += NT) fn(load_scalar<T>(row + v), v);
}

template <typename T>
__global__ __launch_bounds__(1024) void k_accept(AcceptArgs a)
{
    __shared__ AcceptSmem sm;
    const int b = blockIdx.x, tid = threadIdx.x, NT = blockDim.x;
    const int m_max = a.m_max, V = a.vocab;
    int n = a.num_nodes[b];
    if (n < 0 || n > m_max) {
        if (tid == 0) raise_error(a.err, EAGLE_DEVERR_TREE);
        n = n < 0 ? 0 : m_max;
    }
    for (int i = tid; i < kMaxMMax; i += NT) {
        sm.tok[i] = i < n ? a.tokens[(size_t)b * m_max + i] : -1;
        sm.par[i] = i < n ? a.parent[(size_t)b * m_max + i] : -2;
    }
    __syncthreads();

    int cur = -1, len = 0, bonus = -1;
    int32_t *acc = a.accepted + (size_t)b * a.max_accept;
    for (int step = 0; step <= kMaxMMax; ++step) {
        const T *row = static_cast<const T *>(a.target) +
                       ((size_t)b * (m_max + 1) + (size_t)(cur + 1)) * (size_t)a.row_stride;
        if (tid == 0) sm.next = 0x7fffffff;
        int next = -1;
        if (a.mode == EAGLE_ACCEPT_GREEDY) {
            float bv = -__builtin_inff();
            int bi = 0x7fffffff;
            bool nan = false;
            for_each_elem<T>(row, V, a.vec_ok, [&](float f, int id) {
                nan |= (f != f);
                if (before(f, id, bv, bi)) { bv = f; bi = id; }
            });
            if (__any(nan) && (tid & 63) == 0) raise_error(a.err, EAGLE_DEVERR_NONFINITE_ROW);
            block_best(bv, bi, sm.red);
            const int g = bi;
            for (int i = tid; i < n; i += NT)
                if (sm.par[i] == cur && sm.tok[i] == g) atomicMin(&sm.next, i);
            __syncthreads();
            next = sm.next == 0x7fffffff ? -1 : sm.next;
            if (next < 0) bonus = g;
        } else {
            float lmax = -__builtin_inff();
            for_each_elem<T>(row, V, a.vec_ok, [&](float f, int) { lmax = fmaxf(lmax, f); });
            const float M = block_max(lmax, sm.red);
            double ws = 0.0;
            for_each_elem<T>(row, V, a.vec_ok,
                             [&](float f, int) { ws += (double)weight_of_t(f, M, a.temperature, a.unit_t); });
            const double W = block_sum_d(ws, sm.red);
            if (!__builtin_isfinite(M) || !__builtin_isfinite(W)) {
                if (tid == 0) raise_error(a.err, EAGLE_DEVERR_NONFINITE_ROW);
                break;
            }
            // weights of the current node's children
            for (int i = tid; i < n; i += NT)
                if (sm.par[i] == cur) {
                    const int t = sm.tok[i];
                    if (t < 0 || t >= V) {                 // malformed tree: no mass, reported
                        raise_error(a.err, EAGLE_DEVERR_TREE);
                        sm.wchild[i] = 0.0;
                    } else {
                        sm.wchild[i] = (double)weight_of_t(load_scalar<T>(row + t), M, a.temperature, a.unit_t);
                    }
                }
            __syncthreads();
            if (tid == 0) {
                unsigned long long R = (unsigned long long)W;
                int nrem = 0, nx = -1;
                for (int i = 0; i < n; ++i) {
                    if (sm.par[i] != cur) continue;
                    const int t = sm.tok[i];
                    bool gone = false;
                    for (int j = 0; j < nrem; ++j) gone |= sm.removed[j] == t;
                    const unsigned long long wt = gone ? 0ull : (unsigned long long)sm.wchild[i];
                    const unsigned __int128 lhs = (unsigned __int128)a.words[(size_t)b * (m_max + 1) + i] * R;
                    const unsigned __int128 rhs = (unsigned __int128)wt << 32;
                    if (lhs < rhs) { nx = i; break; }
                    R -= wt;
                    if (!gone) sm.removed[nrem++] = t;
                }
                sm.next = nx;
                sm.nrem = nrem;
                sm.R = R;
            }
            __syncthreads();
            next = sm.next;
            if (next < 0) {
                // bonus: smallest v with inclusive cumulative residual weight > s;
                // thread t owns the contiguous range [t*E, (t+1)*E)
                const unsigned long long R = sm.R;
                const int nrem = sm.nrem;
                const unsigned long long s = (unsigned long long)(
                    ((unsigned __int128)a.words[(size_t)b * (m_max + 1) + m_max] * R) >> 32);
                const int E = (V + NT - 1) / NT;
                const int lo = min(V, tid * E), hi = min(V, lo + E);
                double mine = 0.0;
                for (int v = lo; v < hi; ++v) mine += (double)weight_of_t(load_scalar<T>(row + v), M, a.temperature, a.unit_t);
                for (int j = 0; j < nrem; ++j) {
                    const int t = sm.removed[j];
                    if (t >= lo && t < hi) mine -= (double)weight_of_t(load_scalar<T>(row + t), M, a.temperature, a.unit_t);
                }
                const double before_me = block_exclusive_scan_d(mine, sm.part);
                if (tid == 0) sm.bonus = -1;
                __syncthreads();
                const double sd = (double)s;
                if (before_me <= sd && sd < before_me + mine) {
                    double cum = before_me;
                    for (int v = lo; v < hi; ++v) {
                        bool gone = false;
                        for (int j = 0; j < nrem; ++j) gone |= sm.removed[j] == v;
                        if (gone) continue;
                        cum += (double)weight_of_t(load_scalar<T>(row + v), M, a.temperature, a.unit_t);
                        if (cum > sd) { sm.bonus = v; break; }
                    }
                }
                __syncthreads();
                bonus = sm.bonus;
            }
        }
        if (next < 0) break;
        if (len >= a.max_accept) {
            if (tid == 0) raise_error(a.err, EAGLE_DEVERR_PATH);
            break;
        }
        if (tid == 0) acc[len] = next;
        ++len;
        cur = next;
        __syncthreads();
    }
    for (int j = len + tid; j < a.max_accept; j += NT) acc[j] = -1;
    if (tid == 0) {
        a.accept_len[b] = len;
        a.bonus[b] = bonus;
    }
}

// ---------------------------------------------------------------------------
// Register-resident walk (the general form): one workgroup per sequence; at
// each step the current node's target row is read once into registers --
// thread t holds kNV 16-byte vectors, vector q covering elements
// (q*NT + t)*VEC .. +VEC-1 -- and the maximum, the exact weight sum and the
// bonus prefix search all run from there.  Every wave holds node i of the
// sequence in lane i (m_max <= 64), so each wave finds the current node's
// children with a ballot and runs the sequential child tests on wave-uniform
// values itself; the only barriers are those of the row reductions.
// ---------------------------------------------------------------------------
constexpr int kRegMaxVectors = 16;

template <bool B> struct Flag { static constexpr bool value = B; };

struct RegSmem {
    BlockScratch red;
    double part[kRegMaxVectors * 16];   // bonus search: residual weight of (vector q, wave w)
    double before;                      // residual weight ahead of the chosen (q, w)
    int qw;                             // chosen q * waves + w, or -1
    int bonus;
};

__device__ __forceinline__ unsigned long long readlane_u64(unsigned long long v, int k)
{
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, k);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), k);
    return ((unsigned long long)hi << 32) | lo;
}

// exclusive prefix sum over the lanes of one wave (exact integer-valued doubles)
__device__ __forceinline__ double wave_exclusive_scan_d(double v)
{
    const int lane = threadIdx.x & 63;
    double incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const double t = __shfl_up(incl, o);
        if (lane >= o) incl += t;
    }
    return incl - v;
}

// block maximum that propagates NaN (any NaN input makes the result NaN)
__device__ __forceinline__ float block_maximum(float v, BlockScratch &s)
{
    const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = __builtin_elementwise_maximum(v, __shfl_xor(v, o));
    __syncthreads();
    if ((threadIdx.x & 63) == 0) s.f[w] = v;
    __syncthreads();
    float r = s.f[0];
    for (int j = 1; j < nw; ++j) r = __builtin_elementwise_maximum(r, s.f[j]);
    return r;
}

__device__ __forceinline__ int block_min_i(int v, BlockScratch &s)
{
    const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o));
    __syncthreads();
    if ((threadIdx.x & 63) == 0) s.i[w] = v;
    __syncthreads();
    int r = s.i[0];
    for (int j = 1; j < nw; ++j) r = min(r, s.i[j]);
    return r;
}

// exclusive prefix sum over the lanes of one wave (64-bit integers)
__device__ __forceinline__ unsigned long long wave_exclusive_scan_u64(unsigned long long v)
{
    const int lane = threadIdx.x & 63;
    unsigned long long incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const unsigned long long t = __shfl_up(incl, o);
        if (lane >= o) incl += t;
    }
    return incl - v;
}

template <typename T, int kNV, bool kSample>
__global__ __launch_bounds__(1024) void k_accept_reg(AcceptArgs a)
{
    __shared__ RegSmem sm;
    constexpr int VEC = Vec<T>::n;
    const int b = blockIdx.x, tid = threadIdx.x, NT = blockDim.x;
    const int lane = tid & 63, wv = tid >> 6, nw = NT >> 6;
    const int m_max = a.m_max, V = a.vocab, nfull = V / VEC;   // rows aligned, V >= VEC (host)
    const size_t m1 = (size_t)m_max + 1;
    const float T_ = a.temperature;
    const bool unit_t = a.unit_t;
    int n = a.num_nodes[b];
    if (n < 0 || n > m_max) {
        if (tid == 0) raise_error(a.err, EAGLE_DEVERR_TREE);
        n = n < 0 ? 0 : m_max;
    }
    // node `lane` of this sequence, in every wave; padding lanes never match a parent
    const int tok = lane < n ? a.tokens[(size_t)b * m_max + lane] : -1;
    const int par = lane < n ? a.parent[(size_t)b * m_max + lane] : -2;
    const uint32_t word = (kSample && lane < n) ? a.words[(size_t)b * m1 + lane] : 0u;
    const uint32_t word_bonus = kSample ? a.words[(size_t)b * m1 + m_max] : 0u;

    int cur = -1, len = 0, bonus = -1;
    int32_t *acc = a.accepted + (size_t)b * a.max_accept;
    for (int step = 0; step <= kMaxMMax; ++step) {
        const T *row = static_cast<const T *>(a.target) + ((size_t)b * m1 + (size_t)(cur + 1)) * (size_t)a.row_stride;
        // the thread index passes through an opaque move each step, so the
        // per-element indices and bounds tests derived from it are recomputed
        // here rather than hoisted out of the walk and held in registers
        int t_ = tid;
        asm volatile("" : "+v"(t_));
        uint4 x[kNV];
#pragma unroll
        for (int j = 0; j < kNV; ++j) x[j] = load_vec_clamped<T>(row, j * NT + t_, nfull);
#pragma unroll
        for (int j = 0; j < kNV; ++j) fix_tail<T>(x[j], row, j * NT + t_, nfull, V);
        const unsigned long long sib = __ballot(par == cur);   // children of the current node
        int next = -1;
        if constexpr (!kSample) {
            // pass A: the row maximum, NaN-propagating (a NaN anywhere makes it NaN)
            float mt = -__builtin_inff();
#pragma unroll
            for (int j = 0; j < kNV; ++j) {
                float f[VEC];
                unpack<T>(x[j], f);
#pragma unroll
                for (int e = 0; e < VEC; ++e) mt = __builtin_elementwise_maximum(mt, f[e]);
            }
            const float M = block_maximum(mt, sm.red);
#pragma unroll
            for (int j = 0; j < kNV; ++j) x[j] = opaque(x[j]);   // unpack again, not keep the floats
            if (M != M) {
                if (tid == 0) raise_error(a.err, EAGLE_DEVERR_NONFINITE_ROW);
                break;
            }
            // pass B, only in threads that hold the maximum (usually one wave):
            // their first element equal to it, scanning positions j*VEC + e
            // downwards; the block minimum of the ids is the first maximum
            int bi = 0x7fffffff;
            if (mt == M) {
                int bp = 0;
#pragma unroll
                for (int j = kNV - 1; j >= 0; --j) {
                    float f[VEC];
                    unpack<T>(x[j], f);
#pragma unroll
                    for (int e = VEC - 1; e >= 0; --e)
                        if (f[e] == M) bp = j * VEC + e;
                }
                bi = ((bp / VEC) * NT + t_) * VEC + bp % VEC;
            }
            bi = block_min_i(bi, sm.red);
            const unsigned long long hit = __ballot(par == cur && tok == bi);
            if (hit) next = __builtin_ctzll(hit);
            else bonus = bi;
        } else {
            // the children's own logits, loaded with the row and weighed once M is known
            const bool kid = (sib >> lane) & 1ull;
            const bool kid_ok = kid && (unsigned)tok < (unsigned)V;
            float lk = 0.0f;
            if (kid_ok) lk = load_scalar<T>(row + tok);
            float lmax = -__builtin_inff();
#pragma unroll
            for (int j = 0; j < kNV; ++j) {
                float f[VEC];
                unpack<T>(x[j], f);
#pragma unroll
                for (int e = 0; e < VEC; ++e) lmax = fmaxf(lmax, f[e]);
            }
            const float M = block_max(lmax, sm.red);
#pragma unroll
            for (int j = 0; j < kNV; ++j) x[j] = opaque(x[j]);   // unpack again, not keep the floats
            // exact weight sums per (vector j, wave), kept for the bonus search;
            // W is their sum (integers below 2^53: exact in any order).  The
            // temperature branch is taken once, outside the element loops.
            auto parts = [&](auto unit) {
#pragma unroll
                for (int j = 0; j < kNV; ++j) {
                    float f[VEC];
                    unpack<T>(x[j], f);
                    double sj = 0.0;
#pragma unroll
                    for (int e = 0; e < VEC; ++e)
                        sj += (double)(decltype(unit)::value ? weight_of(f[e], M) : weight_from_x((f[e] - M) / T_));
                    sj = wave_sum_d(sj);
                    if (lane == 0) sm.part[j * nw + wv] = sj;
                }
            };
            if (unit_t) parts(Flag<true>{});
            else parts(Flag<false>{});
            __syncthreads();
            const int P = kNV * nw;
            double wl = 0.0;
            for (int i = lane; i < P; i += 64) wl += sm.part[i];
            const double W = wave_sum_d(wl);
            if (!__builtin_isfinite(M) || !__builtin_isfinite(W)) {
                if (tid == 0) raise_error(a.err, EAGLE_DEVERR_NONFINITE_ROW);
                break;
            }
#pragma unroll
            for (int j = 0; j < kNV; ++j) x[j] = opaque(x[j]);
            if (kid && !kid_ok && wv == 0) raise_error(a.err, EAGLE_DEVERR_TREE);   // malformed tree: no mass
            // children in index order: child k is accepted iff r_k * R_k < w_k * 2^32,
            // where R_k is W less the masses of the children before k (all rejected
            // if k is the first to pass); a child repeating an earlier child's token
            // carries no mass.  Every child is tested at once; the first pass wins.
            bool gone = false;
            for (unsigned long long left = sib; left; left &= left - 1) {
                const int k = __builtin_ctzll(left);
                gone |= lane > k && tok == __builtin_amdgcn_readlane(tok, k);
            }
            const unsigned long long wk =
                (kid_ok && !gone) ? (unsigned long long)weight_of_t(lk, M, T_, unit_t) : 0ull;
            const unsigned long long ahead = wave_exclusive_scan_u64(wk);
            const unsigned long long Rk = (unsigned long long)W - ahead;
            const bool pass = kid && (unsigned __int128)word * Rk < ((unsigned __int128)wk << 32);
            const unsigned long long passed = __ballot(pass);
            if (passed) next = __builtin_ctzll(passed);
            if (next < 0) {
                // bonus: every child was rejected; R = W less all their masses, and the
                // bonus is the smallest v whose inclusive cumulative residual weight
                // exceeds s = floor(r * R / 2^32).  In ascending v the elements run by
                // vector q, then wave, then lane, then element.
                const unsigned long long R = (unsigned long long)W - readlane_u64(ahead + wk, 63);
                const unsigned long long s = (unsigned long long)(((unsigned __int128)word_bonus * R) >> 32);
                const double sd = (double)s;
                const unsigned long long removed = __ballot(kid_ok && !gone);
                if (tid == 0) sm.bonus = -1;
                if (wv == 0) {
                    // lane l covers parts [l*c, l*c + c), c <= 4, with the removed
                    // tokens' masses taken out of the parts that hold them
                    const int c = (P + 63) / 64;
                    const int lo = min(P, lane * c), hi = min(P, lo + c);
                    double pv[4];
#pragma unroll
                    for (int u = 0; u < 4; ++u) pv[u] = lo + u < hi ? sm.part[lo + u] : 0.0;
                    for (unsigned long long left = removed; left; left &= left - 1) {
                        const int k = __builtin_ctzll(left);
                        const int v = __builtin_amdgcn_readlane(tok, k);
                        const double wv_k = (double)readlane_u64(wk, k);
                        const int gi = v / VEC, idx = (gi / NT) * nw + ((gi % NT) >> 6);
#pragma unroll
                        for (int u = 0; u < 4; ++u)
                            if (idx == lo + u && lo + u < hi) pv[u] -= wv_k;
                    }
                    double mine = 0.0;
#pragma unroll
                    for (int u = 0; u < 4; ++u) mine += pv[u];
                    const double before = wave_exclusive_scan_d(mine);
                    const bool here = before <= sd && sd < before + mine;
                    if (__ballot(here) == 0ull && lane == 0) sm.qw = -1;
                    if (here) {
                        double cum = before;
#pragma unroll
                        for (int u = 0; u < 4; ++u) {
                            if (lo + u < hi && sd < cum + pv[u]) { sm.qw = lo + u; sm.before = cum; break; }
                            cum += pv[u];
                        }
                    }
                }
                __syncthreads();
                const int qw = sm.qw;
                if (qw >= 0 && wv == qw % nw) {
                    const int qs = qw / nw;
                    float f[VEC];
#pragma unroll
                    for (int j = 0; j < kNV; ++j)
                        if (j == qs) unpack<T>(x[j], f);
                    // this lane's removed elements of vector qs
                    unsigned gone_e = 0u;
                    for (unsigned long long left = removed; left; left &= left - 1) {
                        const int k = __builtin_ctzll(left);
                        const int v = __builtin_amdgcn_readlane(tok, k);
                        if (v / VEC == qs * NT + t_) gone_e |= 1u << (v % VEC);
                    }
                    double mine = 0.0;
#pragma unroll
                    for (int e = 0; e < VEC; ++e)
                        if (!((gone_e >> e) & 1u)) mine += (double)weight_of_t(f[e], M, T_, unit_t);
                    const double before = sm.before + wave_exclusive_scan_d(mine);
                    if (before <= sd && sd < before + mine) {
                        double cum = before;
                        for (int e = 0; e < VEC; ++e) {
                            if ((gone_e >> e) & 1u) continue;
                            cum += (double)weight_of_t(f[e], M, T_, unit_t);
                            if (cum > sd) { sm.bonus = (qs * NT + t_) * VEC + e; break; }
                        }
                    }
                }
                __syncthreads();
                bonus = sm.bonus;
            }
        }
        if (next < 0) break;
        if (len >= a.max_accept) {
            if (tid == 0) raise_error(a.err, EAGLE_DEVERR_PATH);
            break;
        }
        if (tid == 0) acc[len] = next;
        ++len;
        cur = next;
    }
    for (int j = len + tid; j < a.max_accept; j += NT) acc[j] = -1;
    if (tid == 0) {
        a.accept_len[b] = len;
        a.bonus[b] = bonus;
    }
}

// ---------------------------------------------------------------------------
// Greedy acceptance for small batches: the argmax of every row a walk could
// visit (row 0 and the rows of the sequence's nodes) is computed in parallel,
// one workgroup per row; a second kernel walks each tree over those argmaxes.
// ---------------------------------------------------------------------------
template <typename T>
// One part of one row: the first maximum (value desc, id asc) of entries
// [part * span, (part + 1) * span); span is a multiple of 8 entries, so every
// part starts 16-byte aligned where the row does.  Rows past a sequence's
// node count are skipped.
__global__ __launch_bounds__(1024) void k_row_argmax(AcceptArgs a, int2 *g, int parts, int span)
{
    __shared__ BlockScratch red;
    const int m1 = a.m_max + 1;
    const int r = blockIdx.x / parts, part = blockIdx.x - r * parts;
    const int b = r / m1, u = r - b * m1;
    int n = a.num_nodes[b];
    n = n < 0 ? 0 : (n > a.m_max ? a.m_max : n);
    if (u > n) return;
    const int lo = part * span, hi = min(a.vocab, lo + span);
    const T *row = static_cast<const T *>(a.target) + ((size_t)b * m1 + u) * (size_t)a.row_stride + lo;
    float bv = -__builtin_inff();
    int bi = 0x7fffffff;
    bool nan = false;
    if (lo < hi)
        for_each_elem<T>(row, hi - lo, a.vec_ok, [&](float f, int id) {
            nan |= (f != f);
            if (before(f, lo + id, bv, bi)) { bv = f; bi = lo + id; }
        });
    if (__any(nan) && (threadIdx.x & 63) == 0) raise_error(a.err, EAGLE_DEVERR_NONFINITE_ROW);
    block_best(bv, bi, red);
    if (threadIdx.x == 0) g[(size_t)r * parts + part] = make_int2(__float_as_int(bv), bi);
}

__global__ __launch_bounds__(64) void k_greedy_walk(AcceptArgs a, const int2 *g, int parts)
{
    // one wave per sequence; lane i holds node i (m_max <= 64), and the child
    // whose token matches the current argmax is found by a ballot
    __shared__ int gs[kMaxMMax + 1];
    const int b = blockIdx.x, lane = threadIdx.x, m_max = a.m_max;
    int n = a.num_nodes[b];
    if (n < 0 || n > m_max) {
        if (lane == 0) raise_error(a.err, EAGLE_DEVERR_TREE);
        n = n < 0 ? 0 : m_max;
    }
    const int tok = lane < n ? a.tokens[(size_t)b * m_max + lane] : -1;
    const int par = lane < n ? a.parent[(size_t)b * m_max + lane] : -2;
    // each row's argmax: the first of its parts' maxima in (value desc, id asc)
    for (int u = lane; u <= n; u += 64) {
        const int2 *pr = g + ((size_t)b * (m_max + 1) + u) * parts;
        float bv = -__builtin_inff();
        int bi = 0x7fffffff;
        for (int q = 0; q < parts; ++q) {
            const int2 e = pr[q];
            if (before(__int_as_float(e.x), e.y, bv, bi)) { bv = __int_as_float(e.x); bi = e.y; }
        }
        gs[u] = bi;
    }
    __syncthreads();
    int32_t *acc = a.accepted + (size_t)b * a.max_accept;
    int cur = -1, len = 0, bonus = -1;
    while (true) {
        const int gg = gs[cur + 1];
        const unsigned long long hit = __ballot(par == cur && tok == gg);
        if (!hit) { bonus = gg; break; }
        const int next = __builtin_ctzll(hit);
        if (len >= a.max_accept) {
            if (lane == 0) raise_error(a.err, EAGLE_DEVERR_PATH);
            break;
        }
        if (lane == 0) acc[len] = next;
        ++len;
        cur = next;
    }
    for (int j = len + lane; j < a.max_accept; j += 64) acc[j] = -1;
    if (lane == 0) {
        a.accept_len[b] = len;
        a.bonus[b] = bonus;
    }
}

// rows below which greedy acceptance reads every row in parallel
constexpr int kParallelGreedyRows = 512;

// parts per row of the parallel greedy argmax: at least 4096 entries each,
// at most 8 (each part is one workgroup; a row of 32000 bf16 entries takes 7)
static int argmax_parts(int vocab) { return vocab / 4096 < 1 ? 1 : (vocab / 4096 > 8 ? 8 : vocab / 4096); }
static int argmax_span(int vocab, int parts) { return ((vocab + parts - 1) / parts + 7) / 8 * 8; }

size_t accept_layout_bytes(const eagle_accept_params *p, int32_t batch)
{
    size_t o = kWsHeader;
    if (p && p->mode == EAGLE_ACCEPT_GREEDY && (size_t)batch * (p->m_max + 1) <= (size_t)kParallelGreedyRows)
        o = align_up(o + (size_t)batch * (p->m_max + 1) * argmax_parts(p->vocab) * sizeof(int2), 256);
    return o;
}

hipError_t launch_accept(const eagle_accept_params *p, int32_t batch, const void *target,
                         eagle_dtype dt, int64_t row_stride, const int32_t *tokens,
                         const int32_t *parent, const int32_t *num_nodes, const uint32_t *words,
                         int32_t *accepted, int32_t *accept_len, int32_t *bonus, uint32_t *err,
                         hipStream_t st)
{
    if (batch <= 0) return hipSuccess;
    AcceptArgs a;
    a.target = target;
    a.row_stride = row_stride;
    a.m_max = p->m_max;
    a.vocab = p->vocab;
    a.max_accept = p->max_accept;
    a.mode = p->mode;
    a.temperature = p->temperature;
    a.unit_t = p->temperature == 1.0f;
    const size_t esz = dt == EAGLE_F32 ? 4 : 2;
    a.vec_ok = ((uintptr_t)target % 16 == 0) && ((size_t)row_stride * esz % 16 == 0);
    a.tokens = tokens;
    a.parent = parent;
    a.num_nodes = num_nodes;
    a.words = words;
    a.accepted = accepted;
    a.accept_len = accept_len;
    a.bonus = bonus;
    a.err = err;
    const int vec = dt == EAGLE_F32 ? 4 : 8;
    if (p->mode == EAGLE_ACCEPT_GREEDY && (size_t)batch * (p->m_max + 1) <= (size_t)kParallelGreedyRows) {
        const int parts = argmax_parts(p->vocab), span = argmax_span(p->vocab, parts);
        int nt = (span / vec + 63) / 64 * 64;
        nt = nt < 64 ? 64 : (nt > kAcceptThreads ? kAcceptThreads : nt);
        int2 *g = reinterpret_cast<int2 *>(reinterpret_cast<char *>(err) + kWsHeader);
        const dim3 grid((unsigned)(batch * (p->m_max + 1) * parts));
        if (dt == EAGLE_F32)
            hipLaunchKernelGGL(k_row_argmax<float>, grid, dim3(nt), 0, st, a, g, parts, span);
        else
            hipLaunchKernelGGL(k_row_argmax<uint16_t>, grid, dim3(nt), 0, st, a, g, parts, span);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(k_greedy_walk, dim3(batch), dim3(64), 0, st, a, (const int2 *)g, parts);
        return hipGetLastError();
    }
    // register-resident walk: kNV vectors per thread, the fewest threads that hold the row
    const int nvec = (p->vocab + vec - 1) / vec;
    int knv = 1;
    while (knv < kRegMaxVectors && knv * kAcceptThreads < nvec) knv *= 2;
    if (a.vec_ok && p->vocab >= vec && knv * kAcceptThreads >= nvec) {
        int nt = ((nvec + knv - 1) / knv + 63) / 64 * 64;
        nt = nt < 64 ? 64 : nt;
        const dim3 grid((unsigned)batch), block((unsigned)nt);
        const bool sample = p->mode != EAGLE_ACCEPT_GREEDY;
#define EAGLE_ACCEPT_REG(KNV)                                                                    \
    case KNV:                                                                                    \
        if (dt == EAGLE_F32) {                                                                   \
            if (sample) hipLaunchKernelGGL((k_accept_reg<float, KNV, true>), grid, block, 0, st, a); \
            else hipLaunchKernelGGL((k_accept_reg<float, KNV, false>), grid, block, 0, st, a);   \
        } else {                                                                                 \
            if (sample) hipLaunchKernelGGL((k_accept_reg<uint16_t, KNV, true>), grid, block, 0, st, a); \
            else hipLaunchKernelGGL((k_accept_reg<uint16_t, KNV, false>), grid, block, 0, st, a); \
        }                                                                                        \
        break;
        switch (knv) {
            EAGLE_ACCEPT_REG(1)
            EAGLE_ACCEPT_REG(2)
            EAGLE_ACCEPT_REG(4)
            EAGLE_ACCEPT_REG(8)
            EAGLE_ACCEPT_REG(16)
        }
#undef EAGLE_ACCEPT_REG
        return hipGetLastError();
    }
    // unaligned rows, rows shorter than one vector, and rows longer than 16
    // vectors per thread (fp32 beyond 65536 entries): looping walk
    int nt = (p->vocab / vec + 63) / 64 * 64;
    nt = nt < 64 ? 64 : (nt > kAcceptThreads ? kAcceptThreads : nt);
    if (dt == EAGLE_F32)
        hipLaunchKernelGGL(k_accept<float>, dim3(batch), dim3(nt), 0, st, a);
    else
        hipLaunchKernelGGL(k_accept<uint16_t>, dim3(batch), dim3(nt), 0, st, a);
    return hipGetLastError();
}

}  // namespace eagle
