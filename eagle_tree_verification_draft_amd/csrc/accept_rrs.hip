// accept_rrs.hip -- recursive rejection sampling over children drawn from the
// draft (EAGLE-1 explainer, "Verification": a draft token is accepted by the
// ratio of the target and draft distributions, a rejection discards the rest
// and resamples, and the emitted tokens follow the target distribution).
//
// At node u with target weights P (row u + 1 at temperature T, Spec S
// integers, sum SP) and draft weights Q (u's own draft row, temperature 1,
// sum SQ), the children x are tested in draw order:
//   accept iff floor(r_x Q(x) SP / 2^32) < P(x) SQ      (u < p(x) / q(x));
//   else   P <- max(0, P SQ - Q SP) >> s  (the residual max(0, p - q) over the
//          common denominator, shifted to keep its sum below 2^52), and
//          Q(x) <- 0 (q renormalised without x);
// a child with Q(x) = 0 is rejected and changes nothing, and a residual that
// sums to 0 leaves P as it was.  With no child accepted the bonus is the
// inverse-CDF draw from P with the word r_{m_max}.
//
// One workgroup per sequence.  The row maxima take coalesced 16-byte
// vectors; the weight and residual passes one element per lane, so that the
// 64-bit stores coalesce too; the bonus scan sums 64-token segments, scans
// the segment sums, then one segment.  P lives in the workspace (two buffers per
// sequence: a residual is written beside the current P and taken only if it
// is not all zero).  Q is written once per node to a third buffer, and a
// rejected child's entry is set to 0 there, so the residual passes read Q
// instead of recomputing the exact weights.
#include "common.h"
#include "internal.h"
#include "rowvec.h"

namespace eagle {

namespace {

constexpr int kRrsThreads = 1024;

struct RrsSmem {
    unsigned long long part[16];
    float fmax[16];
    int tok[kMaxMMax], par[kMaxMMax], srow[kMaxMMax];
    int removed[kMaxMMax];   // tokens taken out of q at the current node
    unsigned long long seg[kMaxVocab / 64];   // sums of 64-token segments of P
    unsigned long long pick_base;
    int pick, pick_seg;
};

__device__ __forceinline__ unsigned long long rrs_sum(unsigned long long v, RrsSmem &sm)
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

__device__ __forceinline__ float rrs_max(float v, RrsSmem &sm)
{
    const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    __syncthreads();
    if ((threadIdx.x & 63) == 0) sm.fmax[w] = v;
    __syncthreads();
    float r = sm.fmax[0];
    for (int j = 1; j < nw; ++j) r = fmaxf(r, sm.fmax[j]);
    return r;
}

__device__ __forceinline__ unsigned long long rrs_exclusive(unsigned long long v, RrsSmem &sm)
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

__device__ __forceinline__ int bitlen_u128(unsigned __int128 x)
{
    const unsigned long long hi = (unsigned long long)(x >> 64), lo = (unsigned long long)x;
    return hi ? 128 - __clzll(hi) : (lo ? 64 - __clzll(lo) : 0);
}

}  // namespace

struct RrsArgs {
    const void *target, *draft;
    int64_t t_stride, d_stride;
    int m_max, vocab, max_accept, r_max;
    float temperature;
    bool unit_t, t_vec_ok, d_vec_ok;
    const int32_t *tokens, *parent, *src_row, *num_nodes;
    const uint32_t *words;
    int32_t *accepted, *accept_len, *bonus;
    unsigned long long *pbuf;   // [batch][3][vocab]: P, the next P, Q
    uint32_t *err;
};

template <typename T>
__global__ __launch_bounds__(kRrsThreads) void k_accept_rrs(RrsArgs a)
{
    __shared__ RrsSmem sm;
    constexpr int VEC = Vec<T>::n;
    const int b = blockIdx.x, tid = threadIdx.x, NT = blockDim.x, V = a.vocab, m_max = a.m_max;
    // the maxima take 16-byte vectors j = tid + i NT, the weights and
    // residuals one element v = tid + i NT per lane (all coalesced)
    int n = a.num_nodes[b];
    if (n < 0 || n > m_max) {
        if (tid == 0) raise_error(a.err, EAGLE_DEVERR_TREE);
        n = n < 0 ? 0 : m_max;
    }
    for (int i = tid; i < n; i += NT) {
        sm.tok[i] = a.tokens[(size_t)b * m_max + i];
        sm.par[i] = a.parent[(size_t)b * m_max + i];
        sm.srow[i] = a.src_row[(size_t)b * m_max + i];
    }
    __syncthreads();
    const uint32_t *rw = a.words + (size_t)b * (m_max + 1);
    unsigned long long *P = a.pbuf + (size_t)b * 3 * V, *Pn = P + V, *Qw = P + 2 * V;
    int32_t *acc = a.accepted + (size_t)b * a.max_accept;
    int cur = -1, len = 0, bonus = -1;
    while (true) {
        // ---- target weights of node `cur` ----
        const T *trow = static_cast<const T *>(a.target) + ((size_t)b * (m_max + 1) + (size_t)(cur + 1)) * a.t_stride;
        float lmax = -__builtin_inff();
#pragma unroll 4
        for (int j = tid; j * VEC < V; j += NT) {
            float f[VEC];
            unpack<T>(load_vec<T>(trow, j * VEC, V, a.t_vec_ok), f);
#pragma unroll
            for (int e = 0; e < VEC; ++e) lmax = fmaxf(lmax, f[e]);
        }
        const float M = rrs_max(lmax, sm);
        if (!__builtin_isfinite(M)) {
            if (tid == 0) raise_error(a.err, EAGLE_DEVERR_NONFINITE_ROW);
            break;
        }
        // weights with one element per lane, so that the 64-bit stores coalesce
        // (the temperature test is taken outside the loop: the division is
        // computed only where it is used)
        unsigned long long own = 0;
        if (a.unit_t) {
#pragma unroll 8
            for (int v = tid; v < V; v += NT) {
                const unsigned long long w = (unsigned long long)weight_of(load_scalar<T>(trow + v), M);
                P[v] = w;
                own += w;
            }
        } else {
#pragma unroll 8
            for (int v = tid; v < V; v += NT) {
                const unsigned long long w =
                    (unsigned long long)weight_of_t(load_scalar<T>(trow + v), M, a.temperature, false);
                P[v] = w;
                own += w;
            }
        }
        unsigned long long SP = rrs_sum(own, sm);
        if (SP == 0) {
            if (tid == 0) raise_error(a.err, EAGLE_DEVERR_NONFINITE_ROW);
            break;
        }
        bool has_children = false;
        for (int x = 0; x < n; ++x) has_children |= sm.par[x] == cur;
        int next = -1;
        if (has_children) {
            const int dr = cur < 0 ? 0 : sm.srow[cur];
            if (dr < 0 || dr >= a.r_max) {
                if (tid == 0) raise_error(a.err, EAGLE_DEVERR_TREE);
                break;
            }
            const T *drow = static_cast<const T *>(a.draft) + ((size_t)b * a.r_max + dr) * a.d_stride;
            float dmax = -__builtin_inff();
#pragma unroll 4
            for (int j = tid; j * VEC < V; j += NT) {
                float f[VEC];
                unpack<T>(load_vec<T>(drow, j * VEC, V, a.d_vec_ok), f);
#pragma unroll
                for (int e = 0; e < VEC; ++e) dmax = fmaxf(dmax, f[e]);
            }
            const float Md = rrs_max(dmax, sm);
            if (!__builtin_isfinite(Md)) {
                if (tid == 0) raise_error(a.err, EAGLE_DEVERR_NONFINITE_ROW);
                break;
            }
            unsigned long long qown = 0;
#pragma unroll 8
            for (int v = tid; v < V; v += NT) {
                const unsigned long long w = (unsigned long long)weight_of(load_scalar<T>(drow + v), Md);
                Qw[v] = w;
                qown += w;
            }
            unsigned long long SQ = rrs_sum(qown, sm);
            int nrem = 0;
            for (int x = 0; x < n && next < 0; ++x) {
                if (sm.par[x] != cur) continue;
                const int t = sm.tok[x];
                if (t < 0 || t >= V) {
                    if (tid == 0) raise_error(a.err, EAGLE_DEVERR_TREE);
                    continue;
                }
                bool gone = false;
                for (int j = 0; j < nrem; ++j) gone |= sm.removed[j] == t;
                const unsigned long long q = gone ? 0ull : (unsigned long long)weight_of(load_scalar<T>(drow + t), Md);
                if (q == 0) continue;
                const unsigned long long pt = P[t];
                if ((((unsigned __int128)rw[x] * q * SP) >> 32) < (unsigned __int128)pt * SQ) {
                    next = x;
                    break;
                }
                // residual max(0, p - q) over SP * SQ, shifted below 2^52 in sum
                const int bl = bitlen_u128((unsigned __int128)SP * SQ), sh = bl > 52 ? bl - 52 : 0;
                unsigned long long rown = 0;
#pragma unroll 8
                for (int v = tid; v < V; v += NT) {
                    // both products are below 2^105, so a negative difference
                    // sets the top bit; sh < 64 and the shifted value fits in 64 bits
                    const unsigned __int128 df = (unsigned __int128)P[v] * SQ - (unsigned __int128)Qw[v] * SP;
                    const unsigned long long lo = (unsigned long long)df, hi = (unsigned long long)(df >> 64);
                    const unsigned long long d = (long long)hi < 0 ? 0ull : (lo >> sh) | ((hi << 1) << (63 - sh));
                    Pn[v] = d;
                    rown += d;
                }
                const unsigned long long SPn = rrs_sum(rown, sm);
                if (SPn > 0) {
                    unsigned long long *tmp = P;
                    P = Pn;
                    Pn = tmp;
                    SP = SPn;
                }
                if (tid == 0) {
                    sm.removed[nrem] = t;
                    Qw[t] = 0;
                }
                ++nrem;
                SQ -= q;
                __syncthreads();   // the removed list and Q(t) = 0
            }
        }
        if (next < 0) {
            // bonus: inverse CDF of P.  Segments of 64 tokens are summed by
            // waves (coalesced), a block scan over the segment sums finds the
            // segment holding the draw, and one wave scans inside it.
            const unsigned long long s = (unsigned long long)(((unsigned __int128)rw[m_max] * SP) >> 32);
            const int lane = tid & 63, wv = tid >> 6, nw = NT >> 6, nseg = (V + 63) / 64;
            for (int g = wv; g < nseg; g += nw) {
                const int v = g * 64 + lane;
                unsigned long long x = v < V ? P[v] : 0ull;
#pragma unroll
                for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
                if (lane == 0) sm.seg[g] = x;
            }
            if (tid == 0) {
                sm.pick = -1;
                sm.pick_seg = 0;
                sm.pick_base = 0;
            }
            __syncthreads();
            const int sper = (nseg + NT - 1) / NT;
            const int s_lo = min(nseg, tid * sper), s_hi = min(nseg, s_lo + sper);
            unsigned long long sown = 0;
            for (int g = s_lo; g < s_hi; ++g) sown += sm.seg[g];
            const unsigned long long excl = rrs_exclusive(sown, sm);
            if (excl <= s && s < excl + sown) {
                unsigned long long cum = excl;
                for (int g = s_lo; g < s_hi; ++g) {
                    if (s < cum + sm.seg[g]) {
                        sm.pick_seg = g;
                        sm.pick_base = cum;
                        break;
                    }
                    cum += sm.seg[g];
                }
            }
            __syncthreads();
            if (wv == 0) {
                const int g = sm.pick_seg, v = g * 64 + lane;
                unsigned long long incl = v < V ? P[v] : 0ull;
#pragma unroll
                for (int o = 1; o < 64; o <<= 1) {
                    const unsigned long long t = __shfl_up(incl, o);
                    if (lane >= o) incl += t;
                }
                const unsigned long long hit = __ballot(sm.pick_base + incl > s);
                if (lane == 0 && hit) sm.pick = g * 64 + __ffsll((long long)hit) - 1;
            }
            __syncthreads();
            bonus = sm.pick;
            break;
        }
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

size_t accept_rrs_layout_bytes(const eagle_accept_params *p, int32_t batch)
{
    return kWsHeader + align_up((size_t)batch * 3 * (size_t)p->vocab * sizeof(unsigned long long), 256);
}

hipError_t launch_accept_rrs(const eagle_accept_params *p, int32_t batch, const void *target, const void *draft,
                             eagle_dtype dt, int64_t t_stride, int64_t d_stride, int32_t r_max,
                             const int32_t *tokens, const int32_t *parent, const int32_t *src_row,
                             const int32_t *num_nodes, const uint32_t *words, int32_t *accepted,
                             int32_t *accept_len, int32_t *bonus, void *ws, hipStream_t st)
{
    RrsArgs a;
    a.target = target;
    a.draft = draft;
    a.t_stride = t_stride;
    a.d_stride = d_stride;
    a.m_max = p->m_max;
    a.vocab = p->vocab;
    a.max_accept = p->max_accept;
    a.r_max = r_max;
    a.temperature = p->temperature;
    a.unit_t = p->temperature == 1.0f;
    const size_t esz = dt == EAGLE_F32 ? 4 : 2;
    a.t_vec_ok = ((uintptr_t)target % 16 == 0) && ((size_t)t_stride * esz % 16 == 0);
    a.d_vec_ok = ((uintptr_t)draft % 16 == 0) && ((size_t)d_stride * esz % 16 == 0);
    a.tokens = tokens;
    a.parent = parent;
    a.src_row = src_row;
    a.num_nodes = num_nodes;
    a.words = words;
    a.accepted = accepted;
    a.accept_len = accept_len;
    a.bonus = bonus;
    a.err = static_cast<uint32_t *>(ws);
    a.pbuf = reinterpret_cast<unsigned long long *>(static_cast<char *>(ws) + kWsHeader);
    int nt = ((p->vocab + 7) / 8 + 63) / 64 * 64;
    nt = nt < 64 ? 64 : (nt > kRrsThreads ? kRrsThreads : nt);
    if (dt == EAGLE_F32)
        hipLaunchKernelGGL(k_accept_rrs<float>, dim3((unsigned)batch), dim3(nt), 0, st, a);
    else
        hipLaunchKernelGGL(k_accept_rrs<uint16_t>, dim3((unsigned)batch), dim3(nt), 0, st, a);
    return hipGetLastError();
}

}  // namespace eagle
