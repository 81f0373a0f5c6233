// accept.hip -- acceptance walk over the verified tree (EAGLE-1 explainer,
// "Verification"; EAGLE-2 explainer, "Key contributions": lossless by
// rejection sampling).  One workgroup per sequence walks from the root; each
// step reads one target row (the current node's) once from HBM into registers.
#include "common.h"
#include "internal.h"

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

template <typename T> struct AVec;
template <> struct AVec<float> { static constexpr int n = 4; };
template <> struct AVec<uint16_t> { static constexpr int n = 8; };

template <typename T> __device__ __forceinline__ float ld1(const T *p);
template <> __device__ __forceinline__ float ld1<float>(const float *p) { return *p; }
template <> __device__ __forceinline__ float ld1<uint16_t>(const uint16_t *p) { return bf16_to_f32(*p); }

template <typename T>
__device__ __forceinline__ void unpack_a(const uint4 &u, float *o);
template <> __device__ __forceinline__ void unpack_a<float>(const uint4 &u, float *o)
{
    o[0] = __uint_as_float(u.x); o[1] = __uint_as_float(u.y);
    o[2] = __uint_as_float(u.z); o[3] = __uint_as_float(u.w);
}
template <> __device__ __forceinline__ void unpack_a<uint16_t>(const uint4 &u, float *o)
{
    o[0] = bf16_lo(u.x); o[1] = bf16_hi(u.x); o[2] = bf16_lo(u.y); o[3] = bf16_hi(u.y);
    o[4] = bf16_lo(u.z); o[5] = bf16_hi(u.z); o[6] = bf16_lo(u.w); o[7] = bf16_hi(u.w);
}

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
    constexpr int VEC = AVec<T>::n;
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
                unpack_a<T>(u[q], f);
#pragma unroll
                for (int e = 0; e < VEC; ++e) fn(f[e], j * VEC + e);
            }
        }
    }
    for (int v = nvec * VEC + tid; v < V; v += NT) fn(ld1<T>(row + v), v);
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
                        sm.wchild[i] = (double)weight_of_t(ld1<T>(row + t), M, a.temperature, a.unit_t);
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
                for (int v = lo; v < hi; ++v) mine += (double)weight_of_t(ld1<T>(row + v), M, a.temperature, a.unit_t);
                for (int j = 0; j < nrem; ++j) {
                    const int t = sm.removed[j];
                    if (t >= lo && t < hi) mine -= (double)weight_of_t(ld1<T>(row + t), M, a.temperature, a.unit_t);
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
                        cum += (double)weight_of_t(ld1<T>(row + v), M, a.temperature, a.unit_t);
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
// Greedy acceptance for small batches: the argmax of every row a walk could
// visit (row 0 and the rows of the sequence's nodes) is computed in parallel,
// one workgroup per row; a second kernel walks each tree over those argmaxes.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(1024) void k_row_argmax(AcceptArgs a, int32_t *g)
{
    __shared__ BlockScratch red;
    const int m1 = a.m_max + 1;
    const int b = blockIdx.x / m1, u = blockIdx.x % m1;
    int n = a.num_nodes[b];
    n = n < 0 ? 0 : (n > a.m_max ? a.m_max : n);
    if (u > n) return;
    const T *row = static_cast<const T *>(a.target) + ((size_t)b * m1 + u) * (size_t)a.row_stride;
    float bv = -__builtin_inff();
    int bi = 0x7fffffff;
    bool nan = false;
    for_each_elem<T>(row, a.vocab, a.vec_ok, [&](float f, int id) {
        nan |= (f != f);
        if (before(f, id, bv, bi)) { bv = f; bi = id; }
    });
    if (__any(nan) && (threadIdx.x & 63) == 0) raise_error(a.err, EAGLE_DEVERR_NONFINITE_ROW);
    block_best(bv, bi, red);
    if (threadIdx.x == 0) g[(size_t)b * m1 + u] = bi;
}

__global__ __launch_bounds__(64) void k_greedy_walk(AcceptArgs a, const int32_t *g)
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
    for (int u = lane; u <= n; u += 64) gs[u] = g[(size_t)b * (m_max + 1) + u];
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

size_t accept_layout_bytes(const eagle_accept_params *p, int32_t batch)
{
    size_t o = kWsHeader;
    if (p && p->mode == EAGLE_ACCEPT_GREEDY && (size_t)batch * (p->m_max + 1) <= (size_t)kParallelGreedyRows)
        o = align_up(o + (size_t)batch * (p->m_max + 1) * sizeof(int32_t), 256);
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
    int nt = (p->vocab / vec + 63) / 64 * 64;
    nt = nt < 64 ? 64 : (nt > kAcceptThreads ? kAcceptThreads : nt);
    if (p->mode == EAGLE_ACCEPT_GREEDY && (size_t)batch * (p->m_max + 1) <= (size_t)kParallelGreedyRows) {
        int32_t *g = reinterpret_cast<int32_t *>(reinterpret_cast<char *>(err) + kWsHeader);
        const dim3 grid((unsigned)(batch * (p->m_max + 1)));
        if (dt == EAGLE_F32)
            hipLaunchKernelGGL(k_row_argmax<float>, grid, dim3(nt), 0, st, a, g);
        else
            hipLaunchKernelGGL(k_row_argmax<uint16_t>, grid, dim3(nt), 0, st, a, g);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(k_greedy_walk, dim3(batch), dim3(64), 0, st, a, (const int32_t *)g);
        return hipGetLastError();
    }
    if (dt == EAGLE_F32)
        hipLaunchKernelGGL(k_accept<float>, dim3(batch), dim3(nt), 0, st, a);
    else
        hipLaunchKernelGGL(k_accept<uint16_t>, dim3(batch), dim3(nt), 0, st, a);
    return hipGetLastError();
}

}  // namespace eagle
