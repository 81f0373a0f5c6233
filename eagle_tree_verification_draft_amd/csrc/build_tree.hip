// build_tree.hip -- dynamic draft tree construction (EAGLE-2 explainer,
// "Dynamic draft tree construction"): per-row softmax statistics and top-C
// children (kernel 1), then per-sequence expansion, rerank and compaction
// (kernel 2).
#include "common.h"
#include "internal.h"

namespace eagle {

// ---------------------------------------------------------------------------
// Kernel 1: one workgroup per draft row.  The row is read once from HBM with
// 16-byte loads (coalesced across the workgroup) and kept in registers:
//   M = row max; W = sum of exact integer weights (fp64, exact in any order);
//   top-C by (logit desc, id asc): every top-C element is >= T, where T is the
//   largest over waves of the C-th largest lane maximum in that wave (C lanes
//   of that wave hold an element >= T, so the C-th largest of the row is >= T).
//   Elements >= T are appended to an LDS list during the weight pass and
//   ranked there.  If more than kCandCap qualify (heavy ties), C rounds of
//   block argmax over the row select exactly.
// ---------------------------------------------------------------------------
constexpr int kCandCap = 2048;

// threads per row: up to 1024 while a row fits 8 vectors per thread, 512 above
template <int kNV> struct RowMaxThreads { static constexpr int n = kNV <= 8 ? 1024 : 512; };

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

// Loads this thread's part of a row: vector j holds elements [(j*NT + tid)*VEC, +VEC).
// Missing elements read as -inf (never a candidate, weight 0).
template <typename T, int kNV>
__device__ __forceinline__ void load_row(const T *row, int V, bool vec_ok, uint4 (&x)[kNV])
{
    constexpr int VEC = Vec<T>::n;
    const int NT = blockDim.x, tid = threadIdx.x;
#pragma unroll
    for (int j = 0; j < kNV; ++j) {
        const int base = (j * NT + tid) * VEC;
        if (vec_ok && base + VEC <= V) {
            x[j] = ld16_stream(row + base);
        } else {
            float f[8];
#pragma unroll
            for (int e = 0; e < VEC; ++e)
                f[e] = (base + e < V) ? load_scalar<T>(row + base + e) : -__builtin_inff();
            if constexpr (VEC == 4) {
                x[j] = make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                                  __float_as_uint(f[3]));
            } else {
                // re-pack to bf16 pairs (values came from bf16, so truncation is exact)
                uint32_t w[4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    w[e] = (__float_as_uint(f[2 * e]) >> 16) | (__float_as_uint(f[2 * e + 1]) & 0xffff0000u);
                x[j] = make_uint4(w[0], w[1], w[2], w[3]);
            }
        }
    }
}

struct RowStatsSmem {
    BlockScratch red;
    float cand_v[kCandCap + 16];   // +16: segment reads may run past the count
    int cand_i[kCandCap + 16];
    int rank[kCandCap];
    int sel[kMaxChildren];
    float thr[16];
    int count;
};

template <typename T, int kNV>
__global__ __launch_bounds__(RowMaxThreads<kNV>::n) void k_row_stats(RowStatsArgs a)
{
    constexpr int VEC = Vec<T>::n;
    __shared__ RowStatsSmem sm;
    const int b = blockIdx.x / a.r_max, r = blockIdx.x % a.r_max;
    const int kind = a.kind ? a.kind[b] : EAGLE_TREE_DYNAMIC;
    const int rows_needed = kind == EAGLE_TREE_CHAIN ? a.chain_k : a.rows_dyn;
    if (r >= rows_needed) return;
    const int C = kind == EAGLE_TREE_CHAIN ? 1 : a.children;
    const int V = a.vocab, NT = blockDim.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const T *row = static_cast<const T *>(a.logits) + ((size_t)b * a.r_max + r) * (size_t)a.row_stride;

    uint4 x[kNV];
    load_row<T, kNV>(row, V, a.vec_ok, x);

    // row max and per-lane max
    // (the max pass unpacks opaque copies so that the unpacked values are not
    // kept live until the weight pass)
    float lmax = -__builtin_inff();
#pragma unroll
    for (int j = 0; j < kNV; ++j) {
        float f[VEC];
        unpack<T>(opaque(x[j]), f);
#pragma unroll
        for (int e = 0; e < VEC; ++e) lmax = fmaxf(lmax, f[e]);
        if constexpr (kNV > 16) __builtin_amdgcn_sched_barrier(0);
    }
    const float M = block_max(lmax, sm.red);

    // threshold: C-th largest lane max of this wave (bitonic sort, descending)
    float s = lmax;
#pragma unroll
    for (int k = 2; k <= 64; k <<= 1) {
#pragma unroll
        for (int j = k >> 1; j > 0; j >>= 1) {
            const float o = __shfl_xor(s, j);
            const bool keep_max = ((lane & j) == 0) == ((lane & k) == 0);
            s = keep_max ? fmaxf(s, o) : fminf(s, o);
        }
    }
    const float tw = __shfl(s, C - 1);
    if (lane == 0) sm.thr[wv] = tw;
    __syncthreads();
    float thr = sm.thr[0];
    for (int j = 1; j < (NT >> 6); ++j) thr = fmaxf(thr, sm.thr[j]);

    // exact weight sum; elements >= thr are appended to the LDS candidate list
    // (their order there is irrelevant: ranking is by (value, id)).  With
    // thr == -inf (fewer than C lanes per wave hold data) the exact fallback runs.
    if (tid == 0) sm.count = 0;
    __syncthreads();
    const bool use_list = thr != -__builtin_inff();
    double wsum = 0.0;
#pragma unroll
    for (int j = 0; j < kNV; ++j) {
        float f[VEC];
        unpack<T>(x[j], f);
        const int base = (j * NT + tid) * VEC;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            wsum += (double)weight_of(f[e], M);
            if (f[e] >= thr) {
                const int o = atomicAdd(&sm.count, 1);
                if (o < kCandCap) { sm.cand_v[o] = f[e]; sm.cand_i[o] = base + e; }
            }
        }
        if constexpr (kNV > 16) __builtin_amdgcn_sched_barrier(0);
    }
    const double W = block_sum_d(wsum, sm.red);   // contains barriers: the list is complete
    const int total = sm.count;

    if (tid < kMaxChildren) sm.sel[tid] = 0;
    if (use_list && total <= kCandCap) {
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
            const int i = sm.sel[tid];
            const size_t o2 = ((size_t)b * a.r_max + r) * a.children + tid;
            a.top_id[o2] = sm.cand_i[i];
            a.top_w[o2] = (double)weight_of(sm.cand_v[i], M);
        }
    } else {
        // heavy ties or thr == -inf: C rounds of "best element after the
        // previous pick", re-reading the row (rare; exact for any input)
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
            if (tid == 0) {
                const size_t o2 = ((size_t)b * a.r_max + r) * a.children + c;
                a.top_id[o2] = bi;
                a.top_w[o2] = (double)weight_of(bv, M);
            }
            pv = bv;
            pi = bi;
        }
    }
    if (tid == 0) {
        const size_t ro = (size_t)b * a.r_max + r;
        a.M[ro] = M;
        a.W[ro] = W;
        if (!__builtin_isfinite(M) || !__builtin_isfinite(W)) raise_error(a.err, EAGLE_DEVERR_NONFINITE_ROW);
    }
}

// ---------------------------------------------------------------------------
// Kernel 2: one workgroup per sequence.  Candidates live in LDS in creation
// order; every confidence c = w / W is computed once, in parallel, up front.
// Depth by depth, one pass of comparisons (split into segments of kSeg, one
// segment per thread, partial counts added with LDS atomics) yields for each
// depth-d candidate its rank among the depth (the top-k are expanded) and the
// number of entries of the running best-m list that precede it, and for each
// entry of that list the number of depth-d candidates that precede it.
// Those counts are the positions of the merged list, which after the last
// depth is the rerank's top-m in rank order.
// ---------------------------------------------------------------------------
struct Key {
    double v;
    int i;
    int pad;
};

struct TreeSmem {
    double V[kMaxCand];
    int tok[kMaxCand];
    int par[kMaxCand];
    int dep[kMaxCand];
    int row[kMaxCand];
    int rank_of[kMaxCand];
    Key KD[kMaxCand + 16];                  // keys of the current depth (+16: segment reads)
    __attribute__((aligned(16))) float FD[kMaxCand + 16];   // the same V rounded to fp32 (order-preserving prefilter)
    int rankD[kMaxCand];                    // rank of a depth-d candidate within its depth
    int cntS[kMaxCand];                     // best-m entries preceding a depth-d candidate
    double conf[kMaxRows * kMaxChildren];   // c of every (row, child)
    int rowCid[kMaxRows * kMaxChildren];    // token of every (row, child)
    Key KS[kMaxMMax + 16];                  // running best-m list
    __attribute__((aligned(16))) float FS[kMaxMMax + 16];
    Key KSn[kMaxMMax];
    int cntD[kMaxMMax];                     // depth-d candidates preceding a list entry
    int exp_par[kMaxTopk];
};

// (V desc, creation asc)
__device__ __forceinline__ bool kbefore(double va, int ia, double vb, int ib)
{
    return va > vb || (va == vb && ia < ib);
}

// Entries j in [j0, j0 + 16) of (F, K)[0..len), j != self, that come before
// x.  Rounding to fp32 is monotone, so F_j > F_x implies V_j > V_x; only
// equal fp32 keys (rare) need the exact (V, creation) comparison.  The 16
// fp32 keys are read as four 16-byte vectors before any comparison, so the
// segment costs one LDS round trip.
__device__ __forceinline__ int count_seg(const float *F, const Key *K, int len, int j0, int self, float fx,
                                         double vx, int ix)
{
    const float4 *F4 = reinterpret_cast<const float4 *>(F + j0);
    float f[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const float4 v = F4[q];
        f[4 * q] = v.x; f[4 * q + 1] = v.y; f[4 * q + 2] = v.z; f[4 * q + 3] = v.w;
    }
    int cnt = 0;
    uint32_t eq = 0;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        const bool in = j0 + q < len && j0 + q != self;
        cnt += (in && f[q] > fx) ? 1 : 0;
        eq |= (in && f[q] == fx) ? (1u << q) : 0u;
    }
    while (eq) {
        const int q = __builtin_ctz(eq);
        eq &= eq - 1;
        const Key kj = K[j0 + q];
        cnt += kbefore(kj.v, kj.i, vx, ix) ? 1 : 0;
    }
    return cnt;
}

__global__ __launch_bounds__(512) void k_tree_select(TreeSelectArgs a)
{
    __shared__ TreeSmem sm;
    const int b = blockIdx.x, tid = threadIdx.x, NT = blockDim.x;
    const int kind = a.kind ? a.kind[b] : EAGLE_TREE_DYNAMIC;
    const int m_max = a.m_max, Cw = a.children;
    const size_t rb = (size_t)b * a.r_max;
    int32_t *tokens = a.tokens + (size_t)b * m_max, *parent = a.parent + (size_t)b * m_max;
    int32_t *depth = a.depth + (size_t)b * m_max, *src_row = a.src_row + (size_t)b * m_max;
    double *score = a.score + (size_t)b * m_max;

    if (kind == EAGLE_TREE_CHAIN) {
        const int K = a.chain_k;
        if (tid == 0) {
            double Vp = 1.0;
            for (int i = 0; i < K; ++i) {
                const double c = a.top_w[(rb + i) * Cw] / a.W[rb + i];
                Vp = Vp * c;
                tokens[i] = a.top_id[(rb + i) * Cw];
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
        return;
    }

    const int D = a.depth_max, k = a.topk, C = a.children, m = a.m;
    const int R = 1 + (D - 1) * k;
    // confidences of every (row, child), in parallel
    for (int i = tid; i < R * C; i += NT) {
        const int r = i / C, j = i % C;
        sm.conf[i] = a.top_w[(rb + r) * Cw + j] / a.W[rb + r];
        sm.rowCid[i] = a.top_id[(rb + r) * Cw + j];
    }
    __syncthreads();
    // depth 1: children of the root's row 0
    for (int j = tid; j < C; j += NT) {
        sm.V[j] = sm.conf[j];
        sm.KD[j] = Key{sm.conf[j], j, 0};
        sm.FD[j] = (float)sm.conf[j];
        sm.rankD[j] = 0;
        sm.cntS[j] = 0;
        sm.tok[j] = sm.rowCid[j];
        sm.par[j] = -1;
        sm.dep[j] = 1;
        sm.row[j] = -1;
    }
    __syncthreads();
    int begin = 0, end = C, sN = 0;
    for (int d = 1; d <= D; ++d) {
        const int nd = end - begin;
        // ---- counts: rank within the depth, and the merge positions ----
        // items: (segment of D, x in D), (segment of S, x in D), (segment of D, y in S);
        // consecutive threads share a segment
        const int segD = (nd + 15) / 16, segS = (sN + 15) / 16;
        const int itA = segD * nd, itB = segS * nd, itC = segD * sN;
        for (int t = tid; t < itA + itB + itC; t += NT) {
            if (t < itA + itB) {
                const bool vsD = t < itA;
                const int u = vsD ? t : t - itA;
                const int g = u / nd, i = u % nd;
                const Key x = sm.KD[i];
                const float fx = sm.FD[i];
                if (vsD) {
                    const int c = count_seg(sm.FD, sm.KD, nd, 16 * g, i, fx, x.v, x.i);
                    if (c) atomicAdd(&sm.rankD[i], c);
                } else {
                    const int c = count_seg(sm.FS, sm.KS, sN, 16 * g, -1, fx, x.v, x.i);
                    if (c) atomicAdd(&sm.cntS[i], c);
                }
            } else {
                const int u = t - itA - itB;
                const int g = u / sN, q = u % sN;
                const Key y = sm.KS[q];
                const int c = count_seg(sm.FD, sm.KD, nd, 16 * g, -1, sm.FS[q], y.v, y.i);
                if (c) atomicAdd(&sm.cntD[q], c);
            }
        }
        __syncthreads();
        // ---- positions: merged list, expansion ----
        const int ne = d < D ? min(k, nd) : 0;
        for (int t = tid; t < nd + sN; t += NT) {
            if (t < nd) {
                const int rd = sm.rankD[t], pos = rd + sm.cntS[t];
                const Key x = sm.KD[t];
                if (pos < m) sm.KSn[pos] = x;
                if (rd < ne) {
                    sm.exp_par[rd] = x.i;
                    sm.row[x.i] = 1 + (d - 1) * k + rd;
                }
            } else {
                const int q = t - nd, pos = q + sm.cntD[q];
                if (pos < m) sm.KSn[pos] = sm.KS[q];
            }
        }
        __syncthreads();
        // ---- children of the expanded nodes (the next depth's keys); new list ----
        for (int t = tid; t < ne * C; t += NT) {
            const int p = t / C, j = t % C;
            const int pidx = sm.exp_par[p];
            const int r = 1 + (d - 1) * k + p;
            const double v = sm.V[pidx] * sm.conf[r * C + j];
            sm.V[end + t] = v;
            sm.KD[t] = Key{v, end + t, 0};
            sm.FD[t] = (float)v;
            sm.rankD[t] = 0;
            sm.cntS[t] = 0;
            sm.tok[end + t] = sm.rowCid[r * C + j];
            sm.par[end + t] = pidx;
            sm.dep[end + t] = d + 1;
            sm.row[end + t] = -1;
        }
        sN = min(m, sN + nd);
        for (int q = tid; q < sN; q += NT) {
            const Key kq = sm.KSn[q];
            sm.KS[q] = kq;
            sm.FS[q] = (float)kq.v;
            sm.cntD[q] = 0;
        }
        __syncthreads();
        begin = end;
        end += ne * C;
    }
    const int N = begin;
    for (int i = tid; i < N; i += NT) sm.rank_of[i] = -1;
    __syncthreads();
    for (int r = tid; r < m; r += NT) sm.rank_of[sm.KS[r].i] = r;
    __syncthreads();
    // connected tree check (holds by construction: V never grows along a path)
    for (int r = tid; r < m; r += NT) {
        const int i = sm.KS[r].i;
        int q = sm.par[i];
        while (q >= 0) {
            if (sm.rank_of[q] < 0) { raise_error(a.err, EAGLE_DEVERR_CLOSURE); break; }
            q = sm.par[q];
        }
        tokens[r] = sm.tok[i];
        parent[r] = sm.par[i] < 0 ? -1 : sm.rank_of[sm.par[i]];
        depth[r] = sm.dep[i];
        score[r] = sm.V[i];
        src_row[r] = sm.row[i];
    }
    for (int r = m + tid; r < m_max; r += NT) {
        tokens[r] = -1; parent[r] = -1; depth[r] = -1; score[r] = 0.0; src_row[r] = -1;
    }
    if (tid == 0) a.num_nodes[b] = m;
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
    L.off_w = o;      o = align_up(o + rows * p->children * sizeof(double), 256);
    L.total = o;
    return L;
}

// vectors per thread (4, 8, 16 or 32) and threads per row so that one row
// fits the registers of one workgroup; 0 if it does not fit
int row_vectors(int vocab, int vec)
{
    if (vocab <= 1024 * 4 * vec) return 4;
    if (vocab <= 1024 * 8 * vec) return 8;
    if (vocab <= 512 * 16 * vec) return 16;
    if (vocab <= 512 * 32 * vec) return 32;
    return 0;
}

int row_threads(int vocab, int vec)
{
    const int nv = row_vectors(vocab, vec);
    const int per = (nv ? nv : 32) * vec;
    int nt = (vocab + per - 1) / per;
    nt = (nt + 63) / 64 * 64;
    if (nt < 64) nt = 64;
    return nt;
}

hipError_t launch_build_tree(const eagle_tree_params *p, int32_t batch, const void *logits,
                             eagle_dtype dt, int64_t row_stride, const int32_t *kind,
                             int32_t *tokens, int32_t *parent, int32_t *depth, double *score,
                             int32_t *src_row, int32_t *num_nodes, void *ws, hipStream_t st)
{
    const BuildLayout L = build_layout(p, batch);
    char *base = static_cast<char *>(ws);
    RowStatsArgs ra;
    ra.logits = logits;
    ra.row_stride = row_stride;
    ra.r_max = p->r_max;
    ra.vocab = p->vocab;
    ra.children = p->children;
    ra.chain_k = p->chain_k;
    ra.rows_dyn = 1 + (p->depth - 1) * p->topk;
    ra.kind = kind;
    ra.M = reinterpret_cast<float *>(base + L.off_M);
    ra.W = reinterpret_cast<double *>(base + L.off_W);
    ra.top_id = reinterpret_cast<int32_t *>(base + L.off_id);
    ra.top_w = reinterpret_cast<double *>(base + L.off_w);
    ra.err = reinterpret_cast<uint32_t *>(base);
    const size_t esz = dt == EAGLE_F32 ? 4 : 2;
    ra.vec_ok = ((uintptr_t)logits % 16 == 0) && ((size_t)row_stride * esz % 16 == 0);
    const dim3 g1((unsigned)(batch * p->r_max));
    if (batch > 0 && p->r_max > 0) {
        const int vec = dt == EAGLE_F32 ? 4 : 8;
        const dim3 blk(row_threads(p->vocab, vec));
        const int nv = row_vectors(p->vocab, vec);
#define EAGLE_ROWS(T, NV) hipLaunchKernelGGL((k_row_stats<T, NV>), g1, blk, 0, st, ra)
        if (dt == EAGLE_F32) {
            if (nv == 4) EAGLE_ROWS(float, 4);
            else if (nv == 8) EAGLE_ROWS(float, 8);
            else if (nv == 16) EAGLE_ROWS(float, 16);
            else EAGLE_ROWS(float, 32);
        } else {
            if (nv == 4) EAGLE_ROWS(uint16_t, 4);
            else if (nv == 8) EAGLE_ROWS(uint16_t, 8);
            else if (nv == 16) EAGLE_ROWS(uint16_t, 16);
            else EAGLE_ROWS(uint16_t, 32);
        }
#undef EAGLE_ROWS
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    TreeSelectArgs ta;
    ta.kind = kind;
    ta.depth_max = p->depth;
    ta.topk = p->topk;
    ta.children = p->children;
    ta.m = p->m;
    ta.chain_k = p->chain_k;
    ta.m_max = p->m_max;
    ta.r_max = p->r_max;
    ta.W = ra.W;
    ta.top_id = ra.top_id;
    ta.top_w = ra.top_w;
    ta.tokens = tokens;
    ta.parent = parent;
    ta.depth = depth;
    ta.score = score;
    ta.src_row = src_row;
    ta.num_nodes = num_nodes;
    ta.err = ra.err;
    if (batch > 0) {
        hipLaunchKernelGGL(k_tree_select, dim3(batch), dim3(512), 0, st, ta);
        return hipGetLastError();
    }
    return hipSuccess;
}

}  // namespace eagle
