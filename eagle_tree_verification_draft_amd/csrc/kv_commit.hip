// kv_commit.hip -- the accepted path's draft K/V written into the KV cache
// (EAGLE-1 explainer, "Verification": the accepted tokens extend the sequence;
// P-EAGLE in vLLM, "KV cache and CUDA graphs": tokens not kept map to the padding
// slot -1).  One workgroup per sequence: the j-th accepted node goes to
// position prefix_len + j in every kv head.  Wave 0 resolves the node ids and
// cache slots of all accepted tokens at once (one lane each) and finds the
// first one that cannot be written; then K rows are copied in 16-byte pieces
// and V, stored transposed ([head_dim][keys]), from 16-byte pieces of the
// draft rows into head_dim separate key columns.
#include "common.h"
#include "internal.h"

namespace eagle {

constexpr int kCommitThreads = 256;

struct CommitArgs {
    const char *kd, *vd;
    char *kc, *vc;
    const int32_t *block_table, *accepted, *accept_len, *prefix_len;
    int32_t *slot_mapping, *prefix_len_out;
    int Hkv, d, m_max, max_accept, block_size, max_blocks;
    int rows;   // contiguous cache: keys per (sequence, kv head)
    int cap;    // positions a sequence may hold
    uint32_t *err;
};

// cache slot of position pos < cap (contiguous: pos; paged: page * block_size
// + offset), or -1 on an unassigned page
__device__ __forceinline__ long long commit_slot(const CommitArgs &a, int b, int pos)
{
    if (a.block_size == 0) return pos;
    const int page = a.block_table[(size_t)b * a.max_blocks + pos / a.block_size];
    return page < 0 ? -1 : (long long)page * a.block_size + pos % a.block_size;
}

// element offset of key `slot`, kv head h, dimension e in the K cache (e = 0)
// and in the V^T cache
__device__ __forceinline__ size_t k_index(const CommitArgs &a, int b, int h, long long slot)
{
    if (a.block_size == 0) return (((size_t)b * a.Hkv + h) * a.rows + (size_t)slot) * a.d;
    const long long page = slot / a.block_size, off = slot % a.block_size;
    return (((size_t)page * a.Hkv + h) * a.block_size + (size_t)off) * a.d;
}
__device__ __forceinline__ size_t v_index(const CommitArgs &a, int b, int h, int e, long long slot)
{
    if (a.block_size == 0) return (((size_t)b * a.Hkv + h) * a.d + e) * a.rows + (size_t)slot;
    const long long page = slot / a.block_size, off = slot % a.block_size;
    return (((size_t)page * a.Hkv + h) * a.d + e) * a.block_size + (size_t)off;
}

template <typename T>
__global__ __launch_bounds__(kCommitThreads) void k_kv_commit(CommitArgs a)
{
    constexpr int EP = 16 / (int)sizeof(T);   // elements per 16-byte piece
    __shared__ int s_n;                       // tokens committed
    __shared__ int s_node[kMaxMMax];          // their node ids
    __shared__ long long s_slot[kMaxMMax];    // and cache slots
    const int b = blockIdx.x, tid = threadIdx.x;
    const int L = a.prefix_len[b];            // read before the barrier: prefix_len_out may alias it
    const bool l_ok = L >= 0 && L <= a.cap;
    if (tid < 64) {
        const int amax = a.max_accept < a.m_max ? a.max_accept : a.m_max;
        int A = a.accept_len[b];
        const bool clamped = A < 0 || A > amax;
        A = A < 0 ? 0 : (A > amax ? amax : A);
        int node = -1;
        long long slot = -1;
        bool bad_node = false, bad_slot = false;
        if (l_ok && tid < A) {
            node = a.accepted[(size_t)b * a.max_accept + tid];
            bad_node = node < 0 || node >= a.m_max;
            if (!bad_node) {
                bad_slot = L + tid >= a.cap;
                if (!bad_slot) slot = commit_slot(a, b, L + tid);
                bad_slot = bad_slot || slot < 0;
            }
        }
        const unsigned long long bad = __ballot(bad_node || bad_slot);
        const int n = !l_ok ? 0 : (bad ? __ffsll(bad) - 1 : A);
        if (tid < n) {
            s_node[tid] = node;
            s_slot[tid] = slot;
        }
        if (tid == 0) {
            s_n = n;
            const uint32_t e = (clamped ? EAGLE_DEVERR_TREE : 0u) | (l_ok ? 0u : EAGLE_DEVERR_PREFIX);
            if (e) raise_error(a.err, e);
        }
        if (l_ok && tid == n && n < A) raise_error(a.err, bad_node ? EAGLE_DEVERR_TREE : EAGLE_DEVERR_PREFIX);
    }
    __syncthreads();
    const int n = s_n, H = a.Hkv, pieces = a.d / EP;
    const T *kd = reinterpret_cast<const T *>(a.kd);
    const T *vd = reinterpret_cast<const T *>(a.vd);
    T *kc = reinterpret_cast<T *>(a.kc);
    T *vc = reinterpret_cast<T *>(a.vc);
    // work item (token j, kv head h, piece c): one 16-byte K copy and EP V elements
    for (int t = tid; t < n * H * pieces; t += kCommitThreads) {
        const int c = t % pieces, h = (t / pieces) % H, j = t / (pieces * H);
        const size_t src = (((size_t)b * a.m_max + s_node[j]) * H + h) * a.d + (size_t)c * EP;
        const long long slot = s_slot[j];
        *reinterpret_cast<uint4 *>(kc + k_index(a, b, h, slot) + (size_t)c * EP) =
            *reinterpret_cast<const uint4 *>(kd + src);
        const uint4 v = *reinterpret_cast<const uint4 *>(vd + src);
        const T *ve = reinterpret_cast<const T *>(&v);
#pragma unroll
        for (int i = 0; i < EP; ++i) vc[v_index(a, b, h, c * EP + i, slot)] = ve[i];
    }
    // slot of every node: -1 unless committed
    for (int i = tid; i < a.m_max; i += kCommitThreads) {
        long long slot = -1;
        for (int j = 0; j < n; ++j)
            if (s_node[j] == i) slot = s_slot[j];
        a.slot_mapping[(size_t)b * a.m_max + i] = (int32_t)slot;
    }
    if (tid == 0) a.prefix_len_out[b] = l_ok ? L + n : L;
}

hipError_t launch_kv_commit(const eagle_attn_params *p, int32_t batch, const void *k_draft, const void *v_draft,
                            const int32_t *accepted, const int32_t *accept_len, int32_t max_accept,
                            const int32_t *prefix_len, void *k_cache, void *v_cache, const int32_t *block_table,
                            int32_t *slot_mapping, int32_t *prefix_len_out, uint32_t *err, hipStream_t st)
{
    CommitArgs a;
    a.kd = static_cast<const char *>(k_draft);
    a.vd = static_cast<const char *>(v_draft);
    a.kc = static_cast<char *>(k_cache);
    a.vc = static_cast<char *>(v_cache);
    a.block_table = block_table; a.accepted = accepted; a.accept_len = accept_len; a.prefix_len = prefix_len;
    a.slot_mapping = slot_mapping; a.prefix_len_out = prefix_len_out;
    a.Hkv = p->num_kv_heads; a.d = p->head_dim; a.m_max = p->m_max; a.max_accept = max_accept;
    a.block_size = p->block_size; a.max_blocks = p->max_blocks;
    a.rows = p->max_prefix;
    a.cap = commit_capacity(p);
    a.err = err;
    if (p->dtype == EAGLE_F32)
        hipLaunchKernelGGL(k_kv_commit<uint32_t>, dim3((unsigned)batch), dim3(kCommitThreads), 0, st, a);
    else
        hipLaunchKernelGGL(k_kv_commit<uint16_t>, dim3((unsigned)batch), dim3(kCommitThreads), 0, st, a);
    return hipGetLastError();
}

int commit_capacity(const eagle_attn_params *p)
{
    if (p->block_size == 0) return p->max_prefix;
    const long long pc = (long long)p->max_blocks * p->block_size;
    return (p->max_prefix > 0 && p->max_prefix < pc) ? p->max_prefix : (int)pc;
}

}  // namespace eagle
