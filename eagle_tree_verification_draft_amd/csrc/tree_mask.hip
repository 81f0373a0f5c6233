// tree_mask.hip -- ancestor bitmasks and positions (EAGLE-2 explainer,
// "Attention mask adjustment": a draft token sees only its own ancestors).
#include "common.h"
#include "internal.h"

namespace eagle {

// One wave per sequence, lane i = node i.  Pointer jumping: acc_i holds the
// nodes from i up to (not including) jmp_i; each round acc_i |= acc_{jmp_i},
// jmp_i = jmp_{jmp_i}, so the covered path length doubles and ceil(log2 depth)
// + 1 rounds finish any tree of up to 64 nodes.
__global__ __launch_bounds__(64) void k_tree_mask(int m_max, const int32_t *parent,
                                                  const int32_t *num_nodes, const int32_t *prefix_len,
                                                  uint64_t *anc, int32_t *pos, uint32_t *err)
{
    __shared__ uint64_t s_acc[2][kMaxMMax];
    __shared__ int s_jmp[2][kMaxMMax];
    const int b = blockIdx.x, i = threadIdx.x;
    // independent loads first
    int n = num_nodes[b];
    const int L = prefix_len[b];
    int p = i < m_max ? parent[(size_t)b * m_max + i] : -1;
    if (n < 0 || n > m_max) {
        if (i == 0) raise_error(err, EAGLE_DEVERR_TREE);
        n = n < 0 ? 0 : m_max;
    }
    if (i >= n) {
        p = -1;
    } else if (p >= i || p < -1) {          // rank order is topological: parent < child
        raise_error(err, EAGLE_DEVERR_TREE);
        p = -1;
    }
    s_acc[0][i] = i < n ? (uint64_t)1 << i : 0;
    s_jmp[0][i] = p;
    __syncthreads();
    int cur = 0;
    for (int round = 0; round < 7; ++round) {
        const int j = s_jmp[cur][i];
        uint64_t a = s_acc[cur][i];
        int nj = -1;
        if (j >= 0) {
            a |= s_acc[cur][j];
            nj = s_jmp[cur][j];
        }
        s_acc[cur ^ 1][i] = a;
        s_jmp[cur ^ 1][i] = nj;
        __syncthreads();
        cur ^= 1;
        if (!__any(s_jmp[cur][i] >= 0)) break;   // one wave: uniform exit
    }
    if (i < m_max) {
        const uint64_t a = s_acc[cur][i];
        anc[(size_t)b * m_max + i] = a;
        pos[(size_t)b * m_max + i] = i < n ? L + __popcll(a) - 1 : -1;
    }
}

hipError_t launch_tree_mask(int32_t batch, int32_t m_max, const int32_t *parent,
                            const int32_t *num_nodes, const int32_t *prefix_len, uint64_t *anc,
                            int32_t *pos, uint32_t *err, hipStream_t st)
{
    if (batch <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_tree_mask, dim3(batch), dim3(64), 0, st, (int)m_max, parent, num_nodes,
                       prefix_len, anc, pos, err);
    return hipGetLastError();
}

__global__ void k_zero(uint4 *p, size_t n16)
{
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x)
        p[i] = make_uint4(0, 0, 0, 0);
}

hipError_t launch_zero(void *p, size_t bytes, hipStream_t st)
{
    const size_t n16 = bytes / 16;
    if (n16 == 0) return hipSuccess;
    size_t blocks = (n16 + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(k_zero, dim3((unsigned)blocks), dim3(256), 0, st, static_cast<uint4 *>(p), n16);
    return hipGetLastError();
}

}  // namespace eagle
