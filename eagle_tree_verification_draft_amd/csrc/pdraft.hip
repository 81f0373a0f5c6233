// pdraft.hip -- inputs of the next parallel drafting pass (P-EAGLE in vLLM,
// "Unified Triton kernel": token ids and positions copied, the bonus token
// inserted, MASK ids in the parallel slots, and the rejected-token mask,
// mask-token mask and hidden-state mapping produced in one pass; "Hidden-state
// management": the shared learned hidden state broadcast into the MASK slots
// and the target's hidden states mapped to their new positions; "Step 2:
// parallel drafting" for what each slot holds).
//
// Sequence b with prefix length L, A accepted nodes a_0..a_{A-1} and bonus
// token t_A: slot s < A + 1 is position L - 1 + s (slot 0 the root, the last
// prefix token; slot j + 1 the accepted node a_j), paired with the token that
// follows it (t_s: the token of a_s, and the bonus for s = A) and with that
// position's target hidden state; slots A + 1 .. A + K - 1 are the MASK
// positions L + A .. L + A + K - 2 with the shared hidden state.
//
// One workgroup per (sequence, slot): it resolves the slot's metadata (the
// sequence's accepted path is read by the first wave, one node per lane) and
// copies its hidden row in 16-byte pieces; the workgroups of slot 0 also
// write the sequence's rejected-node mask and slot count.
#include "common.h"
#include "internal.h"

namespace eagle {

constexpr int kPrepThreads = 256;

struct PrepArgs {
    int m_max, max_accept, K, H, S, mask_id, esz;
    const int32_t *tokens, *num_nodes, *accepted, *accept_len, *bonus, *prefix_len;
    const char *target_hidden, *h_shared;
    int32_t *input_ids, *positions, *hidden_src, *num_slots;
    uint8_t *is_mask, *rejected;
    char *draft_hidden;
    uint32_t *err;
};

__global__ __launch_bounds__(kPrepThreads) void k_pdraft_prepare(PrepArgs a)
{
    __shared__ int s_A, s_src;
    const int b = blockIdx.x / a.S, s = blockIdx.x % a.S, tid = threadIdx.x;
    const int L = a.prefix_len[b];
    if (tid < 64) {
        // accepted path: its usable length (up to the first invalid node id)
        const int amax = a.max_accept < a.m_max ? a.max_accept : a.m_max;
        // the node ids are read alongside the length (lanes past it are not used)
        const int node = tid < amax ? a.accepted[(size_t)b * a.max_accept + tid] : 0;
        int A = a.accept_len[b];
        const bool clamped = A < 0 || A > amax;
        A = A < 0 ? 0 : (A > amax ? amax : A);
        const unsigned long long bad = __ballot(tid < A && (node < 0 || node >= a.m_max));
        if (bad) A = __ffsll(bad) - 1;
        // the slot's target hidden row: 0 = the root, a_{s-1} + 1 = node a_{s-1}
        const int prev = __shfl(node, s >= 1 && s <= 64 ? s - 1 : 0);
        if (tid == 0) {
            s_A = A;
            s_src = s == 0 ? 0 : (s <= A ? prev + 1 : -1);
            if (s == 0 && (clamped || bad)) raise_error(a.err, EAGLE_DEVERR_TREE);
            if (s == 0 && L < 1) raise_error(a.err, EAGLE_DEVERR_PREFIX);
        }
        if (s == 0) {
            // rejected nodes of the verified tree: present but not on the path
            int n = a.num_nodes[b];
            n = n < 0 ? 0 : (n > a.m_max ? a.m_max : n);
            // lane i checks node i against the path held across the lanes (m_max <= 64)
            bool on_path = false;
            for (int j = 0; j < A; ++j) on_path |= __shfl(node, j) == tid;
            if (tid < a.m_max) a.rejected[(size_t)b * a.m_max + tid] = (tid < n && !on_path) ? 1 : 0;
        }
    }
    __syncthreads();
    const int A = s_A, nslots = A + a.K;
    const int src = s <= A ? s_src : -1;
    const bool mask_slot = s > A && s < nslots;
    if (tid == 0) {
        const size_t o = (size_t)b * a.S + s;
        int id = -1;
        if (s < A) id = a.tokens[(size_t)b * a.m_max + a.accepted[(size_t)b * a.max_accept + s]];
        else if (s == A) id = a.bonus[b];
        else if (mask_slot) id = a.mask_id;
        a.input_ids[o] = id;
        a.positions[o] = s < nslots ? L - 1 + s : -1;
        a.hidden_src[o] = src;
        a.is_mask[o] = mask_slot ? 1 : 0;
        if (s == 0) a.num_slots[b] = nslots;
    }
    // the slot's hidden row: the mapped target row, the shared state, or zeros
    const int pieces = a.H * a.esz / 16;
    const uint4 *from = nullptr;
    if (src >= 0) from = reinterpret_cast<const uint4 *>(a.target_hidden + ((size_t)b * (a.m_max + 1) + src) * a.H * a.esz);
    else if (mask_slot) from = reinterpret_cast<const uint4 *>(a.h_shared);
    uint4 *to = reinterpret_cast<uint4 *>(a.draft_hidden + ((size_t)b * a.S + s) * a.H * a.esz);
    for (int c = tid; c < pieces; c += kPrepThreads) to[c] = from ? from[c] : make_uint4(0u, 0u, 0u, 0u);
}

hipError_t launch_pdraft_prepare(const eagle_pdraft_params *p, int32_t batch, const int32_t *tokens,
                                 const int32_t *num_nodes, const int32_t *accepted, const int32_t *accept_len,
                                 const int32_t *bonus, const int32_t *prefix_len, const void *target_hidden,
                                 const void *h_shared, int32_t *input_ids, int32_t *positions, int32_t *hidden_src,
                                 uint8_t *is_mask, uint8_t *rejected, int32_t *num_slots, void *draft_hidden,
                                 uint32_t *err, hipStream_t st)
{
    PrepArgs a;
    a.m_max = p->m_max; a.max_accept = p->max_accept; a.K = p->k_draft; a.H = p->hidden;
    a.S = p->max_accept + p->k_draft; a.mask_id = p->mask_token_id; a.esz = p->dtype == EAGLE_F32 ? 4 : 2;
    a.tokens = tokens; a.num_nodes = num_nodes; a.accepted = accepted; a.accept_len = accept_len;
    a.bonus = bonus; a.prefix_len = prefix_len;
    a.target_hidden = static_cast<const char *>(target_hidden);
    a.h_shared = static_cast<const char *>(h_shared);
    a.input_ids = input_ids; a.positions = positions; a.hidden_src = hidden_src; a.num_slots = num_slots;
    a.is_mask = is_mask; a.rejected = rejected;
    a.draft_hidden = static_cast<char *>(draft_hidden);
    a.err = err;
    hipLaunchKernelGGL(k_pdraft_prepare, dim3((unsigned)(batch * a.S)), dim3(kPrepThreads), 0, st, a);
    return hipGetLastError();
}

}  // namespace eagle
