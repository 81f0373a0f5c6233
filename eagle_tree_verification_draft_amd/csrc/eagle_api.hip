// eagle_api.hip -- the C ABI declared in include/eagle.h: argument checks on
// the host (before any launch), workspace sizing and kernel dispatch.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "common.h"
#include "internal.h"

using namespace eagle;

// scratch of eagle_build_tree_mask_noalloc (the build workspace of several
// hundred sequences at the largest vocabulary)
constexpr size_t kNoAllocScratch = 4u << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratch];

namespace {

thread_local char g_err[512] = "";

eagle_status fail(eagle_status s, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return s;
}

eagle_status ok()
{
    g_err[0] = 0;
    return EAGLE_OK;
}

eagle_status hip_status(hipError_t e, const char *what)
{
    if (e == hipSuccess) return ok();
    return fail(EAGLE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// The integer a C caller stored in an enum-typed argument or field, read
// without an enum-typed load: values outside the enum are rejected, not used.
template <class T>
int raw_int(const T &v)
{
    static_assert(sizeof(T) == sizeof(int), "enum arguments are int-sized");
    int x;
    std::memcpy(&x, &v, sizeof x);
    return x;
}
bool valid_dtype(const eagle_dtype &d)
{
    const int x = raw_int(d);
    return x == EAGLE_F32 || x == EAGLE_BF16;
}

eagle_status check_workspace(void *ws, size_t have, size_t need)
{
    if (!ws) return fail(EAGLE_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", need);
    if (((uintptr_t)ws & 255u) != 0) return fail(EAGLE_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    if (have < need) return fail(EAGLE_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", have, need);
    return EAGLE_OK;
}

eagle_status check_tree_params(const eagle_tree_params *p, int32_t batch)
{
    if (!p) return fail(EAGLE_ERR_INVALID, "tree params are NULL");
    if (batch < 0) return fail(EAGLE_ERR_INVALID, "batch %d < 0", batch);
    if (p->vocab < 1) return fail(EAGLE_ERR_INVALID, "vocab %d < 1", p->vocab);
    if (p->vocab > kMaxVocab) return fail(EAGLE_ERR_UNSUPPORTED, "vocab %d > %d", p->vocab, kMaxVocab);
    if (p->children < 1 || p->children > p->vocab)
        return fail(EAGLE_ERR_INVALID, "children %d not in [1, vocab]", p->children);
    if (p->children > kMaxChildren) return fail(EAGLE_ERR_UNSUPPORTED, "children %d > %d", p->children, kMaxChildren);
    if (p->depth < 1 || p->topk < 1) return fail(EAGLE_ERR_INVALID, "depth and topk must be >= 1");
    if (p->depth > kMaxDepth || p->topk > kMaxTopk)
        return fail(EAGLE_ERR_UNSUPPORTED, "depth %d / topk %d above %d / %d", p->depth, p->topk, kMaxDepth, kMaxTopk);
    if (p->m_max < 1) return fail(EAGLE_ERR_INVALID, "m_max %d < 1", p->m_max);
    if (p->m_max > kMaxMMax) return fail(EAGLE_ERR_UNSUPPORTED, "m_max %d > %d", p->m_max, kMaxMMax);
    const long long N = (long long)p->children + (long long)(p->depth - 1) * p->topk * p->children;
    if (N > kMaxCand) return fail(EAGLE_ERR_UNSUPPORTED, "%lld candidates > %d", N, kMaxCand);
    // the candidates a tree really generates: a depth with fewer than k nodes
    // expands all of them (depth d + 1 holds min(k, nodes of depth d) x C)
    long long n_gen = 0;
    for (long long d = 0, nn = p->children; d < p->depth; ++d) {
        n_gen += nn;
        nn = (nn < p->topk ? nn : p->topk) * (long long)p->children;
    }
    // the EAGLE-2 rerank keeps m of them; the other policies keep what their
    // rule selects (at most m)
    const long long m_cap = p->policy == EAGLE_POLICY_EAGLE2 ? n_gen : N;
    if (p->m < 1 || p->m > p->m_max || p->m > m_cap)
        return fail(EAGLE_ERR_INVALID, "m %d not in [1, min(m_max %d, candidates %lld)]", p->m, p->m_max, m_cap);
    const long long rows_dyn = 1 + (long long)(p->depth - 1) * p->topk;
    if (rows_dyn > kMaxRows) return fail(EAGLE_ERR_UNSUPPORTED, "dynamic trees use %lld rows > %d", rows_dyn, kMaxRows);
    if (rows_dyn > p->r_max) return fail(EAGLE_ERR_INVALID, "dynamic trees use %lld rows > r_max %d", rows_dyn, p->r_max);
    if (p->chain_k < 0 || p->chain_k > p->m_max || p->chain_k > p->r_max)
        return fail(EAGLE_ERR_INVALID, "chain_k %d not in [0, min(m_max, r_max)]", p->chain_k);
    if (p->policy < EAGLE_POLICY_EAGLE2 || p->policy > EAGLE_POLICY_CONF_NO_RERANK)
        return fail(EAGLE_ERR_INVALID, "tree policy %d", p->policy);
    if (p->policy == EAGLE_POLICY_NO_RERANK || p->policy == EAGLE_POLICY_CONF_NO_RERANK) {
        // every depth's top k: sum over depths of min(k, candidates of the depth)
        long long tot = 0, nn = p->children;
        for (int d = 0; d < p->depth; ++d) {
            tot += nn < p->topk ? nn : p->topk;
            nn = (nn < p->topk ? nn : p->topk) * (long long)p->children;
        }
        if (tot > p->m_max)
            return fail(EAGLE_ERR_INVALID, "a tree without rerank has %lld nodes > m_max %d", tot, p->m_max);
    }
    return EAGLE_OK;
}

eagle_status check_build_mask_args(const eagle_tree_params *p, int32_t batch, const void *draft_logits,
                                   eagle_dtype dtype, int64_t row_stride, const int32_t *prefix_len,
                                   const int32_t *tokens, const int32_t *parent, const int32_t *depth,
                                   const double *score, const int32_t *src_row, const int32_t *num_nodes,
                                   const uint64_t *anc_mask, const int32_t *pos)
{
    eagle_status s = check_tree_params(p, batch);
    if (s != EAGLE_OK) return s;
    if (!valid_dtype(dtype)) return fail(EAGLE_ERR_UNSUPPORTED, "dtype %d", raw_int(dtype));
    if (!draft_logits || !tokens || !parent || !depth || !score || !src_row || !num_nodes || !prefix_len ||
        !anc_mask || !pos)
        return fail(EAGLE_ERR_INVALID, "a required pointer is NULL");
    if (row_stride < p->vocab) return fail(EAGLE_ERR_INVALID, "row_stride %lld < vocab %d", (long long)row_stride, p->vocab);
    return EAGLE_OK;
}

// ---- scratch of the build-and-mask call that allocates nothing ----------
// The static device array `scratch` (above) takes the place of the caller's
// workspace.  Every GPU the library runs on holds its own copy until the
// process ends; its device address is taken once per device, with that
// device current, and kept here.  Host code uses only that address: the
// array's name is a host-side stand-in, not a device address.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

eagle_status scratch_of_current_device(void **out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(EAGLE_ERR_UNSUPPORTED, "device %d >= %d", dev, kMaxDevices);
    std::lock_guard<std::mutex> guard(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return EAGLE_OK;
}

// the call's device error word, copied to the caller's (one lane: a vector store)
__global__ void k_copy_error_word(const uint32_t *src, uint32_t *dst)
{
    const int i = threadIdx.x;
    dst[i] = src[i];
}

}  // namespace

extern "C" {

const char *eagle_status_string(eagle_status s)
{
    switch (s) {
    case EAGLE_OK: return "ok";
    case EAGLE_ERR_INVALID: return "invalid argument";
    case EAGLE_ERR_UNSUPPORTED: return "unsupported configuration";
    case EAGLE_ERR_WORKSPACE: return "workspace missing or too small";
    case EAGLE_ERR_HIP: return "HIP error";
    }
    return "unknown status";
}

const char *eagle_last_error(void) { return g_err; }

eagle_status eagle_workspace_init(void *workspace, size_t workspace_bytes, void *stream)
{
    if (!workspace || workspace_bytes < kWsHeader) return fail(EAGLE_ERR_WORKSPACE, "workspace NULL or below %zu bytes", kWsHeader);
    if (((uintptr_t)workspace & 255u) != 0) return fail(EAGLE_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    return hip_status(launch_zero(workspace, workspace_bytes / 16 * 16, (hipStream_t)stream), "workspace init");
}

eagle_status eagle_read_errors(void *workspace, void *stream, uint32_t *host_bits)
{
    if (!workspace || !host_bits) return fail(EAGLE_ERR_INVALID, "workspace and host_bits must be non-NULL");
    hipStream_t st = (hipStream_t)stream;
    hipError_t e = hipMemcpyAsync(host_bits, workspace, sizeof(uint32_t), hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e == hipSuccess) e = launch_zero(workspace, 16, st);
    return hip_status(e, "read errors");
}

size_t eagle_build_tree_workspace_size(const eagle_tree_params *p, int32_t batch)
{
    if (check_tree_params(p, batch) != EAGLE_OK) return 0;
    return build_layout(p, batch).total;
}

eagle_status eagle_build_tree(const eagle_tree_params *p, int32_t batch, const void *draft_logits,
                              eagle_dtype dtype, int64_t row_stride, const int32_t *kind,
                              int32_t *tokens, int32_t *parent, int32_t *depth, double *score,
                              int32_t *src_row, int32_t *num_nodes, void *workspace,
                              size_t workspace_bytes, void *stream)
{
    eagle_status s = check_tree_params(p, batch);
    if (s != EAGLE_OK) return s;
    if (!valid_dtype(dtype)) return fail(EAGLE_ERR_UNSUPPORTED, "dtype %d", raw_int(dtype));
    if (!draft_logits || !tokens || !parent || !depth || !score || !src_row || !num_nodes)
        return fail(EAGLE_ERR_INVALID, "a required pointer is NULL");
    if (row_stride < p->vocab) return fail(EAGLE_ERR_INVALID, "row_stride %lld < vocab %d", (long long)row_stride, p->vocab);
    s = check_workspace(workspace, workspace_bytes, build_layout(p, batch).total);
    if (s != EAGLE_OK) return s;
    if (batch == 0) return ok();
    return hip_status(launch_build_tree(p, batch, draft_logits, dtype, row_stride, kind, tokens, parent, depth,
                                        score, src_row, num_nodes, workspace, (hipStream_t)stream),
                      "build_tree launch");
}

eagle_status eagle_build_tree_mask(const eagle_tree_params *p, int32_t batch, const void *draft_logits,
                                   eagle_dtype dtype, int64_t row_stride, const int32_t *kind,
                                   const int32_t *prefix_len, int32_t *tokens, int32_t *parent, int32_t *depth,
                                   double *score, int32_t *src_row, int32_t *num_nodes, uint64_t *anc_mask,
                                   int32_t *pos, void *workspace, size_t workspace_bytes, void *stream)
{
    eagle_status s = check_build_mask_args(p, batch, draft_logits, dtype, row_stride, prefix_len, tokens, parent,
                                           depth, score, src_row, num_nodes, anc_mask, pos);
    if (s != EAGLE_OK) return s;
    s = check_workspace(workspace, workspace_bytes, build_layout(p, batch).total);
    if (s != EAGLE_OK) return s;
    if (batch == 0) return ok();
    return hip_status(launch_build_tree_mask(p, batch, draft_logits, dtype, row_stride, kind, prefix_len, tokens,
                                             parent, depth, score, src_row, num_nodes, anc_mask, pos, workspace,
                                             (hipStream_t)stream),
                      "build_tree_mask launch");
}

eagle_status eagle_build_tree_mask_noalloc(const eagle_tree_params *p, int32_t batch, const void *draft_logits,
                                           eagle_dtype dtype, int64_t row_stride, const int32_t *kind,
                                           const int32_t *prefix_len, int32_t *tokens, int32_t *parent,
                                           int32_t *depth, double *score, int32_t *src_row, int32_t *num_nodes,
                                           uint64_t *anc_mask, int32_t *pos, uint32_t *device_errors, void *stream)
{
    eagle_status s = check_build_mask_args(p, batch, draft_logits, dtype, row_stride, prefix_len, tokens, parent,
                                           depth, score, src_row, num_nodes, anc_mask, pos);
    if (s != EAGLE_OK) return s;
    const size_t need = build_layout(p, batch).total;
    if (need > kNoAllocScratch)
        return fail(EAGLE_ERR_WORKSPACE, "the call needs %zu bytes of scratch; the static array holds %zu", need,
                    kNoAllocScratch);
    if (batch == 0) return ok();
    void *ws = nullptr;
    s = scratch_of_current_device(&ws);
    if (s != EAGLE_OK) return s;
    hipStream_t st = (hipStream_t)stream;
    // the error word starts at zero on every call (a fill kernel, no memset node)
    hipError_t e = launch_zero(ws, 16, st);
    if (e == hipSuccess)
        e = launch_build_tree_mask(p, batch, draft_logits, dtype, row_stride, kind, prefix_len, tokens, parent,
                                   depth, score, src_row, num_nodes, anc_mask, pos, ws, st);
    if (e == hipSuccess && device_errors) {
        hipLaunchKernelGGL(k_copy_error_word, dim3(1), dim3(1), 0, st, static_cast<const uint32_t *>(ws),
                           device_errors);
        e = hipGetLastError();
    }
    return hip_status(e, "build_tree_mask_noalloc launch");
}

eagle_status eagle_build_tree_sampled(const eagle_tree_params *p, int32_t batch, const void *draft_logits,
                                      eagle_dtype dtype, int64_t row_stride, const uint32_t *child_words,
                                      int32_t *tokens, int32_t *parent, int32_t *depth, double *score,
                                      int32_t *src_row, int32_t *num_nodes, void *workspace, size_t workspace_bytes,
                                      void *stream)
{
    eagle_status s = check_tree_params(p, batch);
    if (s != EAGLE_OK) return s;
    if (p->policy != EAGLE_POLICY_EAGLE2) return fail(EAGLE_ERR_INVALID, "sampled children take the EAGLE-2 policy");
    long long tot = 0, nn = p->children;
    for (int d = 0; d < p->depth; ++d) {
        tot += nn;
        nn = (nn < p->topk ? nn : p->topk) * (long long)p->children;
    }
    if (tot > p->m_max)
        return fail(EAGLE_ERR_INVALID, "a sampled tree keeps all %lld candidates > m_max %d", tot, p->m_max);
    if (!valid_dtype(dtype)) return fail(EAGLE_ERR_UNSUPPORTED, "dtype %d", raw_int(dtype));
    if (!draft_logits || !child_words || !tokens || !parent || !depth || !score || !src_row || !num_nodes)
        return fail(EAGLE_ERR_INVALID, "a required pointer is NULL");
    if (row_stride < p->vocab) return fail(EAGLE_ERR_INVALID, "row_stride %lld < vocab %d", (long long)row_stride, p->vocab);
    s = check_workspace(workspace, workspace_bytes, build_layout(p, batch).total);
    if (s != EAGLE_OK) return s;
    if (batch == 0) return ok();
    return hip_status(launch_build_tree_sampled(p, batch, draft_logits, dtype, row_stride, child_words, tokens, parent,
                                                depth, score, src_row, num_nodes, workspace, (hipStream_t)stream),
                      "build_tree_sampled launch");
}

eagle_status eagle_build_tree_template(const eagle_tree_params *p, int32_t batch, const void *draft_logits,
                                       eagle_dtype dtype, int64_t row_stride, int32_t n_tmpl,
                                       const int32_t *tmpl_parent, const int32_t *tmpl_child, int32_t *tokens,
                                       int32_t *parent, int32_t *depth, double *score, int32_t *src_row,
                                       int32_t *num_nodes, void *workspace, size_t workspace_bytes, void *stream)
{
    if (!p) return fail(EAGLE_ERR_INVALID, "tree params are NULL");
    if (batch < 0) return fail(EAGLE_ERR_INVALID, "batch %d < 0", batch);
    if (!valid_dtype(dtype)) return fail(EAGLE_ERR_UNSUPPORTED, "dtype %d", raw_int(dtype));
    if (p->vocab < 1) return fail(EAGLE_ERR_INVALID, "vocab %d < 1", p->vocab);
    if (p->vocab > kMaxVocab) return fail(EAGLE_ERR_UNSUPPORTED, "vocab %d > %d", p->vocab, kMaxVocab);
    if (p->children < 1 || p->children > p->vocab)
        return fail(EAGLE_ERR_INVALID, "children %d not in [1, vocab]", p->children);
    if (p->children > kMaxChildren) return fail(EAGLE_ERR_UNSUPPORTED, "children %d > %d", p->children, kMaxChildren);
    if (p->m_max < 1 || p->m_max > kMaxMMax) return fail(EAGLE_ERR_INVALID, "m_max %d not in [1, %d]", p->m_max, kMaxMMax);
    if (p->r_max < 1) return fail(EAGLE_ERR_INVALID, "r_max %d < 1", p->r_max);
    if (n_tmpl < 1 || n_tmpl > p->m_max) return fail(EAGLE_ERR_INVALID, "template of %d nodes not in [1, m_max]", n_tmpl);
    if (!draft_logits || !tmpl_parent || !tmpl_child || !tokens || !parent || !depth || !score || !src_row || !num_nodes)
        return fail(EAGLE_ERR_INVALID, "a required pointer is NULL");
    if (row_stride < p->vocab) return fail(EAGLE_ERR_INVALID, "row_stride %lld < vocab %d", (long long)row_stride, p->vocab);
    eagle_status s = check_workspace(workspace, workspace_bytes, build_layout(p, batch).total);
    if (s != EAGLE_OK) return s;
    if (batch == 0) return ok();
    return hip_status(launch_build_tree_template(p, batch, draft_logits, dtype, row_stride, n_tmpl, tmpl_parent,
                                                 tmpl_child, tokens, parent, depth, score, src_row, num_nodes,
                                                 workspace, (hipStream_t)stream),
                      "build_tree_template launch");
}

eagle_status eagle_tree_expand(const eagle_tree_params *p, int32_t batch, int32_t level,
                               const void *level_logits, eagle_dtype dtype, int64_t row_stride,
                               int32_t *frontier_tokens, int32_t *frontier_parent, double *frontier_score,
                               void *workspace, size_t workspace_bytes, void *stream)
{
    eagle_status s = check_tree_params(p, batch);
    if (s != EAGLE_OK) return s;
    if (!valid_dtype(dtype)) return fail(EAGLE_ERR_UNSUPPORTED, "dtype %d", raw_int(dtype));
    if (level < 0 || level >= p->depth) return fail(EAGLE_ERR_INVALID, "level %d not in [0, depth %d)", level, p->depth);
    if (!level_logits || !frontier_tokens || !frontier_parent || !frontier_score)
        return fail(EAGLE_ERR_INVALID, "a required pointer is NULL");
    if (row_stride < p->vocab) return fail(EAGLE_ERR_INVALID, "row_stride %lld < vocab %d", (long long)row_stride, p->vocab);
    s = check_workspace(workspace, workspace_bytes, build_layout(p, batch).total);
    if (s != EAGLE_OK) return s;
    if (batch == 0) return ok();
    return hip_status(launch_tree_expand(p, batch, level, level_logits, dtype, row_stride, frontier_tokens,
                                         frontier_parent, frontier_score, workspace, (hipStream_t)stream),
                      "tree_expand launch");
}

eagle_status eagle_tree_finish(const eagle_tree_params *p, int32_t batch, int32_t *tokens, int32_t *parent,
                               int32_t *depth, double *score, int32_t *src_row, int32_t *num_nodes,
                               void *workspace, size_t workspace_bytes, void *stream)
{
    eagle_status s = check_tree_params(p, batch);
    if (s != EAGLE_OK) return s;
    if (!tokens || !parent || !depth || !score || !src_row || !num_nodes)
        return fail(EAGLE_ERR_INVALID, "a required pointer is NULL");
    s = check_workspace(workspace, workspace_bytes, build_layout(p, batch).total);
    if (s != EAGLE_OK) return s;
    if (batch == 0) return ok();
    return hip_status(launch_tree_finish(p, batch, tokens, parent, depth, score, src_row, num_nodes, workspace,
                                         (hipStream_t)stream),
                      "tree_finish launch");
}

eagle_status eagle_tree_mask(int32_t batch, int32_t m_max, const int32_t *parent,
                             const int32_t *num_nodes, const int32_t *prefix_len,
                             uint64_t *anc_mask, int32_t *pos, void *workspace,
                             size_t workspace_bytes, void *stream)
{
    if (batch < 0) return fail(EAGLE_ERR_INVALID, "batch %d < 0", batch);
    if (m_max < 1) return fail(EAGLE_ERR_INVALID, "m_max %d < 1", m_max);
    if (m_max > kMaxMMax) return fail(EAGLE_ERR_UNSUPPORTED, "m_max %d > %d", m_max, kMaxMMax);
    if (!parent || !num_nodes || !prefix_len || !anc_mask || !pos) return fail(EAGLE_ERR_INVALID, "a required pointer is NULL");
    uint32_t *err = nullptr;
    if (workspace) {
        eagle_status s = check_workspace(workspace, workspace_bytes, kWsHeader);
        if (s != EAGLE_OK) return s;
        err = static_cast<uint32_t *>(workspace);
    }
    if (batch == 0) return ok();
    return hip_status(launch_tree_mask(batch, m_max, parent, num_nodes, prefix_len, anc_mask, pos, err,
                                       (hipStream_t)stream),
                      "tree_mask launch");
}

static eagle_status check_attn_params(const eagle_attn_params *a, int32_t batch)
{
    if (!a) return fail(EAGLE_ERR_INVALID, "attention params are NULL");
    if (batch < 0) return fail(EAGLE_ERR_INVALID, "batch %d < 0", batch);
    if (!valid_dtype(a->dtype)) return fail(EAGLE_ERR_UNSUPPORTED, "dtype %d", raw_int(a->dtype));
    if (a->num_kv_heads < 1 || a->num_q_heads < 1 || a->num_q_heads % a->num_kv_heads != 0)
        return fail(EAGLE_ERR_INVALID, "num_q_heads %d must be a positive multiple of num_kv_heads %d",
                    a->num_q_heads, a->num_kv_heads);
    if (a->num_q_heads > kMaxHeads) return fail(EAGLE_ERR_UNSUPPORTED, "num_q_heads %d > %d", a->num_q_heads, kMaxHeads);
    if (a->dtype == EAGLE_BF16 && a->head_dim != 128)
        return fail(EAGLE_ERR_UNSUPPORTED, "bf16 head_dim %d (only 128)", a->head_dim);
    if (a->dtype == EAGLE_F32 && a->head_dim != 64 && a->head_dim != 128)
        return fail(EAGLE_ERR_UNSUPPORTED, "fp32 head_dim %d (only 64, 128)", a->head_dim);
    if (a->m_max < 1) return fail(EAGLE_ERR_INVALID, "m_max %d < 1", a->m_max);
    if (a->m_max > kMaxMMax) return fail(EAGLE_ERR_UNSUPPORTED, "m_max %d > %d", a->m_max, kMaxMMax);
    if ((long long)batch * a->num_q_heads * a->m_max > kMaxQueryRows)
        return fail(EAGLE_ERR_UNSUPPORTED, "batch x num_q_heads x m_max above %lld query rows", kMaxQueryRows);
    if (a->block_size < 0 || a->max_prefix < 0) return fail(EAGLE_ERR_INVALID, "negative block_size or max_prefix");
    if (a->dtype == EAGLE_BF16 && a->block_size == 0 && a->max_prefix % 8 != 0)
        return fail(EAGLE_ERR_UNSUPPORTED, "bf16 contiguous cache needs max_prefix %% 8 == 0");
    if (a->block_size == 0 && a->max_prefix > (1 << 24))
        return fail(EAGLE_ERR_UNSUPPORTED, "contiguous cache above 2^24 keys");
    if (a->block_size > 0) {
        if (a->max_blocks < 1) return fail(EAGLE_ERR_INVALID, "paged cache needs max_blocks >= 1");
        if (a->dtype == EAGLE_BF16 && a->block_size % 8 != 0)
            return fail(EAGLE_ERR_UNSUPPORTED, "bf16 paged cache needs block_size %% 8 == 0");
        if ((long long)a->max_blocks * a->block_size > (1ll << 30))
            return fail(EAGLE_ERR_UNSUPPORTED, "paged capacity above 2^30 keys");
    }
    if (!(a->scale == a->scale) || std::isinf(a->scale)) return fail(EAGLE_ERR_INVALID, "scale is not finite");
    return EAGLE_OK;
}

size_t eagle_tree_attn_workspace_size(const eagle_attn_params *a, int32_t batch)
{
    if (check_attn_params(a, batch) != EAGLE_OK) return 0;
    return attn_plan(a, batch).total;
}

eagle_status eagle_tree_attn(const eagle_attn_params *a, int32_t batch, const void *q,
                             const void *k_draft, const void *v_draft, const void *k_cache,
                             const void *v_cache, const int32_t *block_table,
                             const int32_t *prefix_len, const uint64_t *anc_mask,
                             const int32_t *num_nodes, void *out, void *workspace,
                             size_t workspace_bytes, void *stream)
{
    eagle_status s = check_attn_params(a, batch);
    if (s != EAGLE_OK) return s;
    const bool no_cache = a->block_size == 0 && a->max_prefix == 0;   // empty contiguous cache
    if (!q || !k_draft || !v_draft || (!no_cache && (!k_cache || !v_cache)) || !prefix_len || !anc_mask ||
        !num_nodes || !out)
        return fail(EAGLE_ERR_INVALID, "a required pointer is NULL");
    if (a->block_size > 0 && !block_table) return fail(EAGLE_ERR_INVALID, "paged cache needs a block table");
    if (a->dtype == EAGLE_BF16 &&
        !(aligned16(q) && aligned16(k_draft) && aligned16(v_draft) && aligned16(k_cache) && aligned16(v_cache) &&
          aligned16(out)))
        return fail(EAGLE_ERR_UNSUPPORTED, "bf16 tensors must be 16-byte aligned");
    const AttnPlan P = attn_plan(a, batch);
    if (P.total == 0) return fail(EAGLE_ERR_UNSUPPORTED, "more than 2^31 - 1 workgroups in one launch");
    s = check_workspace(workspace, workspace_bytes, P.total);
    if (s != EAGLE_OK) return s;
    if (batch == 0) return ok();
    return hip_status(launch_tree_attn(a, P, batch, q, k_draft, v_draft, k_cache, v_cache, block_table,
                                       prefix_len, anc_mask, num_nodes, out, workspace, (hipStream_t)stream),
                      "tree_attn launch");
}

eagle_status eagle_kv_commit(const eagle_attn_params *a, int32_t batch, const void *k_draft,
                             const void *v_draft, const int32_t *accepted, const int32_t *accept_len,
                             int32_t max_accept, const int32_t *prefix_len, void *k_cache, void *v_cache,
                             const int32_t *block_table, int32_t *slot_mapping, int32_t *prefix_len_out,
                             void *workspace, size_t workspace_bytes, void *stream)
{
    eagle_status s = check_attn_params(a, batch);
    if (s != EAGLE_OK) return s;
    if (max_accept < 1) return fail(EAGLE_ERR_INVALID, "max_accept %d < 1", max_accept);
    const bool no_cache = a->block_size == 0 && a->max_prefix == 0;
    if (!k_draft || !v_draft || !accepted || !accept_len || !prefix_len || (!no_cache && (!k_cache || !v_cache)) ||
        !slot_mapping || !prefix_len_out)
        return fail(EAGLE_ERR_INVALID, "a required pointer is NULL");
    if (a->block_size > 0 && !block_table) return fail(EAGLE_ERR_INVALID, "paged cache needs a block table");
    if (!(aligned16(k_draft) && aligned16(v_draft) && aligned16(k_cache)))
        return fail(EAGLE_ERR_UNSUPPORTED, "k_draft, v_draft and k_cache must be 16-byte aligned");
    s = check_workspace(workspace, workspace_bytes, kWsHeader);
    if (s != EAGLE_OK) return s;
    if (batch == 0) return ok();
    return hip_status(launch_kv_commit(a, batch, k_draft, v_draft, accepted, accept_len, max_accept, prefix_len,
                                       k_cache, v_cache, block_table, slot_mapping, prefix_len_out,
                                       static_cast<uint32_t *>(workspace), (hipStream_t)stream),
                      "kv_commit launch");
}

size_t eagle_accept_workspace_size(const eagle_accept_params *a, int32_t batch)
{
    if (!a || batch < 0 || a->m_max < 1 || a->m_max > kMaxMMax) return kWsHeader;
    return accept_layout_bytes(a, batch);
}

eagle_status eagle_accept(const eagle_accept_params *a, int32_t batch, const void *target_logits,
                          eagle_dtype dtype, int64_t row_stride, const int32_t *tokens,
                          const int32_t *parent, const int32_t *num_nodes,
                          const uint32_t *rand_words, int32_t *accepted, int32_t *accept_len,
                          int32_t *bonus_token, void *workspace, size_t workspace_bytes, void *stream)
{
    if (!a) return fail(EAGLE_ERR_INVALID, "accept params are NULL");
    if (batch < 0) return fail(EAGLE_ERR_INVALID, "batch %d < 0", batch);
    if (raw_int(a->mode) != EAGLE_ACCEPT_GREEDY && raw_int(a->mode) != EAGLE_ACCEPT_SAMPLE)
        return fail(EAGLE_ERR_INVALID, "accept mode %d", raw_int(a->mode));
    if (!valid_dtype(dtype)) return fail(EAGLE_ERR_UNSUPPORTED, "dtype %d", raw_int(dtype));
    if (a->mode == EAGLE_ACCEPT_SAMPLE && !(a->temperature > 0.0f && std::isfinite(a->temperature)))
        return fail(EAGLE_ERR_INVALID, "sampling needs a finite temperature > 0");
    if (a->vocab < 1) return fail(EAGLE_ERR_INVALID, "vocab %d < 1", a->vocab);
    if (a->vocab > kMaxVocab) return fail(EAGLE_ERR_UNSUPPORTED, "vocab %d > %d", a->vocab, kMaxVocab);
    if (a->m_max < 1) return fail(EAGLE_ERR_INVALID, "m_max %d < 1", a->m_max);
    if (a->m_max > kMaxMMax) return fail(EAGLE_ERR_UNSUPPORTED, "m_max %d > %d", a->m_max, kMaxMMax);
    if (a->max_accept < 1) return fail(EAGLE_ERR_INVALID, "max_accept %d < 1", a->max_accept);
    if (row_stride < a->vocab) return fail(EAGLE_ERR_INVALID, "row_stride %lld < vocab %d", (long long)row_stride, a->vocab);
    if (!target_logits || !tokens || !parent || !num_nodes || !accepted || !accept_len || !bonus_token)
        return fail(EAGLE_ERR_INVALID, "a required pointer is NULL");
    if (a->mode == EAGLE_ACCEPT_SAMPLE && !rand_words) return fail(EAGLE_ERR_INVALID, "sampling needs rand_words");
    eagle_status s = check_workspace(workspace, workspace_bytes, accept_layout_bytes(a, batch));
    if (s != EAGLE_OK) return s;
    if (batch == 0) return ok();
    return hip_status(launch_accept(a, batch, target_logits, dtype, row_stride, tokens, parent, num_nodes, rand_words,
                                    accepted, accept_len, bonus_token, static_cast<uint32_t *>(workspace),
                                    (hipStream_t)stream),
                      "accept launch");
}

size_t eagle_accept_rrs_workspace_size(const eagle_accept_params *a, int32_t batch)
{
    if (!a || batch < 0 || a->vocab < 1) return kWsHeader;
    return accept_rrs_layout_bytes(a, batch);
}

eagle_status eagle_accept_rrs(const eagle_accept_params *a, int32_t batch, const void *target_logits,
                              const void *draft_logits, eagle_dtype dtype, int64_t target_row_stride,
                              int64_t draft_row_stride, int32_t r_max, const int32_t *tokens, const int32_t *parent,
                              const int32_t *src_row, const int32_t *num_nodes, const uint32_t *rand_words,
                              int32_t *accepted, int32_t *accept_len, int32_t *bonus_token, void *workspace,
                              size_t workspace_bytes, void *stream)
{
    if (!a) return fail(EAGLE_ERR_INVALID, "accept params are NULL");
    if (batch < 0) return fail(EAGLE_ERR_INVALID, "batch %d < 0", batch);
    if (!valid_dtype(dtype)) return fail(EAGLE_ERR_UNSUPPORTED, "dtype %d", raw_int(dtype));
    if (!(a->temperature > 0.0f && std::isfinite(a->temperature)))
        return fail(EAGLE_ERR_INVALID, "recursive rejection sampling needs a finite temperature > 0");
    if (a->vocab < 1) return fail(EAGLE_ERR_INVALID, "vocab %d < 1", a->vocab);
    if (a->vocab > kMaxVocab) return fail(EAGLE_ERR_UNSUPPORTED, "vocab %d > %d", a->vocab, kMaxVocab);
    if (a->m_max < 1) return fail(EAGLE_ERR_INVALID, "m_max %d < 1", a->m_max);
    if (a->m_max > kMaxMMax) return fail(EAGLE_ERR_UNSUPPORTED, "m_max %d > %d", a->m_max, kMaxMMax);
    if (a->max_accept < 1) return fail(EAGLE_ERR_INVALID, "max_accept %d < 1", a->max_accept);
    if (r_max < 1) return fail(EAGLE_ERR_INVALID, "r_max %d < 1", r_max);
    if (target_row_stride < a->vocab || draft_row_stride < a->vocab)
        return fail(EAGLE_ERR_INVALID, "row strides %lld, %lld below vocab %d", (long long)target_row_stride,
                    (long long)draft_row_stride, a->vocab);
    if (!target_logits || !draft_logits || !tokens || !parent || !src_row || !num_nodes || !rand_words || !accepted ||
        !accept_len || !bonus_token)
        return fail(EAGLE_ERR_INVALID, "a required pointer is NULL");
    eagle_status s = check_workspace(workspace, workspace_bytes, accept_rrs_layout_bytes(a, batch));
    if (s != EAGLE_OK) return s;
    if (batch == 0) return ok();
    return hip_status(launch_accept_rrs(a, batch, target_logits, draft_logits, dtype, target_row_stride,
                                        draft_row_stride, r_max, tokens, parent, src_row, num_nodes, rand_words,
                                        accepted, accept_len, bonus_token, workspace, (hipStream_t)stream),
                      "accept_rrs launch");
}

eagle_status eagle_pdraft_prepare(const eagle_pdraft_params *p, int32_t batch, const int32_t *tokens,
                                  const int32_t *num_nodes, const int32_t *accepted,
                                  const int32_t *accept_len, const int32_t *bonus_token,
                                  const int32_t *prefix_len, const void *target_hidden,
                                  const void *h_shared, int32_t *input_ids, int32_t *positions,
                                  int32_t *hidden_src, uint8_t *is_mask, uint8_t *rejected,
                                  int32_t *num_slots, void *draft_hidden, void *workspace,
                                  size_t workspace_bytes, void *stream)
{
    if (!p) return fail(EAGLE_ERR_INVALID, "parallel-draft params are NULL");
    if (batch < 0) return fail(EAGLE_ERR_INVALID, "batch %d < 0", batch);
    if (!valid_dtype(p->dtype)) return fail(EAGLE_ERR_UNSUPPORTED, "dtype %d", raw_int(p->dtype));
    if (p->m_max < 1 || p->m_max > kMaxMMax) return fail(EAGLE_ERR_INVALID, "m_max %d not in [1, %d]", p->m_max, kMaxMMax);
    if (p->max_accept < 1 || p->k_draft < 1 || p->hidden < 1)
        return fail(EAGLE_ERR_INVALID, "max_accept %d, k_draft %d and hidden %d must be >= 1", p->max_accept,
                    p->k_draft, p->hidden);
    if ((long long)p->max_accept + p->k_draft > (1 << 20))
        return fail(EAGLE_ERR_UNSUPPORTED, "max_accept + k_draft above 2^20");
    const size_t esz = p->dtype == EAGLE_F32 ? 4 : 2;
    if ((size_t)p->hidden * esz % 16 != 0)
        return fail(EAGLE_ERR_UNSUPPORTED, "hidden %d x %zu bytes is not a multiple of 16", p->hidden, esz);
    if (!tokens || !num_nodes || !accepted || !accept_len || !bonus_token || !prefix_len || !target_hidden ||
        !h_shared || !input_ids || !positions || !hidden_src || !is_mask || !rejected || !num_slots || !draft_hidden)
        return fail(EAGLE_ERR_INVALID, "a required pointer is NULL");
    if (!(aligned16(target_hidden) && aligned16(h_shared) && aligned16(draft_hidden)))
        return fail(EAGLE_ERR_UNSUPPORTED, "hidden-state buffers must be 16-byte aligned");
    eagle_status s = check_workspace(workspace, workspace_bytes, kWsHeader);
    if (s != EAGLE_OK) return s;
    if (batch == 0) return ok();
    if ((long long)batch * (p->max_accept + p->k_draft) > 0x7fffffffLL)
        return fail(EAGLE_ERR_UNSUPPORTED, "batch x slots above 2^31");
    return hip_status(launch_pdraft_prepare(p, batch, tokens, num_nodes, accepted, accept_len, bonus_token, prefix_len,
                                            target_hidden, h_shared, input_ids, positions, hidden_src, is_mask,
                                            rejected, num_slots, draft_hidden, static_cast<uint32_t *>(workspace),
                                            (hipStream_t)stream),
                      "pdraft_prepare launch");
}

}  // extern "C"
