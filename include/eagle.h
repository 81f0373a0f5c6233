/*
 * eagle.h -- C ABI of libeagle.so: one EAGLE-2 draft-tree verification step
 * on an MI355X (gfx950), as four asynchronous calls on one HIP stream:
 *
 *   eagle_build_tree   draft logits -> dynamic draft tree (or a K-token chain)
 *   eagle_tree_mask    tree -> packed ancestor bitmasks and positions
 *   eagle_tree_attn    tree-masked attention of the draft queries
 *   eagle_accept       greedy or rejection-sampling acceptance walk
 *
 * Conventions shared by every call
 *   - Pointers named in the signatures are DEVICE pointers owned by the
 *     caller, unless a comment says "host".  The library allocates, frees
 *     and synchronises nothing inside these calls; every call only enqueues
 *     kernels on `stream` (a hipStream_t; NULL = the null stream).
 *   - Arguments are validated on the host before anything is launched; a
 *     call that returns an error launched nothing.  eagle_last_error()
 *     returns a thread-local description of the last failure.
 *   - Faults that only the device can see (non-finite logits, a prefix
 *     longer than the cache, an accepted path longer than the output width)
 *     set bits in the 32-bit error word at the start of that call's
 *     workspace; they never trap.  Read them with eagle_read_errors().
 *   - Padding slots of every integer output are written as -1, the padding
 *     value of paged KV-cache slot maps (P-EAGLE in vLLM, "KV cache and CUDA
 *     graphs").
 *   - dtype: fp32 or bf16 (raw IEEE bfloat16, row-major).
 *   - v1 limits (EAGLE_ERR_UNSUPPORTED otherwise): m_max <= 64 (one 64-bit
 *     mask word per node), children <= 16, vocab <= 131072 (keeps the
 *     softmax weight sums exact), head_dim in {64, 128} (bf16: 128 only).
 *
 * Softmax weights.  Every decision the step takes from floating point (the
 * confidences that rank the tree, the rejection-sampling tests) uses integer
 * weights w_v = floor(exp_s(x_v) * 2^35), x_v = (l_v - max_u l_u) / T in fp32,
 * where exp_s is exp2 range reduction with a degree-6 Taylor polynomial of 2^f
 * (fp32 Horner with fused multiply-adds, coefficients rounded once from
 * ln2^j/j!), and x is clamped below at -32.  Row sums of these weights are
 * exact in fp64, so trees, masks and accepts are reproducible bit for bit.
 */
#ifndef EAGLE_H
#define EAGLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    EAGLE_OK = 0,
    EAGLE_ERR_INVALID = -1,     /* null pointer, size out of range, inconsistent shapes */
    EAGLE_ERR_UNSUPPORTED = -2, /* outside the v1 limits above */
    EAGLE_ERR_WORKSPACE = -3,   /* workspace missing, misaligned or too small */
    EAGLE_ERR_HIP = -4          /* a HIP launch failed; see eagle_last_error() */
} eagle_status;

typedef enum { EAGLE_F32 = 0, EAGLE_BF16 = 1 } eagle_dtype;
typedef enum { EAGLE_TREE_DYNAMIC = 0, EAGLE_TREE_CHAIN = 1 } eagle_tree_kind;
typedef enum { EAGLE_ACCEPT_GREEDY = 0, EAGLE_ACCEPT_SAMPLE = 1 } eagle_accept_mode;
/* dynamic-tree policies; the last three are the ablations of EAGLE-2
   explainer, "Results" (ablation table: no global acceptance probability,
   i.e. ranking by confidence only; no rerank) */
typedef enum {
    EAGLE_POLICY_EAGLE2 = 0,          /* rank by V; rerank: the top m by V */
    EAGLE_POLICY_NO_RERANK = 1,       /* rank by V; the tree is every depth's top k */
    EAGLE_POLICY_CONF = 2,            /* rank by the node's own c; rerank within m (below) */
    EAGLE_POLICY_CONF_NO_RERANK = 3   /* rank by c; the tree is every depth's top k */
} eagle_tree_policy;

/* device error bits (sticky until the workspace is re-initialised) */
#define EAGLE_DEVERR_NONFINITE_ROW 0x1u  /* a logit row had a NaN, +Inf or all -Inf */
#define EAGLE_DEVERR_CLOSURE 0x2u        /* a selected node's ancestor was not selected (never, by construction) */
#define EAGLE_DEVERR_PREFIX 0x4u         /* prefix_len < 0 or above the cache capacity (clamped) */
#define EAGLE_DEVERR_PATH 0x8u           /* accepted path longer than max_accept (truncated) */
#define EAGLE_DEVERR_TREE 0x10u          /* malformed tree input (parent index out of range) */

/* Workspaces hold per-call scratch and the error word.  Allocate at least the
 * queried size (256-byte aligned) and clear it once with eagle_workspace_init
 * before first use; the calls leave it reusable. */
eagle_status eagle_workspace_init(void *workspace, size_t workspace_bytes, void *stream);

/* Copies the error word of a workspace to *host_bits and clears it.
 * Synchronises `stream`; meant for tests and debugging, not the hot path. */
eagle_status eagle_read_errors(void *workspace, void *stream, uint32_t *host_bits);

/* ------------------------------------------------------------------ */
/* Tree construction                                                   */
/* ------------------------------------------------------------------ */
/*
 * Defines (EAGLE-2 explainer, "Draft model calibration" and "Dynamic draft
 * tree construction", equation for V_i and its Python concept sketch):
 *   c  = draft softmax probability of a token under its parent's row;
 *   V_i = product of c over the root path of node i (V_root = 1);
 *   expansion: at each depth d = 1..D-1 the k depth-d nodes with the largest V
 *   get children; the p-th of them (rank p) owns draft row 1 + (d-1)k + p, and
 *   its children are the `children` tokens of that row with the largest logits;
 *   the root owns row 0 and its children are depth 1;
 *   rerank: the m candidates with the largest V among all generated ones;
 *   connected tree: ancestors of selected nodes are selected (already true,
 *   because V never increases along a path and ancestors come first).
 * Orders: children by (logit desc, token id asc); top-k and top-m by (V desc,
 * creation index asc), creation index = BFS order (depth, parent's expansion
 * rank, child rank).  Chain sequences (P-EAGLE, "Parallel drafting": all K
 * tokens from one pass) take token i = argmax of row i (ties -> smallest id),
 * parent i-1, and own row i+1.
 * Policies (EAGLE-2 explainer, "Results", ablation table) change the ranking
 * key and the final selection; the expansion always takes each depth's
 * first k by the key:
 *   EAGLE2:          key V; the top m by V, output in that order;
 *   NO_RERANK:       key V; the tree is every depth's first k (at most
 *                    sum over depths of min(k, depth's candidates) <= m_max
 *                    nodes), output depth by depth in key order;
 *   CONF:            key c, the node's own confidence; the candidates are
 *                    taken in key order, each with its ancestors not yet
 *                    taken (root first), skipping any that would take the
 *                    tree past m nodes (the pages add the ancestors of the
 *                    selected tokens); output in the order taken, so num_nodes
 *                    may be below m;
 *   CONF_NO_RERANK:  key c; as NO_RERANK.
 * score is V in every policy.
 */
typedef struct {
    int32_t depth;      /* D >= 1: draft tokens sit at depths 1..D */
    int32_t topk;       /* k >= 1: nodes expanded per depth */
    int32_t children;   /* C in [1, 16]: children per expanded node */
    int32_t m;          /* nodes kept for dynamic trees, 1 <= m <= min(m_max, C + (D-1)kC);
                           with the EAGLE2 policy m must not exceed the candidates
                           generated, sum over depths of n_d (n_1 = C,
                           n_(d+1) = min(k, n_d) C), which is smaller when k > n_d */
    int32_t chain_k;    /* K for chain sequences, 0 if there are none; K <= m_max */
    int32_t vocab;      /* V in [C, 131072] */
    int32_t m_max;      /* output slots per sequence, <= 64 */
    int32_t r_max;      /* draft rows per sequence in draft_logits (>= rows used) */
    int32_t policy;     /* an eagle_tree_policy value, for dynamic trees (0: EAGLE-2) */
} eagle_tree_params;

size_t eagle_build_tree_workspace_size(const eagle_tree_params *p, int32_t batch);

/*
 * draft_logits [batch][r_max][row_stride] (dtype); row_stride >= vocab, in
 *   elements; rows used: 1 + (D-1)k for dynamic trees, K for chains.
 * kind [batch] eagle_tree_kind, or NULL for all-dynamic.
 * Outputs [batch][m_max], in the policy's output order (topological: parent
 * index < child index), padded with -1 (score 0):
 *   tokens   token ids;            parent   parent's index (-1 = root)
 *   depth    1..D (chains 1..K);   score    V as fp64
 *   src_row  draft row owned by the node if it was expanded, else -1
 * num_nodes [batch]: m for dynamic trees under EAGLE2 (the node count for
 * the other policies), K for chains.
 * Errors: EAGLE_ERR_INVALID for null pointers, m > candidates, rows > r_max,
 * an unknown policy or a tree without rerank larger than m_max;
 * EAGLE_ERR_UNSUPPORTED past the v1 limits; EAGLE_ERR_WORKSPACE if the
 * workspace is smaller than eagle_build_tree_workspace_size().
 * Device errors: NONFINITE_ROW when a used draft row holds a NaN or +Inf or
 * is all -Inf; that sequence's outputs are then unspecified (the other
 * sequences' are not affected).
 */
eagle_status eagle_build_tree(const eagle_tree_params *p, int32_t batch, const void *draft_logits,
                              eagle_dtype dtype, int64_t row_stride, const int32_t *kind,
                              int32_t *tokens, int32_t *parent, int32_t *depth, double *score,
                              int32_t *src_row, int32_t *num_nodes, void *workspace,
                              size_t workspace_bytes, void *stream);

/*
 * eagle_build_tree followed by eagle_tree_mask on its own outputs, in one
 * call with one launch fewer: the same tree outputs, plus anc_mask and pos
 * [batch][m_max] as eagle_tree_mask defines them for prefix_len [batch].
 * Errors: those of eagle_build_tree, and EAGLE_ERR_INVALID for a NULL
 * prefix_len, anc_mask or pos.
 */
eagle_status eagle_build_tree_mask(const eagle_tree_params *p, int32_t batch, const void *draft_logits,
                                   eagle_dtype dtype, int64_t row_stride, const int32_t *kind,
                                   const int32_t *prefix_len, int32_t *tokens, int32_t *parent, int32_t *depth,
                                   double *score, int32_t *src_row, int32_t *num_nodes, uint64_t *anc_mask,
                                   int32_t *pos, void *workspace, size_t workspace_bytes, void *stream);

/*
 * eagle_build_tree_mask without a workspace, for callers that cannot
 * allocate device memory (code under hipGraph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, checks, outputs and
 * kernels as eagle_build_tree_mask; its workspace is a static device array
 * of the library (4 MiB on each GPU it runs on, held until the process
 * ends).  The call allocates and frees nothing.
 * device_errors: NULL, or a caller-owned device uint32 that receives this
 * call's device error bits (EAGLE_DEVERR_*; the array's error word is
 * cleared at the start of every call, by a kernel).  With batch == 0 nothing
 * is launched and device_errors is left as it is.
 * Calls on one GPU share its array and keep the last call's contents: calls
 * that overlap on one GPU (other streams, other threads) race.
 * Errors: those of eagle_build_tree_mask, and EAGLE_ERR_WORKSPACE when
 * eagle_build_tree_workspace_size(p, batch) exceeds the array (4 MiB).
 */
eagle_status eagle_build_tree_mask_noalloc(const eagle_tree_params *p, int32_t batch, const void *draft_logits,
                                           eagle_dtype dtype, int64_t row_stride, const int32_t *kind,
                                           const int32_t *prefix_len, int32_t *tokens, int32_t *parent,
                                           int32_t *depth, double *score, int32_t *src_row, int32_t *num_nodes,
                                           uint64_t *anc_mask, int32_t *pos, uint32_t *device_errors, void *stream);

/*
 * A dynamic tree whose children are drawn from the draft instead of taken
 * as its top tokens, for lossless acceptance by eagle_accept_rrs (EAGLE-1
 * explainer, "Draft generation flow": tokens are sampled from the draft's
 * next-token distribution; "Verification": the ratio test).  Each used row's
 * `children` tokens are drawn without replacement from its softmax at
 * temperature 1, in draw order, by the inverse CDF of the integer weights:
 * with R the weight left and r = child_words[b][row][t], the target is
 * s = floor(r * R / 2^32) and the draw is the first token not yet drawn, in
 * id order, whose inclusive cumulative weight exceeds s (the first token not
 * yet drawn when no weight is left).  c and V as in eagle_build_tree; the
 * expansion takes each depth's top k by V; the tree is every candidate, in
 * creation order (rows [batch][r_max][row_stride], dynamic trees only).
 * child_words [batch][r_max][children] uint32 (device).
 * Errors: those of eagle_build_tree; EAGLE_ERR_INVALID for a policy other
 * than EAGLE2 or when all candidates (children + (depth-1) topk children
 * when children >= topk) exceed m_max.
 */
eagle_status eagle_build_tree_sampled(const eagle_tree_params *p, int32_t batch, const void *draft_logits,
                                      eagle_dtype dtype, int64_t row_stride, const uint32_t *child_words,
                                      int32_t *tokens, int32_t *parent, int32_t *depth, double *score,
                                      int32_t *src_row, int32_t *num_nodes, void *workspace, size_t workspace_bytes,
                                      void *stream);

/*
 * EAGLE-1's static tree (EAGLE-2 explainer, "Differences from EAGLE-1": a
 * fixed tree template, optimised offline, where EAGLE-2 builds the tree from
 * the draft's confidences).  tmpl_parent / tmpl_child [n_tmpl] (device
 * arrays, parents first: tmpl_parent[i] in [-1, i), -1 = the root;
 * tmpl_child[i] in [0, children)): node i is the tmpl_child[i]-th token, by
 * (logit desc, id asc), of its parent's draft row.  The root owns row 0 and
 * the q-th node (in template order) with children owns row 1 + q, so the
 * draft rows are [batch][r_max][row_stride] with r_max >= 1 + (nodes with
 * children); every one of the r_max rows is read.  Outputs as
 * eagle_build_tree, in template order; score is V; num_nodes = n_tmpl.  Uses
 * children, vocab, m_max and r_max of the params.
 * Device errors: EAGLE_DEVERR_TREE for an invalid template or one needing
 * more than r_max rows (every sequence then gets an empty tree);
 * NONFINITE_ROW as eagle_build_tree.
 * Errors: EAGLE_ERR_INVALID for null pointers or n_tmpl outside [1, m_max];
 * the other parameter checks of eagle_build_tree.
 */
eagle_status eagle_build_tree_template(const eagle_tree_params *p, int32_t batch, const void *draft_logits,
                                       eagle_dtype dtype, int64_t row_stride, int32_t n_tmpl,
                                       const int32_t *tmpl_parent, const int32_t *tmpl_child, int32_t *tokens,
                                       int32_t *parent, int32_t *depth, double *score, int32_t *src_row,
                                       int32_t *num_nodes, void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------ */
/* Incremental tree build                                              */
/* ------------------------------------------------------------------ */
/*
 * Defines (EAGLE-2 explainer, "Dynamic draft tree construction": per depth,
 * the top-k nodes by V are expanded and the draft runs on them; EAGLE-1
 * explainer, "Draft generation flow": one draft forward per step).  The same tree
 * as eagle_build_tree, with the draft rows given one level at a time, so a
 * draft forward can run between the calls on the nodes chosen so far:
 *   level 0:      level_logits [batch][1][row_stride], the root's row (row 0);
 *   level l >= 1: level_logits [batch][topk][row_stride], the rows of the
 *                 frontier that level l - 1 returned, in frontier order
 *                 (row 1 + (l - 1) * topk + p of the one-shot layout);
 *                 rows past the frontier's size (when a depth has fewer
 *                 than topk nodes) do not change the tree, but they are
 *                 read and checked as eagle_build_tree checks every row, so
 *                 they must be finite (zeros will do).
 * Each call returns the next frontier: the top-k nodes of depth l + 1 by
 * (V desc, creation index asc) -- the nodes whose draft rows level l + 1
 * brings -- as frontier_tokens / frontier_parent / frontier_score
 * [batch][topk]: the token, the index of its parent in the previous
 * frontier (-1 at level 0: the root), and its V.  Entries past the frontier's
 * size, and the whole frontier at the last level (depth - 1), are -1 / -1 / 0.
 * eagle_tree_finish then writes the tree exactly as eagle_build_tree over the
 * same rows would (dynamic trees; chains are drafted in one pass and use
 * eagle_build_tree).  One workspace (eagle_build_tree_workspace_size, zeroed
 * by eagle_workspace_init before first use) carries the state across the
 * calls of a tree; level 0 starts a new tree.
 * Device errors: EAGLE_DEVERR_TREE when a level comes out of order (that
 * call writes an empty frontier) or eagle_tree_finish runs before every level
 * is in (that sequence gets an empty tree, num_nodes 0); NONFINITE_ROW as in
 * eagle_build_tree.
 * Errors: those of eagle_build_tree; EAGLE_ERR_INVALID for a level outside
 * [0, depth).
 */
eagle_status eagle_tree_expand(const eagle_tree_params *p, int32_t batch, int32_t level,
                               const void *level_logits, eagle_dtype dtype, int64_t row_stride,
                               int32_t *frontier_tokens, int32_t *frontier_parent, double *frontier_score,
                               void *workspace, size_t workspace_bytes, void *stream);

eagle_status eagle_tree_finish(const eagle_tree_params *p, int32_t batch, int32_t *tokens, int32_t *parent,
                               int32_t *depth, double *score, int32_t *src_row, int32_t *num_nodes,
                               void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------ */
/* Ancestor mask                                                       */
/* ------------------------------------------------------------------ */
/*
 * Defines (EAGLE-2 explainer, "Attention mask adjustment"): a draft token may
 * attend only to its own ancestors (and itself, as a causal chain does), so
 * branches share no information.
 * parent [batch][m_max], num_nodes [batch], prefix_len [batch] (inputs);
 * anc_mask [batch][m_max] uint64: bit j of node i is set iff j is i or an
 * ancestor of i (0 for padding rows); pos [batch][m_max]: prefix_len + depth - 1
 * (the root is the last prefix token), -1 for padding rows.
 * Errors: EAGLE_ERR_INVALID for null pointers or m_max outside [1, 64].
 */
/* workspace may be NULL (then malformed-tree errors are not reported). */
eagle_status eagle_tree_mask(int32_t batch, int32_t m_max, const int32_t *parent,
                             const int32_t *num_nodes, const int32_t *prefix_len,
                             uint64_t *anc_mask, int32_t *pos, void *workspace,
                             size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------ */
/* Tree attention                                                      */
/* ------------------------------------------------------------------ */
/*
 * Defines (EAGLE-1 explainer, "Role of Tree Attention": all branches are
 * verified in one pass; EAGLE-2 explainer, "Attention mask adjustment"):
 * for sequence b, node i < num_nodes[b] and query head h (kv head h / G,
 * G = num_q_heads / num_kv_heads),
 *   out[b][i][h] = softmax_j(scale * q . k_j) v_j over the prefix keys
 *   0..prefix_len[b]-1 and the draft keys j whose bit is set in anc_mask[b][i];
 * rows i >= num_nodes[b] are written as zeros.
 * Layouts (row-major):
 *   q, out            [batch][m_max][num_q_heads][head_dim]
 *   k_draft, v_draft  [batch][m_max][num_kv_heads][head_dim]
 *   contiguous cache (block_size == 0):
 *     k_cache [batch][num_kv_heads][max_prefix][head_dim]
 *     v_cache [batch][num_kv_heads][head_dim][max_prefix]   (V stored transposed;
 *     bf16 needs max_prefix % 8 == 0 so that V^T rows are 16-byte aligned;
 *     max_prefix <= 2^24)
 *   paged cache (block_size > 0), block_table [batch][max_blocks] (-1 = unused):
 *     k_cache [num_blocks][num_kv_heads][block_size][head_dim]
 *     v_cache [num_blocks][num_kv_heads][head_dim][block_size]
 * Keys past prefix_len inside the last page are never read into the result
 * (they may hold anything, NaN included).  fp32 accumulation throughout; bf16
 * inputs use bf16 matrix-core products for q.k and p.v.
 * k_cache / v_cache may be NULL for a contiguous cache with max_prefix 0.
 * Errors: EAGLE_ERR_INVALID for null pointers, num_q_heads % num_kv_heads != 0,
 * a missing block table in paged mode; EAGLE_ERR_UNSUPPORTED past the v1
 * limits (num_q_heads <= 1024, batch x num_q_heads x m_max <= 2^26, at most
 * 2^31 - 1 workgroups in the attention launch); EAGLE_ERR_WORKSPACE for a
 * short workspace.
 */
typedef struct {
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t m_max;       /* <= 64 */
    int32_t block_size;  /* 0 = contiguous cache */
    int32_t max_blocks;  /* block_table row length (paged) */
    int32_t max_prefix;  /* contiguous: cache capacity; paged: bound on prefix_len (<= max_blocks*block_size) */
    float scale;         /* <= 0 selects 1/sqrt(head_dim) */
    eagle_dtype dtype;
} eagle_attn_params;

size_t eagle_tree_attn_workspace_size(const eagle_attn_params *a, int32_t batch);

eagle_status eagle_tree_attn(const eagle_attn_params *a, int32_t batch, const void *q,
                             const void *k_draft, const void *v_draft, const void *k_cache,
                             const void *v_cache, const int32_t *block_table,
                             const int32_t *prefix_len, const uint64_t *anc_mask,
                             const int32_t *num_nodes, void *out, void *workspace,
                             size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------ */
/* KV commit                                                           */
/* ------------------------------------------------------------------ */
/*
 * Defines (EAGLE-1 explainer, "Verification": the accepted tokens extend the
 * sequence; P-EAGLE in vLLM, "KV cache and CUDA graphs": tokens that are not
 * kept map to the padding slot -1, so nothing is written for them).  For
 * sequence b with L = prefix_len[b] and A = accept_len[b]: the j-th accepted
 * node (node id accepted[b][j], j < A, root-first as eagle_accept writes
 * them) is the token at position L + j.  Its draft K/V rows
 * (k_draft / v_draft [b][node][kvh][:], every kv head) are written into the
 * cache at that position, in the layouts of eagle_tree_attn (same params):
 *   contiguous: k_cache[b][kvh][L + j][:] and v_cache[b][kvh][:][L + j]
 *   paged:      page p = block_table[b][(L + j) / block_size], slot
 *               t = (L + j) % block_size: k_cache[p][kvh][t][:], v_cache[p][kvh][:][t]
 * slot_mapping[b][i] (i < m_max) = the cache slot of node i if it was
 * committed (contiguous: L + j; paged: p * block_size + t), else -1.
 * prefix_len_out[b] = L + (tokens committed); it may alias prefix_len.
 * Nothing else in the cache is written; if a node id repeats, slot_mapping
 * holds its later position.  accepted is [batch][max_accept]; a sequence's
 * capacity is the bound eagle_tree_attn clamps prefix_len to (contiguous:
 * max_prefix; paged: max_prefix when it is in (0, max_blocks * block_size),
 * else max_blocks * block_size), so prefix_len_out is valid for the next
 * eagle_tree_attn call with the same params.  Page ids in block_table must
 * name pages of the cache (not checked).
 * The commit of a sequence stops at the first token that cannot be written: a
 * node id outside [0, m_max) (EAGLE_DEVERR_TREE), or a position at or past
 * the capacity or on an unassigned page (EAGLE_DEVERR_PREFIX).  L outside
 * [0, capacity] commits nothing and leaves prefix_len_out[b] = L
 * (EAGLE_DEVERR_PREFIX); accept_len outside [0, min(max_accept, m_max)] is
 * clamped to that range (EAGLE_DEVERR_TREE).
 * Workspace: only the error word (eagle_workspace_init'ed, >= 256 bytes).
 * Errors: EAGLE_ERR_INVALID for null pointers or max_accept < 1; the
 * parameter checks of eagle_tree_attn; EAGLE_ERR_UNSUPPORTED unless k_draft,
 * v_draft and k_cache are 16-byte aligned.  A commit must not run
 * concurrently (on another stream) with a call that reads the same cache.
 */
eagle_status eagle_kv_commit(const eagle_attn_params *a, int32_t batch, const void *k_draft,
                             const void *v_draft, const int32_t *accepted, const int32_t *accept_len,
                             int32_t max_accept, const int32_t *prefix_len, void *k_cache, void *v_cache,
                             const int32_t *block_table, int32_t *slot_mapping, int32_t *prefix_len_out,
                             void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------ */
/* Acceptance                                                          */
/* ------------------------------------------------------------------ */
/*
 * Defines (EAGLE-1 explainer, "Verification"; EAGLE-2 explainer, "Key
 * contributions": lossless by rejection sampling).  Target row 0 belongs to
 * the root, row i + 1 to node i.
 * GREEDY: from the root, accept the child whose token is the target argmax
 *   (ties -> smallest id) of the current node's row; bonus = that argmax at
 *   the last accepted node.
 * SAMPLE (temperature T > 0): the children are the draft's deterministic
 *   top choices, so the draft is a point mass on each of them.  At node u with
 *   weights w of row u at temperature T and residual R = sum of w: children x
 *   in index order are accepted iff r_x * R < w_tok(x) * 2^32 (exact integers,
 *   r_x = rand_words[b][x]); a rejection subtracts w_tok(x) from R and removes
 *   that token.  If none is accepted, the bonus is the smallest token v whose
 *   inclusive cumulative residual weight exceeds floor(r * R / 2^32) with
 *   r = rand_words[b][m_max].  The emitted tokens follow the target softmax.
 * Inputs: target_logits [batch][m_max+1][row_stride]; tokens, parent
 *   [batch][m_max] and num_nodes [batch] as produced by eagle_build_tree;
 *   rand_words [batch][m_max+1] uint32 (SAMPLE only, may be NULL for GREEDY).
 * Outputs: accepted [batch][max_accept] node ids root-first, -1 padded;
 *   accept_len [batch]; bonus_token [batch].
 * Errors: EAGLE_ERR_INVALID for null pointers, T <= 0 in SAMPLE mode;
 * EAGLE_ERR_UNSUPPORTED past the v1 limits.  Device errors (workspace error
 * word): EAGLE_DEVERR_NONFINITE_ROW when a target row that is read holds a NaN
 * (GREEDY) or gives a non-finite maximum or weight sum (SAMPLE), after which
 * that sequence's outputs are unspecified (rows read: those on the walk, and in
 * GREEDY for small batches every row of the tree); EAGLE_DEVERR_TREE for a
 * num_nodes outside [0, m_max] or a child token outside [0, vocab);
 * EAGLE_DEVERR_PATH when a path is longer than max_accept.
 */
typedef struct {
    eagle_accept_mode mode;
    float temperature;   /* SAMPLE only */
    int32_t m_max;       /* <= 64 */
    int32_t vocab;       /* <= 131072 */
    int32_t max_accept;  /* width of `accepted`, >= the deepest node */
} eagle_accept_params;

size_t eagle_accept_workspace_size(const eagle_accept_params *a, int32_t batch);

eagle_status eagle_accept(const eagle_accept_params *a, int32_t batch, const void *target_logits,
                          eagle_dtype dtype, int64_t row_stride, const int32_t *tokens,
                          const int32_t *parent, const int32_t *num_nodes,
                          const uint32_t *rand_words, int32_t *accepted, int32_t *accept_len,
                          int32_t *bonus_token, void *workspace, size_t workspace_bytes,
                          void *stream);

/*
 * Recursive rejection sampling over children drawn from the draft
 * (eagle_build_tree_sampled trees; EAGLE-1 explainer, "Verification": draft
 * tokens accepted by the ratio of the target and draft distributions, the
 * rest discarded after a rejection and a token resampled, leaving the target
 * distribution unchanged).  From the root, at node u with target weights P
 * (Spec S integers of row u + 1 at temperature T, sum SP) and draft weights Q
 * (u's own draft row, src_row[u], the root's being row 0, temperature 1, sum
 * SQ), u's children x are tested in index (draw) order:
 *   accept iff floor(r_x * Q(x) * SP / 2^32) < P(x) * SQ, r_x = rand_words[b][x];
 *   otherwise P <- max(0, P * SQ - Q * SP) >> s, s = max(0, bitlen(SP * SQ)
 *   - 52) (the residual max(0, p - q), summing below 2^52), unless it sums to
 *   0, and Q(x) <- 0 (q without x); a child with Q(x) = 0 is skipped.
 * No child accepted: the bonus is the smallest v whose inclusive cumulative
 * P exceeds floor(r * SP / 2^32), r = rand_words[b][m_max].  The emitted
 * tokens follow the target distribution up to the residuals' rounding
 * (relative 2^-52 per element and step).
 * Inputs: target_logits [batch][m_max+1][target_row_stride]; draft_logits
 *   [batch][r_max][draft_row_stride] (the rows the tree was drawn from);
 *   tokens, parent, src_row [batch][m_max] and num_nodes [batch]
 *   (eagle_build_tree_sampled); rand_words [batch][m_max+1].  Uses m_max,
 *   vocab, max_accept and temperature of the params (mode is ignored).
 * Outputs as eagle_accept.  Device errors: NONFINITE_ROW for a row with a
 *   NaN or infinite maximum or no weight; TREE for a num_nodes outside
 *   [0, m_max], a token outside [0, vocab) or a draft row outside [0, r_max);
 *   PATH as eagle_accept.
 * Workspace: eagle_accept_rrs_workspace_size (three buffers of vocab 64-bit
 *   integers per sequence: the target weights, their residual, the draft
 *   weights).
 */
size_t eagle_accept_rrs_workspace_size(const eagle_accept_params *a, int32_t batch);

eagle_status eagle_accept_rrs(const eagle_accept_params *a, int32_t batch, const void *target_logits,
                              const void *draft_logits, eagle_dtype dtype, int64_t target_row_stride,
                              int64_t draft_row_stride, int32_t r_max, const int32_t *tokens, const int32_t *parent,
                              const int32_t *src_row, const int32_t *num_nodes, const uint32_t *rand_words,
                              int32_t *accepted, int32_t *accept_len, int32_t *bonus_token, void *workspace,
                              size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------ */
/* Parallel-draft inputs (P-EAGLE)                                     */
/* ------------------------------------------------------------------ */
/*
 * Defines (P-EAGLE in vLLM, "Step 2: parallel drafting": the prompt positions
 * pair each token with the target hidden state one position earlier, the
 * first drafting position pairs the newly generated token with the last
 * hidden state, and positions 2..K carry the shared MASK embedding and the
 * shared learned hidden state; "Unified Triton kernel" and "Hidden-state
 * management": one pass that writes the ids, positions, MASK ids, the
 * rejected-token and mask-token masks and the hidden-state mapping, and the
 * broadcast copy of the hidden states).  After eagle_accept, for sequence b
 * with L = prefix_len[b], the usable accepted path a_0..a_{A-1}
 * (accepted[b][j], A = accept_len[b]) and the bonus token, with
 * S = max_accept + k_draft slots per sequence:
 *   slot s <= A:        position L - 1 + s (slot 0 is the root, the last
 *                       prefix token; slot j + 1 is node a_j); input_ids =
 *                       tokens[b][a_s] for s < A and bonus_token[b] for
 *                       s = A; hidden_src = 0 for s = 0, a_{s-1} + 1
 *                       otherwise (a row of target_hidden); is_mask 0;
 *   slot A < s < A + K: position L - 1 + s, input_ids = mask_token_id,
 *                       hidden_src = -1, is_mask 1 (hidden state h_shared);
 *   slot s >= A + K:    padding: ids, positions and hidden_src -1, is_mask 0,
 *                       a zero hidden state;
 *   draft_hidden[b][s][:] = target_hidden[b][hidden_src][:], h_shared, or 0;
 *   num_slots[b] = A + K; rejected[b][i] = 1 for nodes i < num_nodes[b] not
 *   on the accepted path (their KV is not kept), else 0.
 * Layouts: tokens [batch][m_max] and num_nodes [batch] (eagle_build_tree);
 *   accepted [batch][max_accept], accept_len and bonus_token [batch]
 *   (eagle_accept); target_hidden [batch][m_max + 1][hidden] (row 0 the
 *   root, row i + 1 node i); h_shared [hidden]; input_ids, positions and
 *   hidden_src [batch][S] int32; is_mask [batch][S] and rejected
 *   [batch][m_max] uint8; num_slots [batch]; draft_hidden [batch][S][hidden].
 * Device errors: EAGLE_DEVERR_TREE for accept_len outside
 *   [0, min(max_accept, m_max)] (clamped) or an accepted node id outside
 *   [0, m_max) (the path is cut before it); EAGLE_DEVERR_PREFIX for L < 1.
 * Errors: EAGLE_ERR_INVALID for null pointers, k_draft < 1, max_accept < 1,
 *   m_max outside [1, 64] or hidden < 1; EAGLE_ERR_UNSUPPORTED unless
 *   hidden * sizeof(dtype) is a multiple of 16 and the three hidden-state
 *   buffers are 16-byte aligned; EAGLE_ERR_WORKSPACE for a short workspace
 *   (only the error word: >= 256 bytes, eagle_workspace_init'ed).
 */
typedef struct {
    int32_t m_max;
    int32_t max_accept;
    int32_t k_draft;        /* K: tokens one parallel drafting pass predicts */
    int32_t hidden;         /* hidden size */
    int32_t mask_token_id;
    eagle_dtype dtype;      /* of target_hidden, h_shared and draft_hidden */
} eagle_pdraft_params;

eagle_status eagle_pdraft_prepare(const eagle_pdraft_params *p, int32_t batch, const int32_t *tokens,
                                  const int32_t *num_nodes, const int32_t *accepted,
                                  const int32_t *accept_len, const int32_t *bonus_token,
                                  const int32_t *prefix_len, const void *target_hidden,
                                  const void *h_shared, int32_t *input_ids, int32_t *positions,
                                  int32_t *hidden_src, uint8_t *is_mask, uint8_t *rejected,
                                  int32_t *num_slots, void *draft_hidden, void *workspace,
                                  size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------ */
const char *eagle_status_string(eagle_status s);
const char *eagle_last_error(void); /* thread-local; never NULL */

#ifdef __cplusplus
}
#endif
#endif /* EAGLE_H */
