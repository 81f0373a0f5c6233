// internal.h -- kernel argument blocks, workspace layouts and launchers of
// libeagle (not part of the public ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/eagle.h"

namespace eagle {

constexpr int kMaxCand = 1024;   // generated candidates per dynamic tree
constexpr int kMaxTopk = 64;     // nodes expanded per depth
constexpr int kMaxDepth = 64;
constexpr int kMaxRows = 128;    // draft rows one dynamic tree uses: 1 + (D-1)k

// ---- tree build ----------------------------------------------------------
struct RowStatsArgs {
    const void *logits;
    int64_t row_stride;
    int rows, r_max, vocab, children, chain_k, rows_dyn;
    int rows_in, row_base;   // input rows per sequence; slot of the first (r_max, 0: all rows)
    const int32_t *kind;
    float *M;          // row max
    double *W;         // exact row weight sum
    int32_t *top_id;   // top-C ids of each row, rank order
    float *top_v;      // and their logits
    uint32_t *err;
    bool vec_ok;
};

// tree-kernel selection for sampled children: every candidate, in creation order
constexpr int kPolicyAllCandidates = 16;

struct TreeSelectArgs {
    const int32_t *kind;
    int depth_max, topk, children, m, chain_k, m_max, r_max, policy;
    const float *M;
    const double *W;
    const int32_t *top_id;
    const float *top_v;
    int32_t *tokens, *parent, *depth;
    double *score;
    int32_t *src_row, *num_nodes;
    const int32_t *levels;   // incremental build: levels given per sequence (NULL: one-shot)
    const int32_t *prefix_len;   // with anc / pos: the ancestor masks and positions too
    uint64_t *anc;
    int32_t *pos;
    uint32_t *err;
};

// incremental build: one level of draft rows at a time
struct FrontierArgs {
    int level, depth_max, topk, children, r_max, policy;
    const float *M;
    const double *W;
    const int32_t *top_id;
    const float *top_v;
    double *fV;        // [batch][kMaxTopk] V of the current frontier
    int32_t *fn;       // [batch] its size
    int32_t *levels;   // [batch] levels given so far
    int32_t *f_tok, *f_par;
    double *f_score;   // outputs [batch][topk]
    uint32_t *err;
};

// EAGLE-1 static template tree
struct TemplateArgs {
    int n_t, children, r_max, m_max;
    const int32_t *tparent, *tchild;
    const float *M;
    const double *W;
    const int32_t *top_id;
    const float *top_v;
    int32_t *tokens, *parent, *depth;
    double *score;
    int32_t *src_row, *num_nodes;
    uint32_t *err;
};

struct BuildLayout {
    size_t off_M, off_W, off_id, off_v;
    size_t off_fV, off_fn, off_lv;   // incremental-build state
    size_t total;
};
BuildLayout build_layout(const eagle_tree_params *p, int32_t batch);
int row_vectors(int vocab, int vec);
int row_threads(int vocab, int vec);

hipError_t launch_build_tree(const eagle_tree_params *p, int32_t batch, const void *logits,
                             eagle_dtype dt, int64_t row_stride, const int32_t *kind,
                             int32_t *tokens, int32_t *parent, int32_t *depth, double *score,
                             int32_t *src_row, int32_t *num_nodes, void *ws, hipStream_t st);

hipError_t launch_build_tree_mask(const eagle_tree_params *p, int32_t batch, const void *logits,
                                  eagle_dtype dt, int64_t row_stride, const int32_t *kind,
                                  const int32_t *prefix_len, int32_t *tokens, int32_t *parent, int32_t *depth,
                                  double *score, int32_t *src_row, int32_t *num_nodes, uint64_t *anc,
                                  int32_t *pos, void *ws, hipStream_t st);
hipError_t launch_build_tree_sampled(const eagle_tree_params *p, int32_t batch, const void *logits,
                                    eagle_dtype dt, int64_t row_stride, const uint32_t *child_words,
                                    int32_t *tokens, int32_t *parent, int32_t *depth, double *score,
                                    int32_t *src_row, int32_t *num_nodes, void *ws, hipStream_t st);
hipError_t launch_build_tree_template(const eagle_tree_params *p, int32_t batch, const void *logits,
                                     eagle_dtype dt, int64_t row_stride, int32_t n_tmpl, const int32_t *tparent,
                                     const int32_t *tchild, int32_t *tokens, int32_t *parent, int32_t *depth,
                                     double *score, int32_t *src_row, int32_t *num_nodes, void *ws, hipStream_t st);
hipError_t launch_tree_expand(const eagle_tree_params *p, int32_t batch, int32_t level, const void *logits,
                              eagle_dtype dt, int64_t row_stride, int32_t *f_tok, int32_t *f_par,
                              double *f_score, void *ws, hipStream_t st);
hipError_t launch_tree_finish(const eagle_tree_params *p, int32_t batch, int32_t *tokens, int32_t *parent,
                              int32_t *depth, double *score, int32_t *src_row, int32_t *num_nodes, void *ws,
                              hipStream_t st);

// ---- mask ----------------------------------------------------------------
hipError_t launch_tree_mask(int32_t batch, int32_t m_max, const int32_t *parent,
                            const int32_t *num_nodes, const int32_t *prefix_len, uint64_t *anc,
                            int32_t *pos, uint32_t *err, hipStream_t st);

// ---- attention -----------------------------------------------------------
struct AttnPlan {
    int G;              // q heads per kv head
    int rows;           // m_max * G query rows per (sequence, kv head)
    int row_groups;     // workgroups along the query rows
    int waves;          // waves per workgroup (32 rows each, bf16 path)
    int chunk;          // keys per split
    int nsplit;         // splits per (sequence, kv head)
    int max_prefix;     // cache capacity: every prefix_len is clamped to it
    int sched;          // 1: blocks follow the longest-first table at off_cnt (k_attn_schedule)
    size_t off_part, off_ml, off_cnt, total;
};
AttnPlan attn_plan(const eagle_attn_params *a, int32_t batch);

hipError_t launch_tree_attn(const eagle_attn_params *a, const AttnPlan &P, int32_t batch,
                            const void *q, const void *k_draft, const void *v_draft,
                            const void *k_cache, const void *v_cache, const int32_t *block_table,
                            const int32_t *prefix_len, const uint64_t *anc, const int32_t *num_nodes,
                            void *out, void *ws, hipStream_t st);

// ---- KV commit -----------------------------------------------------------
// positions a sequence's cache may hold: contiguous max_prefix; paged
// max_prefix when it is in (0, max_blocks * block_size), else the pages' total
int commit_capacity(const eagle_attn_params *p);

hipError_t launch_kv_commit(const eagle_attn_params *p, int32_t batch, const void *k_draft, const void *v_draft,
                            const int32_t *accepted, const int32_t *accept_len, int32_t max_accept,
                            const int32_t *prefix_len, void *k_cache, void *v_cache, const int32_t *block_table,
                            int32_t *slot_mapping, int32_t *prefix_len_out, uint32_t *err, hipStream_t st);

// ---- parallel-draft inputs ------------------------------------------------
hipError_t launch_pdraft_prepare(const eagle_pdraft_params *p, int32_t batch, const int32_t *tokens,
                                 const int32_t *num_nodes, const int32_t *accepted, const int32_t *accept_len,
                                 const int32_t *bonus, const int32_t *prefix_len, const void *target_hidden,
                                 const void *h_shared, int32_t *input_ids, int32_t *positions, int32_t *hidden_src,
                                 uint8_t *is_mask, uint8_t *rejected, int32_t *num_slots, void *draft_hidden,
                                 uint32_t *err, hipStream_t st);

// ---- accept --------------------------------------------------------------
hipError_t launch_accept(const eagle_accept_params *a, int32_t batch, const void *target,
                         eagle_dtype dt, int64_t row_stride, const int32_t *tokens,
                         const int32_t *parent, const int32_t *num_nodes, const uint32_t *words,
                         int32_t *accepted, int32_t *accept_len, int32_t *bonus, uint32_t *err,
                         hipStream_t st);

size_t accept_layout_bytes(const eagle_accept_params *p, int32_t batch);

// recursive rejection sampling over drawn children
size_t accept_rrs_layout_bytes(const eagle_accept_params *p, int32_t batch);
hipError_t launch_accept_rrs(const eagle_accept_params *p, int32_t batch, const void *target, const void *draft,
                             eagle_dtype dt, int64_t t_stride, int64_t d_stride, int32_t r_max,
                             const int32_t *tokens, const int32_t *parent, const int32_t *src_row,
                             const int32_t *num_nodes, const uint32_t *words, int32_t *accepted,
                             int32_t *accept_len, int32_t *bonus, void *ws, hipStream_t st);

// ---- misc ----------------------------------------------------------------
hipError_t launch_zero(void *p, size_t bytes, hipStream_t st);

}  // namespace eagle
