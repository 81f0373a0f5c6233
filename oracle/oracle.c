/*
 * oracle.c -- plain, slow CPU oracle for one EAGLE-2 draft-tree verification
 * step.  TEST INFRASTRUCTURE ONLY: it is called by the tests, by the smoke
 * check and by the benchmark's CPU-baseline leg, never by the product path.
 * It shares no source with the GPU library.
 *
 * What it computes, and where the pages define it:
 *   - confidences c = draft softmax probability of a token under its parent's
 *     row (EAGLE-2 explainer, "Draft model calibration": c_i is the probability
 *     the draft model gives token t_i);
 *   - global acceptance V_i = product of c along the root path (EAGLE-2
 *     explainer, "Dynamic draft tree construction", equation for V_i);
 *   - expansion: per depth, the top-k nodes by V get children; rerank: top-m of
 *     all generated candidates by V; connected tree: ancestors of selected
 *     nodes are included (same section, and its Python concept sketch);
 *   - attention mask: each token sees only its own ancestors (section
 *     "Attention mask adjustment"); tree attention processes the branches in
 *     one pass (EAGLE-1 explainer, "Role of Tree Attention");
 *   - KV commit: the accepted tokens extend the sequence (EAGLE-1 explainer,
 *     "Verification"), so the accepted path's draft K/V are written at the
 *     next cache positions; tokens not kept map to slot -1 (P-EAGLE in vLLM, "KV
 *     cache and CUDA graphs");
 *   - parallel-draft inputs: the ids, positions, masks and hidden states
 *     of the next P-EAGLE drafting pass (P-EAGLE in vLLM, "Step 2: parallel
 *     drafting", "Unified Triton kernel", "Hidden-state management");
 *   - acceptance: draft tokens are accepted by comparing draft and target
 *     distributions, the rest discarded after a rejection and a token
 *     resampled, leaving the target distribution unchanged (EAGLE-1 explainer,
 *     "Verification"); greedy at temperature 0.
 *
 * Softmax arithmetic ("Spec S"; the pages fix no precision):
 *   x  = (l - M) / T  in fp32, M = row max (fmaxf), T = temperature (1 for c)
 *   x  = -32 if x < -32 (NaN stays NaN)
 *   y  = x * L2E (fp32), n = rint(y), f = y - n
 *   p  = Taylor polynomial of 2^f of degree 6 evaluated by Horner with fmaf,
 *        coefficients RN32(ln2^j / j!)
 *   w  = floor(p * 2^(n + 35))    -- an exact integer in [0, 2^35]
 *   W  = sum of w over the row    -- exact in fp64 for V <= 2^17
 *   c  = w / W (fp64 RN); V_child = V_parent * c (fp64 RN); V_root = 1.
 * Orders: children of a row by (logit desc, token id asc); per-depth top-k and
 * global top-m by (V desc, creation index asc); argmax ties to the smallest id.
 *
 * Build: gcc -O2 -std=c11 -fopenmp -ffp-contract=off -fPIC -shared (no fast-math).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef unsigned __int128 u128;

#define ORC_OK 0
#define ORC_ERR_ARG (-1)
#define ORC_ERR_DATA (-2)     /* non-finite row statistics */
#define ORC_ERR_CLOSURE (-3)  /* selected set not closed under ancestors */
#define ORC_ERR_PATH (-4)     /* accepted path longer than the output width */

/* ------------------------------------------------------------------ */
/* element access                                                      */
/* ------------------------------------------------------------------ */

static float bf16_bits_to_f32(uint16_t h)
{
    uint32_t u = ((uint32_t)h) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* dtype 0 = fp32, 1 = bf16 */
static float elem_f32(const void *base, int dtype, int64_t i)
{
    if (dtype == 0) return ((const float *)base)[i];
    return bf16_bits_to_f32(((const uint16_t *)base)[i]);
}

/* ------------------------------------------------------------------ */
/* Spec S exponential and integer weights                              */
/* ------------------------------------------------------------------ */

static const float L2E = 0x1.715476p+0f; /* RN32(1/ln 2) */
static const float EXP_C[7] = {
    0x1.000000p+0f,  /* 1          */
    0x1.62e430p-1f,  /* ln2        */
    0x1.ebfbe0p-3f,  /* ln2^2/2!   */
    0x1.c6b08ep-5f,  /* ln2^3/3!   */
    0x1.3b2ab6p-7f,  /* ln2^4/4!   */
    0x1.5d87fep-10f, /* ln2^5/5!   */
    0x1.430912p-13f, /* ln2^6/6!   */
};

/* p and n with exp(x) ~= p * 2^n, for x already clamped to [-32, 0]. */
static void exp_parts(float x, float *p_out, int *n_out)
{
    float y = x * L2E;
    float n = rintf(y);
    float f = y - n;
    float p = EXP_C[6];
    for (int j = 5; j >= 0; --j) p = fmaf(p, f, EXP_C[j]);
    *p_out = p;
    *n_out = (int)n;
}

float orc_exp_spec(float x)
{
    if (isnan(x)) return x;
    if (x < -32.0f) x = -32.0f;
    float p;
    int n;
    exp_parts(x, &p, &n);
    return ldexpf(p, n);
}

/* w = floor(exp_spec(x) * 2^35); NaN in -> NaN out. */
static double weight_x(float x)
{
    if (isnan(x)) return (double)x;
    if (x < -32.0f) x = -32.0f;
    float p;
    int n;
    exp_parts(x, &p, &n);
    return (double)floorf(ldexpf(p, n + 35));
}

static double weight_l(float l, float M, float T)
{
    float x = (l - M) / T;
    return weight_x(x);
}

double orc_weight(float l, float M, float T) { return weight_l(l, M, T); }

/* ------------------------------------------------------------------ */
/* row statistics: max, exact weight sum, top-C children               */
/* ------------------------------------------------------------------ */

static int beats(float la, int ia, float lb, int ib)
{
    return la > lb || (la == lb && ia < ib);
}

/* One row: M, W, and the top-C tokens by (logit desc, id asc) with weights. */
static int row_stats_one(const void *row, int dtype, int V, int C, float T,
                         float *M_out, double *W_out, int *top_id, double *top_w)
{
    float M = -INFINITY;
    for (int v = 0; v < V; ++v) M = fmaxf(M, elem_f32(row, dtype, v));
    double W = 0.0;
    for (int v = 0; v < V; ++v) W += weight_l(elem_f32(row, dtype, v), M, T);
    *M_out = M;
    *W_out = W;
    if (!isfinite(M) || !isfinite(W)) return ORC_ERR_DATA;
    /* insertion into a sorted list of at most C entries */
    int cnt = 0;
    float tl[64];
    int ti[64];
    for (int v = 0; v < V; ++v) {
        float l = elem_f32(row, dtype, v);
        int pos = cnt;
        while (pos > 0 && beats(l, v, tl[pos - 1], ti[pos - 1])) --pos;
        if (pos >= C) continue;
        int last = cnt < C ? cnt : C - 1;
        for (int j = last; j > pos; --j) { tl[j] = tl[j - 1]; ti[j] = ti[j - 1]; }
        tl[pos] = l;
        ti[pos] = v;
        if (cnt < C) ++cnt;
    }
    for (int j = 0; j < C; ++j) {
        if (j < cnt) {
            top_id[j] = ti[j];
            top_w[j] = weight_l(tl[j], M, T);
        } else {
            top_id[j] = -1;
            top_w[j] = 0.0;
        }
    }
    return ORC_OK;
}

/*
 * C tokens drawn without replacement from the row's softmax at temperature 1
 * (the draft's own distribution), in draw order, by exact inverse-CDF draws
 * on the integer weights: with R the weight left, draw t takes word r_t and
 * s = floor(r_t * R / 2^32), and returns the smallest token not yet drawn
 * whose inclusive cumulative weight (over tokens not yet drawn, in id order)
 * exceeds s; if no weight is left it returns the smallest token not yet drawn.
 */
static int row_draws_one(const void *row, int dtype, int V, int C, const uint32_t *words,
                         float *M_out, double *W_out, int *ids, double *ws)
{
    float M = -INFINITY;
    for (int v = 0; v < V; ++v) M = fmaxf(M, elem_f32(row, dtype, v));
    double W = 0.0;
    for (int v = 0; v < V; ++v) W += weight_l(elem_f32(row, dtype, v), M, 1.0f);
    *M_out = M;
    *W_out = W;
    if (!isfinite(M) || !isfinite(W)) return ORC_ERR_DATA;
    uint64_t R = (uint64_t)W;
    for (int t = 0; t < C; ++t) {
        const uint64_t target = (uint64_t)(((u128)words[t] * R) >> 32);
        uint64_t cum = 0;
        int x = -1, first_free = -1;
        for (int v = 0; v < V && x < 0; ++v) {
            int drawn = 0;
            for (int q = 0; q < t; ++q) drawn |= ids[q] == v;
            if (drawn) continue;
            if (first_free < 0) first_free = v;
            cum += (uint64_t)weight_l(elem_f32(row, dtype, v), M, 1.0f);
            if (cum > target) x = v;
        }
        if (x < 0) x = first_free;
        ids[t] = x;
        ws[t] = x < 0 ? 0.0 : weight_l(elem_f32(row, dtype, x), M, 1.0f);
        R -= (uint64_t)ws[t];
    }
    return ORC_OK;
}

/* rows x V block with the given row stride (elements). C <= 64. */
int orc_row_stats(const void *logits, int dtype, int64_t row_stride, int rows, int V, int C,
                  float T, float *M, double *W, int *top_id, double *top_w)
{
    if (!logits || rows < 0 || V <= 0 || C <= 0 || C > 64 || C > V || !(T > 0.0f)) return ORC_ERR_ARG;
    int err = ORC_OK;
    size_t esz = dtype == 0 ? 4 : 2;
#pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < rows; ++r) {
        const char *row = (const char *)logits + (size_t)r * (size_t)row_stride * esz;
        int e = row_stats_one(row, dtype, V, C, T, &M[r], &W[r], &top_id[(size_t)r * C],
                              &top_w[(size_t)r * C]);
        if (e != ORC_OK) {
#pragma omp critical
            err = e;
        }
    }
    return err;
}

/* ------------------------------------------------------------------ */
/* tree construction                                                   */
/* ------------------------------------------------------------------ */

typedef struct {
    int token;
    int parent;   /* creation index of the parent, -1 = root */
    int depth;    /* 1..D */
    double V;
    double key;   /* ranking key: V, or the node's own confidence c (confidence policies) */
    int row;      /* draft row owned by this node if it was expanded, else -1 */
} Cand;

/* plain selection sort keeps this thread-safe and obviously correct */
static void sort_by_rank(const Cand *c, int *idx, int n)
{
    for (int i = 0; i < n; ++i) {
        int best = i;
        for (int j = i + 1; j < n; ++j) {
            const Cand *x = &c[idx[j]], *y = &c[idx[best]];
            if (x->key > y->key || (x->key == y->key && idx[j] < idx[best])) best = j;
        }
        int t = idx[i];
        idx[i] = idx[best];
        idx[best] = t;
    }
}

/*
 * policy (EAGLE-2 explainer, "Results", ablation table: without the global
 * acceptance probability, ranking by confidence only; without reranking):
 *   0: nodes ranked by V for the expansion and the rerank (EAGLE-2);
 *   1: ranked by V; no rerank: the tree is every depth's top-k;
 *   2: ranked by the node's own confidence c; rerank: candidates taken in
 *      that order, each with its missing ancestors, while the tree stays
 *      within m nodes (the pages add the ancestors of selected tokens);
 *   3: ranked by c; no rerank.
 */
typedef struct {
    int depth, topk, children, m, chain_k, vocab, policy;
} orc_tree_params;

/*
 * One sequence.  rows: [R][row_stride] draft logits of this sequence.
 * Outputs (rank order) tokens/parent/depth/score/src_row [m_max], *num_nodes.
 * Optional debug outputs in creation order (may be NULL): cand_* [N_max],
 * cand_rank (-1 if not selected), and *n_cand.
 */
static int build_one(const orc_tree_params *p, int kind, const void *rows, int dtype,
                     int64_t row_stride, int m_max, const uint32_t *child_words,
                     int *tokens, int *parent, int *depth, double *score, int *src_row, int *num_nodes,
                     int *n_cand, int *cand_token, int *cand_parent, int *cand_depth, double *cand_V,
                     int *cand_row, int *cand_rank)
{
    const int D = p->depth, k = p->topk, C = p->children, V = p->vocab;
    size_t esz = dtype == 0 ? 4 : 2;
    for (int i = 0; i < m_max; ++i) {
        tokens[i] = -1; parent[i] = -1; depth[i] = -1; score[i] = 0.0; src_row[i] = -1;
    }
    if (kind == 1) {
        /* chain: token i = argmax of row i, parent i-1 */
        const int K = p->chain_k;
        if (K <= 0 || K > m_max) return ORC_ERR_ARG;
        double Vp = 1.0;
        for (int i = 0; i < K; ++i) {
            float M;
            double W, tw;
            int tid;
            int e = row_stats_one((const char *)rows + (size_t)i * row_stride * esz, dtype, V, 1, 1.0f,
                                  &M, &W, &tid, &tw);
            if (e != ORC_OK) return e;
            double c = tw / W;
            Vp = Vp * c;
            tokens[i] = tid; parent[i] = i - 1; depth[i] = i + 1; score[i] = Vp;
            src_row[i] = (i + 1 < K) ? i + 1 : -1;
            if (cand_token) {
                cand_token[i] = tid; cand_parent[i] = i - 1; cand_depth[i] = i + 1; cand_V[i] = Vp;
                cand_row[i] = src_row[i]; cand_rank[i] = i;
            }
        }
        *num_nodes = K;
        if (n_cand) *n_cand = K;
        return ORC_OK;
    }

    if (D < 1 || k < 1 || C < 1 || p->m < 1 || p->m > m_max) return ORC_ERR_ARG;
    if (p->policy < 0 || p->policy > 3 || D > 64) return ORC_ERR_ARG;
    const int conf_key = p->policy >= 2, rerank = p->policy == 0 || p->policy == 2;
    const int R = 1 + (D - 1) * k;
    const int Nmax = C + (D - 1) * k * C;
    Cand *cand = (Cand *)malloc(sizeof(Cand) * (size_t)Nmax);
    int *idx = (int *)malloc(sizeof(int) * (size_t)Nmax);
    int *rank_of = (int *)malloc(sizeof(int) * (size_t)Nmax);
    float *Mr = (float *)malloc(sizeof(float) * (size_t)R);
    double *Wr = (double *)malloc(sizeof(double) * (size_t)R);
    int *tid = (int *)malloc(sizeof(int) * (size_t)R * C);
    double *tw = (double *)malloc(sizeof(double) * (size_t)R * C);
    int err = ORC_OK;

    for (int r = 0; r < R && err == ORC_OK; ++r)
        err = child_words
                  ? row_draws_one((const char *)rows + (size_t)r * row_stride * esz, dtype, V, C,
                                  child_words + (size_t)r * C, &Mr[r], &Wr[r], &tid[(size_t)r * C], &tw[(size_t)r * C])
                  : row_stats_one((const char *)rows + (size_t)r * row_stride * esz, dtype, V, C, 1.0f,
                                  &Mr[r], &Wr[r], &tid[(size_t)r * C], &tw[(size_t)r * C]);
    if (err != ORC_OK) goto done;

    /* depth 1: the children of the root's row 0 */
    int N = 0;
    for (int j = 0; j < C; ++j) {
        cand[N].token = tid[j];
        cand[N].parent = -1;
        cand[N].depth = 1;
        cand[N].V = 1.0 * (tw[j] / Wr[0]);
        cand[N].key = conf_key ? tw[j] / Wr[0] : cand[N].V;
        cand[N].row = -1;
        ++N;
    }
    int begin = 0, end = N;
    /* expansion: at depth d take the top-k depth-d nodes; the p-th owns row 1+(d-1)k+p */
    for (int d = 1; d <= D - 1; ++d) {
        int cnt = end - begin;
        for (int i = 0; i < cnt; ++i) idx[i] = begin + i;
        sort_by_rank(cand, idx, cnt);
        int ne = cnt < k ? cnt : k;
        for (int pr = 0; pr < ne; ++pr) {
            int par = idx[pr];
            int r = 1 + (d - 1) * k + pr;
            cand[par].row = r;
            for (int j = 0; j < C; ++j) {
                cand[N].token = tid[(size_t)r * C + j];
                cand[N].parent = par;
                cand[N].depth = d + 1;
                cand[N].V = cand[par].V * (tw[(size_t)r * C + j] / Wr[r]);
                cand[N].key = conf_key ? tw[(size_t)r * C + j] / Wr[r] : cand[N].V;
                cand[N].row = -1;
                ++N;
            }
        }
        begin = end;
        end = N;
    }
    /* selection, in output order (idx[0..m)) */
    int m = p->m;
    for (int i = 0; i < N; ++i) rank_of[i] = -1;
    if (child_words) {
        /* sampled children: the tree is every candidate, in creation order */
        if (N > m_max) { err = ORC_ERR_ARG; goto done; }
        for (int i = 0; i < N; ++i) idx[i] = i;
        m = N;
    } else if (rerank && !conf_key) {
        /* rerank: top-m of every generated candidate */
        if (N < m) { err = ORC_ERR_ARG; goto done; }
        for (int i = 0; i < N; ++i) idx[i] = i;
        sort_by_rank(cand, idx, N);
    } else if (rerank) {
        /* candidates in key order, each added with its missing ancestors (root
           first) while the tree stays within m nodes */
        int *order = (int *)malloc(sizeof(int) * (size_t)N);
        int chain[64];
        for (int i = 0; i < N; ++i) order[i] = i;
        sort_by_rank(cand, order, N);
        int n_sel = 0;
        for (int t = 0; t < N && n_sel < m; ++t) {
            int nc = 0;
            for (int a = order[t]; a >= 0 && rank_of[a] < 0; a = cand[a].parent) chain[nc++] = a;
            if (nc == 0 || n_sel + nc > m) continue;
            for (int q = nc - 1; q >= 0; --q) {
                rank_of[chain[q]] = n_sel;
                idx[n_sel++] = chain[q];
            }
        }
        free(order);
        m = n_sel;
    } else {
        /* no rerank: every depth's top-k by the key, depth by depth */
        int n_sel = 0;
        for (int d = 1; d <= D; ++d) {
            int *lvl = idx + n_sel, cnt = 0;
            for (int i = 0; i < N; ++i)
                if (cand[i].depth == d) lvl[cnt++] = i;
            sort_by_rank(cand, lvl, cnt);
            n_sel += cnt < k ? cnt : k;
        }
        m = n_sel;
        if (m > m_max) { err = ORC_ERR_ARG; goto done; }
    }
    for (int r = 0; r < m; ++r) rank_of[idx[r]] = r;
    /* connected tree: every ancestor of a selected node must be selected */
    for (int r = 0; r < m; ++r) {
        int a = cand[idx[r]].parent;
        while (a >= 0) {
            if (rank_of[a] < 0) { err = ORC_ERR_CLOSURE; goto done; }
            a = cand[a].parent;
        }
    }
    for (int r = 0; r < m; ++r) {
        const Cand *c = &cand[idx[r]];
        tokens[r] = c->token;
        parent[r] = c->parent < 0 ? -1 : rank_of[c->parent];
        depth[r] = c->depth;
        score[r] = c->V;
        src_row[r] = c->row;
    }
    *num_nodes = m;
    if (n_cand) {
        *n_cand = N;
        for (int i = 0; i < N; ++i) {
            cand_token[i] = cand[i].token; cand_parent[i] = cand[i].parent;
            cand_depth[i] = cand[i].depth; cand_V[i] = cand[i].V; cand_row[i] = cand[i].row;
            cand_rank[i] = rank_of[i];
        }
    }
done:
    free(cand); free(idx); free(rank_of); free(Mr); free(Wr); free(tid); free(tw);
    return err;
}

/* child_words [batch][r_max][children] (may be NULL): children drawn from the
   draft rows instead of taken as their top tokens; the tree is then every
   candidate, in creation order (dynamic trees only) */
int orc_build_tree(const orc_tree_params *p, int batch, const void *draft_logits, int dtype,
                   int64_t row_stride, int r_max, const int *kind, int m_max, const uint32_t *child_words,
                   int *tokens, int *parent, int *depth, double *score, int *src_row, int *num_nodes,
                   int n_max_dbg, int *n_cand, int *cand_token, int *cand_parent, int *cand_depth,
                   double *cand_V, int *cand_row, int *cand_rank)
{
    if (!p || batch < 0 || !draft_logits || m_max <= 0 || p->vocab <= 0) return ORC_ERR_ARG;
    if (p->children > 64 || p->vocab > (1 << 17) || row_stride < p->vocab) return ORC_ERR_ARG;
    int err = ORC_OK;
    size_t esz = dtype == 0 ? 4 : 2;
#pragma omp parallel for schedule(dynamic, 1)
    for (int b = 0; b < batch; ++b) {
        int kd = kind ? kind[b] : 0;
        int rows_needed = kd == 1 ? p->chain_k : 1 + (p->depth - 1) * p->topk;
        int e;
        if (rows_needed > r_max) {
            e = ORC_ERR_ARG;
        } else {
            const char *rows = (const char *)draft_logits + (size_t)b * r_max * row_stride * esz;
            e = build_one(p, kd, rows, dtype, row_stride, m_max,
                          child_words && kd == 0 ? child_words + (size_t)b * r_max * p->children : NULL,
                          tokens + (size_t)b * m_max, parent + (size_t)b * m_max,
                          depth + (size_t)b * m_max, score + (size_t)b * m_max,
                          src_row + (size_t)b * m_max, num_nodes + b,
                          n_cand ? n_cand + b : NULL,
                          cand_token ? cand_token + (size_t)b * n_max_dbg : NULL,
                          cand_parent ? cand_parent + (size_t)b * n_max_dbg : NULL,
                          cand_depth ? cand_depth + (size_t)b * n_max_dbg : NULL,
                          cand_V ? cand_V + (size_t)b * n_max_dbg : NULL,
                          cand_row ? cand_row + (size_t)b * n_max_dbg : NULL,
                          cand_rank ? cand_rank + (size_t)b * n_max_dbg : NULL);
        }
        if (e != ORC_OK) {
#pragma omp critical
            err = e;
        }
    }
    return err;
}

/*
 * EAGLE-1's static tree (EAGLE-2 explainer, "Differences from EAGLE-1": a
 * fixed tree template, optimised offline, where EAGLE-2 builds the tree from
 * the draft's confidences).  Template node i (parents first: tparent[i] in
 * [-1, i), -1 = the root) is the tchild[i]-th token, by (logit desc, id asc),
 * of its parent's draft row; the root owns row 0 and the q-th template node
 * (in template order) that has children owns row 1 + q.  c and V as in the
 * dynamic build; outputs in template order.
 */
int orc_build_tree_template(int batch, int n_t, const int *tparent, const int *tchild, int C, int V,
                            const void *draft_logits, int dtype, int64_t row_stride, int r_max, int m_max,
                            int *tokens, int *parent, int *depth, double *score, int *src_row, int *num_nodes)
{
    if (batch < 0 || n_t < 1 || n_t > m_max || m_max > 64 || C < 1 || C > 64 || V < C || V > (1 << 17))
        return ORC_ERR_ARG;
    int row_of[64], internal = 0;
    for (int i = 0; i < n_t; ++i) {
        if (tparent[i] < -1 || tparent[i] >= i || tchild[i] < 0 || tchild[i] >= C) return ORC_ERR_ARG;
        row_of[i] = -1;
    }
    for (int i = 0; i < n_t; ++i)
        for (int j = i + 1; j < n_t; ++j)
            if (tparent[j] == i) { row_of[i] = 1 + internal++; break; }
    if (1 + internal > r_max) return ORC_ERR_ARG;
    const size_t esz = dtype == 0 ? 4 : 2;
    int err = ORC_OK;
#pragma omp parallel for schedule(dynamic, 1)
    for (int b = 0; b < batch; ++b) {
        float M[65];
        double W[65], tw[65 * 64], Vn[64];
        int tid[65 * 64], dep[64];
        const char *rows = (const char *)draft_logits + (size_t)b * r_max * row_stride * esz;
        int e = ORC_OK;
        for (int r = 0; r <= internal && e == ORC_OK; ++r)
            e = row_stats_one(rows + (size_t)r * row_stride * esz, dtype, V, C, 1.0f, &M[r], &W[r],
                              &tid[r * C], &tw[r * C]);
        int *tk = tokens + (size_t)b * m_max, *pa = parent + (size_t)b * m_max, *de = depth + (size_t)b * m_max;
        int *sr = src_row + (size_t)b * m_max;
        double *sc = score + (size_t)b * m_max;
        for (int i = 0; i < m_max; ++i) { tk[i] = -1; pa[i] = -1; de[i] = -1; sc[i] = 0.0; sr[i] = -1; }
        if (e == ORC_OK) {
            for (int i = 0; i < n_t; ++i) {
                const int p = tparent[i], r = p < 0 ? 0 : row_of[p], j = tchild[i];
                Vn[i] = (p < 0 ? 1.0 : Vn[p]) * (tw[r * C + j] / W[r]);
                dep[i] = p < 0 ? 1 : dep[p] + 1;
                tk[i] = tid[r * C + j]; pa[i] = p; de[i] = dep[i]; sc[i] = Vn[i]; sr[i] = row_of[i];
            }
            num_nodes[b] = n_t;
        } else {
#pragma omp critical
            err = e;
        }
    }
    return err;
}

/* ------------------------------------------------------------------ */
/* ancestor mask and positions                                          */
/* ------------------------------------------------------------------ */

/* anc[b][i] bit j set iff j is i or an ancestor of i; pos = L + depth - 1. m_max <= 64. */
int orc_tree_mask(int batch, int m_max, const int *parent, const int *num_nodes,
                  const int *prefix_len, uint64_t *anc, int *pos)
{
    if (m_max <= 0 || m_max > 64) return ORC_ERR_ARG;
    for (int b = 0; b < batch; ++b) {
        int n = num_nodes[b];
        for (int i = 0; i < m_max; ++i) {
            uint64_t bits = 0;
            int dep = 0;
            if (i < n) {
                int a = i;
                while (a >= 0) {
                    if (a >= n) return ORC_ERR_ARG;
                    bits |= (uint64_t)1 << a;
                    ++dep;
                    a = parent[(size_t)b * m_max + a];
                }
            }
            anc[(size_t)b * m_max + i] = bits;
            pos[(size_t)b * m_max + i] = i < n ? prefix_len[b] + dep - 1 : -1;
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* tree attention, fp64                                                 */
/* ------------------------------------------------------------------ */

typedef struct {
    int num_q_heads, num_kv_heads, head_dim, m_max, block_size, max_blocks, max_prefix;
    int dtype;        /* 0 fp32, 1 bf16 */
    double scale;     /* softmax scale (1/sqrt(d)) */
} orc_attn_params;

/* element index of key position t, kv head kvh, dimension e in the K cache
   ([..][t][e]) and in the V cache (stored transposed, [..][e][t]) */
static int64_t k_idx(const orc_attn_params *a, const int *block_table, int b, int kvh, int t, int e)
{
    int d = a->head_dim, Hkv = a->num_kv_heads;
    if (a->block_size == 0) return (((int64_t)b * Hkv + kvh) * a->max_prefix + t) * d + e;
    int blk = block_table[(size_t)b * a->max_blocks + t / a->block_size];
    return (((int64_t)blk * Hkv + kvh) * a->block_size + t % a->block_size) * d + e;
}

static int64_t v_idx(const orc_attn_params *a, const int *block_table, int b, int kvh, int t, int e)
{
    int d = a->head_dim, Hkv = a->num_kv_heads;
    if (a->block_size == 0) return (((int64_t)b * Hkv + kvh) * d + e) * a->max_prefix + t;
    int blk = block_table[(size_t)b * a->max_blocks + t / a->block_size];
    return (((int64_t)blk * Hkv + kvh) * d + e) * a->block_size + t % a->block_size;
}

static double kelem(const orc_attn_params *a, const void *k_cache, const int *block_table,
                    int b, int kvh, int t, int e)
{
    return (double)elem_f32(k_cache, a->dtype, k_idx(a, block_table, b, kvh, t, e));
}

static double velem(const orc_attn_params *a, const void *v_cache, const int *block_table,
                    int b, int kvh, int t, int e)
{
    return (double)elem_f32(v_cache, a->dtype, v_idx(a, block_table, b, kvh, t, e));
}

/* Output row for (b, i, h): softmax over prefix keys and ancestor-or-self draft keys. */
static void attn_row(const orc_attn_params *a, const void *q, const void *k_draft, const void *v_draft,
                     const void *k_cache, const void *v_cache, const int *block_table,
                     const int *prefix_len, const uint64_t *anc, int b, int i, int h, double *out)
{
    const int d = a->head_dim, Hq = a->num_q_heads, Hkv = a->num_kv_heads, M = a->m_max;
    const int G = Hq / Hkv, kvh = h / G, L = prefix_len[b];
    const uint64_t bits = anc[(size_t)b * M + i];
    double *qv = (double *)malloc(sizeof(double) * d);
    int nkeys = L + M;
    double *s = (double *)malloc(sizeof(double) * (size_t)nkeys);
    for (int e = 0; e < d; ++e) qv[e] = (double)elem_f32(q, a->dtype, (((int64_t)b * M + i) * Hq + h) * d + e);
    double mx = -INFINITY;
    for (int t = 0; t < L; ++t) {
        double acc = 0.0;
        for (int e = 0; e < d; ++e) acc += qv[e] * kelem(a, k_cache, block_table, b, kvh, t, e);
        s[t] = acc * a->scale;
        if (s[t] > mx) mx = s[t];
    }
    for (int j = 0; j < M; ++j) {
        if (!((bits >> j) & 1)) continue;
        double acc = 0.0;
        for (int e = 0; e < d; ++e)
            acc += qv[e] * (double)elem_f32(k_draft, a->dtype, (((int64_t)b * M + j) * Hkv + kvh) * d + e);
        s[L + j] = acc * a->scale;
        if (s[L + j] > mx) mx = s[L + j];
    }
    double den = 0.0;
    for (int t = 0; t < L; ++t) { s[t] = exp(s[t] - mx); den += s[t]; }
    for (int j = 0; j < M; ++j)
        if ((bits >> j) & 1) { s[L + j] = exp(s[L + j] - mx); den += s[L + j]; }
    for (int e = 0; e < d; ++e) {
        double acc = 0.0;
        for (int t = 0; t < L; ++t) acc += s[t] * velem(a, v_cache, block_table, b, kvh, t, e);
        for (int j = 0; j < M; ++j)
            if ((bits >> j) & 1)
                acc += s[L + j] * (double)elem_f32(v_draft, a->dtype, (((int64_t)b * M + j) * Hkv + kvh) * d + e);
        out[e] = acc / den;
    }
    free(qv);
    free(s);
}

/* Selected output rows: sel_b/sel_i/sel_h [n_sel]; out [n_sel][d]. */
int orc_tree_attn_rows(const orc_attn_params *a, const void *q, const void *k_draft, const void *v_draft,
                       const void *k_cache, const void *v_cache, const int *block_table,
                       const int *prefix_len, const uint64_t *anc, int n_sel, const int *sel_b,
                       const int *sel_i, const int *sel_h, double *out)
{
    if (!a || a->num_kv_heads <= 0 || a->num_q_heads % a->num_kv_heads != 0 || a->m_max > 64) return ORC_ERR_ARG;
#pragma omp parallel for schedule(dynamic, 1)
    for (int s = 0; s < n_sel; ++s)
        attn_row(a, q, k_draft, v_draft, k_cache, v_cache, block_table, prefix_len, anc, sel_b[s],
                 sel_i[s], sel_h[s], out + (size_t)s * a->head_dim);
    return ORC_OK;
}

/* All rows: out [B][m_max][Hq][d] (fp64); rows i >= num_nodes[b] are zero. */
int orc_tree_attn(const orc_attn_params *a, int batch, const void *q, const void *k_draft,
                  const void *v_draft, const void *k_cache, const void *v_cache,
                  const int *block_table, const int *prefix_len, const uint64_t *anc,
                  const int *num_nodes, double *out)
{
    if (!a || a->num_kv_heads <= 0 || a->num_q_heads % a->num_kv_heads != 0 || a->m_max > 64) return ORC_ERR_ARG;
    const int M = a->m_max, Hq = a->num_q_heads, d = a->head_dim;
    const int64_t units = (int64_t)batch * M * Hq;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t u = 0; u < units; ++u) {
        int h = (int)(u % Hq), i = (int)((u / Hq) % M), b = (int)(u / ((int64_t)Hq * M));
        double *o = out + (size_t)u * d;
        if (i >= num_nodes[b]) {
            for (int e = 0; e < d; ++e) o[e] = 0.0;
            continue;
        }
        attn_row(a, q, k_draft, v_draft, k_cache, v_cache, block_table, prefix_len, anc, b, i, h, o);
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* KV commit                                                            */
/* ------------------------------------------------------------------ */

/*
 * The accepted tokens extend the sequence (EAGLE-1 explainer, "Verification"),
 * so the j-th accepted node of sequence b is the token at position
 * L + j (L = prefix_len[b]) and its draft K/V rows, every kv head, are stored
 * in the cache at that position; nodes that are not kept map to slot -1 and
 * nothing is written for them (P-EAGLE in vLLM, "KV cache and CUDA graphs").
 * cap = positions a sequence may hold.  A sequence stops at the first node id
 * outside [0, m_max) (flags[0]) or the first position >= cap or on a page id
 * < 0 (flags[1]); L outside [0, cap] commits nothing and keeps L (flags[1]);
 * accept_len outside [0, min(max_accept, m_max)] is clamped (flags[0]).
 * flags count these events.  slot_mapping [B][m_max]: the slot (contiguous:
 * position; paged: page * block_size + offset) of each committed node, else -1.
 */
int orc_kv_commit(const orc_attn_params *a, int cap, int batch, const void *k_draft, const void *v_draft,
                  const int *accepted, const int *accept_len, int max_accept, const int *prefix_len,
                  void *k_cache, void *v_cache, const int *block_table, int *slot_mapping,
                  int *prefix_len_out, int *flags)
{
    if (!a || batch < 0 || max_accept < 1 || a->m_max < 1 || a->m_max > 64) return ORC_ERR_ARG;
    const size_t esz = a->dtype == 0 ? 4 : 2;
    const int M = a->m_max, H = a->num_kv_heads, d = a->head_dim, bs = a->block_size;
    const int amax = max_accept < M ? max_accept : M;
    flags[0] = flags[1] = 0;
    for (int b = 0; b < batch; ++b) {
        const int L = prefix_len[b];
        int A = accept_len[b];
        if (A < 0 || A > amax) {
            A = A < 0 ? 0 : amax;
            flags[0]++;
        }
        for (int i = 0; i < M; ++i) slot_mapping[(size_t)b * M + i] = -1;
        if (L < 0 || L > cap) {
            flags[1]++;
            prefix_len_out[b] = L;
            continue;
        }
        int n = 0;
        for (int j = 0; j < A; ++j) {
            const int node = accepted[(size_t)b * max_accept + j];
            if (node < 0 || node >= M) { flags[0]++; break; }
            const int pos = L + j;
            if (pos >= cap) { flags[1]++; break; }
            int slot = pos;
            if (bs > 0) {
                const int page = block_table[(size_t)b * a->max_blocks + pos / bs];
                if (page < 0) { flags[1]++; break; }
                slot = page * bs + pos % bs;
            }
            for (int h = 0; h < H; ++h)
                for (int e = 0; e < d; ++e) {
                    const int64_t src = (((int64_t)b * M + node) * H + h) * d + e;
                    memcpy((char *)k_cache + k_idx(a, block_table, b, h, pos, e) * esz,
                           (const char *)k_draft + src * esz, esz);
                    memcpy((char *)v_cache + v_idx(a, block_table, b, h, pos, e) * esz,
                           (const char *)v_draft + src * esz, esz);
                }
            slot_mapping[(size_t)b * M + node] = slot;
            ++n;
        }
        prefix_len_out[b] = L + n;
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* parallel-draft inputs                                                */
/* ------------------------------------------------------------------ */

/*
 * The inputs of the next parallel drafting pass (P-EAGLE in vLLM, "Step 2:
 * parallel drafting": a known position pairs its target hidden state with the
 * token that follows it, the first drafting position pairs the new token with
 * the last hidden state, and the K - 1 further positions carry the MASK token
 * and the shared hidden state; "Unified Triton kernel" and "Hidden-state
 * management" for the outputs).  For sequence b: L = prefix_len[b], the
 * accepted path a_0..a_{A-1} (cut at the first node id outside [0, m_max),
 * flags[0]; A clamped to [0, min(max_accept, m_max)], flags[0]), bonus t_A.
 * The known positions are the root (the last prefix token, position L - 1,
 * hidden row 0) and the accepted nodes (position L + j, hidden row a_j + 1);
 * the token that follows position L - 1 + s is the token of a_s, or the bonus
 * after the last.  S = max_accept + K slots; L < 1 is flagged (flags[1]).
 * esz = bytes per hidden element; hidden rows are H elements.
 */
int orc_pdraft_prepare(int batch, int m_max, int max_accept, int K, int H, int mask_id, int esz,
                       const int *tokens, const int *num_nodes, const int *accepted, const int *accept_len,
                       const int *bonus, const int *prefix_len, const void *target_hidden, const void *h_shared,
                       int *input_ids, int *positions, int *hidden_src, uint8_t *is_mask, uint8_t *rejected,
                       int *num_slots, void *draft_hidden, int *flags)
{
    if (batch < 0 || m_max < 1 || m_max > 64 || max_accept < 1 || K < 1 || H < 1) return ORC_ERR_ARG;
    const int S = max_accept + K;
    const size_t row = (size_t)H * esz;
    flags[0] = flags[1] = 0;
    for (int b = 0; b < batch; ++b) {
        const int L = prefix_len[b];
        const int amax = max_accept < m_max ? max_accept : m_max;
        int A = accept_len[b];
        if (A < 0 || A > amax) {
            A = A < 0 ? 0 : amax;
            flags[0]++;
        }
        const int *acc = accepted + (size_t)b * max_accept;
        for (int j = 0; j < A; ++j)
            if (acc[j] < 0 || acc[j] >= m_max) {
                A = j;
                flags[0]++;
                break;
            }
        if (L < 1) flags[1]++;
        num_slots[b] = A + K;
        for (int s = 0; s < S; ++s) {
            const size_t o = (size_t)b * S + s;
            char *dst = (char *)draft_hidden + o * row;
            const void *src = NULL;
            if (s <= A) {
                /* a known position: the root (s = 0) or accepted node a_{s-1} */
                input_ids[o] = s < A ? tokens[(size_t)b * m_max + acc[s]] : bonus[b];
                positions[o] = L - 1 + s;
                hidden_src[o] = s == 0 ? 0 : acc[s - 1] + 1;
                is_mask[o] = 0;
                src = (const char *)target_hidden + ((size_t)b * (m_max + 1) + hidden_src[o]) * row;
            } else if (s < A + K) {
                /* a parallel-drafting position */
                input_ids[o] = mask_id;
                positions[o] = L - 1 + s;
                hidden_src[o] = -1;
                is_mask[o] = 1;
                src = h_shared;
            } else {
                input_ids[o] = -1;
                positions[o] = -1;
                hidden_src[o] = -1;
                is_mask[o] = 0;
            }
            if (src) memcpy(dst, src, row);
            else memset(dst, 0, row);
        }
        int n = num_nodes[b];
        n = n < 0 ? 0 : (n > m_max ? m_max : n);
        for (int i = 0; i < m_max; ++i) {
            int on_path = 0;
            for (int j = 0; j < A; ++j) on_path |= acc[j] == i;
            rejected[(size_t)b * m_max + i] = (uint8_t)(i < n && !on_path);
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* acceptance                                                           */
/* ------------------------------------------------------------------ */

/* argmax by (value desc, id asc); -1 if the row holds a NaN */
static int argmax_row(const void *row, int dtype, int V)
{
    int best = 0;
    float bl = elem_f32(row, dtype, 0);
    for (int v = 0; v < V; ++v) {
        float l = elem_f32(row, dtype, v);
        if (isnan(l)) return -1;
        if (l > bl) { bl = l; best = v; }
    }
    return best;
}

/*
 * mode 0 greedy: follow the child whose token is the target argmax of the
 * current node's row; bonus = argmax at the last accepted node.
 * mode 1 sample: point-mass rejection sampling with exact integer weights.
 * At node u with residual R (initially W_u): child x (in index order) is
 * accepted iff r_x * R < w_tok * 2^32; otherwise R -= w_tok and the token is
 * removed.  With no child accepted, the bonus is the smallest v whose inclusive
 * cumulative residual weight exceeds floor(r_bonus * R / 2^32).
 * Target row of the root is row 0, of node i row i + 1.  rand_words [B][m_max+1]:
 * word i tests node i, word m_max draws the bonus.
 */
int orc_accept(int mode, float T, int batch, int m_max, int max_accept, int V,
               const void *target_logits, int dtype, int64_t row_stride,
               const int *tokens, const int *parent, const int *num_nodes, const uint32_t *rand_words,
               int *accepted, int *accept_len, int *bonus)
{
    if (batch < 0 || m_max <= 0 || max_accept <= 0 || V <= 0 || V > (1 << 17) || !(T > 0.0f)) return ORC_ERR_ARG;
    if (mode == 1 && !rand_words) return ORC_ERR_ARG;
    int err = ORC_OK;
    size_t esz = dtype == 0 ? 4 : 2;
#pragma omp parallel for schedule(dynamic, 1)
    for (int b = 0; b < batch; ++b) {
        const int *tk = tokens + (size_t)b * m_max;
        const int *pa = parent + (size_t)b * m_max;
        const int n = num_nodes[b];
        int *acc = accepted + (size_t)b * max_accept;
        for (int j = 0; j < max_accept; ++j) acc[j] = -1;
        int len = 0, cur = -1, e = ORC_OK;
        int bon = -1;
        while (1) {
            const char *row = (const char *)target_logits +
                              ((size_t)b * (m_max + 1) + (size_t)(cur + 1)) * row_stride * esz;
            int next = -1;
            if (mode == 0) {
                int g = argmax_row(row, dtype, V);
                if (g < 0) { e = ORC_ERR_DATA; break; }
                for (int x = 0; x < n; ++x)
                    if (pa[x] == cur && tk[x] == g) { next = x; break; }
                if (next < 0) bon = g;
            } else {
                float M = -INFINITY;
                for (int v = 0; v < V; ++v) M = fmaxf(M, elem_f32(row, dtype, v));
                double Wd = 0.0;
                for (int v = 0; v < V; ++v) Wd += weight_l(elem_f32(row, dtype, v), M, T);
                if (!isfinite(M) || !isfinite(Wd)) { e = ORC_ERR_DATA; break; }
                uint64_t R = (uint64_t)Wd;
                int removed[64];
                int nrem = 0;
                for (int x = 0; x < n && next < 0; ++x) {
                    if (pa[x] != cur) continue;
                    int t = tk[x];
                    int is_removed = 0;
                    for (int j = 0; j < nrem; ++j) if (removed[j] == t) is_removed = 1;
                    uint64_t wt = is_removed ? 0 : (uint64_t)weight_l(elem_f32(row, dtype, t), M, T);
                    uint64_t r = rand_words[(size_t)b * (m_max + 1) + x];
                    if ((u128)r * R < ((u128)wt << 32)) {
                        next = x;
                    } else {
                        R -= wt;
                        if (!is_removed && nrem < 64) removed[nrem++] = t;
                    }
                }
                if (next < 0) {
                    uint64_t rb = rand_words[(size_t)b * (m_max + 1) + m_max];
                    uint64_t s = (uint64_t)(((u128)rb * R) >> 32);
                    uint64_t cum = 0;
                    for (int v = 0; v < V; ++v) {
                        int is_removed = 0;
                        for (int j = 0; j < nrem; ++j) if (removed[j] == v) is_removed = 1;
                        if (is_removed) continue;
                        cum += (uint64_t)weight_l(elem_f32(row, dtype, v), M, T);
                        if (cum > s) { bon = v; break; }
                    }
                }
            }
            if (next < 0) break;
            if (len >= max_accept) { e = ORC_ERR_PATH; break; }
            acc[len++] = next;
            cur = next;
        }
        accept_len[b] = len;
        bonus[b] = bon;
        if (e != ORC_OK) {
#pragma omp critical
            err = e;
        }
    }
    return err;
}

/* bit length of x (0 for 0) */
static int bitlen128(u128 x)
{
    int n = 0;
    while (x) { ++n; x >>= 1; }
    return n;
}

/*
 * Recursive rejection sampling over drawn children (EAGLE-1 explainer,
 * "Verification": tokens accepted by the ratio of the target and draft
 * distributions, the rest discarded after a rejection and a token
 * resampled, leaving the target distribution unchanged).  The children of a
 * node are draws without replacement from its draft row's softmax q (the
 * sampled build); at node u with target weights P (row u + 1 at temperature
 * T) and draft weights Q (u's draft row, temperature 1), the children x in
 * draw order are tested:
 *   accept iff floor(r_x * Q(x) * SP / 2^32) < P(x) * SQ  (u < p(x) / q(x));
 *   otherwise P <- max(0, P * SQ - Q * SP) >> s, with s the shift that keeps
 *   the sum below 2^52 (the residual max(0, p - q), renormalised), and
 *   Q(x) <- 0 (q renormalised without x).  A child with Q(x) = 0 is rejected
 *   and changes nothing; a residual that sums to 0 leaves P unchanged.
 * With no child accepted the bonus is the inverse-CDF draw from P with
 * r = rand_words[b][m_max].  src_row [B][m_max] gives each node's draft row
 * (the root's is row 0); draft_logits [B][r_max][V].
 */
int orc_accept_rrs(float T, int batch, int m_max, int max_accept, int V, const void *target_logits,
                   const void *draft_logits, int r_max, int dtype, const int *tokens, const int *parent,
                   const int *src_row, const int *num_nodes, const uint32_t *rand_words, int *accepted,
                   int *accept_len, int *bonus)
{
    if (batch < 0 || m_max <= 0 || m_max > 64 || max_accept <= 0 || V <= 0 || V > (1 << 17) || !(T > 0.0f))
        return ORC_ERR_ARG;
    const size_t esz = dtype == 0 ? 4 : 2;
    int err = ORC_OK;
#pragma omp parallel for schedule(dynamic, 1)
    for (int b = 0; b < batch; ++b) {
        uint64_t *P = (uint64_t *)malloc(sizeof(uint64_t) * (size_t)V);
        uint64_t *Q = (uint64_t *)malloc(sizeof(uint64_t) * (size_t)V);
        uint64_t *Pn = (uint64_t *)malloc(sizeof(uint64_t) * (size_t)V);
        const int *tk = tokens + (size_t)b * m_max, *pa = parent + (size_t)b * m_max;
        const int *sr = src_row + (size_t)b * m_max;
        const uint32_t *rw = rand_words + (size_t)b * (m_max + 1);
        const int n = num_nodes[b];
        int *acc = accepted + (size_t)b * max_accept;
        for (int j = 0; j < max_accept; ++j) acc[j] = -1;
        int len = 0, cur = -1, bon = -1, e = ORC_OK;
        while (1) {
            /* target weights of the current node */
            const char *trow = (const char *)target_logits + ((size_t)b * (m_max + 1) + (size_t)(cur + 1)) * V * esz;
            float M = -INFINITY;
            for (int v = 0; v < V; ++v) M = fmaxf(M, elem_f32(trow, dtype, v));
            uint64_t SP = 0;
            for (int v = 0; v < V; ++v) {
                P[v] = (uint64_t)weight_l(elem_f32(trow, dtype, v), M, T);
                SP += P[v];
            }
            if (!isfinite(M) || SP == 0) { e = ORC_ERR_DATA; break; }
            int next = -1, has_children = 0;
            for (int x = 0; x < n; ++x) has_children |= pa[x] == cur;
            if (has_children) {
                const int dr = cur < 0 ? 0 : sr[cur];
                if (dr < 0 || dr >= r_max) { e = ORC_ERR_ARG; break; }
                const char *drow = (const char *)draft_logits + ((size_t)b * r_max + (size_t)dr) * V * esz;
                float Md = -INFINITY;
                for (int v = 0; v < V; ++v) Md = fmaxf(Md, elem_f32(drow, dtype, v));
                uint64_t SQ = 0;
                for (int v = 0; v < V; ++v) {
                    Q[v] = (uint64_t)weight_l(elem_f32(drow, dtype, v), Md, 1.0f);
                    SQ += Q[v];
                }
                for (int x = 0; x < n && next < 0; ++x) {
                    if (pa[x] != cur) continue;
                    const int t = tk[x];
                    const uint64_t q = Q[t], pt = P[t];
                    if (q == 0) continue;
                    if ((((u128)rw[x] * q * SP) >> 32) < (u128)pt * SQ) {
                        next = x;
                        break;
                    }
                    /* residual max(0, p - q) over the common denominator SP * SQ, shifted so
                       that its sum stays below 2^52 */
                    const int bl = bitlen128((u128)SP * SQ), sh = bl > 52 ? bl - 52 : 0;
                    uint64_t SPn = 0;
                    for (int v = 0; v < V; ++v) {
                        const u128 a = (u128)P[v] * SQ, c = (u128)Q[v] * SP;
                        Pn[v] = a > c ? (uint64_t)((a - c) >> sh) : 0;
                        SPn += Pn[v];
                    }
                    if (SPn > 0) {
                        for (int v = 0; v < V; ++v) P[v] = Pn[v];
                        SP = SPn;
                    }
                    Q[t] = 0;
                    SQ -= q;
                }
            }
            if (next < 0) {
                const uint64_t target = (uint64_t)(((u128)rw[m_max] * SP) >> 32);
                uint64_t cum = 0;
                for (int v = 0; v < V; ++v) {
                    cum += P[v];
                    if (cum > target) { bon = v; break; }
                }
                break;
            }
            if (len >= max_accept) { e = ORC_ERR_PATH; break; }
            acc[len++] = next;
            cur = next;
        }
        accept_len[b] = len;
        bonus[b] = bon;
        free(P);
        free(Q);
        free(Pn);
        if (e != ORC_OK) {
#pragma omp critical
            err = e;
        }
    }
    return err;
}

/* thread count the OpenMP runtime will use (for reporting) */
int orc_num_threads(void)
{
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        {
#ifdef _OPENMP
            extern int omp_get_num_threads(void);
            n = omp_get_num_threads();
#endif
        }
    }
    return n;
}
