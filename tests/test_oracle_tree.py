"""Pins for the oracle's dynamic draft tree (EAGLE-2 explainer, "Dynamic draft
tree construction" and its Python concept sketch) and ancestor mask ("Attention
mask adjustment").

Pins: a hand-derived golden example; the concept sketch's own special case
(every parent at a depth shares one children list) against brute force over
the full C-ary tree; invariants recomputed with
library sorts and exact integer weights; degenerate shapes that reduce to a
sort of one row or to a greedy chain; brute-force reflexive-transitive closure
for the mask.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import spec_emul
import synth
from conftest import to_np

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _hand():
    with open(os.path.join(GOLD, "hand_tree.json")) as f:
        return json.load(f)


def test_hand_example_tree_mask_greedy(orc):
    g = _hand()
    p = g["params"]
    logits = np.array(g["draft_logits"], np.float32)[None]
    t = orc.build_tree(logits, p["depth"], p["topk"], p["children"], p["m"])
    e = g["tree"]
    assert list(t["tokens"][0]) == e["tokens"]
    assert list(t["parent"][0]) == e["parent"]
    assert list(t["depth"][0]) == e["depth"]
    assert list(t["src_row"][0]) == e["src_row"]
    assert [float.fromhex(h) for h in e["score_hex"]] == list(t["score"][0])
    assert t["num_nodes"][0] == e["num_nodes"]
    anc, pos = orc.tree_mask(t["parent"], t["num_nodes"], [g["mask"]["prefix_len"]])
    assert [int(v) for v in anc[0]] == g["mask"]["anc"]
    assert list(pos[0]) == g["mask"]["pos"]
    for case in g["greedy_cases"]:
        tl = np.array(case["target_logits"], np.float32)[None]
        acc, alen, bon = orc.accept(0, tl, t["tokens"], t["parent"], t["num_nodes"], p["depth"])
        assert list(acc[0]) == case["accepted"], case["why"]
        assert alen[0] == case["accept_len"] and bon[0] == case["bonus"], case["why"]


# ---------------------------------------------------------------------------
# the concept sketch's special case: shared children per depth, against brute
# force over the full C-ary tree
# ---------------------------------------------------------------------------

def _brute_force_shared_children(per_depth, m, k, max_depth):
    """Every node of the full C-ary tree of depth max_depth, identified by its
    path of child ranks; V is the explicit product of the confidences along
    the path, multiplied root first.  A node of depth d >= 2 is generated iff
    its parent is generated and among the first k generated nodes of depth
    d - 1 in the order (V desc, creation asc), where creation order is
    (depth, the parent's rank in that order, child rank).  Returns the
    generated nodes' records and the first m of them in (V desc, creation asc)
    order."""
    C = len(per_depth[0])
    rec = {}                                    # path -> dict(V, depth, creation key, token)
    rank_in_depth = {}
    for d in range(1, max_depth + 1):
        if d - 1 >= len(per_depth):
            break
        if d == 1:
            gen = [(r,) for r in range(C)]
        else:
            gen = [p + (r,) for p in rec if len(p) == d - 1 and rank_in_depth[p] < k for r in range(C)]
        for p in gen:
            v = 1.0
            for depth_i, r in enumerate(p):
                v = v * per_depth[depth_i][r][1]
            parent_rank = rank_in_depth[p[:-1]] if d > 1 else 0
            rec[p] = dict(V=v, depth=d, key=(d, parent_rank, p[-1]), token=per_depth[d - 1][p[-1]][0])
        order = sorted(gen, key=lambda p: (-rec[p]["V"], rec[p]["key"]))
        for r, p in enumerate(order):
            rank_in_depth[p] = r
    ranked = sorted(rec, key=lambda p: (-rec[p]["V"], rec[p]["key"]))
    return rec, ranked[:m]


@pytest.mark.parametrize("seed,V,dt", [(0, 50, "f32"), (1, 300, "bf16"), (2, 1000, "f32"), (3, 40, "ties")])
def test_sketch_special_case_shared_children(orc, seed, V, dt):
    D, k, C, m = 4, 3, 4, 12
    rng = np.random.default_rng(seed)
    base = (rng.standard_normal((D, V)) * 2).astype(np.float32)
    if dt == "ties":
        # few distinct logits: equal confidences among siblings and equal V
        # across nodes, so the creation-order tie rule decides the ranking
        base = rng.integers(0, 3, size=(D, V)).astype(np.float32)
    R = 1 + (D - 1) * k
    rows = np.zeros((R, V), np.float32)
    rows[0] = base[0]
    for d in range(1, D):
        rows[1 + (d - 1) * k: 1 + d * k] = base[d]          # every parent at depth d shares a row
    if dt == "bf16":
        rows = torch.from_numpy(rows).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    t = orc.build_tree(rows[None], D, k, C, m)
    # the sketch consumes per-depth (token, conf) lists with conf = w / W of that row
    per_depth = []
    for d in range(D):
        r = 0 if d == 0 else 1 + (d - 1) * k
        M, W, ids, ws = spec_emul.row_stats(rows[r], C)
        per_depth.append([(int(i), w / W) for i, w in zip(ids, ws)])
    rec, chosen = _brute_force_shared_children(per_depth, m, k, D)
    assert len(chosen) == m
    assert all(p[:-1] in chosen for p in chosen if len(p) > 1)   # closed: adding ancestors adds nothing
    assert list(t["tokens"][0]) == [rec[p]["token"] for p in chosen]
    assert list(t["score"][0]) == [rec[p]["V"] for p in chosen]
    assert list(t["depth"][0]) == [rec[p]["depth"] for p in chosen]
    pos_of = {p: r for r, p in enumerate(chosen)}
    assert list(t["parent"][0]) == [-1 if len(p) == 1 else pos_of[p[:-1]] for p in chosen]


# ---------------------------------------------------------------------------
# invariants on random trees, recomputed independently
# ---------------------------------------------------------------------------

def _rows_np(w, seed):
    return to_np(synth.draft_logits(w, seed))


@pytest.mark.parametrize("base,seed,B", [(1, 11, 1), (2, 12, 2), (3, 13, 1)])
def test_tree_invariants(orc, base, seed, B):
    w = synth.small_workload(base, batch=B)
    logits = _rows_np(w, seed)
    t = orc.build_tree(logits, w.depth, w.topk, w.children, w.m, debug=True)
    D, k, C, m = w.depth, w.topk, w.children, w.m
    for b in range(B):
        cd = {kk: v[b] for kk, v in t["cand"].items()}
        N = int(cd["n"])
        assert N == C + (D - 1) * k * C
        stats = {}

        def row(r):
            if r not in stats:
                stats[r] = spec_emul.row_stats(logits[b, r], C)
            return stats[r]

        # (1) children = top-C of the parent's row; V = fl64(V_parent * fl64(w / W))
        sib_rank = {}
        for i in range(N):
            par = int(cd["parent"][i])
            r = 0 if par < 0 else int(cd["row"][par])
            assert r >= 0
            j = sib_rank.get(par, 0)
            sib_rank[par] = j + 1
            M, W, ids, ws = row(r)
            assert cd["token"][i] == ids[j]
            pv = 1.0 if par < 0 else float(cd["V"][par])
            assert cd["V"][i] == pv * (ws[j] / W)
            assert cd["depth"][i] == (1 if par < 0 else cd["depth"][par] + 1)
        # (2) expansion: the top-k of each depth by (V desc, creation asc) own rows 1+(d-1)k+p
        for d in range(1, D):
            at_d = [i for i in range(N) if cd["depth"][i] == d]
            top = sorted(at_d, key=lambda i: (-cd["V"][i], i))[:k]
            assert [int(cd["row"][i]) for i in top] == [1 + (d - 1) * k + p for p in range(len(top))]
            assert all(cd["row"][i] < 0 for i in at_d if i not in top)
        assert all(cd["row"][i] < 0 for i in range(N) if cd["depth"][i] == D)
        # (3) rerank: the selection is the first m of the total order, in that order
        order = sorted(range(N), key=lambda i: (-cd["V"][i], i))[:m]
        assert [int(cd["rank"][i]) for i in order] == list(range(m))
        assert sum(1 for i in range(N) if cd["rank"][i] >= 0) == m
        # (4) closed under ancestors, exactly m nodes
        for i in order:
            a = int(cd["parent"][i])
            while a >= 0:
                assert cd["rank"][a] >= 0
                a = int(cd["parent"][a])
        # (5) outputs are the selection in rank order
        assert t["num_nodes"][b] == m
        for r_, i in enumerate(order):
            assert t["tokens"][b, r_] == cd["token"][i]
            assert t["score"][b, r_] == cd["V"][i]
            assert t["depth"][b, r_] == cd["depth"][i]
            assert t["src_row"][b, r_] == cd["row"][i]
            par = int(cd["parent"][i])
            assert t["parent"][b, r_] == (-1 if par < 0 else cd["rank"][par])
            assert t["parent"][b, r_] < r_                      # rank order is topological
        # (6) V equals the product of confidences along the root path (any order)
        for r_ in range(m):
            cs, a = [], r_
            while a >= 0:
                par = int(t["parent"][b, a])
                pv = 1.0 if par < 0 else float(t["score"][b, par])
                cs.append(float(t["score"][b, a]) / pv if pv > 0 else 0.0)
                a = par
            assert math.isclose(math.prod(reversed(cs)), t["score"][b, r_], rel_tol=1e-13, abs_tol=1e-300)


def test_depth_one_is_top_m_of_root_row(orc):
    rng = np.random.default_rng(5)
    row = (rng.standard_normal((1, 1, 500)) * 2).astype(np.float32)
    t = orc.build_tree(row, 1, 4, 16, 9)
    M, W, ids, ws = spec_emul.row_stats(row[0, 0], 16)
    assert list(t["tokens"][0]) == list(ids[:9])
    assert list(t["score"][0]) == [x / W for x in ws[:9]]
    assert list(t["parent"][0]) == [-1] * 9


def test_k1_c1_tree_equals_chain(orc):
    w = synth.small_workload(2, batch=1)
    logits = _rows_np(w, 21)
    D = 6
    t = orc.build_tree(logits[:, :D], D, 1, 1, D)
    c = orc.build_tree(logits[:, :D], D, 1, 1, D, chain_k=D, kinds=[1])
    for kk in ("tokens", "parent", "depth", "score"):
        assert np.array_equal(t[kk], c[kk])
    assert list(t["parent"][0]) == [-1, 0, 1, 2, 3, 4]
    # chain tokens are row argmaxes (ties to the smallest id)
    for i in range(D):
        lf = spec_emul.to_f32(logits[0, i])
        assert c["tokens"][0, i] == int(np.flatnonzero(lf == lf.max())[0])


def test_m_equals_n_selects_everything(orc):
    rng = np.random.default_rng(6)
    D, k, C = 3, 2, 3
    R = 1 + (D - 1) * k
    N = C + (D - 1) * k * C
    rows = (rng.standard_normal((1, R, 40))).astype(np.float32)
    t = orc.build_tree(rows, D, k, C, N, debug=True)
    assert t["num_nodes"][0] == N and (t["cand"]["rank"][0][:N] >= 0).all()
    with pytest.raises(orc.OracleError):
        orc.build_tree(rows, D, k, C, N + 1)


def test_chain_mode_src_rows_and_padding(orc):
    w = synth.small_workload(5, batch=2, vocab=2000)
    logits = _rows_np(w, 31)
    t = orc.build_tree(logits, w.depth, w.topk, w.children, w.m, chain_k=7, kinds=[0, 1], m_max=60)
    assert t["num_nodes"].tolist() == [60, 7]
    assert list(t["src_row"][1, :7]) == [1, 2, 3, 4, 5, 6, -1]
    assert (t["tokens"][1, 7:] == -1).all() and (t["parent"][1, 7:] == -1).all()


# ---------------------------------------------------------------------------
# mask: reflexive-transitive closure of parent
# ---------------------------------------------------------------------------

def test_mask_is_ancestor_closure(orc):
    w = synth.small_workload(5, batch=4, vocab=3000)
    logits = _rows_np(w, 41)
    kinds = [0, 1, 0, 1]
    t = orc.build_tree(logits, w.depth, w.topk, w.children, w.m, chain_k=7, kinds=kinds, m_max=60)
    plen = np.array([100, 7, 1, 33], np.int32)
    anc, pos = orc.tree_mask(t["parent"], t["num_nodes"], plen)
    for b in range(4):
        n = int(t["num_nodes"][b])
        par = t["parent"][b]
        reach = np.eye(60, dtype=bool)
        for _ in range(64):                                  # closure by repeated composition
            step = reach.copy()
            for i in range(n):
                if par[i] >= 0:
                    step[i] |= reach[par[i]]
            reach = step
        for i in range(60):
            bits = int(anc[b, i])
            want = sum(1 << j for j in range(60) if i < n and reach[i, j])
            assert bits == want
            if i < n:
                assert bin(bits).count("1") == t["depth"][b, i]
                assert pos[b, i] == plen[b] + t["depth"][b, i] - 1
            else:
                assert pos[b, i] == -1
        if kinds[b] == 1:                                    # chain -> lower triangular
            assert [int(anc[b, i]) for i in range(7)] == [(1 << (i + 1)) - 1 for i in range(7)]


@pytest.mark.parametrize("base,seed,B,k", [(1, 21, 2, 10), (2, 22, 1, 4), (3, 23, 2, 1)])
def test_frontiers_follow_level_by_level_expansion(orc, base, seed, B, k):
    """The oracle's per-depth expanded nodes (what an incremental build returns
    after each level) equal a level-by-level restatement that sees only the
    rows of the nodes chosen so far: level 0 ranks the root row's top-C by V
    = w / W; level l ranks the children of level l - 1's frontier, in frontier
    order, by V = V_parent * w / W and (V desc, creation asc)."""
    w = synth.small_workload(base, batch=B, topk=k)
    logits = _rows_np(w, seed)
    D, C = w.depth, w.children
    tok, par, score = orc.tree_frontiers(logits, D, k, C, w.m)
    assert (tok[D - 1] == -1).all() and (par[D - 1] == -1).all()
    for b in range(B):
        front = [(1.0, None)]          # (V, row) of the nodes whose rows the next level brings
        for lv in range(D - 1):
            cands = []
            for p, (vp, r) in enumerate(front):
                M, W, ids, ws = spec_emul.row_stats(logits[b, 0 if lv == 0 else r], C)
                for j in range(C):
                    cands.append((vp * (ws[j] / W), len(cands), ids[j], -1 if lv == 0 else p))
            top = sorted(cands, key=lambda c: (-c[0], c[1]))[:k]
            assert [int(x) for x in tok[lv, b, :len(top)]] == [c[2] for c in top]
            assert [int(x) for x in par[lv, b, :len(top)]] == [c[3] for c in top]
            assert [float(x) for x in score[lv, b, :len(top)]] == [c[0] for c in top]
            assert (tok[lv, b, len(top):] == -1).all()
            front = [(c[0], 1 + lv * k + p) for p, c in enumerate(top)]


def _cand_conf(logits_b, cd, C):
    """c of every candidate (w / W of its parent's row at its sibling rank),
    from the Spec S restatement in spec_emul."""
    N = int(cd["n"])
    stats, conf, sib = {}, np.zeros(N), {}
    for i in range(N):
        q = int(cd["parent"][i])
        r = 0 if q < 0 else int(cd["row"][q])
        if r not in stats:
            stats[r] = spec_emul.row_stats(logits_b[r], C)
        j = sib.get(q, 0)
        sib[q] = j + 1
        _, W, ids, ws = stats[r]
        assert cd["token"][i] == ids[j]
        conf[i] = ws[j] / W
    return conf


@pytest.mark.parametrize("base,seed", [(1, 31), (2, 32), (3, 33)])
def test_no_rerank_policy_is_every_depths_top_k(orc, base, seed):
    """Policy 1 (V, no rerank): the nodes of depths < D are exactly the nodes
    the EAGLE-2 build expands (same V ranking), depth D adds its top-k by V;
    output depth by depth, rank order inside a depth."""
    w = synth.small_workload(base, batch=2)
    logits = _rows_np(w, seed)
    D, k, C = w.depth, w.topk, w.children
    t0 = orc.build_tree(logits, D, k, C, w.m, m_max=64, debug=True, policy=0)
    t1 = orc.build_tree(logits, D, k, C, w.m, m_max=64, debug=True, policy=1)
    for b in range(2):
        cd = {kk: v[b] for kk, v in t0["cand"].items()}
        N = int(cd["n"])
        want = []
        for d in range(1, D + 1):
            at_d = sorted([i for i in range(N) if cd["depth"][i] == d], key=lambda i: (-cd["V"][i], i))[:k]
            if d < D:
                assert all(cd["row"][i] >= 0 for i in at_d)   # the expanded nodes
            want += at_d
        n = int(t1["num_nodes"][b])
        assert n == len(want) == min(C, k) + (D - 1) * k
        assert t1["tokens"][b, :n].tolist() == [int(cd["token"][i]) for i in want]
        assert t1["score"][b, :n].tolist() == [float(cd["V"][i]) for i in want]
        assert all(t1["parent"][b, r] < r for r in range(n))
        assert (t1["tokens"][b, n:] == -1).all()


@pytest.mark.parametrize("base,seed", [(1, 41), (2, 42)])
def test_confidence_policies(orc, base, seed):
    """Policy 3 (c, no rerank): each depth's nodes are the top-k by c of the
    children of the previous depth's nodes.  Policy 2 (c, rerank): a closed
    tree of at most m nodes whose every node either ranks among the first by
    c or is an ancestor of one that does; with rows made flatter at every
    depth (c falls along every path), it is exactly the top-m by c."""
    w = synth.small_workload(base, batch=1)
    logits = _rows_np(w, seed)
    D, k, C, m = w.depth, w.topk, w.children, w.m
    t3 = orc.build_tree(logits, D, k, C, m, m_max=64, debug=True, policy=3)
    cd = {kk: v[0] for kk, v in t3["cand"].items()}
    conf = _cand_conf(logits[0], cd, C)
    N = int(cd["n"])
    front = [-1]
    sel3 = []
    for d in range(1, D + 1):
        at_d = [i for i in range(N) if cd["depth"][i] == d and int(cd["parent"][i]) in front]
        assert len(at_d) == sum(1 for i in range(N) if cd["depth"][i] == d)   # children of the kept nodes only
        top = sorted(at_d, key=lambda i: (-conf[i], i))[:k]
        sel3 += top
        front = top
    n3 = int(t3["num_nodes"][0])
    assert t3["tokens"][0, :n3].tolist() == [int(cd["token"][i]) for i in sel3]
    # policy 2 on rows whose top-C logits fall with the owner's depth (all
    # others 0): c falls along every path, so the c order is closed under
    # ancestors and the selection is the top-m by c
    rng = np.random.default_rng(seed)
    V = logits.shape[2]
    flat = np.zeros((1, logits.shape[1], V), np.float32)
    for r in range(flat.shape[1]):
        dr = 0 if r == 0 else 1 + (r - 1) // k
        flat[0, r, rng.choice(V, size=C, replace=False)] = 8.0 - 1.5 * dr
    t2 = orc.build_tree(flat, D, k, C, m, m_max=64, debug=True, policy=2)
    cd2 = {kk: v[0] for kk, v in t2["cand"].items()}
    conf2 = _cand_conf(flat[0], cd2, C)
    N2 = int(cd2["n"])
    par = cd2["parent"]
    assert all(conf2[i] < conf2[int(par[i])] for i in range(N2) if par[i] >= 0)
    order = sorted(range(N2), key=lambda i: (-conf2[i], i))[:m]
    n2 = int(t2["num_nodes"][0])
    assert n2 == m
    assert t2["tokens"][0, :n2].tolist() == [int(cd2["token"][i]) for i in order]
    # policy 2 on the original rows: closed, within m, nodes in selection order
    t2o = orc.build_tree(logits, D, k, C, m, m_max=64, debug=True, policy=2)
    n = int(t2o["num_nodes"][0])
    assert 0 < n <= m
    assert all(t2o["parent"][0, r] < r for r in range(n))


def test_confidence_rerank_hand_example(orc):
    """Policy 2 with a candidate whose missing ancestors do not fit: D = 3,
    k = 1, C = 2, vocabulary 4.  Root row: token 0 (c ~ .88), token 1 (~ .12);
    token 0's row: tokens 2 (~ .52) and 3 (~ .48); token 2's row: token 0
    (c ~ 1) and token 1.  By c the deepest token 0 comes first but needs its
    two ancestors: with m = 2 it is skipped, and tokens 0 then 2 are taken
    (depths 1 and 2); with m = 3 it fits, ancestors first."""
    logits = np.array([[[2.0, 0.0, -10.0, -10.0],
                        [-10.0, -10.0, 5.0, 4.9],
                        [10.0, -10.0, -10.0, -10.0]]], np.float32)
    t = orc.build_tree(logits, 3, 1, 2, 2, m_max=4, policy=2)
    assert t["num_nodes"][0] == 2
    assert t["tokens"][0, :2].tolist() == [0, 2] and t["parent"][0, :2].tolist() == [-1, 0]
    assert t["depth"][0, :2].tolist() == [1, 2]
    t = orc.build_tree(logits, 3, 1, 2, 3, m_max=4, policy=2)
    assert t["tokens"][0, :3].tolist() == [0, 2, 0] and t["parent"][0, :3].tolist() == [-1, 0, 1]
    assert t["depth"][0, :3].tolist() == [1, 2, 3]
    # no rerank by c: depth 1 keeps token 0, depth 2 token 2, depth 3 token 0
    t = orc.build_tree(logits, 3, 1, 2, 2, m_max=4, policy=3)
    assert t["num_nodes"][0] == 3 and t["tokens"][0, :3].tolist() == [0, 2, 0]


def test_template_chain_equals_chain_mode(orc):
    """A chain template (node i the top token of node i-1's row) is the chain
    mode of the build: same tokens, parents, depths, rows and V bit for bit."""
    w = synth.small_workload(2, batch=2, vocab=3000)
    logits = _rows_np(w, 61)[:, :7]
    K = 7
    tc = orc.build_tree(logits, 1, 1, 1, 1, chain_k=K, kinds=[1, 1], m_max=K)
    tt = orc.build_tree_template(logits, list(range(-1, K - 1)), [0] * K, children=4, m_max=K)
    for k in ("tokens", "parent", "depth", "score", "src_row", "num_nodes"):
        assert np.array_equal(tt[k], tc[k]), k


@pytest.mark.parametrize("seed", [62, 63])
def test_template_nodes_follow_their_parents_rows(orc, seed):
    """A random template: each node is the chosen rank of its parent's row
    (spec_emul restatement of Spec S), V the product of c from the root down,
    rows owned by the nodes with children in template order."""
    rng = np.random.default_rng(seed)
    C, n_t = 5, 30
    tp = [-1] + [int(rng.integers(-1, i)) for i in range(1, n_t)]
    tch = [int(rng.integers(0, C)) for _ in range(n_t)]
    internal = [i for i in range(n_t) if i in tp[i + 1:]]
    w = synth.small_workload(1, batch=2, vocab=1000)
    logits = _rows_np(w, seed)
    R = 1 + len(internal)
    if logits.shape[1] < R:
        logits = np.concatenate([logits] * (R // logits.shape[1] + 1), axis=1)
    logits = np.ascontiguousarray(logits[:, :R])
    t = orc.build_tree_template(logits, tp, tch, children=C, m_max=32)
    row_of = {i: 1 + q for q, i in enumerate(internal)}
    for b in range(2):
        V = {}
        for i in range(n_t):
            p = tp[i]
            r = 0 if p < 0 else row_of[p]
            _, W, ids, ws = spec_emul.row_stats(logits[b, r], C)
            V[i] = (1.0 if p < 0 else V[p]) * (ws[tch[i]] / W)
            assert t["tokens"][b, i] == ids[tch[i]]
            assert t["score"][b, i] == V[i]
            assert t["parent"][b, i] == p
            assert t["src_row"][b, i] == row_of.get(i, -1)
        assert t["num_nodes"][b] == n_t and (t["tokens"][b, n_t:] == -1).all()
