"""GPU parity over seeded random shapes: every output of the step against the
oracle for configurations drawn across the library's limits (dtype, GQA
ratio, tree depth / expansion / children / rerank size, chains of any
length, paged caches of every supported page size or contiguous ones,
ragged and empty prefixes, poisoned tails, greedy and sampled acceptance).

The same seeded draws cover the other entry points: every tree policy and
the incremental build, sampled children with recursive rejection sampling,
the KV commit, the parallel-draft inputs and EAGLE-1 templates.

The draws are fixed by their seeds, so every run checks the same cases.
Trees, masks, accepts and commits are compared bit for bit; attention row
by row for every (node, head) within the tolerance of its dtype.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import pytest
import torch

import eagle_tree_verification_draft_amd as E
import oracle
import synth
from conftest import to_np
from gpu_harness import (BF16_TOL, F32_TOL, assert_accept_equal, assert_tree_equal, check_attn_rows, make_case,
                         sample_rows,
                         oracle_mask, run_gpu, say)

pytestmark = pytest.mark.gpu

N_CASES = 64


def random_workload(i: int) -> synth.Workload:
    rng = np.random.default_rng(7000 + i)
    fp32 = rng.random() < 0.25
    if fp32:
        w = dataclasses.replace(synth.workload(1))
        w.head_dim = int(rng.choice([64, 128]))
        w.block_size = int(rng.choice([0, 16, 32]))
    else:
        w = dataclasses.replace(synth.workload(2))
        w.block_size = int(rng.choice([0, 8, 16, 24, 32, 64]))
    kv = int(rng.choice([1, 2, 4, 8]))
    g = int(rng.choice([1, 2, 4, 8]))
    w.num_kv_heads, w.num_q_heads = kv, kv * g
    # tree shape within the limits: rows 1 + (D-1)k <= 128, candidates
    # C + (D-1)kC <= 1024, m <= min(64, candidates generated) (a depth with
    # fewer than k nodes expands all of them)
    while True:
        depth = int(rng.integers(1, 7))
        children = int(rng.integers(1, 17))
        topk = int(rng.integers(1, 17))
        rows = 1 + (depth - 1) * topk
        cand = children + (depth - 1) * topk * children
        if rows <= 128 and cand <= 1024:
            break
    gen, nd = 0, children
    for _ in range(depth):
        gen += nd
        nd = min(topk, nd) * children
    w.depth, w.children, w.topk = depth, children, topk
    w.m = int(rng.integers(1, min(64, gen) + 1))
    w.batch = int(rng.integers(1, 4))
    w.chain_k = int(rng.integers(1, 65)) if rng.random() < 0.5 else 0
    w.kinds = [int(rng.random() < 0.5) if w.chain_k else 0 for _ in range(w.batch)]
    if synth.TREE_DYNAMIC not in w.kinds:
        # the tree parameters are validated whatever the kinds (batches of
        # chains only are covered by the fixed cases)
        w.kinds[0] = synth.TREE_DYNAMIC
    if synth.TREE_CHAIN not in w.kinds:
        w.chain_k = 0   # chain_k is bounded by the m_max and r_max of the batch's kinds
    w.vocab = int(rng.integers(max(children, 16), 9000))
    lo = int(rng.integers(0, 2000))
    w.prefix = (lo, int(rng.integers(lo, 2600)))
    w.poison_tail = bool(rng.random() < 0.5)
    w.accept_mode = synth.ACCEPT_SAMPLE if rng.random() < 0.4 else synth.ACCEPT_GREEDY
    w.temperature = float(rng.choice([1.0, 0.7]))
    w.target_kind = "draft_plus_noise"
    w.name = f"random-{i}"
    return w


@pytest.fixture(scope="module", params=range(N_CASES))
def random_case(request):
    w = random_workload(request.param)
    say(f"[random {request.param}] {w}")
    c = make_case(w, seed=100 + request.param, plant=(w.accept_mode == synth.ACCEPT_GREEDY))
    run_gpu(c)
    return c


def test_random_shape_all_outputs(random_case):
    c = random_case
    assert_tree_equal(c)
    anc, pos = oracle_mask(c)
    assert np.array_equal(c.step.anc.cpu().numpy().view(np.uint64), anc)
    assert np.array_equal(c.step.pos.cpu().numpy(), pos)
    sel = [(b, i, h) for b in range(c.w.batch) for i in range(int(c.otree["num_nodes"][b]))
           for h in range(c.w.num_q_heads)]
    tol = BF16_TOL if c.w.dtype == torch.bfloat16 else F32_TOL
    check_attn_rows(c, sel, tol)
    assert_accept_equal(c)
    assert c.step.errors() == 0


# ---------------------------------------------------------------------------
# tree policies and the incremental build over random tree shapes
# ---------------------------------------------------------------------------
N_TREES = 32
M_OUT = 64   # output width (m_max) of these calls


def random_tree_shape(i: int):
    rng = np.random.default_rng(8000 + i)
    w = dataclasses.replace(synth.workload(1 if rng.random() < 0.25 else 2))
    while True:
        depth = int(rng.integers(1, 7))
        children = int(rng.integers(1, 17))
        topk = int(rng.integers(1, 17))
        if 1 + (depth - 1) * topk <= 128 and children + (depth - 1) * topk * children <= 1024:
            break
    gen, per_depth, nd = 0, 0, children
    for _ in range(depth):
        gen += nd
        per_depth += min(topk, nd)
        nd = min(topk, nd) * children
    w.depth, w.children, w.topk = depth, children, topk
    w.m = int(rng.integers(1, min(M_OUT, gen) + 1))
    w.batch = int(rng.integers(1, 5))
    w.kinds = [synth.TREE_DYNAMIC] * w.batch
    w.chain_k = 0
    w.vocab = int(rng.integers(max(children, 16), 9000))
    policies = [E.EAGLE_POLICY_EAGLE2, E.EAGLE_POLICY_CONF]
    if per_depth <= M_OUT:   # a tree without rerank keeps every depth's first k
        policies += [E.EAGLE_POLICY_NO_RERANK, E.EAGLE_POLICY_CONF_NO_RERANK]
    return w, policies


def _tree_bufs(B):
    i32 = dict(dtype=torch.int32, device="cuda")
    return dict(tokens=torch.empty((B, M_OUT), **i32), parent=torch.empty((B, M_OUT), **i32),
                depth=torch.empty((B, M_OUT), **i32),
                score=torch.empty((B, M_OUT), dtype=torch.float64, device="cuda"),
                src_row=torch.empty((B, M_OUT), **i32), num_nodes=torch.empty((B,), **i32))


def _assert_tree(t, ot):
    for k in ("tokens", "parent", "depth", "score", "src_row", "num_nodes"):
        assert np.array_equal(t[k].cpu().numpy(), ot[k]), k


@pytest.mark.parametrize("i", range(N_TREES))
def test_random_tree_policies_and_incremental_build(i):
    w, policies = random_tree_shape(i)
    say(f"[random tree {i}] B={w.batch} V={w.vocab} D={w.depth} k={w.topk} C={w.children} m={w.m} "
        f"policies={policies} {w.dtype}")
    draft = synth.draft_logits(w, 300 + i, device="cuda")
    dn = to_np(draft)
    kinds = synth.kinds_tensor(w, "cuda")
    for policy in policies:
        ot = oracle.build_tree(dn, w.depth, w.topk, w.children, w.m, kinds=w.kinds, m_max=M_OUT, policy=policy)
        p = E.TreeParams(w.depth, w.topk, w.children, w.m, 0, w.vocab, M_OUT, w.r_max, policy)
        ws = torch.empty(max(256, E.build_tree_workspace_size(p, w.batch)), dtype=torch.uint8, device="cuda")
        E.workspace_init(ws)
        # one-shot build with its masks
        t = _tree_bufs(w.batch)
        plen = torch.randint(0, 3000, (w.batch,), dtype=torch.int32, device="cuda")
        anc = torch.empty((w.batch, M_OUT), dtype=torch.int64, device="cuda")
        pos = torch.empty((w.batch, M_OUT), dtype=torch.int32, device="cuda")
        E.build_tree_mask(p, w.batch, draft, kinds, plen, t["tokens"], t["parent"], t["depth"], t["score"],
                          t["src_row"], t["num_nodes"], anc, pos, ws)
        torch.cuda.synchronize()
        assert E.read_errors(ws) == 0, policy
        _assert_tree(t, ot)
        oanc, opos = oracle.tree_mask(ot["parent"], ot["num_nodes"], plen.cpu().numpy())
        assert np.array_equal(anc.cpu().numpy().view(np.uint64), oanc)
        assert np.array_equal(pos.cpu().numpy(), opos)
        # the same tree built one depth at a time
        ftok, fpar, fsc = oracle.tree_frontiers(dn, w.depth, w.topk, w.children, w.m, m_max=M_OUT, policy=policy)
        k = w.topk
        for lv in range(w.depth):
            rows = draft[:, 0:1] if lv == 0 else draft[:, 1 + (lv - 1) * k:1 + lv * k]
            ft = torch.empty((w.batch, k), dtype=torch.int32, device="cuda")
            fp = torch.empty_like(ft)
            fs = torch.empty((w.batch, k), dtype=torch.float64, device="cuda")
            E.tree_expand(p, w.batch, lv, rows.contiguous(), ft, fp, fs, ws)
            torch.cuda.synchronize()
            assert np.array_equal(ft.cpu().numpy(), ftok[lv]), (policy, lv)
            assert np.array_equal(fp.cpu().numpy(), fpar[lv]), (policy, lv)
            assert np.array_equal(fs.cpu().numpy(), fsc[lv]), (policy, lv)
        t2 = _tree_bufs(w.batch)
        E.tree_finish(p, w.batch, t2["tokens"], t2["parent"], t2["depth"], t2["score"], t2["src_row"],
                      t2["num_nodes"], ws)
        torch.cuda.synchronize()
        assert E.read_errors(ws) == 0, policy
        _assert_tree(t2, ot)


# ---------------------------------------------------------------------------
# sampled children and recursive rejection sampling over random shapes
# ---------------------------------------------------------------------------
N_SAMPLED = 24


def random_sampled_shape(i: int):
    rng = np.random.default_rng(9000 + i)
    dtype = torch.float32 if rng.random() < 0.3 else torch.bfloat16
    while True:
        D = int(rng.integers(1, 5))
        k = int(rng.integers(1, 5))
        C = int(rng.integers(1, 17))
        n_all, nd = 0, C
        for _ in range(D):
            n_all += nd
            nd = min(k, nd) * C
        if n_all <= 64 and 1 + (D - 1) * k <= 128:   # the sampled tree keeps every candidate
            break
    V = int(rng.choice([int(rng.integers(max(C, 2), 200)), int(rng.integers(200, 40000)),
                        int(rng.integers(65537, 1 << 17))]))
    B = int(rng.integers(1, 7))
    T = float(rng.choice([1.0, 0.7, 0.9, 1.3]))
    return rng, dtype, B, V, D, k, C, T


@pytest.mark.parametrize("i", range(N_SAMPLED))
def test_random_sampled_build_and_rrs(i):
    from test_gpu_rrs import _gpu_build, _gpu_rrs, _words
    rng, dtype, B, V, D, k, C, T = random_sampled_shape(i)
    say(f"[random sampled {i}] {dtype} B={B} V={V} D={D} k={k} C={C} T={T}")
    R = 1 + (D - 1) * k
    draft_f = (rng.standard_normal((B, R, V)) * float(rng.choice([0.5, 1.5, 3.0]))).astype(np.float32)
    draft = torch.from_numpy(draft_f).to(dtype).to("cuda")
    cw = _words(rng, (B, R, C))
    t, N, errs = _gpu_build(draft, D, k, C, cw)
    assert errs == 0
    ot = oracle.build_tree(to_np(draft), D, k, C, 1, m_max=N, child_words=cw)
    _assert_tree_n(t, ot)
    tgt = np.empty((B, N + 1, V), np.float32)
    tgt[:, 0] = draft_f[:, 0]
    for b in range(B):
        for j in range(N):
            r = ot["src_row"][b, j]
            tgt[b, j + 1] = draft_f[b, r] if r >= 0 else draft_f[b, 0]
    tgt += (rng.standard_normal(tgt.shape) * float(rng.choice([0.2, 0.5, 1.0]))).astype(np.float32)
    target = torch.from_numpy(tgt).to(dtype).to("cuda")
    words = _words(rng, (B, N + 1))
    o_acc, o_len, o_bon = oracle.accept_rrs(to_np(target), to_np(draft), ot["tokens"], ot["parent"], ot["src_row"],
                                            ot["num_nodes"], D, words, T=T)
    acc, alen, bon, errs = _gpu_rrs(target, draft, t, N, D, words, T)
    assert errs == 0
    assert np.array_equal(alen, o_len) and np.array_equal(acc, o_acc) and np.array_equal(bon, o_bon)


def _assert_tree_n(t, ot):
    for k in ("tokens", "parent", "depth", "score", "src_row", "num_nodes"):
        assert np.array_equal(t[k].cpu().numpy(), ot[k]), k


# ---------------------------------------------------------------------------
# KV commit over random cache shapes
# ---------------------------------------------------------------------------
N_COMMIT = 24


@pytest.mark.parametrize("i", range(N_COMMIT))
def test_random_kv_commit(i):
    from test_gpu_commit import _compare, _inputs, _oracle, _run
    rng = np.random.default_rng(9500 + i)
    if rng.random() < 0.3:
        dtype, d = torch.float32, int(rng.choice([64, 128]))
        bs = int(rng.choice([0, 16, 32]))
    else:
        dtype, d = torch.bfloat16, 128
        bs = int(rng.choice([0, 8, 16, 24, 32, 64]))
    B = int(rng.integers(1, 9))
    M = int(rng.integers(1, 65))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    P = int(rng.integers(M, 600))
    if dtype == torch.bfloat16 and bs == 0:
        P = (P + 7) // 8 * 8
    max_accept = int(rng.integers(1, M + 1))
    name = f"random-commit-{i}"
    say(f"[{name}] {dtype} bs={bs} B={B} M={M} Hkv={Hkv} d={d} capacity={P} max_accept={max_accept}")
    x = _inputs(name, dtype, bs, B, M, Hkv, d, P, max_accept)
    _compare(_run(x, dtype, bs, M, Hkv, d, P), _oracle(x))


# ---------------------------------------------------------------------------
# parallel-draft inputs over random shapes
# ---------------------------------------------------------------------------
N_PDRAFT = 16


@pytest.mark.parametrize("i", range(N_PDRAFT))
def test_random_pdraft_prepare(i):
    from test_gpu_pdraft import _compare, _inputs
    rng = np.random.default_rng(9700 + i)
    dtype = torch.float32 if rng.random() < 0.3 else torch.bfloat16
    B = int(rng.integers(1, 65))
    M = int(rng.integers(1, 65))
    MA = int(rng.integers(1, M + 1))
    H = int(rng.choice([8, 64, 128, 1000, 4096, 5120]))
    K = int(rng.integers(1, 9))
    name = f"random-pdraft-{i}"
    say(f"[{name}] {dtype} B={B} M={M} max_accept={MA} hidden={H} K={K}")
    _compare(_inputs(name, B, M, MA, H, dtype), K, 128255, dtype)


# ---------------------------------------------------------------------------
# EAGLE-1 static templates over random shapes
# ---------------------------------------------------------------------------
N_TEMPLATE = 16


@pytest.mark.parametrize("i", range(N_TEMPLATE))
def test_random_template(i):
    from test_gpu_template import _run, _template
    rng = np.random.default_rng(9900 + i)
    base = 1 if rng.random() < 0.3 else 2
    n = int(rng.integers(1, 65))
    C = int(rng.integers(1, 17))
    B = int(rng.integers(1, 5))
    V = int(rng.choice([int(rng.integers(max(C, 16), 3000)), int(rng.integers(3000, 40000)),
                        int(rng.integers(65537, 1 << 17))]))
    tp, tc = _template(9900 + i, n, C)
    R = 1 + sum(1 for j in range(n) if j in tp[j + 1:])
    say(f"[random template {i}] base={base} B={B} V={V} nodes={n} C={C} rows={R}")
    w = synth.small_workload(base, batch=B, vocab=V)
    w.depth, w.topk = 1, 1
    draft = synth.draft_logits(w, 400 + i, device="cuda")
    while draft.shape[1] < R:
        draft = torch.cat([draft, draft], dim=1)
    draft = draft[:, :R].contiguous()
    ot = oracle.build_tree_template(to_np(draft), tp, tc, children=C, m_max=64)
    got, errs = _run(draft, tp, tc, C, V, 64, R)
    assert errs == 0
    for k in ("tokens", "parent", "depth", "score", "src_row", "num_nodes"):
        assert np.array_equal(got[k], ot[k]), k


# ---------------------------------------------------------------------------
# larger random attention shapes (key splits, merge, longest-first order),
# with planted draft keys so that the check sees the tree at long prefixes
# ---------------------------------------------------------------------------
N_LARGE = 8


def random_large_workload(i: int) -> synth.Workload:
    rng = np.random.default_rng(9800 + i)
    w = dataclasses.replace(synth.workload(5))
    kv = int(rng.choice([2, 4, 8]))
    g = int(rng.choice([1, 2, 4, 8]))
    w.num_kv_heads, w.num_q_heads = kv, kv * g
    w.block_size = int(rng.choice([0, 16, 32, 64]))
    w.batch = int(rng.integers(4, 25))
    w.m = int(rng.integers(20, 65))
    w.chain_k = int(rng.integers(1, 9))
    w.kinds = [int(rng.random() < 0.5) for _ in range(w.batch)]
    w.kinds[0] = synth.TREE_DYNAMIC
    w.vocab = int(rng.integers(2000, 6000))
    lo = int(rng.integers(500, 8000))
    w.prefix = (lo, int(rng.integers(lo + 1, 24000)))
    w.poison_tail = bool(rng.random() < 0.5)
    w.name = f"random-large-{i}"
    return w


@pytest.mark.parametrize("i", range(N_LARGE))
def test_random_large_attention_planted(i):
    w = random_large_workload(i)
    say(f"[random large {i}] {w}")
    c = make_case(w, seed=500 + i)
    c.attn = synth.plant_draft_keys(c.attn, w, c.seed)
    run_gpu(c)
    assert_tree_equal(c)
    rng = np.random.default_rng(600 + i)
    sel = sample_rows(c, 96, rng)
    mx, rl2 = check_attn_rows(c, sel, BF16_TOL, power=0.1)
    say(f"[random large {i}] max-abs {mx:.3g}, relative L2 {rl2:.3g}")
    assert rl2 <= 1e-2
    assert_accept_equal(c)
    assert c.step.errors() == 0
