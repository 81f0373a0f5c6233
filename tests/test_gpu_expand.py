"""Incremental tree build through the C ABI: the draft rows given one level at
a time (eagle_tree_expand), then eagle_tree_finish.  Bit-exact against the
oracle: every level's frontier (the nodes whose rows the next level brings)
against the oracle's expanded nodes of that depth, and the finished tree
against both the oracle's tree and the one-shot eagle_build_tree over the
same rows.  Cases cover fp32 and bf16, the register and the streaming row
kernels (each side may take a different one), a depth whose frontier is
smaller than topk, depth 1, a restart in the same workspace, and the
out-of-order errors."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import eagle_tree_verification_draft_amd as E
import oracle
import synth
from conftest import to_np
from gpu_harness import say

pytestmark = pytest.mark.gpu

# (name, workload base, overrides)
CASES = [
    ("f32-v1000", 1, dict(batch=2)),
    ("bf16-v32000-b1", 2, dict(batch=1)),
    ("bf16-b8-k4", 3, dict(batch=8, topk=4, vocab=8000)),
    ("bf16-c3-k5", 2, dict(batch=3, children=3, topk=5, vocab=5000)),
    ("bf16-v128256-stream", 2, dict(batch=2, vocab=128256)),
    ("bf16-b8-one-shot-streams", 2, dict(batch=8, vocab=32000)),
    ("bf16-depth1", 2, dict(batch=2, depth=1, m=8, vocab=3000)),
]


def _workload(base, over):
    w = synth.small_workload(base, **over)
    w.kinds = [synth.TREE_DYNAMIC] * w.batch
    w.chain_k = 0
    return w


def _level_rows(draft, lv, k):
    if lv == 0:
        return draft[:, 0:1].contiguous()
    return draft[:, 1 + (lv - 1) * k:1 + lv * k].contiguous()


def _tree_bufs(w, dev):
    i32 = dict(dtype=torch.int32, device=dev)
    B, M = w.batch, w.m_max
    return dict(tokens=torch.empty((B, M), **i32), parent=torch.empty((B, M), **i32),
                depth=torch.empty((B, M), **i32), score=torch.empty((B, M), dtype=torch.float64, device=dev),
                src_row=torch.empty((B, M), **i32), num_nodes=torch.empty((B,), **i32))


def _incremental(w, p, draft, ws, dev="cuda", levels=None):
    """Runs the given levels (default all) and finish; returns (frontiers, tree)."""
    B, k = w.batch, w.topk
    fr = []
    for lv in (range(w.depth) if levels is None else levels):
        ft = torch.empty((B, k), dtype=torch.int32, device=dev)
        fp = torch.empty((B, k), dtype=torch.int32, device=dev)
        fs = torch.empty((B, k), dtype=torch.float64, device=dev)
        E.tree_expand(p, B, lv, _level_rows(draft, lv, k), ft, fp, fs, ws)
        fr.append((lv, ft, fp, fs))
    t = _tree_bufs(w, dev)
    E.tree_finish(p, B, t["tokens"], t["parent"], t["depth"], t["score"], t["src_row"], t["num_nodes"], ws)
    torch.cuda.synchronize()
    fr = [(lv, ft.cpu().numpy(), fp.cpu().numpy(), fs.cpu().numpy()) for lv, ft, fp, fs in fr]
    return fr, {kk: v.cpu().numpy() for kk, v in t.items()}


def _params(w):
    return E.TreeParams(w.depth, w.topk, w.children, w.m, 0, w.vocab, w.m_max, w.r_max)


def _workspace(p, B, dev="cuda"):
    ws = torch.empty(max(256, E.build_tree_workspace_size(p, B)), dtype=torch.uint8, device=dev)
    E.workspace_init(ws)
    return ws


@pytest.mark.parametrize("name,base,over", CASES, ids=[c[0] for c in CASES])
def test_incremental_equals_one_shot_and_oracle(name, base, over):
    w = _workload(base, over)
    say(f"[expand {name}] B={w.batch} V={w.vocab} D={w.depth} k={w.topk} C={w.children} m={w.m}")
    dev = "cuda"
    draft = synth.draft_logits(w, 31, device=dev)
    dn = to_np(draft)
    ot = oracle.build_tree(dn, w.depth, w.topk, w.children, w.m, m_max=w.m_max)
    otok, opar, oscore = oracle.tree_frontiers(dn, w.depth, w.topk, w.children, w.m, m_max=w.m_max)
    p = _params(w)
    ws = _workspace(p, w.batch)
    fr, tree = _incremental(w, p, draft, ws)
    assert E.read_errors(ws) == 0
    for lv, ft, fp, fs in fr:
        assert np.array_equal(ft, otok[lv]), (lv, ft, otok[lv])
        assert np.array_equal(fp, opar[lv]), lv
        assert np.array_equal(fs, oscore[lv]), lv
    for kk in ("tokens", "parent", "depth", "score", "src_row", "num_nodes"):
        assert np.array_equal(tree[kk], ot[kk]), kk
    # the one-shot build over the same rows, in its own workspace
    one = _tree_bufs(w, dev)
    ws1 = _workspace(p, w.batch)
    E.build_tree(p, w.batch, draft, None, one["tokens"], one["parent"], one["depth"], one["score"],
                 one["src_row"], one["num_nodes"], ws1)
    torch.cuda.synchronize()
    for kk in ("tokens", "parent", "depth", "score", "src_row", "num_nodes"):
        assert np.array_equal(one[kk].cpu().numpy(), tree[kk]), kk


def test_restart_in_the_same_workspace():
    w = _workload(2, dict(batch=3, vocab=6000))
    say("[expand restart]")
    p = _params(w)
    ws = _workspace(p, w.batch)
    for seed in (41, 42):
        draft = synth.draft_logits(w, seed, device="cuda")
        ot = oracle.build_tree(to_np(draft), w.depth, w.topk, w.children, w.m, m_max=w.m_max)
        _, tree = _incremental(w, p, draft, ws)
        assert E.read_errors(ws) == 0
        for kk in ("tokens", "parent", "score", "num_nodes"):
            assert np.array_equal(tree[kk], ot[kk]), (seed, kk)


def test_levels_out_of_order_are_reported():
    w = _workload(2, dict(batch=2, vocab=3000))
    say("[expand out of order]")
    p = _params(w)
    draft = synth.draft_logits(w, 43, device="cuda")
    # level 2 right after level 0: an empty frontier and the TREE bit
    ws = _workspace(p, w.batch)
    fr, tree = _incremental(w, p, draft, ws, levels=[0, 2])
    assert E.read_errors(ws) & E.DEVERR_TREE
    assert (fr[1][1] == -1).all()
    # finish after levels 0..2 of 6: every sequence gets an empty tree
    assert (tree["num_nodes"] == 0).all() and (tree["tokens"] == -1).all()
    ws = _workspace(p, w.batch)
    _, tree = _incremental(w, p, draft, ws, levels=[0, 1, 2])
    assert E.read_errors(ws) == E.DEVERR_TREE
    assert (tree["num_nodes"] == 0).all() and (tree["parent"] == -1).all()
    # a restart at level 0 then succeeds in the same workspace
    ot = oracle.build_tree(to_np(draft), w.depth, w.topk, w.children, w.m, m_max=w.m_max)
    _, tree = _incremental(w, p, draft, ws)
    assert E.read_errors(ws) == 0
    assert np.array_equal(tree["tokens"], ot["tokens"]) and np.array_equal(tree["score"], ot["score"])
