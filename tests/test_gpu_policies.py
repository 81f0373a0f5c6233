"""Tree-policy ablations (confidence ranking, no rerank) through the C ABI
against the oracle, bit-exact: trees from eagle_build_tree, masks from
eagle_build_tree_mask, and the incremental build's frontiers and tree, for
every policy, on fp32 and bf16 rows, register and streaming row kernels, and
mixed trees and chains."""
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

M_MAX = 64
CASES = [
    ("f32-v1000", 1, dict(batch=2)),
    ("bf16-v32000", 2, dict(batch=2)),
    ("bf16-b8-stream", 3, dict(batch=8, vocab=70001)),
    ("bf16-mixed-chains", 5, dict(batch=4, vocab=5000, kinds=[0, 1, 0, 1])),
    ("bf16-k4-c6", 2, dict(batch=3, topk=4, children=6, m=24, vocab=3000)),
]
POLICIES = [E.EAGLE_POLICY_NO_RERANK, E.EAGLE_POLICY_CONF, E.EAGLE_POLICY_CONF_NO_RERANK]


def _params(w, policy):
    return E.TreeParams(w.depth, w.topk, w.children, w.m, w.chain_k, w.vocab, M_MAX, w.r_max, policy)


def _bufs(B, dev="cuda"):
    i32 = dict(dtype=torch.int32, device=dev)
    return dict(tokens=torch.empty((B, M_MAX), **i32), parent=torch.empty((B, M_MAX), **i32),
                depth=torch.empty((B, M_MAX), **i32), score=torch.empty((B, M_MAX), dtype=torch.float64, device=dev),
                src_row=torch.empty((B, M_MAX), **i32), num_nodes=torch.empty((B,), **i32))


def _workspace(p, B):
    ws = torch.empty(max(256, E.build_tree_workspace_size(p, B)), dtype=torch.uint8, device="cuda")
    E.workspace_init(ws)
    return ws


def _check_tree(got, ot):
    for k in ("tokens", "parent", "depth", "score", "src_row", "num_nodes"):
        g = got[k].cpu().numpy() if torch.is_tensor(got[k]) else got[k]
        assert np.array_equal(g, ot[k]), k


@pytest.mark.parametrize("policy", POLICIES)
@pytest.mark.parametrize("name,base,over", CASES, ids=[c[0] for c in CASES])
def test_policy_build_and_mask(name, base, over, policy):
    w = synth.small_workload(base, **over)
    say(f"[policy {policy} {name}] B={w.batch} V={w.vocab} D={w.depth} k={w.topk} C={w.children} m={w.m}")
    draft = synth.draft_logits(w, 51, device="cuda")
    kinds = synth.kinds_tensor(w, "cuda")
    ot = oracle.build_tree(to_np(draft), w.depth, w.topk, w.children, w.m, chain_k=w.chain_k, kinds=w.kinds,
                           m_max=M_MAX, policy=policy)
    p = _params(w, policy)
    t = _bufs(w.batch)
    ws = _workspace(p, w.batch)
    E.build_tree(p, w.batch, draft, kinds, t["tokens"], t["parent"], t["depth"], t["score"], t["src_row"],
                 t["num_nodes"], ws)
    torch.cuda.synchronize()
    assert E.read_errors(ws) == 0
    _check_tree(t, ot)
    # the fused call: same tree, and the masks of it
    plen = torch.randint(1, 5000, (w.batch,), dtype=torch.int32, device="cuda")
    anc = torch.empty((w.batch, M_MAX), dtype=torch.int64, device="cuda")
    pos = torch.empty((w.batch, M_MAX), dtype=torch.int32, device="cuda")
    t2 = _bufs(w.batch)
    E.build_tree_mask(p, w.batch, draft, kinds, plen, t2["tokens"], t2["parent"], t2["depth"], t2["score"],
                      t2["src_row"], t2["num_nodes"], anc, pos, ws)
    torch.cuda.synchronize()
    _check_tree(t2, ot)
    oanc, opos = oracle.tree_mask(ot["parent"], ot["num_nodes"], plen.cpu().numpy())
    assert np.array_equal(anc.cpu().numpy().view(np.uint64), oanc)
    assert np.array_equal(pos.cpu().numpy(), opos)


@pytest.mark.parametrize("policy", POLICIES)
def test_policy_incremental_build(policy):
    w = synth.small_workload(2, batch=3, vocab=6000)
    w.kinds = [synth.TREE_DYNAMIC] * 3
    say(f"[policy {policy} incremental]")
    draft = synth.draft_logits(w, 52, device="cuda")
    dn = to_np(draft)
    ot = oracle.build_tree(dn, w.depth, w.topk, w.children, w.m, m_max=M_MAX, policy=policy)
    ftok, fpar, fsc = oracle.tree_frontiers(dn, w.depth, w.topk, w.children, w.m, m_max=M_MAX, policy=policy)
    p = E.TreeParams(w.depth, w.topk, w.children, w.m, 0, w.vocab, M_MAX, w.r_max, policy)
    ws = _workspace(p, w.batch)
    k = w.topk
    for lv in range(w.depth):
        rows = draft[:, 0:1] if lv == 0 else draft[:, 1 + (lv - 1) * k:1 + lv * k]
        ft = torch.empty((w.batch, k), dtype=torch.int32, device="cuda")
        fp = torch.empty_like(ft)
        fs = torch.empty((w.batch, k), dtype=torch.float64, device="cuda")
        E.tree_expand(p, w.batch, lv, rows.contiguous(), ft, fp, fs, ws)
        torch.cuda.synchronize()
        assert np.array_equal(ft.cpu().numpy(), ftok[lv]), lv
        assert np.array_equal(fp.cpu().numpy(), fpar[lv]), lv
        assert np.array_equal(fs.cpu().numpy(), fsc[lv]), lv
    t = _bufs(w.batch)
    E.tree_finish(p, w.batch, t["tokens"], t["parent"], t["depth"], t["score"], t["src_row"], t["num_nodes"], ws)
    torch.cuda.synchronize()
    assert E.read_errors(ws) == 0
    _check_tree(t, ot)
