"""EAGLE-1 static template trees through the C ABI against the oracle,
bit-exact: random templates, a chain template (equal to the chain mode) and a
star template, fp32 and bf16 rows, register and streaming row kernels, and an
invalid template (reported, empty trees)."""
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


def _template(seed, n, C):
    rng = np.random.default_rng(seed)
    tp = [-1] + [int(rng.integers(-1, i)) for i in range(1, n)]
    tc = [int(rng.integers(0, C)) for _ in range(n)]
    return tp, tc


def _run(draft, tp, tc, C, V, m_max, r_max):
    B = draft.shape[0]
    p = E.TreeParams(1, 1, C, 1, 0, V, m_max, r_max, 0)
    ws = torch.empty(max(256, E.build_tree_workspace_size(p, B)), dtype=torch.uint8, device="cuda")
    E.workspace_init(ws)
    i32 = dict(dtype=torch.int32, device="cuda")
    t = dict(tokens=torch.empty((B, m_max), **i32), parent=torch.empty((B, m_max), **i32),
             depth=torch.empty((B, m_max), **i32), score=torch.empty((B, m_max), dtype=torch.float64, device="cuda"),
             src_row=torch.empty((B, m_max), **i32), num_nodes=torch.empty((B,), **i32))
    E.build_tree_template(p, B, draft, torch.tensor(tp, **i32), torch.tensor(tc, **i32), t["tokens"], t["parent"],
                          t["depth"], t["score"], t["src_row"], t["num_nodes"], ws)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in t.items()}, E.read_errors(ws)


# (name, workload base, batch, vocab, template nodes, children, seed)
CASES = [
    ("f32-v1000-n26", 1, 2, 1000, 26, 4, 71),
    ("bf16-v32000-n60", 2, 2, 32000, 60, 10, 72),
    ("bf16-v70001-stream-n40", 2, 3, 70001, 40, 8, 73),
    ("bf16-v3000-n64", 2, 4, 3000, 64, 16, 74),
]


@pytest.mark.parametrize("name,base,B,V,n,C,seed", CASES, ids=[c[0] for c in CASES])
def test_template_matches_oracle(name, base, B, V, n, C, seed):
    say(f"[template {name}]")
    tp, tc = _template(seed, n, C)
    R = 1 + sum(1 for i in range(n) if i in tp[i + 1:])
    w = synth.small_workload(base, batch=B, vocab=V)
    draft = synth.draft_logits(w, seed, device="cuda")
    while draft.shape[1] < R:
        draft = torch.cat([draft, draft], dim=1)
    draft = draft[:, :R].contiguous()
    ot = oracle.build_tree_template(to_np(draft), tp, tc, children=C, m_max=64)
    got, errs = _run(draft, tp, tc, C, V, 64, R)
    assert errs == 0
    for k in ("tokens", "parent", "depth", "score", "src_row", "num_nodes"):
        assert np.array_equal(got[k], ot[k]), k


def test_chain_and_star_templates():
    say("[template chain and star]")
    w = synth.small_workload(2, batch=2, vocab=5000)
    draft = synth.draft_logits(w, 75, device="cuda")
    K = 7
    chain = oracle.build_tree(to_np(draft[:, :K]), 1, 1, 1, 1, chain_k=K, kinds=[1, 1], m_max=K)
    got, errs = _run(draft[:, :K].contiguous(), list(range(-1, K - 1)), [0] * K, 3, 5000, K, K)
    assert errs == 0
    for k in ("tokens", "parent", "depth", "score", "src_row", "num_nodes"):
        assert np.array_equal(got[k], chain[k]), k
    star = oracle.build_tree_template(to_np(draft[:, :1]), [-1] * 10, list(range(10)), children=10, m_max=10)
    got, errs = _run(draft[:, :1].contiguous(), [-1] * 10, list(range(10)), 10, 5000, 10, 1)
    assert errs == 0 and np.array_equal(got["tokens"], star["tokens"]) and np.array_equal(got["score"], star["score"])


def test_invalid_template_is_reported():
    say("[template invalid]")
    w = synth.small_workload(2, batch=2, vocab=3000)
    draft = synth.draft_logits(w, 76, device="cuda")[:, :4].contiguous()
    for tp, tc in (([-1, 1, 0], [0, 0, 0]),       # a parent after its child
                   ([-1, 0, 0], [0, 5, 0]),       # a child rank past `children`
                   ([-1, 0, 1, 2, 3], [0] * 5)):  # 5 rows needed, 4 given
        got, errs = _run(draft, tp, tc, 4, 3000, 8, 4)
        assert errs & E.DEVERR_TREE
        assert (got["num_nodes"] == 0).all() and (got["tokens"] == -1).all()
