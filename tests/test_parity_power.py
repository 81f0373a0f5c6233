"""Power of the attention parity check at full prefix lengths (oracle only, CPU).

The tree mask admits each draft query to its ancestors and itself among the
draft keys (EAGLE-2 explainer, "Attention mask adjustment").  With N(0, 1)
inputs and a prefix of 8k-32k keys, the draft keys hold a tiny share of the
softmax mass, so a kernel that mishandled them would still pass a 2e-2
max-abs check.  The planted inputs (synth.plant_draft_keys) give the draft
keys most of the mass.  This test shows, with the oracle alone, that on the
planted inputs the GPU tests' check rejects three plausible kernel mistakes
at every workload's longest prefix:
  - no draft keys at all,
  - the draft block unmasked (every node sees every node),
  - a parent-only mask (self and parent, no deeper ancestors),
and records how little the same mistakes move the unplanted outputs.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from conftest import to_np

TOL = {torch.bfloat16: 2e-2, torch.float32: 1e-5}


def _reduced(n):
    """Workload n's attention shape and tree parameters at its longest prefix,
    with one or two sequences (one tree and, for workload 5, one chain)."""
    w = synth.workload(n)
    L = w.prefix if isinstance(w.prefix, int) else w.prefix[1]
    kinds = [synth.TREE_DYNAMIC, synth.TREE_CHAIN] if w.chain_k else [synth.TREE_DYNAMIC]
    return synth.small_workload(n, batch=len(kinds), kinds=kinds, vocab=3000, prefix=L)


def _mutants(parent, num_nodes, anc):
    B, M = anc.shape
    none = np.zeros_like(anc)
    full = np.zeros_like(anc)
    par_only = np.zeros_like(anc)
    for b in range(B):
        n = int(num_nodes[b])
        allbits = np.uint64((1 << n) - 1) if n < 64 else np.uint64(0xFFFFFFFFFFFFFFFF)
        for i in range(n):
            full[b, i] = allbits
            bits = 1 << i
            if parent[b, i] >= 0:
                bits |= 1 << int(parent[b, i])
            par_only[b, i] = np.uint64(bits)
    return {"no draft keys": none, "unmasked draft block": full, "parent-only mask": par_only}


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
def test_check_rejects_mask_mutants_at_full_prefix(n):
    w = _reduced(n)
    seed = 300 + n
    draft = to_np(synth.draft_logits(w, seed))
    t = oracle.build_tree(draft, w.depth, w.topk, w.children, w.m, chain_k=w.chain_k, kinds=w.kinds,
                          m_max=w.m_max)
    attn = synth.attn_inputs(w, seed)
    planted = synth.plant_draft_keys(attn, w, seed)
    plen = to_np(attn.prefix_len)
    anc, _ = oracle.tree_mask(t["parent"], t["num_nodes"], plen)
    # every node of every sequence, first and last q head (as the GPU tests add)
    sel = [(b, i, h) for b in range(w.batch) for i in range(int(t["num_nodes"][b]))
           for h in (0, w.num_q_heads - 1)]
    tol = TOL[w.dtype]
    report = {}
    for label, a in (("unplanted", attn), ("planted", planted)):
        host = [to_np(x) for x in (a.q, a.k_draft, a.v_draft, a.k_cache, a.v_cache)]
        bt = None if a.block_table is None else to_np(a.block_table)
        ref = oracle.tree_attn_rows(*host, bt, plen, anc, sel)
        gaps = {}
        for name, m in _mutants(t["parent"], t["num_nodes"], anc).items():
            mut = oracle.tree_attn_rows(*host, bt, plen, m, sel)
            gaps[name] = float(np.abs(mut - ref).max())
        report[label] = gaps
    print(f"workload {n} (L = {int(plen.max())}): max-abs gap to each mutant {report}")
    for name, gap in report["planted"].items():
        assert gap > 10 * tol, f"planted inputs: the '{name}' mutant moves the output by only {gap}"
