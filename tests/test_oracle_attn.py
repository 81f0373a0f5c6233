"""Pins for the oracle's tree attention (EAGLE-1 explainer, "Role of Tree
Attention"; EAGLE-2 explainer, "Attention mask adjustment": a draft token
attends to the prefix and to its own ancestors only).

Pins: every node's output equals plain causal attention of one query over
[prefix, its root path] computed as a separate chain; torch's
scaled_dot_product_attention in float64 with the explicit boolean mask; GQA
equals MHA with repeated KV heads; paged equals contiguous under any block
permutation; invariance under a permutation of prefix positions.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from conftest import to_np


def _case(seed, B=2, Hq=4, Hkv=2, d=16, L=(37, 21), vocab=400, kinds=(0, 1), paged=False):
    w = synth.small_workload(5, batch=B, vocab=vocab, num_q_heads=Hq, num_kv_heads=Hkv,
                             head_dim=d, kinds=list(kinds), m=12, depth=4, topk=3, children=3,
                             chain_k=5, dtype=torch.float32, prefix=0, block_size=0,
                             poison_tail=False)
    logits = to_np(synth.draft_logits(w, seed))
    t = oracle.build_tree(logits, w.depth, w.topk, w.children, w.m, chain_k=w.chain_k,
                          kinds=list(kinds), m_max=w.m_max)
    rng = np.random.default_rng(seed)
    M = w.m_max
    Lmax = max(L)
    plen = np.array(L[:B], np.int32)
    q = rng.standard_normal((B, M, Hq, d)).astype(np.float32)
    kd = rng.standard_normal((B, M, Hkv, d)).astype(np.float32)
    vd = rng.standard_normal((B, M, Hkv, d)).astype(np.float32)
    kc = rng.standard_normal((B, Hkv, Lmax, d)).astype(np.float32)
    vc = rng.standard_normal((B, Hkv, d, Lmax)).astype(np.float32)
    return dict(w=w, t=t, q=q, kd=kd, vd=vd, kc=kc, vc=vc, plen=plen)


def _mask(orc, c):
    anc, _ = orc.tree_mask(c["t"]["parent"], c["t"]["num_nodes"], c["plen"])
    return anc


def test_chain_equivalence(orc):
    c = _case(3)
    anc = _mask(orc, c)
    out = orc.tree_attn(c["q"], c["kd"], c["vd"], c["kc"], c["vc"], None, c["plen"], anc,
                        c["t"]["num_nodes"])
    B, M, Hq, d = c["q"].shape
    G = Hq // c["kd"].shape[2]
    for b in range(B):
        n = int(c["t"]["num_nodes"][b])
        L = int(c["plen"][b])
        for i in range(n):
            path = []
            a = i
            while a >= 0:
                path.append(a)
                a = int(c["t"]["parent"][b, a])
            path = path[::-1]                                # root-first chain ending at i
            for h in range(Hq):
                kv = h // G
                keys = np.concatenate([c["kc"][b, kv, :L].astype(np.float64),
                                       c["kd"][b, path, kv].astype(np.float64)])
                vals = np.concatenate([c["vc"][b, kv, :, :L].T.astype(np.float64),
                                       c["vd"][b, path, kv].astype(np.float64)])
                s = keys @ c["q"][b, i, h].astype(np.float64) / np.sqrt(d)
                p = np.exp(s - s.max())
                ref = (p / p.sum()) @ vals
                assert np.abs(out[b, i, h] - ref).max() < 1e-12
        assert (out[b, n:] == 0).all()


def test_matches_torch_sdpa_float64(orc):
    c = _case(4, B=2, Hq=6, Hkv=3, d=32, L=(50, 9))
    anc = _mask(orc, c)
    out = orc.tree_attn(c["q"], c["kd"], c["vd"], c["kc"], c["vc"], None, c["plen"], anc,
                        c["t"]["num_nodes"])
    B, M, Hq, d = c["q"].shape
    Hkv = c["kd"].shape[2]
    for b in range(B):
        n = int(c["t"]["num_nodes"][b])
        L = int(c["plen"][b])
        bits = np.array([[(int(anc[b, i]) >> j) & 1 for j in range(M)] for i in range(n)], bool)
        mask = torch.from_numpy(np.concatenate([np.ones((n, L), bool), bits], axis=1))
        for kv in range(Hkv):
            K = torch.from_numpy(np.concatenate([c["kc"][b, kv, :L], c["kd"][b, :, kv]])).double()
            V = torch.from_numpy(np.concatenate([c["vc"][b, kv, :, :L].T, c["vd"][b, :, kv]])).double()
            for h in range(kv * (Hq // Hkv), (kv + 1) * (Hq // Hkv)):
                Q = torch.from_numpy(c["q"][b, :n, h]).double()
                ref = torch.nn.functional.scaled_dot_product_attention(
                    Q[None, None], K[None, None], V[None, None], attn_mask=mask[None, None])[0, 0]
                assert np.abs(out[b, :n, h] - ref.numpy()).max() < 1e-12


def test_gqa_equals_mha_with_repeated_kv(orc):
    c = _case(5, Hq=6, Hkv=2)
    anc = _mask(orc, c)
    G = 3
    out = orc.tree_attn(c["q"], c["kd"], c["vd"], c["kc"], c["vc"], None, c["plen"], anc,
                        c["t"]["num_nodes"])
    rep = lambda a, ax: np.ascontiguousarray(np.repeat(a, G, axis=ax))
    out2 = orc.tree_attn(c["q"], rep(c["kd"], 2), rep(c["vd"], 2), rep(c["kc"], 1), rep(c["vc"], 1),
                         None, c["plen"], anc, c["t"]["num_nodes"])
    assert np.array_equal(out, out2)


def test_paged_equals_contiguous_any_block_permutation(orc):
    c = _case(6, L=(37, 21))
    anc = _mask(orc, c)
    ref = orc.tree_attn(c["q"], c["kd"], c["vd"], c["kc"], c["vc"], None, c["plen"], anc,
                        c["t"]["num_nodes"])
    bs = 8
    B, Hkv, Lmax, d = c["kc"].shape
    nb = [(int(x) + bs - 1) // bs for x in c["plen"]]
    total = sum(nb) + 3                                    # spare blocks never referenced
    perm = np.random.default_rng(0).permutation(total)
    kp = np.full((total, Hkv, bs, d), np.nan, np.float32)   # unused slots poisoned
    vp = np.full((total, Hkv, d, bs), np.nan, np.float32)
    table = np.full((B, max(nb)), -1, np.int32)
    o = 0
    for b in range(B):
        for j in range(nb[b]):
            blk = perm[o]
            o += 1
            table[b, j] = blk
            n = min(bs, int(c["plen"][b]) - j * bs)
            kp[blk, :, :n] = c["kc"][b, :, j * bs: j * bs + n]
            vp[blk, :, :, :n] = c["vc"][b, :, :, j * bs: j * bs + n]
    out = orc.tree_attn(c["q"], c["kd"], c["vd"], kp, vp, table, c["plen"], anc, c["t"]["num_nodes"])
    assert np.array_equal(out, ref)
    sel = [(0, 3, 1), (1, 2, 0), (0, 0, 3)]
    rows = orc.tree_attn_rows(c["q"], c["kd"], c["vd"], kp, vp, table, c["plen"], anc, sel)
    for s, (b, i, h) in enumerate(sel):
        assert np.array_equal(rows[s], ref[b, i, h])


def test_prefix_permutation_invariance(orc):
    c = _case(7, L=(30, 30))
    anc = _mask(orc, c)
    ref = orc.tree_attn(c["q"], c["kd"], c["vd"], c["kc"], c["vc"], None, c["plen"], anc,
                        c["t"]["num_nodes"])
    perm = np.random.default_rng(1).permutation(30)
    kc = np.ascontiguousarray(c["kc"][:, :, perm])
    vc = np.ascontiguousarray(c["vc"][:, :, :, perm])
    out = orc.tree_attn(c["q"], c["kd"], c["vd"], kc, vc, None, c["plen"], anc, c["t"]["num_nodes"])
    assert np.abs(out - ref).max() < 1e-13
