"""Children drawn from the draft (eagle_build_tree_sampled) and recursive
rejection sampling over them (eagle_accept_rrs) through the C ABI against the
oracle, bit-exact: the drawn trees, and the accepted paths and bonus tokens,
for fp32 and bf16 rows, vocabularies from 6 to 70001 (chunks that end inside
and past the row), one to four levels, temperatures 1 and 0.7; and the
emitted first token's distribution over 200 000 GPU trials."""
from __future__ import annotations

import zlib

import numpy as np
import pytest
import scipy.stats
import torch

import eagle_tree_verification_draft_amd as E
import oracle
import synth
from conftest import to_np
from gpu_harness import say

pytestmark = pytest.mark.gpu


def _words(rng, shape):
    return rng.integers(0, 1 << 32, size=shape, dtype=np.uint64).astype(np.uint32)


def _as_i32(u32):
    return torch.from_numpy(np.ascontiguousarray(u32).view(np.int32))


def _gpu_build(draft, D, k, C, cw):
    B, R, V = draft.shape
    N, nn = 0, C
    for _ in range(D):
        N += nn
        nn = min(k, nn) * C
    p = E.TreeParams(D, k, C, 1, 0, V, N, R, 0)
    ws = torch.empty(max(256, E.build_tree_workspace_size(p, B)), dtype=torch.uint8, device="cuda")
    E.workspace_init(ws)
    i32 = dict(dtype=torch.int32, device="cuda")
    t = dict(tokens=torch.empty((B, N), **i32), parent=torch.empty((B, N), **i32), depth=torch.empty((B, N), **i32),
             score=torch.empty((B, N), dtype=torch.float64, device="cuda"), src_row=torch.empty((B, N), **i32),
             num_nodes=torch.empty((B,), **i32))
    E.build_tree_sampled(p, B, draft, _as_i32(cw).to("cuda"), t["tokens"], t["parent"], t["depth"], t["score"],
                         t["src_row"], t["num_nodes"], ws)
    torch.cuda.synchronize()
    return t, N, E.read_errors(ws)


def _gpu_rrs(target, draft, t, N, max_accept, words, T):
    B, _, V = target.shape
    a = E.AcceptParams(E.EAGLE_ACCEPT_SAMPLE, T, N, V, max_accept)
    ws = torch.empty(E.accept_rrs_workspace_size(a, B), dtype=torch.uint8, device="cuda")
    E.workspace_init(ws)
    i32 = dict(dtype=torch.int32, device="cuda")
    acc = torch.empty((B, max_accept), **i32)
    alen = torch.empty((B,), **i32)
    bon = torch.empty((B,), **i32)
    E.accept_rrs(a, B, target, draft, t["tokens"], t["parent"], t["src_row"], t["num_nodes"],
                 _as_i32(words).to("cuda"), acc, alen, bon, ws)
    torch.cuda.synchronize()
    return acc.cpu().numpy(), alen.cpu().numpy(), bon.cpu().numpy(), E.read_errors(ws)


# (name, dtype, batch, vocab, D, k, C, temperature)
CASES = [
    ("f32-v1000-d3", torch.float32, 4, 1000, 3, 2, 3, 1.0),
    ("bf16-v32000-d4", torch.bfloat16, 3, 32000, 4, 2, 3, 1.0),
    ("bf16-v70001-d2-T0.7", torch.bfloat16, 2, 70001, 2, 4, 4, 0.7),
    ("bf16-v6-d2", torch.bfloat16, 8, 6, 2, 2, 2, 1.0),
    ("f32-v300-d1-c8", torch.float32, 5, 300, 1, 1, 8, 1.0),
    # the largest vocabulary (two 64-token pieces per draw walk, two segments
    # per thread in the bonus scan) and the most children per row
    ("bf16-vmax-d2-T0.9", torch.bfloat16, 2, 1 << 17, 2, 2, 3, 0.9),
    ("bf16-v2000-d2-c16", torch.bfloat16, 3, 2000, 2, 1, 16, 1.0),
]


@pytest.mark.parametrize("name,dtype,B,V,D,k,C,T", CASES, ids=[c[0] for c in CASES])
def test_sampled_build_and_rrs_match_oracle(name, dtype, B, V, D, k, C, T):
    say(f"[rrs {name}]")
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    R = 1 + (D - 1) * k
    draft_f = (rng.standard_normal((B, R, V)) * 1.5).astype(np.float32)
    draft = torch.from_numpy(draft_f).to(dtype).to("cuda")
    cw = _words(rng, (B, R, C))
    t, N, errs = _gpu_build(draft, D, k, C, cw)
    assert errs == 0
    ot = oracle.build_tree(to_np(draft), D, k, C, 1, m_max=N, child_words=cw)
    for kk in ("tokens", "parent", "depth", "score", "src_row", "num_nodes"):
        assert np.array_equal(t[kk].cpu().numpy(), ot[kk]), kk
    # targets near the draft of each node's own row (so paths go several levels)
    tgt = np.empty((B, N + 1, V), np.float32)
    tgt[:, 0] = draft_f[:, 0]
    for b in range(B):
        for i in range(N):
            r = ot["src_row"][b, i]
            tgt[b, i + 1] = draft_f[b, r] if r >= 0 else draft_f[b, 0]
    tgt += (rng.standard_normal(tgt.shape) * 0.5).astype(np.float32)
    target = torch.from_numpy(tgt).to(dtype).to("cuda")
    words = _words(rng, (B, N + 1))
    max_accept = D
    o_acc, o_len, o_bon = oracle.accept_rrs(to_np(target), to_np(draft), ot["tokens"], ot["parent"], ot["src_row"],
                                            ot["num_nodes"], max_accept, words, T=T)
    acc, alen, bon, errs = _gpu_rrs(target, draft, t, N, max_accept, words, T)
    assert errs == 0
    assert np.array_equal(alen, o_len) and np.array_equal(acc, o_acc) and np.array_equal(bon, o_bon)
    say(f"[rrs {name}] accept lengths {o_len.tolist()}")
    if D >= 2 and C <= 4:
        # the walk goes past the first level (with many children and one
        # expanded, the accepted child is mostly a leaf)
        assert o_len.max() >= 2


def test_rrs_first_token_distribution_on_gpu():
    """200 000 sequences, vocabulary 6, two levels: the first emitted token
    follows the target (chi-square), and the GPU agrees with the oracle on
    every sequence."""
    say("[rrs distribution]")
    rng = np.random.default_rng(99)
    V, D, k, C, B = 6, 2, 2, 2, 200_000
    target_row = np.array([1.0, 0.2, -0.5, 0.7, -2.0, 0.0], np.float32)
    draft_row = np.array([-0.3, 1.2, 0.4, -1.0, 0.9, 0.1], np.float32)
    R = 1 + (D - 1) * k
    draft = torch.from_numpy(np.tile(draft_row, (B, R, 1))).to("cuda")
    cw = _words(rng, (B, R, C))
    t, N, errs = _gpu_build(draft, D, k, C, cw)
    assert errs == 0
    target = torch.from_numpy(np.tile(target_row, (B, N + 1, 1))).to("cuda")
    words = _words(rng, (B, N + 1))
    acc, alen, bon, errs = _gpu_rrs(target, draft, t, N, D, words, 1.0)
    assert errs == 0
    tok = t["tokens"].cpu().numpy()
    first = np.where(alen > 0, tok[np.arange(B), np.maximum(acc[:, 0], 0)], bon)
    w = np.array([oracle.weight(float(x), float(target_row.max()), 1.0) for x in target_row])
    p = w / w.sum()
    assert scipy.stats.chisquare(np.bincount(first, minlength=V), p * B).pvalue > 1e-3
    ot = oracle.build_tree(draft.cpu().numpy(), D, k, C, 1, m_max=N, child_words=cw)
    o_acc, o_len, o_bon = oracle.accept_rrs(target.cpu().numpy(), draft.cpu().numpy(), ot["tokens"], ot["parent"],
                                            ot["src_row"], ot["num_nodes"], D, words)
    assert np.array_equal(alen, o_len) and np.array_equal(acc, o_acc) and np.array_equal(bon, o_bon)
