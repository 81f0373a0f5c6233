"""Acceptance through the C ABI against the oracle, bit-exact, on every kernel
route the library chooses between: the parallel greedy argmax (few rows), the
register-resident walk (aligned rows of up to 16 vectors per thread, greedy and
sampling, padded rows whose vocabulary ends inside a vector), and the looping
walk (unaligned rows, rows shorter than one vector, long fp32 rows).

Trees are random but valid (parents precede children), with repeated sibling
tokens so that a rejected token's later siblings carry no mass, and target rows
planted so that walks go several levels deep."""
from __future__ import annotations

import math
import zlib

import numpy as np
import pytest
import torch

import eagle_tree_verification_draft_amd as E
import oracle
from conftest import to_np
from gpu_harness import say

pytestmark = pytest.mark.gpu


def _random_tree(rng, B, m_max, V, n_lo):
    tokens = np.zeros((B, m_max), np.int32)
    parent = np.zeros((B, m_max), np.int32)
    nn = rng.integers(n_lo, m_max + 1, size=B).astype(np.int32)
    for b in range(B):
        for i in range(int(nn[b])):
            parent[b, i] = rng.integers(-1, i) if i else -1
            sib = [j for j in range(i) if parent[b, j] == parent[b, i]]
            # a quarter of the nodes repeat an earlier sibling's token
            tokens[b, i] = tokens[b, sib[-1]] if sib and rng.random() < 0.25 else rng.integers(0, V)
    return tokens, parent, nn


def _target(rng, B, m_max, V, tokens, parent, nn, dtype, boost):
    """N(0, 2) rows; along one random root-to-leaf path per sequence the row of
    each node (root: row 0) is raised at its child's token."""
    t = rng.standard_normal((B, m_max + 1, V)).astype(np.float32) * 2.0
    for b in range(B):
        n = int(nn[b])
        if n == 0:
            continue
        a = int(rng.integers(0, n))
        while a >= 0:
            p = int(parent[b, a])
            t[b, p + 1, tokens[b, a]] += boost
            a = p
    return torch.from_numpy(t).to(dtype)


# (name, dtype, V, mode, batch, m_max, row padding, temperature)
ROUTES = [
    ("greedy-parallel-bf16", torch.bfloat16, 3000, 0, 4, 40, 0, 1.0),
    ("greedy-reg-bf16-2vec", torch.bfloat16, 16000, 0, 10, 60, 0, 1.0),
    ("greedy-reg-bf16-padded-ragged", torch.bfloat16, 16001, 0, 10, 60, 15, 1.0),
    ("greedy-reg-f32-16vec", torch.float32, 60001, 0, 9, 60, 3, 1.0),
    ("greedy-reg-bf16-vmax", torch.bfloat16, 1 << 17, 0, 9, 60, 0, 1.0),
    ("greedy-loop-bf16-unaligned", torch.bfloat16, 2001, 0, 10, 60, 0, 1.0),
    ("sample-reg-bf16-1vec", torch.bfloat16, 5000, 1, 10, 50, 0, 1.0),
    ("sample-reg-bf16-padded-ragged", torch.bfloat16, 5001, 1, 6, 50, 7, 1.0),
    ("sample-reg-bf16-4vec-T0.6", torch.bfloat16, 32000, 1, 5, 48, 0, 0.6),
    ("sample-reg-f32-16vec", torch.float32, 60001, 1, 6, 30, 3, 1.0),
    ("sample-reg-bf16-vmax", torch.bfloat16, 1 << 17, 1, 3, 30, 0, 1.0),
    ("sample-loop-bf16-unaligned", torch.bfloat16, 2001, 1, 6, 50, 0, 1.0),
    ("sample-loop-f32-long", torch.float32, 70001, 1, 3, 30, 3, 1.0),
    ("sample-loop-bf16-tiny", torch.bfloat16, 5, 1, 8, 6, 0, 1.0),
    ("greedy-loop-f32-tiny", torch.float32, 3, 0, 90, 6, 0, 1.0),
]


def _inputs(name, dtype, V, mode, B, m_max, pad, T):
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    tokens, parent, nn = _random_tree(rng, B, m_max, V, n_lo=1)
    # greedy: a large boost walks the planted path; sampling: one that gives the
    # planted token most (not all) of the mass against V N(0, 2) logits
    boost = 30.0 if mode == 0 else math.log(V) + 3.0
    target = _target(rng, B, m_max, V, tokens, parent, nn, dtype, boost=boost)
    words = rng.integers(0, 1 << 32, size=(B, m_max + 1), dtype=np.uint64).astype(np.uint32)
    return tokens, parent, nn, target, words


def _run_gpu(dtype, V, mode, B, m_max, pad, T, tokens, parent, nn, target, words):
    """(accepted, accept_len, bonus, device error bits) from the C ABI."""
    dev = "cuda"
    if pad:
        # rows inside a wider buffer whose padding holds large values: any read
        # past the vocabulary would change the argmax or the weights
        buf = torch.full((B, m_max + 1, V + pad), 1.0e4, dtype=dtype)
        buf[..., :V] = target
        tg = buf.to(dev)[..., :V]
    else:
        tg = target.to(dev)
    a = E.AcceptParams(mode, T, m_max, V, m_max)
    ws = torch.empty(max(256, E.accept_workspace_size(a, B)), dtype=torch.uint8, device=dev)
    E.workspace_init(ws)
    acc = torch.empty((B, m_max), dtype=torch.int32, device=dev)
    alen = torch.empty(B, dtype=torch.int32, device=dev)
    bon = torch.empty(B, dtype=torch.int32, device=dev)
    w_dev = torch.from_numpy(words.view(np.int32)).to(dev) if mode == 1 else None
    E.accept(a, B, tg, torch.from_numpy(tokens).to(dev), torch.from_numpy(parent).to(dev),
             torch.from_numpy(nn).to(dev), w_dev, acc, alen, bon, ws)
    torch.cuda.synchronize()
    return acc.cpu().numpy(), alen.cpu().numpy(), bon.cpu().numpy(), E.read_errors(ws)


@pytest.mark.parametrize("name,dtype,V,mode,B,m_max,pad,T", ROUTES, ids=[r[0] for r in ROUTES])
def test_accept_route(name, dtype, V, mode, B, m_max, pad, T):
    say(f"[accept {name}] B={B} m_max={m_max} V={V} pad={pad}")
    tokens, parent, nn, target, words = _inputs(name, dtype, V, mode, B, m_max, pad, T)
    o_acc, o_len, o_bon = oracle.accept(mode, to_np(target), tokens, parent, nn, m_max,
                                        rand_words=words if mode == 1 else None, T=T)
    acc, alen, bon, errs = _run_gpu(dtype, V, mode, B, m_max, pad, T, tokens, parent, nn, target, words)
    assert errs == 0
    assert np.array_equal(alen, o_len), (alen, o_len)
    assert np.array_equal(acc, o_acc)
    assert np.array_equal(bon, o_bon)
    say(f"[accept {name}] mean accepted length {o_len.mean():.2f}, max {o_len.max()}")
    # the walks must go beyond the root for the case to mean anything
    assert o_len.max() >= 2


NAN_ROUTES = ["greedy-parallel-bf16", "greedy-reg-bf16-2vec", "greedy-reg-bf16-vmax", "sample-reg-bf16-1vec",
              "greedy-loop-bf16-unaligned", "sample-loop-bf16-unaligned"]


@pytest.mark.parametrize("name", NAN_ROUTES)
def test_accept_nan_row_reported(name):
    """A NaN in the root row of sequence 1 raises NONFINITE_ROW; the other
    sequences' results are those of the clean rows."""
    route = {r[0]: r for r in ROUTES}[name]
    _, dtype, V, mode, B, m_max, pad, T = route
    say(f"[accept nan {name}]")
    tokens, parent, nn, target, words = _inputs(*route)
    o_acc, o_len, o_bon = oracle.accept(mode, to_np(target), tokens, parent, nn, m_max,
                                        rand_words=words if mode == 1 else None, T=T)
    bad = target.clone()
    bad[1, 0, V // 3] = float("nan")
    acc, alen, bon, errs = _run_gpu(dtype, V, mode, B, m_max, pad, T, tokens, parent, nn, bad, words)
    assert errs & E.DEVERR_NONFINITE_ROW
    keep = np.arange(B) != 1
    assert np.array_equal(alen[keep], o_len[keep])
    assert np.array_equal(acc[keep], o_acc[keep])
    assert np.array_equal(bon[keep], o_bon[keep])
