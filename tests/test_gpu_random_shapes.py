"""GPU parity over seeded random shapes: every output of the step against the
oracle for configurations drawn across the library's limits (dtype, GQA
ratio, tree depth / expansion / children / rerank size, chains of any
length, paged caches of every supported page size or contiguous ones,
ragged and empty prefixes, poisoned tails, greedy and sampled acceptance).

The draws are fixed by their seeds, so every run checks the same cases.
Trees, masks and accepts are compared bit for bit; attention row by row
for every (node, head) within the tolerance of its dtype.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import pytest
import torch

import synth
from gpu_harness import (BF16_TOL, F32_TOL, assert_accept_equal, assert_tree_equal, check_attn_rows, make_case,
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
