"""Pins for the oracle's KV commit (EAGLE-1 explainer, "Verification": the
accepted tokens extend the sequence; P-EAGLE in vLLM, "KV cache and CUDA
graphs": tokens that are not kept map to slot -1 and are not written).

Pins:
  - commit-then-attend: after the commit, one query's attention over the
    prefix of L + A cache keys (no draft keys) equals its attention over the
    old L keys plus the accepted path's draft keys under the tree mask, in
    fp64 -- a wrong position, head, row or V transpose changes the result;
  - every element outside the committed positions is untouched and every
    committed one is the draft's (bit-exact, against positions worked out in
    the test);
  - slot numbers of a hand-worked paged example;
  - two commits in a row equal one commit of the joined path;
  - the stop and clamp rules at the capacity, an unassigned page, an invalid
    node id, a prefix past the capacity and an accept length out of range.
"""
import numpy as np
import pytest

import oracle


def _tree_path(rng, M, depth):
    """Random parents (parents precede children) with a root path of `depth`
    nodes planted; returns (parent, path root-first)."""
    parent = np.array([rng.integers(-1, i) if i else -1 for i in range(M)], np.int32)
    path = sorted(rng.choice(M, size=depth, replace=False).tolist())
    for k, x in enumerate(path):
        parent[x] = path[k - 1] if k else -1
    return parent, path


def _caches(rng, B, Hkv, d, P, paged, bs, dtype=np.float32):
    def fill(shape):
        if dtype == np.uint16:
            return rng.integers(0, 1 << 16, shape).astype(np.uint16)
        return rng.standard_normal(shape).astype(dtype)
    if not paged:
        return fill((B, Hkv, P, d)), fill((B, Hkv, d, P)), None
    nblk = (P + bs - 1) // bs
    table = rng.permutation(B * nblk).astype(np.int32).reshape(B, nblk)
    return fill((B * nblk, Hkv, bs, d)), fill((B * nblk, Hkv, d, bs)), table


@pytest.mark.parametrize("paged", [False, True])
def test_commit_then_attend(paged):
    rng = np.random.default_rng(11 + paged)
    B, M, Hq, Hkv, d, P, bs = 3, 20, 4, 2, 16, 64, 8
    kc, vc, table = _caches(rng, B, Hkv, d, P, paged, bs)
    kd = rng.standard_normal((B, M, Hkv, d)).astype(np.float32)
    vd = rng.standard_normal((B, M, Hkv, d)).astype(np.float32)
    q = rng.standard_normal((B, M, Hq, d)).astype(np.float32)
    L = np.array([0, 17, 40], np.int32)
    depths = [5, 3, 7]
    parents, paths = zip(*[_tree_path(rng, M, depths[b]) for b in range(B)])
    parent = np.stack(parents)
    acc = np.full((B, M), -1, np.int32)
    for b in range(B):
        acc[b, :depths[b]] = paths[b]
    alen = np.array(depths, np.int32)
    nn = np.full(B, M, np.int32)
    anc, _ = oracle.tree_mask(parent, nn, L)
    kc2, vc2, slot, L2, flags = oracle.kv_commit(kd, vd, acc, alen, L, kc, vc, table)
    assert flags == (0, 0)
    assert np.array_equal(L2, L + alen)
    no_draft = np.zeros_like(anc)
    for b in range(B):
        last = paths[b][-1]
        sel = [(b, last, h) for h in range(Hq)]
        before = oracle.tree_attn_rows(q, kd, vd, kc, vc, table, L, anc, sel)
        after = oracle.tree_attn_rows(q, kd, vd, kc2, vc2, table, L2, no_draft, sel)
        np.testing.assert_allclose(after, before, rtol=1e-12, atol=1e-12)
        # and every accepted node's own row: its ancestors are the path's first nodes
        for k, x in enumerate(paths[b]):
            sel = [(b, x, 0)]
            before = oracle.tree_attn_rows(q, kd, vd, kc, vc, table, L, anc, sel)
            Lk = L.copy()
            Lk[b] = L[b] + k + 1
            after = oracle.tree_attn_rows(q, kd, vd, kc2, vc2, table, Lk, no_draft, sel)
            np.testing.assert_allclose(after, before, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("paged", [False, True])
def test_only_committed_positions_change(paged):
    rng = np.random.default_rng(5 + paged)
    B, M, Hkv, d, P, bs = 2, 12, 3, 8, 32, 8
    kc, vc, table = _caches(rng, B, Hkv, d, P, paged, bs, np.uint16)
    kd = rng.integers(0, 1 << 16, (B, M, Hkv, d)).astype(np.uint16)
    vd = rng.integers(0, 1 << 16, (B, M, Hkv, d)).astype(np.uint16)
    acc = np.array([[4, 9, 2, -1], [7, -1, -1, -1]], np.int32)
    alen = np.array([3, 1], np.int32)
    L = np.array([13, 0], np.int32)
    kc2, vc2, slot, L2, flags = oracle.kv_commit(kd, vd, acc, alen, L, kc, vc, table)
    assert flags == (0, 0)
    assert (kc2 != kc).sum() <= 4 * Hkv * d and (vc2 != vc).sum() <= 4 * Hkv * d
    # every element outside the committed slots is untouched; inside it is the draft's
    kexp, vexp = kc.copy(), vc.copy()
    for b in range(B):
        for j in range(int(alen[b])):
            pos = int(L[b]) + j
            node = int(acc[b, j])
            if paged:
                pg, off = int(table[b, pos // bs]), pos % bs
                kexp[pg, :, off, :] = kd[b, node]
                vexp[pg, :, :, off] = vd[b, node]
            else:
                kexp[b, :, pos, :] = kd[b, node]
                vexp[b, :, :, pos] = vd[b, node]
    assert np.array_equal(kc2, kexp) and np.array_equal(vc2, vexp)
    assert (slot >= 0).sum() == alen.sum()


def test_paged_slots_hand_example():
    # block table [3, 0, 2], 4-key pages, prefix 3: positions 3, 4, 5 sit in
    # page 3 offset 3, page 0 offset 0, page 0 offset 1 -> slots 15, 0, 1
    Hkv, d, bs, M = 1, 8, 4, 8
    kc = np.zeros((4, Hkv, bs, d), np.float32)
    vc = np.zeros((4, Hkv, d, bs), np.float32)
    kd = np.arange(M * d, dtype=np.float32).reshape(1, M, Hkv, d) + 1
    vd = -kd
    acc = np.array([[5, 2, 7]], np.int32)
    kc2, vc2, slot, L2, flags = oracle.kv_commit(kd, vd, acc, np.array([3], np.int32),
                                                 np.array([3], np.int32), kc, vc,
                                                 np.array([[3, 0, 2]], np.int32))
    assert flags == (0, 0) and L2[0] == 6
    want = np.full((1, M), -1, np.int32)
    want[0, 5], want[0, 2], want[0, 7] = 15, 0, 1
    assert np.array_equal(slot, want)
    assert np.array_equal(kc2[3, 0, 3], kd[0, 5, 0]) and np.array_equal(vc2[3, 0, :, 3], vd[0, 5, 0])
    assert np.array_equal(kc2[0, 0, 0], kd[0, 2, 0]) and np.array_equal(kc2[0, 0, 1], kd[0, 7, 0])
    assert not kc2[2].any() and not kc2[1].any()


def test_two_commits_equal_one():
    rng = np.random.default_rng(3)
    B, M, Hkv, d, P = 1, 16, 2, 8, 40
    kc, vc, _ = _caches(rng, B, Hkv, d, P, False, 0)
    kd1 = rng.standard_normal((B, M, Hkv, d)).astype(np.float32)
    kd2 = rng.standard_normal((B, M, Hkv, d)).astype(np.float32)
    vd1, vd2 = -kd1, 2 * kd2
    a1, a2 = [3, 8, 1], [0, 5]
    # the joined path as one commit of a draft tensor holding both steps' rows
    kdj = np.concatenate([kd1, kd2], axis=1)[:, :M]
    vdj = np.concatenate([vd1, vd2], axis=1)[:, :M]
    kdj[:, 9], vdj[:, 9] = kd2[:, 0], vd2[:, 0]
    kdj[:, 10], vdj[:, 10] = kd2[:, 5], vd2[:, 5]
    L = np.array([11], np.int32)
    k1, v1, _, L1, _ = oracle.kv_commit(kd1, vd1, np.array([a1], np.int32), np.array([3], np.int32), L, kc, vc)
    k2, v2, _, L2, _ = oracle.kv_commit(kd2, vd2, np.array([a2], np.int32), np.array([2], np.int32), L1, k1, v1)
    kj, vj, _, Lj, _ = oracle.kv_commit(kdj, vdj, np.array([[3, 8, 1, 9, 10]], np.int32),
                                        np.array([5], np.int32), L, kc, vc)
    assert L2[0] == Lj[0] == 16
    assert np.array_equal(k2, kj) and np.array_equal(v2, vj)


def test_stop_and_clamp_rules():
    rng = np.random.default_rng(8)
    B, M, Hkv, d, bs = 6, 10, 1, 8, 4
    kc, vc, table = _caches(rng, B, Hkv, d, 12, True, bs)   # 3 pages per sequence, capacity 12
    table[3, 2] = -1                                           # sequence 3: third page unassigned
    kd = rng.standard_normal((B, M, Hkv, d)).astype(np.float32)
    vd = rng.standard_normal((B, M, Hkv, d)).astype(np.float32)
    acc = np.tile(np.array([1, 2, 3, 4, 5], np.int32), (B, 1))
    acc[2, 2] = M                                              # sequence 2: invalid third node
    alen = np.array([5, 5, 5, 5, 0, 9], np.int32)              # 9 > max_accept: clamped to 5
    L = np.array([10, 13, 0, 6, 4, 1], np.int32)
    kc2, vc2, slot, L2, flags = oracle.kv_commit(kd, vd, acc, alen, L, kc, vc, table)
    # 0: positions 10, 11 fit, 12 is past the capacity; 1: L past capacity;
    # 2: stops at the invalid node; 3: positions 6, 7 fit, 8 is on the unassigned page;
    # 4: nothing to commit; 5: clamped to 5 tokens at positions 1..5
    assert L2.tolist() == [12, 13, 2, 8, 4, 6]
    assert flags == (2, 3)
    assert (slot >= 0).sum(axis=1).tolist() == [2, 0, 2, 2, 0, 5]
    # the max_prefix bound on paged caches
    _, _, _, L3, f3 = oracle.kv_commit(kd, vd, acc, np.full(B, 2, np.int32), np.zeros(B, np.int32), kc, vc,
                                       table, max_prefix=1)
    assert L3.tolist() == [1] * 6 and f3 == (0, 6)
