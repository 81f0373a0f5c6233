"""Pins for the oracle's parallel-draft inputs (P-EAGLE in vLLM, "Step 2:
parallel drafting": a known position pairs its target hidden state with the
token that follows it, the first drafting position pairs the new token with
the last hidden state, positions 2..K carry the MASK token and the shared
hidden state; "Unified Triton kernel", "Hidden-state management").

Pins: a hand-worked example; the known slots' positions agree with the KV
commit's positions of the same accepted nodes (a separately pinned
function); the slot tokens are the accepted sequence shifted by one; counts
of MASK, padding and rejected entries; the edge cases of an empty path and of
cut or clamped paths.
"""
import numpy as np
import pytest

import oracle


def _hidden(rng, B, M, H):
    return rng.standard_normal((B, M + 1, H)).astype(np.float32), rng.standard_normal(H).astype(np.float32)


def test_hand_worked_example():
    # tree tokens 10..17, 6 nodes, accepted path nodes 2 then 4, bonus 99,
    # prefix 100 (the root is position 99), K = 3, MASK id 7, max_accept 4
    tokens = np.arange(10, 18, dtype=np.int32)[None]
    th = np.arange(9 * 4, dtype=np.float32).reshape(1, 9, 4)
    hs = np.full(4, -1.0, np.float32)
    acc = np.array([[2, 4, -1, -1]], np.int32)
    o = oracle.pdraft_prepare(tokens, [6], acc, [2], [99], [100], th, hs, K=3, mask_id=7)
    # slot: 0 root, 1 node 2, 2 node 4, 3-4 MASK, 5-6 padding
    assert o["positions"][0].tolist() == [99, 100, 101, 102, 103, -1, -1]
    assert o["input_ids"][0].tolist() == [12, 14, 99, 7, 7, -1, -1]
    assert o["hidden_src"][0].tolist() == [0, 3, 5, -1, -1, -1, -1]
    assert o["is_mask"][0].tolist() == [0, 0, 0, 1, 1, 0, 0]
    assert o["num_slots"][0] == 5
    assert o["rejected"][0].tolist() == [1, 1, 0, 1, 0, 1, 0, 0]
    d = o["draft_hidden"][0]
    assert np.array_equal(d[0], th[0, 0]) and np.array_equal(d[1], th[0, 3]) and np.array_equal(d[2], th[0, 5])
    assert np.array_equal(d[3], hs) and np.array_equal(d[4], hs) and not d[5:].any()
    assert o["flags"] == (0, 0)


def test_nothing_accepted():
    # the bonus token follows the root directly; K - 1 MASK slots after it
    tokens = np.arange(5, dtype=np.int32)[None]
    th, hs = _hidden(np.random.default_rng(1), 1, 5, 8)
    o = oracle.pdraft_prepare(tokens, [5], np.full((1, 3), -1, np.int32), [0], [42], [17], th, hs, K=4, mask_id=0)
    assert o["input_ids"][0].tolist() == [42, 0, 0, 0, -1, -1, -1]
    assert o["positions"][0].tolist() == [16, 17, 18, 19, -1, -1, -1]
    assert o["rejected"][0].tolist() == [1] * 5
    assert o["num_slots"][0] == 4


@pytest.mark.parametrize("seed", [3, 4, 5])
def test_invariants_and_agreement_with_kv_commit(seed):
    rng = np.random.default_rng(seed)
    B, M, MA, K, H = 6, 20, 7, 5, 16
    tokens = rng.integers(0, 1000, (B, M)).astype(np.int32)
    nn = rng.integers(1, M + 1, B).astype(np.int32)
    alen = np.array([min(int(rng.integers(0, MA + 1)), int(n)) for n in nn], np.int32)
    acc = np.full((B, MA), -1, np.int32)
    for b in range(B):
        acc[b, :alen[b]] = rng.choice(int(nn[b]), size=int(alen[b]), replace=False)
    bonus = rng.integers(0, 1000, B).astype(np.int32)
    L = rng.integers(1, 500, B).astype(np.int32)
    th, hs = _hidden(rng, B, M, H)
    o = oracle.pdraft_prepare(tokens, nn, acc, alen, bonus, L, th, hs, K=K, mask_id=-5)
    assert o["flags"] == (0, 0)
    # the KV commit of the same path, contiguous cache with room
    kd = rng.standard_normal((B, M, 1, 8)).astype(np.float32)
    kc = np.zeros((B, 1, 512, 8), np.float32)
    vc = np.zeros((B, 1, 8, 512), np.float32)
    _, _, slot, _, _ = oracle.kv_commit(kd, kd, acc, alen, L, kc, vc)
    for b in range(B):
        A = int(alen[b])
        assert o["num_slots"][b] == A + K
        assert o["positions"][b, :A + K].tolist() == list(range(L[b] - 1, L[b] - 1 + A + K))
        assert (o["positions"][b, A + K:] == -1).all()
        # known slot j + 1 is accepted node a_j: the same position the commit gives it
        for j in range(A):
            assert o["positions"][b, j + 1] == slot[b, acc[b, j]] == L[b] + j
            assert o["hidden_src"][b, j + 1] == acc[b, j] + 1
        # tokens: the accepted sequence (path tokens, then the bonus), one position ahead
        seq = [int(tokens[b, a]) for a in acc[b, :A]] + [int(bonus[b])]
        assert o["input_ids"][b, :A + 1].tolist() == seq
        assert o["is_mask"][b].sum() == K - 1 and (o["input_ids"][b, A + 1:A + K] == -5).all()
        assert o["rejected"][b].sum() == int(nn[b]) - A
        for s in range(MA + K):
            src = int(o["hidden_src"][b, s])
            want = th[b, src] if src >= 0 else (hs if o["is_mask"][b, s] else np.zeros(H, np.float32))
            assert np.array_equal(o["draft_hidden"][b, s], want)


def test_cut_and_clamped_paths():
    tokens = np.arange(40, dtype=np.int32).reshape(2, 20)
    th, hs = _hidden(np.random.default_rng(2), 2, 20, 8)
    acc = np.array([[3, 7, 25, 4], [1, 2, 3, 4]], np.int32)     # node 25 is outside [0, 20)
    o = oracle.pdraft_prepare(tokens, [20, 20], acc, [4, 9], [0, 0], [10, 0], th, hs, K=2, mask_id=-1)
    # sequence 0 is cut before node 25; sequence 1's length 9 is clamped to 4; L = 0 is flagged
    assert o["num_slots"].tolist() == [2 + 2, 4 + 2]
    assert o["flags"] == (2, 1)
    assert o["input_ids"][0, :3].tolist() == [3, 7, 0]
