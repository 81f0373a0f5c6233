"""Pins for the oracle's sampled children and recursive rejection sampling
(EAGLE-1 explainer, "Verification": tokens are accepted by the ratio of the
target and draft distributions and a rejection resamples, which leaves the
target distribution unchanged; the children are draws from the draft).

Pins:
  - each child draw is the inverse CDF of the draft's integer weights over
    the tokens not yet drawn (numpy cumsum/searchsorted on spec_emul weights);
  - the sampled tree is every candidate, in creation order;
  - the first emitted token follows the target distribution (chi-square over
    200 000 seeded trials on a 6-token vocabulary, one and two levels, two and
    three children), and the test has the power to see a 5% shift;
  - a draft equal to the target accepts the first child every time; a draft
    whose mass sits on a token the target never emits is always rejected.
"""
import numpy as np
import pytest
import scipy.stats

import oracle
import spec_emul


def _words(rng, shape):
    return rng.integers(0, 1 << 32, size=shape, dtype=np.uint64).astype(np.uint32)


def test_draws_are_inverse_cdf_without_replacement():
    rng = np.random.default_rng(1)
    B, V, C = 20, 300, 6
    logits = (rng.standard_normal((B, 1, V)) * 2).astype(np.float32)
    cw = _words(rng, (B, 1, C))
    t = oracle.build_tree(logits, 1, 1, C, C, m_max=C, child_words=cw)
    for b in range(B):
        row = logits[b, 0]
        w = spec_emul.weights(row, np.float32(row.max())).astype(np.float64)
        left = np.ones(V, bool)
        R = int(w.sum())
        want = []
        for q in range(C):
            target = (int(cw[b, 0, q]) * R) >> 32
            cum = np.cumsum(np.where(left, w, 0.0))
            x = int(np.searchsorted(cum, target, side="right"))
            want.append(x)
            left[x] = False
            R -= int(w[x])
        assert t["tokens"][b, :C].tolist() == want
        assert t["parent"][b, :C].tolist() == [-1] * C


def test_sampled_tree_is_every_candidate_in_creation_order():
    rng = np.random.default_rng(2)
    D, k, C, V = 3, 2, 3, 200
    R = 1 + (D - 1) * k
    logits = (rng.standard_normal((2, R, V)) * 2).astype(np.float32)
    cw = _words(rng, (2, R, C))
    t = oracle.build_tree(logits, D, k, C, 1, m_max=64, child_words=cw, debug=True)
    N = C + (D - 1) * k * C
    for b in range(2):
        cd = {kk: v[b] for kk, v in t["cand"].items()}
        assert t["num_nodes"][b] == N == int(cd["n"])
        assert t["tokens"][b, :N].tolist() == cd["token"][:N].tolist()
        assert t["depth"][b, :N].tolist() == cd["depth"][:N].tolist()
        # siblings are distinct tokens (drawn without replacement)
        for q in range(-1, N):
            sib = [int(cd["token"][i]) for i in range(N) if cd["parent"][i] == q]
            assert len(sib) == len(set(sib))


def _first_tokens(target, draft, D, k, C, trials, seed, T=1.0):
    """Build a sampled tree per trial and run the recursive test; returns the
    first emitted token of every trial."""
    rng = np.random.default_rng(seed)
    V = target.shape[-1]
    R = 1 + (D - 1) * k
    N = C + (D - 1) * k * C
    dl = np.broadcast_to(draft, (trials, R, V)).copy()
    tl = np.broadcast_to(target, (trials, N + 1, V)).copy()
    t = oracle.build_tree(dl, D, k, C, 1, m_max=N, child_words=_words(rng, (trials, R, C)))
    acc, alen, bon = oracle.accept_rrs(tl, dl, t["tokens"], t["parent"], t["src_row"], t["num_nodes"], D,
                                       _words(rng, (trials, N + 1)), T=T)
    first = np.where(alen > 0, t["tokens"][np.arange(trials), np.maximum(acc[:, 0], 0)], bon)
    return first


def _target_probs(row, T=1.0):
    w = spec_emul.weights(row, np.float32(row.max()), T).astype(np.float64)
    return w / w.sum()


def test_second_token_follows_the_target():
    """Two levels, every row the same target and draft: after an accepted
    first child the walk tests that node's own children, and the second
    emitted token (an accepted grandchild or the bonus) follows the target."""
    rng = np.random.default_rng(17)
    V, D, k, C, trials = 6, 2, 2, 2, 200_000
    target_row = np.array([1.0, 0.2, -0.5, 0.7, -2.0, 0.0], np.float32)
    draft_row = np.array([-0.3, 1.2, 0.4, -1.0, 0.9, 0.1], np.float32)
    R, N = 1 + (D - 1) * k, C + (D - 1) * k * C
    dl = np.tile(draft_row, (trials, R, 1))
    tl = np.tile(target_row, (trials, N + 1, 1))
    t = oracle.build_tree(dl, D, k, C, 1, m_max=N, child_words=_words(rng, (trials, R, C)))
    acc, alen, bon = oracle.accept_rrs(tl, dl, t["tokens"], t["parent"], t["src_row"], t["num_nodes"], D,
                                       _words(rng, (trials, N + 1)))
    sel = alen >= 1
    idx = np.arange(trials)[sel]
    second = np.where(alen[sel] >= 2, t["tokens"][idx, np.maximum(acc[sel, 1], 0)], bon[sel])
    assert (alen >= 2).sum() > 1000      # the second level is exercised
    counts = np.bincount(second, minlength=V)
    p = _target_probs(target_row)
    assert scipy.stats.chisquare(counts, p * sel.sum()).pvalue > 1e-3


@pytest.mark.parametrize("D,k,C", [(1, 1, 2), (1, 1, 3), (2, 2, 2)])
def test_first_token_follows_the_target(D, k, C):
    V = 6
    target_row = np.array([1.0, 0.2, -0.5, 0.7, -2.0, 0.0], np.float32)
    draft_row = np.array([-0.3, 1.2, 0.4, -1.0, 0.9, 0.1], np.float32)
    R, N = 1 + (D - 1) * k, C + (D - 1) * k * C
    draft = np.tile(draft_row, (R, 1))[None]
    target = np.tile(target_row, (N + 1, 1))[None]
    trials = 200_000
    first = _first_tokens(target, draft, D, k, C, trials, seed=10 + C + D)
    counts = np.bincount(first, minlength=V)
    p = _target_probs(target_row)
    assert scipy.stats.chisquare(counts, p * trials).pvalue > 1e-3
    # power: a 5% shift of one token's mass is detected
    q = p.copy()
    q[0] *= 1.05
    q /= q.sum()
    assert scipy.stats.chisquare(counts, q * trials).pvalue < 1e-6


def test_draft_equal_to_target_always_accepts_the_first_child():
    row = np.array([0.3, -1.0, 2.0, 0.5], np.float32)
    rng = np.random.default_rng(5)
    trials, C = 5000, 2
    t = oracle.build_tree(np.tile(row, (trials, 1, 1)), 1, 1, C, 1, m_max=C, child_words=_words(rng, (trials, 1, C)))
    acc, alen, _ = oracle.accept_rrs(np.tile(row, (trials, C + 1, 1)), np.tile(row, (trials, 1, 1)), t["tokens"],
                                     t["parent"], t["src_row"], t["num_nodes"], 1, _words(rng, (trials, C + 1)))
    assert (alen == 1).all() and (acc[:, 0] == 0).all()


def test_draft_on_a_token_the_target_never_emits_is_rejected():
    # the draft puts (nearly) all its mass on token 3, which the target gives weight 0
    target_row = np.array([0.0, 1.0, 0.5, -60.0], np.float32)
    draft_row = np.array([-60.0, -60.0, -60.0, 0.0], np.float32)
    rng = np.random.default_rng(6)
    trials = 20000
    t = oracle.build_tree(np.tile(draft_row, (trials, 1, 1)), 1, 1, 1, 1, m_max=1,
                          child_words=_words(rng, (trials, 1, 1)))
    assert (t["tokens"][:, 0] == 3).all()
    acc, alen, bon = oracle.accept_rrs(np.tile(target_row, (trials, 2, 1)), np.tile(draft_row, (trials, 1, 1)),
                                       t["tokens"], t["parent"], t["src_row"], t["num_nodes"], 1,
                                       _words(rng, (trials, 2)))
    assert (alen == 0).all()
    counts = np.bincount(bon, minlength=4)
    p = _target_probs(target_row)
    assert counts[3] == 0 and scipy.stats.chisquare(counts[:3], p[:3] / p[:3].sum() * trials).pvalue > 1e-3


def test_bonus_after_one_rejection_is_the_exact_residual_inverse_cdf():
    """One child x with q(x) > p(x), rejected by a word at the top of its
    range; the bonus token for a word r must be the inverse CDF at r / 2^32 of
    the residual max(0, p - q) / sum, computed here in exact rationals from the
    Spec S weights (the oracle works in shifted integers; words closer than
    1e-6 to a CDF step are skipped)."""
    from fractions import Fraction
    V = 6
    target_row = np.array([1.0, 0.2, -0.5, 0.7, -2.0, 0.0], np.float32)
    draft_row = np.array([-0.3, 1.2, 0.4, -1.0, 0.9, 0.1], np.float32)
    P = [int(w) for w in spec_emul.weights(target_row, np.float32(target_row.max()))]
    Q = [int(w) for w in spec_emul.weights(draft_row, np.float32(draft_row.max()))]
    SP, SQ = sum(P), sum(Q)
    x = 1
    assert Fraction(P[x], SP) < Fraction(Q[x], SQ)
    # child word in the middle of token x's draft interval
    cw = ((sum(Q[:x]) * 2 + Q[x]) << 31) // SQ
    res = [max(Fraction(0), Fraction(P[v], SP) - Fraction(Q[v], SQ)) for v in range(V)]
    Z = sum(res)
    cdf = np.cumsum([float(r / Z) for r in res])
    words_r = np.linspace(0, (1 << 32) - 1, 4001).astype(np.uint64)
    keep = np.array([np.min(np.abs(cdf - float(r) / 2**32)) > 1e-6 for r in words_r])
    words_r = words_r[keep].astype(np.uint32)
    T = len(words_r)
    t = oracle.build_tree(np.tile(draft_row, (T, 1, 1)), 1, 1, 1, 1, m_max=1,
                          child_words=np.full((T, 1, 1), cw, np.uint32))
    assert (t["tokens"][:, 0] == x).all()
    words = np.stack([np.full(T, (1 << 32) - 1, np.uint32), words_r], axis=1)
    acc, alen, bon = oracle.accept_rrs(np.tile(target_row, (T, 2, 1)), np.tile(draft_row, (T, 1, 1)), t["tokens"],
                                       t["parent"], t["src_row"], t["num_nodes"], 1, words)
    assert (alen == 0).all()
    want = np.searchsorted(cdf, words_r.astype(np.float64) / 2**32, side="right")
    assert np.array_equal(bon, want)
    assert res[x] == 0 and not (bon == x).any()
