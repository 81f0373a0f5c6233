"""Pins for the oracle's acceptance walk (EAGLE-1 explainer, "Verification":
draft tokens are accepted by comparing the draft and target distributions, the
remainder is discarded after a rejection and a token is resampled, so the
output follows the target distribution; EAGLE-2 explainer, "Key
contributions": lossless through rejection sampling).

EAGLE-2's children are the top-k of the draft row, not samples from it, so
the draft is a point mass on each child and the lossless test accepts child x
with the target's residual probability of x (the rule this oracle follows).

Pins: greedy equals the brute-force longest matching path; planted paths give
the full depth; rejection sampling reproduces the target distribution
(chi-square over 10^6 trials on a tiny vocabulary); reach probabilities and the
mean accepted length equal their closed forms; one-hot and zero-mass targets
behave as the definitions force; a naive ratio rule with top-k children fails
the same chi-square test (the test has power).
"""
import numpy as np
import pytest
import scipy.stats
import torch

import oracle
import spec_emul
import synth
from conftest import to_np


def _argmax(row):
    lf = spec_emul.to_f32(row)
    return int(np.flatnonzero(lf == lf.max())[0])


def _greedy_bruteforce(tokens, parent, n, target):
    """node i is matched iff token(i) == argmax of its parent's target row; the
    accepted path ends at the deepest node whose whole root path is matched."""
    g = [_argmax(target[u]) for u in range(n + 1)]
    matched = [tokens[i] == g[parent[i] + 1] for i in range(n)]
    best, best_depth = -1, 0
    for i in range(n):
        a, ok, dep = i, True, 0
        while a >= 0:
            ok &= matched[a]
            dep += 1
            a = parent[a]
        if ok and dep > best_depth:
            best, best_depth = i, dep
    path = []
    a = best
    while a >= 0:
        path.append(a)
        a = parent[a]
    path = path[::-1]
    return path, g[best + 1]


@pytest.mark.parametrize("base,seed,plant", [(1, 51, False), (2, 52, True), (2, 53, False),
                                             (5, 54, True)])
def test_greedy_equals_bruteforce(orc, base, seed, plant):
    over = dict(batch=3)
    if base == 5:
        over.update(vocab=3000, kinds=[0, 1, 0])
    w = synth.small_workload(base, **over)
    d = synth.draft_logits(w, seed)
    t = orc.build_tree(to_np(d), w.depth, w.topk, w.children, w.m, chain_k=w.chain_k,
                       kinds=w.kinds, m_max=w.m_max)
    tgt = synth.target_logits(w, seed, d, torch.from_numpy(t["src_row"]),
                              torch.from_numpy(t["num_nodes"]))
    if plant:
        for b in range(w.batch):
            # plant the path through the deepest node 0 -> ... chain of first children
            n = int(t["num_nodes"][b])
            deepest = max(range(n), key=lambda i: (t["depth"][b, i], -i))
            path, a = [], deepest
            while a >= 0:
                path.append(a)
                a = int(t["parent"][b, a])
            synth.plant_path(tgt, w, b, path[::-1], torch.from_numpy(t["tokens"]))
    tn = to_np(tgt)
    acc, alen, bon = orc.accept(0, tn, t["tokens"], t["parent"], t["num_nodes"], w.max_accept)
    for b in range(w.batch):
        n = int(t["num_nodes"][b])
        path, bonus = _greedy_bruteforce(list(t["tokens"][b]), list(t["parent"][b]), n, tn[b])
        assert list(acc[b, :alen[b]]) == path
        assert (acc[b, alen[b]:] == -1).all()
        assert bon[b] == bonus
        if plant:
            assert alen[b] == max(t["depth"][b, :n])


# ---------------------------------------------------------------------------
# rejection sampling on a tiny vocabulary
# ---------------------------------------------------------------------------

V8 = 8
# tree: node 0 (token 2) and node 1 (token 5) are root children; node 2 (token 7) is node 0's child
TOK = np.array([[2, 5, 7]], np.int32)
PAR = np.array([[-1, -1, 0]], np.int32)


def _tiny_target(seed, T_scale=1.5):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((1, 4, V8)) * T_scale).astype(np.float32)


def _run_trials(orc, target, n, seed, T=1.0):
    rng = np.random.default_rng(seed)
    words = rng.integers(0, 1 << 32, size=(n, 4), dtype=np.uint64).astype(np.uint32)
    tg = np.ascontiguousarray(np.broadcast_to(target, (n, 4, V8)))
    toks = np.ascontiguousarray(np.broadcast_to(TOK, (n, 3)))
    pars = np.ascontiguousarray(np.broadcast_to(PAR, (n, 3)))
    nn = np.full(n, 3, np.int32)
    return orc.accept(1, tg, toks, pars, nn, 2, rand_words=words, T=T)


def _first_emitted(acc, alen, bon):
    first = np.where(alen > 0, TOK[0][np.maximum(acc[:, 0], 0)], bon)
    return first


def _pdist(target_row, T=1.0):
    lf = target_row.astype(np.float32)
    w = spec_emul.weights(lf, lf.max(), T)
    return w / w.sum()


@pytest.mark.parametrize("T", [1.0, 0.6])
def test_rejection_sampling_reproduces_target_chi_square(orc, T):
    target = _tiny_target(7)
    n = 1_000_000
    acc, alen, bon = _run_trials(orc, target, n, 100, T=T)
    # first emitted token ~ p(root row)
    first = _first_emitted(acc, alen, bon)
    obs = np.bincount(first, minlength=V8)
    exp = _pdist(target[0, 0], T) * n
    keep = exp > 0
    assert obs[~keep].sum() == 0
    chi = scipy.stats.chisquare(obs[keep], exp[keep])
    assert chi.pvalue > 1e-3, chi
    # second emitted token given node 0 (token 2) accepted ~ p(node 0's row = row 1)
    sel = (alen >= 1) & (acc[:, 0] == 0)
    second = np.where(alen[sel] >= 2, 7, bon[sel])
    obs2 = np.bincount(second, minlength=V8)
    exp2 = _pdist(target[0, 1], T) * sel.sum()
    keep2 = exp2 > 0
    chi2 = scipy.stats.chisquare(obs2[keep2], exp2[keep2])
    assert chi2.pvalue > 1e-3, chi2


def test_reach_probabilities_closed_form(orc):
    target = _tiny_target(8)
    n = 400_000
    acc, alen, bon = _run_trials(orc, target, n, 5)
    p0 = _pdist(target[0, 0])
    p1 = _pdist(target[0, 1])
    reach = {0: p0[2], 1: p0[5], 2: p0[2] * p1[7]}
    for node, pr in reach.items():
        freq = np.mean((acc == node).any(axis=1))
        assert abs(freq - pr) < 5 * np.sqrt(pr * (1 - pr) / n) + 1e-9
    e_tau = reach[0] + reach[1] + reach[2]
    sd = np.sqrt(alen.var() / n)
    assert abs(alen.mean() - e_tau) < 5 * sd + 1e-9


def test_one_hot_and_zero_mass_targets(orc):
    # one-hot on node 0's token at the root: always accepted; zero mass on both
    # root children: never accepted and the bonus follows p
    t = np.full((1, 4, V8), -100.0, np.float32)
    t[0, 0, 2] = 0.0
    t[0, 1] = 0.0
    acc, alen, bon = _run_trials(orc, t, 20_000, 3)
    assert (acc[:, 0] == 0).all()
    t2 = _tiny_target(9)
    t2[0, 0, 2] = -200.0
    t2[0, 0, 5] = -200.0
    acc, alen, bon = _run_trials(orc, t2, 200_000, 4)
    assert (alen == 0).all()
    obs = np.bincount(bon, minlength=V8)
    exp = _pdist(t2[0, 0]) * len(bon)
    keep = exp > 0
    assert obs[~keep].sum() == 0
    assert scipy.stats.chisquare(obs[keep], exp[keep]).pvalue > 1e-3


def test_naive_ratio_rule_with_topk_children_fails(orc):
    """Negative control: accept child x with min(1, p(x)/q(x)) and resample
    from max(0, p - q) -- the sampled-children rule -- applied to deterministic
    top-k children.  Its first-token distribution is not p; the chi-square test
    used above must reject it."""
    rng = np.random.default_rng(11)
    p = _pdist(_tiny_target(7)[0, 0])
    ql = (rng.standard_normal(V8) * 1.5).astype(np.float32)
    q = np.exp(ql - ql.max())
    q /= q.sum()
    kids = list(np.argsort(-q, kind="stable")[:2])
    n = 1_000_000
    u = rng.random((n, 3))
    out = np.empty(n, np.int64)
    res = np.maximum(p - q, 0)
    res /= res.sum()
    cres = np.cumsum(res)
    for j in range(n):
        for c_i, x in enumerate(kids):
            if u[j, c_i] < min(1.0, p[x] / q[x]):
                out[j] = x
                break
        else:
            out[j] = min(int(np.searchsorted(cres, u[j, 2], side="right")), V8 - 1)
    obs = np.bincount(out, minlength=V8)
    exp = p * n
    keep = exp > 0
    pv = scipy.stats.chisquare(obs[keep], exp[keep] * obs[keep].sum() / exp[keep].sum()).pvalue
    assert pv < 1e-6
