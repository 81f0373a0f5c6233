"""Helpers for the GPU parity tests: seeded inputs, the oracle on the host,
the HIP path through the C ABI, element-by-element comparison."""
from __future__ import annotations

import dataclasses
import sys

import numpy as np
import torch

import eagle_tree_verification_draft_amd as E
import oracle
import synth
from conftest import to_np

BF16_TOL = 2e-2   # max-abs, bf16 inputs with fp32 accumulation
F32_TOL = 1e-5    # max-abs, fp32 path


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


@dataclasses.dataclass
class Case:
    w: synth.Workload
    seed: int
    draft: torch.Tensor          # on device
    kinds: torch.Tensor          # on device
    attn: synth.AttnInputs       # on device
    words: torch.Tensor          # on device
    otree: dict                  # oracle tree (host)
    target: torch.Tensor         # on device
    step: E.VerifyStep


def make_case(w: synth.Workload, seed: int, device="cuda", gen_device="cuda", plant=False) -> Case:
    draft = synth.draft_logits(w, seed, device=gen_device).to(device)
    kinds = synth.kinds_tensor(w, device)
    ot = oracle.build_tree(to_np(draft), w.depth, w.topk, w.children, w.m, chain_k=w.chain_k,
                           kinds=w.kinds, m_max=w.m_max)
    target = synth.target_logits(w, seed, draft.to(gen_device), torch.from_numpy(ot["src_row"]),
                                 torch.from_numpy(ot["num_nodes"]), device=gen_device).to(device)
    if plant:
        for b in range(w.batch):
            n = int(ot["num_nodes"][b])
            deepest = max(range(n), key=lambda i: (ot["depth"][b, i], -i))
            path, a = [], deepest
            while a >= 0:
                path.append(a)
                a = int(ot["parent"][b, a])
            synth.plant_path(target, w, b, path[::-1], torch.from_numpy(ot["tokens"]))
    attn = synth.attn_inputs(w, seed, device=gen_device)
    attn = dataclasses.replace(
        attn, q=attn.q.to(device), k_draft=attn.k_draft.to(device), v_draft=attn.v_draft.to(device),
        k_cache=attn.k_cache.to(device), v_cache=attn.v_cache.to(device),
        block_table=None if attn.block_table is None else attn.block_table.to(device),
        prefix_len=attn.prefix_len.to(device))
    words = synth.rand_words(w, seed, device)
    step = E.VerifyStep(E.StepShape(**synth.step_dims(w, attn)), device)
    return Case(w, seed, draft, kinds, attn, words, ot, target, step)


def run_gpu(c: Case):
    a = c.attn
    c.step.run(c.draft, c.kinds, a.prefix_len, a.q, a.k_draft, a.v_draft, a.k_cache, a.v_cache,
               a.block_table, c.target, c.words if c.w.accept_mode == synth.ACCEPT_SAMPLE else None)
    torch.cuda.synchronize()


def assert_tree_equal(c: Case, b_list=None):
    s, ot = c.step, c.otree
    for k in ("tokens", "parent", "depth", "src_row"):
        got = getattr(s, k).cpu().numpy()
        if b_list is not None:
            got, want = got[b_list], ot[k][b_list]
        else:
            want = ot[k]
        bad = np.argwhere(got != want)
        assert bad.size == 0, f"{k} differs at {bad[:5].tolist()}: gpu {got[tuple(bad[0])]} oracle {want[tuple(bad[0])]}"
    got = s.score.cpu().numpy().view(np.uint64)
    want = ot["score"].view(np.uint64)
    if b_list is not None:
        got, want = got[b_list], want[b_list]
    assert np.array_equal(got, want), "score bits differ"
    assert np.array_equal(s.num_nodes.cpu().numpy(), ot["num_nodes"])


def oracle_mask(c: Case):
    return oracle.tree_mask(c.otree["parent"], c.otree["num_nodes"], c.attn.prefix_len.cpu().numpy())


def attn_host(c: Case, attn=None):
    a = c.attn if attn is None else attn
    return dict(q=to_np(a.q), k_draft=to_np(a.k_draft), v_draft=to_np(a.v_draft), k_cache=to_np(a.k_cache),
                v_cache=to_np(a.v_cache), block_table=None if a.block_table is None else to_np(a.block_table),
                prefix_len=to_np(a.prefix_len))


def gpu_out_f64(c: Case) -> np.ndarray:
    return c.step.out.to(torch.float64).cpu().numpy()


def oracle_attn_rows(h: dict, sel, anc) -> np.ndarray:
    return oracle.tree_attn_rows(h["q"], h["k_draft"], h["v_draft"], h["k_cache"], h["v_cache"],
                                 h["block_table"], h["prefix_len"], anc, sel)


def check_attn_rows(c: Case, sel, tol, attn=None, power=None):
    """Compares selected output rows (b, i, h) against the oracle.

    Returns (max-abs error, relative L2 error over the selected rows).  With
    power = f, each row's error must also stay below f times that row's
    max-abs gap between the oracle with and without the draft keys, so the
    check is sensitive to the tree part of the keys."""
    anc, _ = oracle_mask(c)
    h = attn_host(c, attn)
    ref = oracle_attn_rows(h, sel, anc)
    got = gpu_out_f64(c)
    g = np.stack([got[b, i, hh] for b, i, hh in sel])
    err = np.abs(g - ref)
    assert np.isfinite(g).all(), "non-finite attention output"
    mx = float(err.max()) if err.size else 0.0
    den = float(np.sqrt((ref * ref).sum()))
    rl2 = float(np.sqrt(((g - ref) ** 2).sum())) / den if den > 0 else 0.0
    assert mx <= tol, f"attention max-abs error {mx} > {tol} at row {sel[int(np.argmax(err.max(axis=1)))]}"
    if power is not None:
        nodraft = oracle_attn_rows(h, sel, np.zeros_like(anc))
        gap = np.abs(nodraft - ref).max(axis=1)
        row_err = err.max(axis=1)
        worst = int(np.argmax(row_err / np.maximum(gap, 1e-300)))
        assert (row_err <= power * gap).all(), \
            f"row {sel[worst]}: error {row_err[worst]} not below {power} x draft-key gap {gap[worst]}"
        assert float(gap.min()) > 10 * tol, f"draft keys move row {sel[int(np.argmin(gap))]} by only {gap.min()}"
    return mx, rl2


def sample_rows(c: Case, n_rows: int, rng) -> list:
    nn = c.otree["num_nodes"]
    out = []
    for _ in range(n_rows):
        b = int(rng.integers(0, c.w.batch))
        i = int(rng.integers(0, max(1, int(nn[b]))))
        h = int(rng.integers(0, c.w.num_q_heads))
        out.append((b, i, h))
    return out


def oracle_accept(c: Case, b_list=None):
    tn = to_np(c.target)
    words = to_np(c.words) if c.w.accept_mode == synth.ACCEPT_SAMPLE else None
    tok, par, nn = c.otree["tokens"], c.otree["parent"], c.otree["num_nodes"]
    if b_list is not None:
        tn, tok, par, nn = tn[b_list], tok[b_list], par[b_list], nn[b_list]
        words = None if words is None else words[b_list]
    return oracle.accept(c.w.accept_mode, tn, tok, par, nn, c.w.max_accept, rand_words=words,
                         T=c.w.temperature)


def assert_accept_equal(c: Case, b_list=None):
    acc, alen, bon = oracle_accept(c, b_list)
    g_acc, g_len, g_bon = (c.step.accepted.cpu().numpy(), c.step.accept_len.cpu().numpy(),
                           c.step.bonus.cpu().numpy())
    if b_list is not None:
        g_acc, g_len, g_bon = g_acc[b_list], g_len[b_list], g_bon[b_list]
    assert np.array_equal(g_len, alen), f"accept_len gpu {g_len[:8]} oracle {alen[:8]}"
    assert np.array_equal(g_acc, acc), "accepted nodes differ"
    assert np.array_equal(g_bon, bon), f"bonus gpu {g_bon[:8]} oracle {bon[:8]}"
    return alen
