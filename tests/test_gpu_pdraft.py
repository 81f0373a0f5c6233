"""Parallel-draft inputs (eagle_pdraft_prepare) through the C ABI against the
oracle, bit-exact: ids, positions, hidden-state mapping, MASK and rejected
masks, slot counts, the copied hidden states and the device error bits; in
bf16 and fp32, K = 1 and K = 8, a batch of 64, the path edge cases (nothing
accepted, a full path, a cut path, a clamped length, an empty prefix), and
end to end after a greedy step's eagle_accept."""
from __future__ import annotations

import zlib

import numpy as np
import pytest
import torch

import eagle_tree_verification_draft_amd as E
import oracle
import synth
from conftest import to_np
from gpu_harness import make_case, run_gpu, say

pytestmark = pytest.mark.gpu


def _inputs(name, B, M, MA, H, dtype):
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    tokens = rng.integers(0, 50000, (B, M)).astype(np.int32)
    nn = rng.integers(1, M + 1, B).astype(np.int32)
    alen = np.array([min(int(rng.integers(0, MA + 1)), int(n)) for n in nn], np.int32)
    acc = np.full((B, MA), -1, np.int32)
    for b in range(B):
        acc[b, :alen[b]] = rng.choice(int(nn[b]), size=int(alen[b]), replace=False)
    bonus = rng.integers(0, 50000, B).astype(np.int32)
    L = rng.integers(1, 30000, B).astype(np.int32)
    th = torch.from_numpy(rng.standard_normal((B, M + 1, H)).astype(np.float32)).to(dtype)
    hs = torch.from_numpy(rng.standard_normal(H).astype(np.float32)).to(dtype)
    return dict(tokens=tokens, nn=nn, acc=acc, alen=alen, bonus=bonus, L=L, th=th, hs=hs)


def _run(x, K, mask_id, dtype):
    dev = "cuda"
    B, M = x["tokens"].shape
    MA, H = x["acc"].shape[1], x["th"].shape[-1]
    S = MA + K
    p = E.PdraftParams(M, MA, K, H, mask_id, E.dtype_code(dtype))
    i32 = dict(dtype=torch.int32, device=dev)
    out = dict(input_ids=torch.full((B, S), -9, **i32), positions=torch.full((B, S), -9, **i32),
               hidden_src=torch.full((B, S), -9, **i32), is_mask=torch.full((B, S), 9, dtype=torch.uint8, device=dev),
               rejected=torch.full((B, M), 9, dtype=torch.uint8, device=dev), num_slots=torch.full((B,), -9, **i32),
               draft_hidden=torch.full((B, S, H), 7.0, dtype=dtype, device=dev))
    ws = torch.empty(256, dtype=torch.uint8, device=dev)
    E.workspace_init(ws)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    E.pdraft_prepare(p, B, t(x["tokens"]), t(x["nn"]), t(x["acc"]), t(x["alen"]), t(x["bonus"]), t(x["L"]),
                     x["th"].to(dev), x["hs"].to(dev), out["input_ids"], out["positions"], out["hidden_src"],
                     out["is_mask"], out["rejected"], out["num_slots"], out["draft_hidden"], ws)
    torch.cuda.synchronize()
    got = {k: (to_np(v) if k == "draft_hidden" else v.cpu().numpy()) for k, v in out.items()}
    return got, E.read_errors(ws)


def _compare(x, K, mask_id, dtype):
    got, errs = _run(x, K, mask_id, dtype)
    want = oracle.pdraft_prepare(x["tokens"], x["nn"], x["acc"], x["alen"], x["bonus"], x["L"], to_np(x["th"]),
                                 to_np(x["hs"]), K=K, mask_id=mask_id)
    for k in ("input_ids", "positions", "hidden_src", "is_mask", "rejected", "num_slots", "draft_hidden"):
        assert np.array_equal(got[k], want[k]), k
    ftree, fprefix = want["flags"]
    assert bool(errs & E.DEVERR_TREE) == (ftree > 0) and bool(errs & E.DEVERR_PREFIX) == (fprefix > 0), errs
    assert errs & ~(E.DEVERR_TREE | E.DEVERR_PREFIX) == 0
    return want


# (name, batch, m_max, max_accept, hidden, K, dtype)
CASES = [
    ("bf16-h4096-k7", 4, 60, 6, 4096, 7, torch.bfloat16),
    ("bf16-h4096-b64-k7", 64, 60, 7, 4096, 7, torch.bfloat16),
    ("bf16-h8-k1", 5, 16, 16, 8, 1, torch.bfloat16),
    ("f32-h256-k8", 3, 33, 64, 256, 8, torch.float32),
]


@pytest.mark.parametrize("name,B,M,MA,H,K,dtype", CASES, ids=[c[0] for c in CASES])
def test_prepare_matches_oracle(name, B, M, MA, H, K, dtype):
    say(f"[pdraft {name}]")
    _compare(_inputs(name, B, M, MA, H, dtype), K, 31999, dtype)


def test_prepare_edge_paths():
    """Per sequence: nothing accepted; a full path; a path cut at an invalid
    node id; a length above max_accept (clamped); a negative length; an empty
    prefix (flagged)."""
    say("[pdraft edges]")
    x = _inputs("edges", 6, 12, 5, 64, torch.bfloat16)
    x["nn"][:] = 12
    x["acc"] = np.tile(np.array([4, 9, 1, 0, 7], np.int32), (6, 1))
    x["acc"][2, 2] = 12
    x["alen"] = np.array([0, 5, 5, 8, -1, 3], np.int32)
    x["L"][5] = 0
    want = _compare(x, 3, 2, torch.bfloat16)
    assert want["num_slots"].tolist() == [3, 8, 5, 8, 3, 6]
    assert want["flags"] == (3, 1)


def test_prepare_after_accept_end_to_end():
    """A greedy step with planted paths: eagle_accept's path and bonus feed
    eagle_pdraft_prepare; the result equals the oracle's accept followed by
    the oracle's preparation."""
    w = synth.small_workload(2, batch=4, vocab=4000, num_q_heads=8, num_kv_heads=4, prefix=(30, 90))
    say(f"[pdraft e2e] {w.name}")
    c = make_case(w, 43, plant=True)
    run_gpu(c)
    s = c.step
    o_acc, o_len, o_bon = oracle.accept(w.accept_mode, to_np(c.target), c.otree["tokens"], c.otree["parent"],
                                        c.otree["num_nodes"], w.max_accept)
    assert o_len.max() >= 2
    H, K = 512, 7
    rng = np.random.default_rng(5)
    th = torch.from_numpy(rng.standard_normal((w.batch, w.m_max + 1, H)).astype(np.float32)).to(torch.bfloat16)
    hs = torch.from_numpy(rng.standard_normal(H).astype(np.float32)).to(torch.bfloat16)
    want = oracle.pdraft_prepare(c.otree["tokens"], c.otree["num_nodes"], o_acc, o_len, o_bon,
                                 c.attn.prefix_len.cpu().numpy(), to_np(th), to_np(hs), K=K, mask_id=3)
    x = dict(tokens=s.tokens.cpu().numpy(), nn=s.num_nodes.cpu().numpy(), acc=s.accepted.cpu().numpy(),
             alen=s.accept_len.cpu().numpy(), bonus=s.bonus.cpu().numpy(), L=c.attn.prefix_len.cpu().numpy(),
             th=th, hs=hs)
    got, errs = _run(x, K, 3, torch.bfloat16)
    assert errs == 0
    for k in ("input_ids", "positions", "hidden_src", "is_mask", "rejected", "num_slots", "draft_hidden"):
        assert np.array_equal(got[k], want[k]), k
