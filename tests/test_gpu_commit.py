"""KV commit through the C ABI against the oracle, bit-exact: both caches
(every element, committed or not), the slot mapping, the new prefix lengths
and the device error bits, for contiguous and paged caches (pages of 8, 16, 24
and 64 keys) in bf16 and fp32, GQA and MHA head counts, and per sequence the
edge cases of the commit rules: nothing accepted, a path that runs into the
capacity, an unassigned page, an invalid node id, a prefix past the capacity,
accept lengths out of range, prefix_len_out aliasing prefix_len.  The last
test commits the path eagle_accept chose on a full small step and checks the
result against the oracle's accept followed by the oracle's commit."""
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


def _randn(rng, shape, dtype):
    return torch.from_numpy(rng.standard_normal(shape).astype(np.float32)).to(dtype)


def _inputs(name, dtype, bs, B, M, Hkv, d, P, max_accept, spare_pages=3):
    """Draft K/V, caches of capacity P (paged: ceil(P / bs) pages per sequence
    in a random permutation plus spare pages), prefix lengths leaving room for
    most paths, accepted node ids (distinct, -1 padded) and their count."""
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    kd, vd = _randn(rng, (B, M, Hkv, d), dtype), _randn(rng, (B, M, Hkv, d), dtype)
    if bs == 0:
        kc, vc, table = _randn(rng, (B, Hkv, P, d), dtype), _randn(rng, (B, Hkv, d, P), dtype), None
    else:
        nblk = (P + bs - 1) // bs
        pages = B * nblk + spare_pages
        table = torch.from_numpy(rng.permutation(pages)[:B * nblk].astype(np.int32).reshape(B, nblk))
        kc, vc = _randn(rng, (pages, Hkv, bs, d), dtype), _randn(rng, (pages, Hkv, d, bs), dtype)
    amax = min(max_accept, M)
    alen = rng.integers(0, amax + 1, size=B).astype(np.int32)
    L = rng.integers(0, P - amax // 2 + 1, size=B).astype(np.int32)
    acc = np.full((B, max_accept), -1, np.int32)
    for b in range(B):
        acc[b, :alen[b]] = rng.choice(M, size=int(alen[b]), replace=False)
    return dict(kd=kd, vd=vd, kc=kc, vc=vc, table=table, L=L, alen=alen, acc=acc)


def _run(x, dtype, bs, M, Hkv, d, P, max_prefix=0, alias=False):
    """(k_cache, v_cache, slot_mapping, prefix_len_out, error bits) from the C ABI."""
    dev = "cuda"
    B = x["kd"].shape[0]
    maxb = 0 if x["table"] is None else x["table"].shape[1]
    a = E.AttnParams(Hkv, Hkv, d, M, bs, maxb, P if bs == 0 else max_prefix, 0.0, E.dtype_code(dtype))
    kc, vc = x["kc"].to(dev), x["vc"].to(dev)
    ws = torch.empty(256, dtype=torch.uint8, device=dev)
    E.workspace_init(ws)
    pl = torch.from_numpy(x["L"]).to(dev)
    plo = pl if alias else torch.full((B,), -7, dtype=torch.int32, device=dev)
    slot = torch.full((B, M), -7, dtype=torch.int32, device=dev)
    E.kv_commit(a, B, x["kd"].to(dev), x["vd"].to(dev), torch.from_numpy(x["acc"]).to(dev),
                torch.from_numpy(x["alen"]).to(dev), pl, kc, vc,
                None if x["table"] is None else x["table"].to(dev), slot, plo, ws)
    torch.cuda.synchronize()
    return kc.cpu(), vc.cpu(), slot.cpu().numpy(), plo.cpu().numpy(), E.read_errors(ws)


def _oracle(x, max_prefix=0):
    return oracle.kv_commit(to_np(x["kd"]), to_np(x["vd"]), x["acc"], x["alen"], x["L"], to_np(x["kc"]),
                            to_np(x["vc"]), None if x["table"] is None else x["table"].numpy(),
                            max_prefix=max_prefix)


def _compare(got, want):
    kc, vc, slot, plo, errs = got
    okc, ovc, oslot, oplo, (ftree, fprefix) = want
    assert np.array_equal(plo, oplo), (plo, oplo)
    assert np.array_equal(slot, oslot)
    assert np.array_equal(to_np(kc), okc)
    assert np.array_equal(to_np(vc), ovc)
    assert bool(errs & E.DEVERR_TREE) == (ftree > 0), (errs, ftree)
    assert bool(errs & E.DEVERR_PREFIX) == (fprefix > 0), (errs, fprefix)
    assert errs & ~(E.DEVERR_TREE | E.DEVERR_PREFIX) == 0


# (name, dtype, block_size, batch, m_max, kv heads, head_dim, capacity, max_accept)
CASES = [
    ("bf16-contig-gqa8", torch.bfloat16, 0, 6, 60, 8, 128, 256, 60),
    ("bf16-contig-mha32", torch.bfloat16, 0, 2, 60, 32, 128, 2112, 60),
    ("bf16-paged16", torch.bfloat16, 16, 6, 60, 8, 128, 200, 60),
    ("bf16-paged8", torch.bfloat16, 8, 5, 40, 4, 128, 120, 16),
    ("bf16-paged24", torch.bfloat16, 24, 4, 64, 2, 128, 100, 64),
    ("bf16-paged64", torch.bfloat16, 64, 3, 30, 8, 128, 300, 30),
    ("f32-contig-d64", torch.float32, 0, 4, 24, 4, 64, 90, 24),
    ("f32-paged16-d128", torch.float32, 16, 4, 24, 2, 128, 70, 24),
    ("bf16-contig-batch64", torch.bfloat16, 0, 64, 16, 2, 128, 64, 16),
]


@pytest.mark.parametrize("name,dtype,bs,B,M,Hkv,d,P,max_accept", CASES, ids=[c[0] for c in CASES])
def test_commit_matches_oracle(name, dtype, bs, B, M, Hkv, d, P, max_accept):
    say(f"[commit {name}] B={B} M={M} Hkv={Hkv} d={d} capacity={P} bs={bs}")
    x = _inputs(name, dtype, bs, B, M, Hkv, d, P, max_accept)
    _compare(_run(x, dtype, bs, M, Hkv, d, P), _oracle(x))


@pytest.mark.parametrize("bs", [0, 8])
def test_commit_edge_rules(bs):
    """Per sequence: 0 nothing accepted; 1 the path runs past the capacity;
    2 an invalid node id mid-path; 3 a prefix past the capacity; 4 an accept
    length above max_accept; 5 a negative one; 6 a prefix exactly at the
    capacity with nothing accepted; 7 (paged) a path onto an unassigned page;
    8 a full-length path that fits."""
    name = f"edges-{bs}"
    M, Hkv, d, P, ma = 12, 2, 128, 48, 8
    say(f"[commit {name}]")
    x = _inputs(name, torch.bfloat16, bs, 9, M, Hkv, d, P, ma)
    acc = np.tile(np.arange(1, ma + 1, dtype=np.int32), (9, 1))
    acc[2, 3] = M + 5
    x["acc"] = acc
    x["alen"] = np.array([0, 6, 6, 3, ma + 4, -2, 0, 5, ma], np.int32)
    x["L"] = np.array([5, P - 2, 0, P + 1, 10, 3, P, 15, 20], np.int32)
    if bs:
        x["table"][7, 2] = -1          # positions 16..23 of sequence 7
    got, want = _run(x, torch.bfloat16, bs, M, Hkv, d, P), _oracle(x)
    _compare(got, want)
    assert want[3].tolist()[:7] == [5, P, 3, P + 1, 18, 3, P]
    assert want[3][7] == (16 if bs else 20) and want[3][8] == 28


@pytest.mark.parametrize("bs", [0, 16])
def test_commit_prefix_aliased(bs):
    name = f"alias-{bs}"
    say(f"[commit {name}]")
    x = _inputs(name, torch.bfloat16, bs, 7, 32, 4, 128, 160, 32)
    want = _oracle(x)
    _compare(_run(x, torch.bfloat16, bs, 32, 4, 128, 160, alias=True), want)
    assert (want[3] > x["L"]).any()


def test_commit_paged_max_prefix_bound():
    """A paged cache with max_prefix below the pages' total: positions at or
    past max_prefix are not written."""
    say("[commit paged max_prefix]")
    x = _inputs("maxp", torch.bfloat16, 16, 5, 40, 2, 128, 128, 40)
    x["L"] = np.array([90, 95, 100, 0, 60], np.int32)
    x["alen"] = np.array([8, 8, 3, 8, 0], np.int32)
    for b in range(5):
        x["acc"][b, :8] = np.arange(8) + b
    want = _oracle(x, max_prefix=100)
    _compare(_run(x, torch.bfloat16, 16, 40, 2, 128, 128, max_prefix=100), want)
    assert want[3].tolist() == [98, 100, 100, 8, 60]


def test_commit_after_accept_end_to_end():
    """One small greedy step with planted paths: eagle_accept's path committed
    by eagle_kv_commit equals the oracle's accept followed by its commit."""
    w = synth.small_workload(2, batch=4, vocab=4000, num_q_heads=8, num_kv_heads=4, block_size=16,
                             prefix=(30, 90))
    say(f"[commit e2e] {w.name}")
    c = make_case(w, 41, plant=True)
    run_gpu(c)
    s, a = c.step, c.attn
    # a cache with room: the synthetic one plus pages for the longest path
    kc, vc, table = a.k_cache, a.v_cache, a.block_table
    nblk = table.shape[1]
    extra = (w.max_accept + w.block_size - 1) // w.block_size + 1
    pages = kc.shape[0]
    new = torch.arange(pages, pages + w.batch * extra, dtype=torch.int32, device=table.device).view(w.batch, extra)
    table2 = torch.cat([table, new], dim=1).contiguous()
    # the last page of each prefix may be partial; give every sequence its own fresh pages after it
    for b in range(w.batch):
        used = (int(a.prefix_len[b]) + w.block_size - 1) // w.block_size
        table2[b, used:] = -1
        table2[b, used:used + extra] = new[b]
    kc2 = torch.cat([kc, torch.zeros((w.batch * extra,) + tuple(kc.shape[1:]), dtype=kc.dtype,
                                     device=kc.device)]).contiguous()
    vc2 = torch.cat([vc, torch.zeros((w.batch * extra,) + tuple(vc.shape[1:]), dtype=vc.dtype,
                                     device=vc.device)]).contiguous()
    o_acc, o_len, _ = oracle.accept(w.accept_mode, to_np(c.target), c.otree["tokens"], c.otree["parent"],
                                    c.otree["num_nodes"], w.max_accept)
    assert np.array_equal(s.accept_len.cpu().numpy(), o_len)
    assert o_len.max() >= 2
    want = oracle.kv_commit(to_np(a.k_draft), to_np(a.v_draft), o_acc, o_len, a.prefix_len.cpu().numpy(),
                            to_np(kc2), to_np(vc2), table2.cpu().numpy())
    plen = a.prefix_len.clone()
    # the step's attention params with the wider block table
    ap = E.AttnParams.from_buffer_copy(s.attn)
    ap.max_blocks = table2.shape[1]
    E.kv_commit(ap, w.batch, a.k_draft, a.v_draft, s.accepted, s.accept_len, plen, kc2, vc2, table2,
                s.slot_mapping, plen, s.ws_commit)
    torch.cuda.synchronize()
    errs = s.errors()
    got = (kc2.cpu(), vc2.cpu(), s.slot_mapping.cpu().numpy(), plen.cpu().numpy(), errs)
    _compare(got, want)
    assert np.array_equal(plen.cpu().numpy(), a.prefix_len.cpu().numpy() + o_len)
