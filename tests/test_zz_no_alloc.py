"""The fused build-and-mask call without a workspace (for callers that cannot
allocate): through the C ABI, its outputs must equal those of
eagle_build_tree_mask bit for bit, on two calls in a row (the second with a
smaller batch, so the static scratch holds the first call's contents), and its
device error word must report this call's errors only."""
import numpy as np
import pytest
import torch

import eagle_tree_verification_draft_amd as E
import synth
from gpu_harness import say

pytestmark = pytest.mark.gpu

OUTS = ("tokens", "parent", "depth", "score", "src_row", "num_nodes", "anc", "pos")


def _outputs(w, m_max, dev):
    i32 = dict(dtype=torch.int32, device=dev)
    B = w.batch
    o = {k: torch.full((B, m_max), -7, **i32) for k in ("tokens", "parent", "depth", "src_row", "pos")}
    o["score"] = torch.full((B, m_max), -7.0, dtype=torch.float64, device=dev)
    o["num_nodes"] = torch.full((B,), -7, **i32)
    o["anc"] = torch.zeros((B, m_max), dtype=torch.int64, device=dev)
    return o


def _params(w):
    return E.TreeParams(w.depth, w.topk, w.children, w.m, w.chain_k, w.vocab, w.m_max, w.r_max, 0)


def _run_both(w, seed, dev, poison=False):
    draft = synth.draft_logits(w, seed, dev)
    if poison:
        draft[w.batch - 1, 0, 5] = float("nan")
    kinds = synth.kinds_tensor(w, dev)
    plen = synth.prefix_lengths(w, seed).to(dev)
    p = _params(w)
    ref = _outputs(w, w.m_max, dev)
    ws = torch.empty(E.build_tree_workspace_size(p, w.batch), dtype=torch.uint8, device=dev)
    E.workspace_init(ws)
    E.build_tree_mask(p, w.batch, draft, kinds, plen, ref["tokens"], ref["parent"], ref["depth"], ref["score"],
                      ref["src_row"], ref["num_nodes"], ref["anc"], ref["pos"], ws)
    got = _outputs(w, w.m_max, dev)
    err = torch.full((1,), -1, dtype=torch.int32, device=dev)
    E.build_tree_mask_noalloc(p, w.batch, draft, kinds, plen, got["tokens"], got["parent"], got["depth"],
                              got["score"], got["src_row"], got["num_nodes"], got["anc"], got["pos"], err)
    torch.cuda.synchronize()
    return ref, got, int(err.item()) & 0xFFFFFFFF, E.read_errors(ws)


def _assert_equal(ref, got, seqs=None):
    for k in OUTS:
        a, b = ref[k], got[k]
        if seqs is not None:
            a, b = a[seqs], b[seqs]
        if a.dtype == torch.float64:
            a, b = a.view(torch.int64), b.view(torch.int64)
        assert torch.equal(a, b), f"{k} differs from eagle_build_tree_mask"


def test_noalloc_build_mask_equals_the_workspace_call():
    dev = "cuda"
    big = synth.small_workload(5, batch=12, vocab=7001, prefix=(10, 3000),
                               kinds=[0, 1, 0, 0, 1, 0, 1, 1, 0, 0, 1, 0])
    small = synth.small_workload(5, batch=3, vocab=5003, prefix=(10, 900), kinds=[1, 0, 0])
    for label, w, seed in (("first call, batch 12", big, 41), ("second call, batch 3", small, 42)):
        say(f"[no-alloc build+mask] {label}")
        ref, got, err, ref_err = _run_both(w, seed, dev)
        _assert_equal(ref, got)
        assert err == 0 and ref_err == 0
        assert int(got["num_nodes"].min().item()) > 0


def test_noalloc_error_word_is_per_call():
    dev = "cuda"
    w = synth.small_workload(2, batch=2, vocab=4000, prefix=100)
    say("[no-alloc build+mask] non-finite draft row")
    ref, got, err, ref_err = _run_both(w, 5, dev, poison=True)
    assert err & E.DEVERR_NONFINITE_ROW and ref_err & E.DEVERR_NONFINITE_ROW
    # the poisoned (last) sequence's outputs are unspecified; the others' are not
    _assert_equal(ref, got, seqs=slice(0, w.batch - 1))
    say("[no-alloc build+mask] clean rows after it")
    ref, got, err, ref_err = _run_both(w, 6, dev)
    assert err == 0
    _assert_equal(ref, got)
