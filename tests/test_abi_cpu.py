"""C-ABI checks that need no GPU: libeagle.so loads, exports every function
include/eagle.h declares, and rejects invalid arguments before any launch."""
import ctypes as C
import os
import re

import numpy as np
import pytest

import eagle_tree_verification_draft_amd as E
import oracle

HDR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "eagle.h")


def _declared():
    txt = open(HDR).read()
    return sorted(set(re.findall(r"\b(eagle_[a-z_]+)\s*\(", txt)))


def test_exports_match_header():
    L = E.lib()
    decl = _declared()
    assert sorted(E.EXPORTS) == decl
    for name in decl:
        assert hasattr(L, name), name


def test_status_strings():
    L = E.lib()
    for s in (0, -1, -2, -3, -4):
        assert L.eagle_status_string(s)


def _tree(**over):
    d = dict(depth=6, topk=10, children=10, m=60, chain_k=0, vocab=32000, m_max=60, r_max=51)
    d.update(over)
    return E.TreeParams(**d)


def _call_build(p, batch=1, logits=1 << 20, dtype=E.EAGLE_BF16, stride=None, ws=1 << 21, wsb=1 << 30):
    L = E.lib()
    out = C.c_void_p(1 << 24)
    return L.eagle_build_tree(C.byref(p), batch, C.c_void_p(logits) if logits else None, dtype,
                              p.vocab if stride is None else stride, None, out, out, out, out, out, out,
                              C.c_void_p(ws) if ws else None, wsb, None)


@pytest.mark.parametrize("over,want", [
    (dict(m=0), E.EAGLE_ERR_INVALID),
    (dict(m=61), E.EAGLE_ERR_INVALID),
    (dict(m_max=65, m=60), E.EAGLE_ERR_UNSUPPORTED),
    (dict(children=17), E.EAGLE_ERR_UNSUPPORTED),
    (dict(vocab=(1 << 17) + 1), E.EAGLE_ERR_UNSUPPORTED),
    (dict(r_max=50), E.EAGLE_ERR_INVALID),
    (dict(depth=0), E.EAGLE_ERR_INVALID),
    (dict(chain_k=61), E.EAGLE_ERR_INVALID),
    (dict(depth=8, topk=16, children=16, m=60), E.EAGLE_ERR_UNSUPPORTED),   # 1808 candidates
    # k = 5 > C = 2: depth 1 has 2 nodes to expand, so 2 + 4 = 6 candidates are
    # generated (C + (D-1)kC = 12 bounds them); the rerank cannot keep 8
    (dict(depth=2, topk=5, children=2, m=8, m_max=8, r_max=6), E.EAGLE_ERR_INVALID),
])
def test_build_tree_rejects_bad_params(over, want):
    assert _call_build(_tree(**over)) == want
    assert E.lib().eagle_last_error()


def test_m_up_to_the_generated_candidates_is_accepted():
    # the same k > C tree keeping all 6 generated candidates is valid, and the
    # oracle builds it (its own check is against the generated count too)
    p = _tree(depth=2, topk=5, children=2, m=6, m_max=8, r_max=6)
    assert E.lib().eagle_build_tree_workspace_size(C.byref(p), 1) > 0
    rng = np.random.default_rng(3)
    logits = rng.standard_normal((1, 6, 100)).astype(np.float32)
    t = oracle.build_tree(logits, 2, 5, 2, 6, m_max=8)
    assert int(t["num_nodes"][0]) == 6
    with pytest.raises(oracle.OracleError):
        oracle.build_tree(logits, 2, 5, 2, 7, m_max=8)


def test_build_tree_rejects_null_stride_and_workspace():
    p = _tree()
    assert _call_build(p, logits=0) == E.EAGLE_ERR_INVALID
    assert _call_build(p, stride=31999) == E.EAGLE_ERR_INVALID
    assert _call_build(p, ws=0) == E.EAGLE_ERR_WORKSPACE
    assert _call_build(p, wsb=16) == E.EAGLE_ERR_WORKSPACE
    assert _call_build(p, ws=(1 << 21) + 8) == E.EAGLE_ERR_WORKSPACE          # misaligned
    assert _call_build(p, dtype=7) == E.EAGLE_ERR_UNSUPPORTED
    # rows of any length up to 2^17 are handled (long ones by the streaming kernel);
    # above it the exact fp64 weight sums are no longer guaranteed
    assert _call_build(_tree(vocab=(1 << 17) + 1), dtype=E.EAGLE_F32) == E.EAGLE_ERR_UNSUPPORTED
    assert E.lib().eagle_build_tree_workspace_size(C.byref(_tree(m=0)), 1) == 0
    assert E.lib().eagle_build_tree_workspace_size(C.byref(p), 4) > 0


def _attn(**over):
    d = dict(num_q_heads=32, num_kv_heads=8, head_dim=128, m_max=60, block_size=16, max_blocks=4,
             max_prefix=0, scale=0.0, dtype=E.EAGLE_BF16)
    d.update(over)
    return E.AttnParams(**d)


def _call_attn(a, bt=True, align=0, ws=1 << 21, wsb=1 << 30):
    L = E.lib()
    p = C.c_void_p((1 << 24) + align)
    return L.eagle_tree_attn(C.byref(a), 2, p, p, p, p, p, C.c_void_p(1 << 22) if bt else None,
                             p, p, p, p, C.c_void_p(ws), wsb, None)


@pytest.mark.parametrize("over,want", [
    (dict(num_q_heads=30), E.EAGLE_ERR_INVALID),
    (dict(head_dim=64), E.EAGLE_ERR_UNSUPPORTED),
    (dict(dtype=E.EAGLE_F32, head_dim=96), E.EAGLE_ERR_UNSUPPORTED),
    (dict(m_max=65), E.EAGLE_ERR_UNSUPPORTED),
    (dict(block_size=12), E.EAGLE_ERR_UNSUPPORTED),
    (dict(block_size=0, max_blocks=0, max_prefix=13), E.EAGLE_ERR_UNSUPPORTED),
    (dict(max_blocks=0), E.EAGLE_ERR_INVALID),
    (dict(scale=float("nan")), E.EAGLE_ERR_INVALID),
    (dict(num_q_heads=2048), E.EAGLE_ERR_UNSUPPORTED),
    (dict(num_q_heads=(1 << 31) - 1, num_kv_heads=1), E.EAGLE_ERR_UNSUPPORTED),
])
def test_tree_attn_rejects_bad_params(over, want):
    assert _call_attn(_attn(**over)) == want


def test_tree_attn_rejects_missing_table_misalignment_and_workspace():
    assert _call_attn(_attn(), bt=False) == E.EAGLE_ERR_INVALID
    assert _call_attn(_attn(), align=2) == E.EAGLE_ERR_UNSUPPORTED
    assert _call_attn(_attn(), wsb=8) == E.EAGLE_ERR_WORKSPACE
    assert E.lib().eagle_tree_attn_workspace_size(C.byref(_attn()), 2) >= 256


def test_tree_attn_size_limits():
    """Query rows and the launch's workgroup count stay within their stated
    limits; past them the size query returns 0 and the call is unsupported."""
    L = E.lib()
    a = _attn(num_q_heads=64, num_kv_heads=64, m_max=64, block_size=16, max_blocks=4)
    assert L.eagle_tree_attn_workspace_size(C.byref(a), 1 << 14) > 0          # 2^26 query rows
    assert L.eagle_tree_attn_workspace_size(C.byref(a), (1 << 14) + 1) == 0
    big = _attn(num_q_heads=64, num_kv_heads=64, m_max=64, block_size=1 << 16, max_blocks=1 << 14)
    assert L.eagle_tree_attn_workspace_size(C.byref(big), 1 << 14) == 0        # > 2^31 - 1 workgroups
    assert L.eagle_tree_attn_workspace_size(C.byref(big), 1) > 0


def _call_commit(a, max_accept=6, bt=True, align=0, null_slot=False, ws=1 << 21, wsb=256):
    L = E.lib()
    p = C.c_void_p(1 << 24)
    kd = C.c_void_p((1 << 24) + align)
    return L.eagle_kv_commit(C.byref(a), 2, kd, p, p, p, max_accept, p, p, p,
                             C.c_void_p(1 << 22) if bt else None, None if null_slot else p, p,
                             C.c_void_p(ws), wsb, None)


def test_kv_commit_rejects_bad_params():
    assert _call_commit(_attn(num_q_heads=30)) == E.EAGLE_ERR_INVALID
    assert _call_commit(_attn(head_dim=64)) == E.EAGLE_ERR_UNSUPPORTED
    assert _call_commit(_attn(), max_accept=0) == E.EAGLE_ERR_INVALID
    assert _call_commit(_attn(), bt=False) == E.EAGLE_ERR_INVALID
    assert _call_commit(_attn(), null_slot=True) == E.EAGLE_ERR_INVALID
    assert _call_commit(_attn(), align=4) == E.EAGLE_ERR_UNSUPPORTED
    assert _call_commit(_attn(), wsb=8) == E.EAGLE_ERR_WORKSPACE
    assert _call_commit(_attn(), ws=(1 << 21) + 16) == E.EAGLE_ERR_WORKSPACE


def test_tree_expand_and_finish_reject_bad_params():
    L = E.lib()
    p = _tree()
    x = C.c_void_p(1 << 24)
    ws = C.c_void_p(1 << 21)
    need = L.eagle_build_tree_workspace_size(C.byref(p), 2)

    def expand(level, params=p, ptr=x, stride=32000, wsb=need, dtype=E.EAGLE_BF16):
        return L.eagle_tree_expand(C.byref(params), 2, level, x, dtype, stride, ptr, x, x, ws, wsb, None)

    assert expand(-1) == E.EAGLE_ERR_INVALID
    assert expand(6) == E.EAGLE_ERR_INVALID          # levels are 0 .. depth - 1
    assert expand(0, ptr=None) == E.EAGLE_ERR_INVALID
    assert expand(0, stride=100) == E.EAGLE_ERR_INVALID
    assert expand(0, wsb=need - 256) == E.EAGLE_ERR_WORKSPACE
    assert expand(0, dtype=7) == E.EAGLE_ERR_UNSUPPORTED
    assert expand(0, params=_tree(children=17)) == E.EAGLE_ERR_UNSUPPORTED
    assert L.eagle_tree_finish(C.byref(p), 2, x, x, x, None, x, x, ws, need, None) == E.EAGLE_ERR_INVALID
    assert L.eagle_tree_finish(C.byref(p), 2, x, x, x, x, x, x, ws, 256, None) == E.EAGLE_ERR_WORKSPACE
    assert L.eagle_tree_expand(C.byref(p), 0, 3, x, E.EAGLE_BF16, 32000, x, x, x, ws, need, None) == E.EAGLE_OK
    assert L.eagle_tree_finish(C.byref(p), 0, x, x, x, x, x, x, ws, need, None) == E.EAGLE_OK


def test_pdraft_prepare_rejects_bad_params():
    L = E.lib()
    x = C.c_void_p(1 << 24)
    ws = C.c_void_p(1 << 21)

    def call(p, align=0, wsb=256, null_hidden=False, batch=2):
        th = C.c_void_p((1 << 24) + align)
        return L.eagle_pdraft_prepare(C.byref(p), batch, x, x, x, x, x, x, None if null_hidden else th, x, x, x, x, x,
                                      x, x, x, ws, wsb, None)

    ok = E.PdraftParams(60, 6, 7, 4096, 5, E.EAGLE_BF16)
    assert call(E.PdraftParams(60, 6, 0, 4096, 5, E.EAGLE_BF16)) == E.EAGLE_ERR_INVALID
    assert call(E.PdraftParams(65, 6, 7, 4096, 5, E.EAGLE_BF16)) == E.EAGLE_ERR_INVALID
    assert call(E.PdraftParams(60, 0, 7, 4096, 5, E.EAGLE_BF16)) == E.EAGLE_ERR_INVALID
    assert call(E.PdraftParams(60, 6, 7, 4095, 5, E.EAGLE_BF16)) == E.EAGLE_ERR_UNSUPPORTED
    assert call(E.PdraftParams(60, 6, 7, 4096, 5, 3)) == E.EAGLE_ERR_UNSUPPORTED
    assert call(ok, null_hidden=True) == E.EAGLE_ERR_INVALID
    assert call(ok, align=8) == E.EAGLE_ERR_UNSUPPORTED
    assert call(ok, wsb=8) == E.EAGLE_ERR_WORKSPACE
    assert call(ok, batch=0) == E.EAGLE_OK


def test_tree_policy_validation():
    L = E.lib()
    x = C.c_void_p(1 << 24)

    def call(**over):
        p = _tree(**over)
        need = max(256, L.eagle_build_tree_workspace_size(C.byref(p), 1))
        return L.eagle_build_tree(C.byref(p), 0, x, 1, 32000, None, x, x, x, x, x, x, C.c_void_p(1 << 21), need, None)

    assert call(policy=4) == E.EAGLE_ERR_INVALID
    assert call(policy=-1) == E.EAGLE_ERR_INVALID
    assert call(policy=E.EAGLE_POLICY_CONF) == E.EAGLE_OK
    # without rerank the tree has 10 + 5 * 10 = 60 nodes: m_max 59 is too small
    assert call(policy=E.EAGLE_POLICY_NO_RERANK, m_max=59, m=50) == E.EAGLE_ERR_INVALID
    assert call(policy=E.EAGLE_POLICY_CONF_NO_RERANK, m_max=60, m=50) == E.EAGLE_OK


def test_build_tree_template_rejects_bad_params():
    L = E.lib()
    x = C.c_void_p(1 << 24)
    ws = C.c_void_p(1 << 21)

    def call(n=10, tmpl=True, **over):
        p = _tree(**over)
        need = max(256, L.eagle_build_tree_workspace_size(C.byref(_tree()), 2))
        return L.eagle_build_tree_template(C.byref(p), 2, x, 1, 32000, n, x if tmpl else None, x, x, x, x, x, x, x,
                                           ws, need, None)

    assert call(n=0) == E.EAGLE_ERR_INVALID
    assert call(n=61) == E.EAGLE_ERR_INVALID          # above m_max 60
    assert call(tmpl=False) == E.EAGLE_ERR_INVALID
    assert call(children=17) == E.EAGLE_ERR_UNSUPPORTED
    assert call(r_max=0) == E.EAGLE_ERR_INVALID
    assert L.eagle_build_tree_template(C.byref(_tree()), 0, x, 1, 32000, 10, x, x, x, x, x, x, x, x, ws, 1 << 20,
                                       None) == E.EAGLE_OK


def test_sampled_build_and_rrs_reject_bad_params():
    L = E.lib()
    x = C.c_void_p(1 << 24)
    ws = C.c_void_p(1 << 21)

    # (every call below is rejected before a launch, or has batch 0)
    def build(batch=2, **over):
        d = dict(depth=3, topk=2, children=3, m=3, m_max=15, r_max=5)
        d.update(over)
        p = _tree(**d)
        need = max(256, L.eagle_build_tree_workspace_size(C.byref(_tree(**d)), 2))
        return L.eagle_build_tree_sampled(C.byref(p), batch, x, 1, 32000, x, x, x, x, x, x, x, ws, need, None)

    assert build(batch=0) == E.EAGLE_OK                   # 3 + 6 + 6 = 15 candidates fit m_max 15
    assert build(m_max=14) == E.EAGLE_ERR_INVALID
    assert build(policy=E.EAGLE_POLICY_CONF) == E.EAGLE_ERR_INVALID

    def rrs(T=1.0, wsb=None, tgt=x, **over):
        d = dict(mode=E.EAGLE_ACCEPT_SAMPLE, temperature=T, m_max=21, vocab=32000, max_accept=3)
        d.update(over)
        a = E.AcceptParams(**d)
        need = L.eagle_accept_rrs_workspace_size(C.byref(a), 2) if wsb is None else wsb
        return L.eagle_accept_rrs(C.byref(a), 2, tgt, x, 1, 32000, 32000, 5, x, x, x, x, x, x, x, x, ws, need, None)

    assert rrs(T=0.0) == E.EAGLE_ERR_INVALID
    assert rrs(tgt=None) == E.EAGLE_ERR_INVALID
    assert rrs(wsb=256) == E.EAGLE_ERR_WORKSPACE
    assert rrs(max_accept=0) == E.EAGLE_ERR_INVALID
    assert L.eagle_accept_rrs_workspace_size(C.byref(E.AcceptParams(1, 1.0, 21, 32000, 3)), 2) >= 2 * 3 * 32000 * 8


def test_accept_and_mask_reject_bad_params():
    L = E.lib()
    p = C.c_void_p(1 << 24)
    ws = C.c_void_p(1 << 21)
    bad_t = E.AcceptParams(E.EAGLE_ACCEPT_SAMPLE, 0.0, 60, 32000, 6)
    assert L.eagle_accept(C.byref(bad_t), 1, p, 1, 32000, p, p, p, p, p, p, p, ws, 256, None) == E.EAGLE_ERR_INVALID
    no_words = E.AcceptParams(E.EAGLE_ACCEPT_SAMPLE, 1.0, 60, 32000, 6)
    assert L.eagle_accept(C.byref(no_words), 1, p, 1, 32000, p, p, p, None, p, p, p, ws, 256, None) == E.EAGLE_ERR_INVALID
    big = E.AcceptParams(E.EAGLE_ACCEPT_GREEDY, 1.0, 65, 32000, 6)
    assert L.eagle_accept(C.byref(big), 1, p, 1, 32000, p, p, p, None, p, p, p, ws, 256, None) == E.EAGLE_ERR_UNSUPPORTED
    ok = E.AcceptParams(E.EAGLE_ACCEPT_GREEDY, 1.0, 60, 32000, 6)
    assert L.eagle_accept(C.byref(ok), 1, p, 1, 31999, p, p, p, None, p, p, p, ws, 256, None) == E.EAGLE_ERR_INVALID
    assert L.eagle_accept(C.byref(ok), 1, p, 1, 32000, p, p, p, None, p, p, p, ws, 8, None) == E.EAGLE_ERR_WORKSPACE
    assert L.eagle_tree_mask(1, 65, p, p, p, p, p, None, 0, None) == E.EAGLE_ERR_UNSUPPORTED
    assert L.eagle_tree_mask(1, 60, None, p, p, p, p, None, 0, None) == E.EAGLE_ERR_INVALID
    assert L.eagle_workspace_init(None, 0, None) == E.EAGLE_ERR_WORKSPACE


def test_zero_batch_launches_nothing():
    # batch 0 is valid and returns before touching any pointer or the GPU
    L = E.lib()
    p = _tree()
    out = C.c_void_p(1 << 24)
    assert L.eagle_build_tree(C.byref(p), 0, out, 1, 32000, None, out, out, out, out, out, out,
                              C.c_void_p(1 << 21), 1 << 20, None) == E.EAGLE_OK
    assert L.eagle_kv_commit(C.byref(_attn()), 0, out, out, out, out, 6, out, out, out, out, out, out,
                             C.c_void_p(1 << 21), 256, None) == E.EAGLE_OK


def test_build_tree_mask_noalloc_checks_before_any_launch():
    # the call with no workspace: same argument checks as the fused call, a
    # size check against its static scratch, and batch 0 launches nothing
    L = E.lib()
    p = _tree()
    out = C.c_void_p(1 << 24)
    f = L.eagle_build_tree_mask_noalloc
    assert f(C.byref(p), 1, None, 1, 32000, None, out, out, out, out, out, out, out, out, out, None, None) \
        == E.EAGLE_ERR_INVALID
    assert f(C.byref(p), 1, out, 1, 31999, None, out, out, out, out, out, out, out, out, out, None, None) \
        == E.EAGLE_ERR_INVALID
    assert f(C.byref(p), 1, out, 1, 32000, None, None, out, out, out, out, out, out, out, out, None, None) \
        == E.EAGLE_ERR_INVALID
    big = 100000
    assert E.build_tree_workspace_size(p, big) > 4 << 20
    assert f(C.byref(p), big, out, 1, 32000, None, out, out, out, out, out, out, out, out, out, None, None) \
        == E.EAGLE_ERR_WORKSPACE
    assert b"static array holds" in L.eagle_last_error()
    assert f(C.byref(p), 0, out, 1, 32000, None, out, out, out, out, out, out, out, out, out, None, None) \
        == E.EAGLE_OK


def test_logit_rows_marshalling():
    """Rows inside a wider buffer pass their stride; anything else is refused."""
    import torch
    assert E._rows(torch.zeros(2, 3, 10))[1] == 10
    assert E._rows(torch.zeros(2, 3, 16)[..., :10])[1] == 16
    assert E._rows(torch.zeros(4, 1, 16)[..., :10])[1] == 16
    assert E._rows(torch.zeros(1, 1, 10))[1] == 10
    with pytest.raises(ValueError):
        E._rows(torch.zeros(2, 3, 16)[:, :2, :10])      # rows not evenly spaced
    with pytest.raises(ValueError):
        E._rows(torch.zeros(3, 10).t())                 # elements not contiguous
