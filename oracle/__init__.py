"""CPU oracle for one EAGLE-2 draft-tree verification step (test infrastructure).

Only the tests, the smoke check and the benchmark's CPU-baseline leg use this
package; the product path never does.  It wraps ``oracle.c`` (plain C loops,
fp64 attention) through ctypes and takes numpy arrays on the host.  bf16
inputs are passed as their raw uint16 bit patterns.

Every function follows the passages named in ``oracle.c``'s header; the
arithmetic of the softmax weights is defined there ("Spec S").
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_CFLAGS = ["-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]

OK, ERR_ARG, ERR_DATA, ERR_CLOSURE, ERR_PATH = 0, -1, -2, -3, -4


def build(force: bool = False) -> str:
    """Compile liboracle.so with gcc (always when force=True)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *_CFLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    """Loads liboracle.so (built here when missing or stale), or the library
    ORACLE_LIB names (a sanitizer build, see tests/sanitize.py)."""
    global _lib
    if _lib is None:
        path = os.environ.get("ORACLE_LIB")
        if not path:
            build()
            path = _LIB
        L = C.CDLL(path)
        vp, i32, i64, f32, f64 = C.c_void_p, C.c_int, C.c_int64, C.c_float, C.c_double
        L.orc_exp_spec.restype = f32
        L.orc_exp_spec.argtypes = [f32]
        L.orc_weight.restype = f64
        L.orc_weight.argtypes = [f32, f32, f32]
        L.orc_row_stats.argtypes = [vp, i32, i64, i32, i32, i32, f32, vp, vp, vp, vp]
        L.orc_build_tree.argtypes = [vp, i32, vp, i32, i64, i32, vp, i32, vp, vp, vp, vp, vp, vp, vp,
                                     i32, vp, vp, vp, vp, vp, vp, vp]
        L.orc_build_tree_template.argtypes = [i32, i32, vp, vp, i32, i32, vp, i32, i64, i32, i32] + [vp] * 6
        L.orc_tree_mask.argtypes = [i32, i32, vp, vp, vp, vp, vp]
        L.orc_tree_attn.argtypes = [vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.orc_tree_attn_rows.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp]
        L.orc_kv_commit.argtypes = [vp, i32, i32, vp, vp, vp, vp, i32, vp, vp, vp, vp, vp, vp, vp]
        L.orc_pdraft_prepare.argtypes = [i32] * 7 + [vp] * 16
        L.orc_accept_rrs.argtypes = [f32, i32, i32, i32, i32, vp, vp, i32, i32] + [vp] * 8
        L.orc_accept.argtypes = [i32, f32, i32, i32, i32, i32, vp, i32, i64, vp, vp, vp, vp, vp, vp, vp]
        for f in ("orc_row_stats", "orc_build_tree", "orc_tree_mask", "orc_tree_attn",
                  "orc_tree_attn_rows", "orc_build_tree_template", "orc_kv_commit", "orc_pdraft_prepare", "orc_accept_rrs", "orc_accept", "orc_num_threads"):
            getattr(L, f).restype = i32
        _lib = L
    return _lib


class OracleError(RuntimeError):
    def __init__(self, code, what):
        super().__init__(f"oracle {what} failed with code {code}")
        self.code = code


def _check(code, what):
    if code != OK:
        raise OracleError(code, what)


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _logits(a):
    """(array, dtype code): fp32 stays fp32, uint16 is bf16 bits."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.float32:
        return a, 0
    if a.dtype == np.uint16:
        return a, 1
    raise TypeError(f"logits must be float32 or uint16 (bf16 bits), got {a.dtype}")


def num_threads() -> int:
    return lib().orc_num_threads()


def exp_spec(x) -> np.ndarray:
    x = np.asarray(x, dtype=np.float32)
    f = lib().orc_exp_spec
    return np.array([f(float(v)) for v in x.ravel()], dtype=np.float32).reshape(x.shape)


def weight(l, M, T=1.0) -> float:
    return lib().orc_weight(float(l), float(M), float(T))


def row_stats(logits, C: int, T: float = 1.0):
    """logits [rows][V] -> (M [rows] f32, W [rows] f64, top_id [rows][C], top_w [rows][C] f64)."""
    a, dt = _logits(logits)
    rows, V = a.shape
    M = np.zeros(rows, np.float32)
    W = np.zeros(rows, np.float64)
    tid = np.zeros((rows, C), np.int32)
    tw = np.zeros((rows, C), np.float64)
    _check(lib().orc_row_stats(_p(a), dt, V, rows, V, C, T, _p(M), _p(W), _p(tid), _p(tw)), "row_stats")
    return M, W, tid, tw


class _TreeParams(C.Structure):
    _fields_ = [(n, C.c_int) for n in ("depth", "topk", "children", "m", "chain_k", "vocab", "policy")]


def build_tree(draft_logits, depth, topk, children, m, chain_k=0, kinds=None, m_max=None,
               debug=False, policy=0, child_words=None):
    """draft_logits [B][R_max][V] -> dict of tree arrays (output order), plus candidates if debug.
    policy: 0 EAGLE-2, 1 no rerank, 2 confidence ranking, 3 confidence ranking without rerank
    (see oracle.c).  child_words [B][R_max][children] uint32: children drawn from
    the draft rows (the tree is then every candidate, in creation order)."""
    a, dt = _logits(draft_logits)
    B, R, V = a.shape
    if m_max is None:
        m_max = m
    kinds = np.zeros(B, np.int32) if kinds is None else np.ascontiguousarray(kinds, dtype=np.int32)
    p = _TreeParams(depth, topk, children, m, chain_k, V, policy)
    out = {k: np.zeros((B, m_max), np.int32) for k in ("tokens", "parent", "depth", "src_row")}
    out["score"] = np.zeros((B, m_max), np.float64)
    out["num_nodes"] = np.zeros(B, np.int32)
    nmax = max(children + (depth - 1) * topk * children, chain_k)
    dbg = {}
    if debug:
        dbg = {k: np.zeros((B, nmax), np.int32) for k in ("token", "parent", "depth", "row", "rank")}
        dbg["V"] = np.zeros((B, nmax), np.float64)
        dbg["n"] = np.zeros(B, np.int32)
    cw = None if child_words is None else np.ascontiguousarray(child_words).view(np.uint32)
    if cw is not None and cw.shape != (B, R, children):
        raise ValueError("child_words must be [B][R_max][children]")
    code = lib().orc_build_tree(
        C.byref(p), B, _p(a), dt, V, R, _p(kinds), m_max, _p(cw),
        _p(out["tokens"]), _p(out["parent"]), _p(out["depth"]), _p(out["score"]), _p(out["src_row"]),
        _p(out["num_nodes"]), nmax, _p(dbg.get("n")), _p(dbg.get("token")), _p(dbg.get("parent")),
        _p(dbg.get("depth")), _p(dbg.get("V")), _p(dbg.get("row")), _p(dbg.get("rank")))
    _check(code, "build_tree")
    if debug:
        out["cand"] = dbg
    return out


def build_tree_template(draft_logits, tmpl_parent, tmpl_child, children, m_max=None):
    """EAGLE-1 static tree: template node i is the tmpl_child[i]-th top token of
    its parent's row (see oracle.c).  draft_logits [B][R_max][V]."""
    a, dt = _logits(draft_logits)
    B, R, V = a.shape
    tp = np.ascontiguousarray(tmpl_parent, dtype=np.int32)
    tc = np.ascontiguousarray(tmpl_child, dtype=np.int32)
    n_t = len(tp)
    m_max = n_t if m_max is None else m_max
    out = {k: np.zeros((B, m_max), np.int32) for k in ("tokens", "parent", "depth", "src_row")}
    out["score"] = np.zeros((B, m_max), np.float64)
    out["num_nodes"] = np.zeros(B, np.int32)
    _check(lib().orc_build_tree_template(B, n_t, _p(tp), _p(tc), children, V, _p(a), dt, V, R, m_max,
                                         _p(out["tokens"]), _p(out["parent"]), _p(out["depth"]), _p(out["score"]),
                                         _p(out["src_row"]), _p(out["num_nodes"])), "build_tree_template")
    return out


def tree_frontiers(draft_logits, depth, topk, children, m, m_max=None, policy=0):
    """The nodes expanded at each depth of the dynamic trees, as an incremental
    build returns them level by level: level l's frontier is the expanded
    nodes of depth l + 1 in expansion order (they own rows 1 + l * topk + p).
    Returns tokens, parent (index in the previous frontier, -1 at level 0) and
    score (V), each [depth][B][topk], padded with -1 / -1 / 0; the last level
    is empty (depth `depth` is not expanded)."""
    t = build_tree(draft_logits, depth, topk, children, m, m_max=m_max, debug=True, policy=policy)
    cd = t["cand"]
    B = cd["n"].shape[0]
    tok = np.full((depth, B, topk), -1, np.int32)
    par = np.full((depth, B, topk), -1, np.int32)
    score = np.zeros((depth, B, topk), np.float64)
    for b in range(B):
        for g in range(int(cd["n"][b])):
            r = int(cd["row"][b, g])
            if r < 0:
                continue
            lv = int(cd["depth"][b, g]) - 1          # level whose call returns this node
            p = r - 1 - lv * topk
            tok[lv, b, p] = cd["token"][b, g]
            score[lv, b, p] = cd["V"][b, g]
            q = int(cd["parent"][b, g])
            par[lv, b, p] = -1 if q < 0 else int(cd["row"][b, q]) - 1 - (lv - 1) * topk
    return tok, par, score


def tree_mask(parent, num_nodes, prefix_len):
    parent = np.ascontiguousarray(parent, dtype=np.int32)
    num_nodes = np.ascontiguousarray(num_nodes, dtype=np.int32)
    prefix_len = np.ascontiguousarray(prefix_len, dtype=np.int32)
    B, M = parent.shape
    anc = np.zeros((B, M), np.uint64)
    pos = np.zeros((B, M), np.int32)
    _check(lib().orc_tree_mask(B, M, _p(parent), _p(num_nodes), _p(prefix_len), _p(anc), _p(pos)),
           "tree_mask")
    return anc, pos


class _AttnParams(C.Structure):
    _fields_ = [("num_q_heads", C.c_int), ("num_kv_heads", C.c_int), ("head_dim", C.c_int),
                ("m_max", C.c_int), ("block_size", C.c_int), ("max_blocks", C.c_int),
                ("max_prefix", C.c_int), ("dtype", C.c_int), ("scale", C.c_double)]


def _attn_common(q, k_draft, v_draft, k_cache, v_cache, block_table, prefix_len, anc, scale):
    arrs = [np.ascontiguousarray(x) for x in (q, k_draft, v_draft, k_cache, v_cache)]
    dt = 0 if arrs[0].dtype == np.float32 else 1
    for x in arrs:
        if (x.dtype == np.float32) != (dt == 0) or x.dtype not in (np.float32, np.uint16):
            raise TypeError("attention inputs must all be float32 or all uint16 (bf16 bits)")
    q_, kd, vd, kc, vc = arrs
    B, M, Hq, d = q_.shape
    Hkv = kd.shape[2]
    if block_table is None:
        bs, maxb, maxp = 0, 0, kc.shape[2]
        bt = None
    else:
        bt = np.ascontiguousarray(block_table, dtype=np.int32)
        bs, maxb, maxp = kc.shape[2], bt.shape[1], 0
    p = _AttnParams(Hq, Hkv, d, M, bs, maxb, maxp, dt, scale if scale is not None else 1.0 / np.sqrt(d))
    pl = np.ascontiguousarray(prefix_len, dtype=np.int32)
    an = np.ascontiguousarray(anc, dtype=np.uint64)
    return p, (q_, kd, vd, kc, vc, bt, pl, an)


def tree_attn(q, k_draft, v_draft, k_cache, v_cache, block_table, prefix_len, anc, num_nodes,
              scale=None):
    """All output rows in fp64: [B][m_max][Hq][d]; rows past num_nodes are zero."""
    p, (q_, kd, vd, kc, vc, bt, pl, an) = _attn_common(q, k_draft, v_draft, k_cache, v_cache,
                                                      block_table, prefix_len, anc, scale)
    nn = np.ascontiguousarray(num_nodes, dtype=np.int32)
    out = np.zeros(q_.shape, np.float64)
    _check(lib().orc_tree_attn(C.byref(p), q_.shape[0], _p(q_), _p(kd), _p(vd), _p(kc), _p(vc),
                               _p(bt), _p(pl), _p(an), _p(nn), _p(out)), "tree_attn")
    return out


def tree_attn_rows(q, k_draft, v_draft, k_cache, v_cache, block_table, prefix_len, anc, sel,
                   scale=None):
    """Selected rows: sel = list of (b, i, h); returns [n_sel][d] fp64."""
    p, (q_, kd, vd, kc, vc, bt, pl, an) = _attn_common(q, k_draft, v_draft, k_cache, v_cache,
                                                      block_table, prefix_len, anc, scale)
    sel = np.asarray(sel, dtype=np.int32).reshape(-1, 3)
    sb, si, sh = (np.ascontiguousarray(sel[:, j]) for j in range(3))
    out = np.zeros((len(sel), q_.shape[3]), np.float64)
    _check(lib().orc_tree_attn_rows(C.byref(p), _p(q_), _p(kd), _p(vd), _p(kc), _p(vc), _p(bt),
                                    _p(pl), _p(an), len(sel), _p(sb), _p(si), _p(sh), _p(out)),
           "tree_attn_rows")
    return out


def kv_commit(k_draft, v_draft, accepted, accept_len, prefix_len, k_cache, v_cache, block_table=None,
              max_prefix=0):
    """The accepted path's draft K/V written into copies of the caches.

    Layouts as in tree_attn (contiguous [B][Hkv][P][d] / [B][Hkv][d][P]; paged
    [pages][Hkv][bs][d] / [pages][Hkv][d][bs] with block_table [B][max_blocks]).
    Capacity: contiguous P; paged max_prefix if it is in (0, max_blocks * bs),
    else max_blocks * bs.  Returns (k_cache, v_cache, slot_mapping [B][m_max],
    prefix_len_out [B], (tree_flags, prefix_flags))."""
    kd, vd = np.ascontiguousarray(k_draft), np.ascontiguousarray(v_draft)
    kc, vc = np.array(k_cache, copy=True, order="C"), np.array(v_cache, copy=True, order="C")
    dt = 0 if kd.dtype == np.float32 else 1
    for x in (kd, vd, kc, vc):
        if (x.dtype == np.float32) != (dt == 0) or x.dtype not in (np.float32, np.uint16):
            raise TypeError("K/V inputs must all be float32 or all uint16 (bf16 bits)")
    B, M, Hkv, d = kd.shape
    acc = np.ascontiguousarray(accepted, dtype=np.int32)
    alen = np.ascontiguousarray(accept_len, dtype=np.int32)
    pl = np.ascontiguousarray(prefix_len, dtype=np.int32)
    if block_table is None:
        bt, bs, maxb, rows = None, 0, 0, kc.shape[2]
        cap = rows
    else:
        bt = np.ascontiguousarray(block_table, dtype=np.int32)
        bs, maxb, rows = kc.shape[2], bt.shape[1], 0
        cap = max_prefix if 0 < max_prefix < maxb * bs else maxb * bs
    p = _AttnParams(Hkv, Hkv, d, M, bs, maxb, rows, dt, 1.0)
    slot = np.zeros((B, M), np.int32)
    plo = np.zeros(B, np.int32)
    flags = np.zeros(2, np.int32)
    _check(lib().orc_kv_commit(C.byref(p), cap, B, _p(kd), _p(vd), _p(acc), _p(alen), acc.shape[1], _p(pl),
                               _p(kc), _p(vc), _p(bt), _p(slot), _p(plo), _p(flags)), "kv_commit")
    return kc, vc, slot, plo, (int(flags[0]), int(flags[1]))


def pdraft_prepare(tokens, num_nodes, accepted, accept_len, bonus, prefix_len, target_hidden, h_shared, K,
                   mask_id):
    """Inputs of the next parallel drafting pass (see oracle.c).  target_hidden
    [B][m_max+1][H] and h_shared [H] as float32 or uint16 (bf16 bits).  Returns
    a dict of input_ids, positions, hidden_src [B][S], is_mask [B][S],
    rejected [B][m_max], num_slots [B], draft_hidden [B][S][H], flags."""
    tok = np.ascontiguousarray(tokens, dtype=np.int32)
    B, M = tok.shape
    acc = np.ascontiguousarray(accepted, dtype=np.int32)
    MA = acc.shape[1]
    th = np.ascontiguousarray(target_hidden)
    hs = np.ascontiguousarray(h_shared)
    if th.dtype not in (np.float32, np.uint16) or hs.dtype != th.dtype:
        raise TypeError("hidden states must be float32 or uint16 (bf16 bits), both the same")
    H = th.shape[-1]
    S = MA + K
    out = dict(input_ids=np.zeros((B, S), np.int32), positions=np.zeros((B, S), np.int32),
               hidden_src=np.zeros((B, S), np.int32), is_mask=np.zeros((B, S), np.uint8),
               rejected=np.zeros((B, M), np.uint8), num_slots=np.zeros(B, np.int32),
               draft_hidden=np.zeros((B, S, H), th.dtype))
    flags = np.zeros(2, np.int32)
    arr = [np.ascontiguousarray(x, dtype=np.int32) for x in (num_nodes, accept_len, bonus, prefix_len)]
    _check(lib().orc_pdraft_prepare(B, M, MA, K, H, mask_id, th.itemsize, _p(tok), _p(arr[0]), _p(acc), _p(arr[1]),
                                    _p(arr[2]), _p(arr[3]), _p(th), _p(hs), _p(out["input_ids"]),
                                    _p(out["positions"]), _p(out["hidden_src"]), _p(out["is_mask"]),
                                    _p(out["rejected"]), _p(out["num_slots"]), _p(out["draft_hidden"]), _p(flags)),
           "pdraft_prepare")
    out["flags"] = (int(flags[0]), int(flags[1]))
    return out


def accept_rrs(target_logits, draft_logits, tokens, parent, src_row, num_nodes, max_accept, rand_words, T=1.0):
    """Recursive rejection sampling over drawn children (see oracle.c):
    target_logits [B][m_max+1][V], draft_logits [B][R_max][V] (same dtype),
    tree arrays [B][m_max], rand_words [B][m_max+1] uint32.
    -> (accepted [B][max_accept], accept_len [B], bonus [B])."""
    t, dt = _logits(target_logits)
    d, dd = _logits(draft_logits)
    if dd != dt:
        raise TypeError("target and draft logits must share a dtype")
    B, M1, V = t.shape
    arrs = [np.ascontiguousarray(x, dtype=np.int32) for x in (tokens, parent, src_row, num_nodes)]
    rw = np.ascontiguousarray(rand_words).view(np.uint32)
    acc = np.zeros((B, max_accept), np.int32)
    alen = np.zeros(B, np.int32)
    bon = np.zeros(B, np.int32)
    _check(lib().orc_accept_rrs(T, B, M1 - 1, max_accept, V, _p(t), _p(d), d.shape[1], dt, _p(arrs[0]),
                                _p(arrs[1]), _p(arrs[2]), _p(arrs[3]), _p(rw), _p(acc), _p(alen), _p(bon)),
           "accept_rrs")
    return acc, alen, bon


def accept(mode, target_logits, tokens, parent, num_nodes, max_accept, rand_words=None, T=1.0):
    """mode 0 greedy / 1 sample -> (accepted [B][max_accept], accept_len [B], bonus [B])."""
    a, dt = _logits(target_logits)
    B, M1, V = a.shape
    tokens = np.ascontiguousarray(tokens, dtype=np.int32)
    parent = np.ascontiguousarray(parent, dtype=np.int32)
    nn = np.ascontiguousarray(num_nodes, dtype=np.int32)
    rw = None if rand_words is None else np.ascontiguousarray(rand_words).view(np.uint32)
    acc = np.zeros((B, max_accept), np.int32)
    alen = np.zeros(B, np.int32)
    bon = np.zeros(B, np.int32)
    _check(lib().orc_accept(mode, T, B, M1 - 1, max_accept, V, _p(a), dt, V, _p(tokens), _p(parent),
                            _p(nn), _p(rw), _p(acc), _p(alen), _p(bon)), "accept")
    return acc, alen, bon
