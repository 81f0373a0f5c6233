"""Python binding of libeagle.so: one EAGLE-2 draft-tree verification step on
an MI355X (gfx950).

The functions here carry the names of the C entry points declared in
``include/eagle.h`` and only marshal arguments: torch tensors become device
pointers, the current torch stream becomes the HIP stream, and a non-OK
status becomes an ``EagleError``.  Every step of the computation runs in the
HIP kernels of libeagle.so; there is no fallback.  ``VerifyStep`` allocates
the outputs and workspaces of one step for fixed shapes and runs its calls
in order on one stream.
"""
from __future__ import annotations

import ctypes as C
import dataclasses
import math
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# EAGLE_LIB may name another build of the same sources (the host-sanitizer
# build of tests/sanitize.py)
LIB_PATH = os.environ.get("EAGLE_LIB") or os.path.join(_HERE, "libeagle.so")

EAGLE_OK, EAGLE_ERR_INVALID, EAGLE_ERR_UNSUPPORTED, EAGLE_ERR_WORKSPACE, EAGLE_ERR_HIP = 0, -1, -2, -3, -4
EAGLE_F32, EAGLE_BF16 = 0, 1
EAGLE_TREE_DYNAMIC, EAGLE_TREE_CHAIN = 0, 1
EAGLE_ACCEPT_GREEDY, EAGLE_ACCEPT_SAMPLE = 0, 1
EAGLE_POLICY_EAGLE2, EAGLE_POLICY_NO_RERANK, EAGLE_POLICY_CONF, EAGLE_POLICY_CONF_NO_RERANK = 0, 1, 2, 3
DEVERR_NONFINITE_ROW, DEVERR_CLOSURE, DEVERR_PREFIX, DEVERR_PATH, DEVERR_TREE = 0x1, 0x2, 0x4, 0x8, 0x10

# every function exported by libeagle.so (the declarations of include/eagle.h)
EXPORTS = (
    "eagle_workspace_init", "eagle_read_errors",
    "eagle_build_tree_workspace_size", "eagle_build_tree",
    "eagle_build_tree_mask", "eagle_build_tree_mask_noalloc", "eagle_build_tree_sampled", "eagle_build_tree_template", "eagle_tree_expand", "eagle_tree_finish",
    "eagle_tree_mask",
    "eagle_tree_attn_workspace_size", "eagle_tree_attn",
    "eagle_kv_commit",
    "eagle_accept_workspace_size", "eagle_accept",
    "eagle_pdraft_prepare", "eagle_accept_rrs_workspace_size", "eagle_accept_rrs",
    "eagle_status_string", "eagle_last_error",
)


class EagleError(RuntimeError):
    def __init__(self, status: int, what: str, detail: str):
        super().__init__(f"{what}: status {status} ({detail})")
        self.status = status


class TreeParams(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("depth", "topk", "children", "m", "chain_k", "vocab", "m_max", "r_max",
                                         "policy")]


class AttnParams(C.Structure):
    _fields_ = [("num_q_heads", C.c_int32), ("num_kv_heads", C.c_int32), ("head_dim", C.c_int32),
                ("m_max", C.c_int32), ("block_size", C.c_int32), ("max_blocks", C.c_int32),
                ("max_prefix", C.c_int32), ("scale", C.c_float), ("dtype", C.c_int)]


class PdraftParams(C.Structure):
    _fields_ = [("m_max", C.c_int32), ("max_accept", C.c_int32), ("k_draft", C.c_int32), ("hidden", C.c_int32),
                ("mask_token_id", C.c_int32), ("dtype", C.c_int)]


class AcceptParams(C.Structure):
    _fields_ = [("mode", C.c_int), ("temperature", C.c_float), ("m_max", C.c_int32),
                ("vocab", C.c_int32), ("max_accept", C.c_int32)]


_lib = None


def lib() -> C.CDLL:
    """Loads libeagle.so (built in-tree); raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m eagle_tree_verification_draft_amd.build`")
        L = C.CDLL(LIB_PATH)
        vp, i32, i64, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
        L.eagle_workspace_init.argtypes = [vp, sz, vp]
        L.eagle_read_errors.argtypes = [vp, vp, C.POINTER(C.c_uint32)]
        L.eagle_build_tree_workspace_size.argtypes = [C.POINTER(TreeParams), i32]
        L.eagle_build_tree_workspace_size.restype = sz
        L.eagle_build_tree.argtypes = [C.POINTER(TreeParams), i32, vp, C.c_int, i64, vp, vp, vp, vp, vp, vp, vp,
                                       vp, sz, vp]
        L.eagle_build_tree_mask.argtypes = [C.POINTER(TreeParams), i32, vp, C.c_int, i64, vp, vp, vp, vp, vp, vp,
                                            vp, vp, vp, vp, vp, sz, vp]
        L.eagle_build_tree_mask_noalloc.argtypes = [C.POINTER(TreeParams), i32, vp, C.c_int, i64] + [vp] * 11 + [vp]
        L.eagle_build_tree_sampled.argtypes = [C.POINTER(TreeParams), i32, vp, C.c_int, i64] + [vp] * 8 + [sz, vp]
        L.eagle_build_tree_template.argtypes = [C.POINTER(TreeParams), i32, vp, C.c_int, i64, i32] + [vp] * 9 + [sz, vp]
        L.eagle_tree_expand.argtypes = [C.POINTER(TreeParams), i32, i32, vp, C.c_int, i64, vp, vp, vp, vp, sz, vp]
        L.eagle_tree_finish.argtypes = [C.POINTER(TreeParams), i32, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.eagle_tree_mask.argtypes = [i32, i32, vp, vp, vp, vp, vp, vp, sz, vp]
        L.eagle_tree_attn_workspace_size.argtypes = [C.POINTER(AttnParams), i32]
        L.eagle_tree_attn_workspace_size.restype = sz
        L.eagle_tree_attn.argtypes = [C.POINTER(AttnParams), i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.eagle_kv_commit.argtypes = [C.POINTER(AttnParams), i32, vp, vp, vp, vp, i32, vp, vp, vp, vp, vp, vp,
                                      vp, sz, vp]
        L.eagle_accept_workspace_size.argtypes = [C.POINTER(AcceptParams), i32]
        L.eagle_accept_workspace_size.restype = sz
        L.eagle_accept.argtypes = [C.POINTER(AcceptParams), i32, vp, C.c_int, i64, vp, vp, vp, vp, vp, vp, vp, vp,
                                   sz, vp]
        L.eagle_accept_rrs_workspace_size.argtypes = [C.POINTER(AcceptParams), i32]
        L.eagle_accept_rrs_workspace_size.restype = sz
        L.eagle_accept_rrs.argtypes = [C.POINTER(AcceptParams), i32, vp, vp, C.c_int, i64, i64, i32] + [vp] * 9 + [sz, vp]
        L.eagle_pdraft_prepare.argtypes = [C.POINTER(PdraftParams), i32] + [vp] * 16 + [sz, vp]
        L.eagle_status_string.argtypes = [C.c_int]
        L.eagle_status_string.restype = C.c_char_p
        L.eagle_last_error.argtypes = []
        L.eagle_last_error.restype = C.c_char_p
        for f in ("eagle_workspace_init", "eagle_read_errors", "eagle_build_tree", "eagle_build_tree_mask",
                  "eagle_build_tree_mask_noalloc",
                  "eagle_build_tree_sampled", "eagle_build_tree_template", "eagle_tree_expand", "eagle_tree_finish",
                  "eagle_tree_mask", "eagle_tree_attn", "eagle_kv_commit", "eagle_accept", "eagle_accept_rrs",
                  "eagle_pdraft_prepare"):
            getattr(L, f).restype = C.c_int
        _lib = L
    return _lib


def _check(status: int, what: str):
    if status != EAGLE_OK:
        raise EagleError(status, what, lib().eagle_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libeagle must be contiguous")
    return C.c_void_p(t.data_ptr())


def _rows(t: torch.Tensor):
    """(pointer, row stride in elements) of a [..., V] logit tensor whose rows are
    contiguous and evenly spaced, e.g. the [..., :V] slice of a wider buffer."""
    if t.dim() < 2 or t.stride(-1) != 1:
        raise ValueError("logit rows passed to libeagle must be contiguous")
    lead = [d for d in range(t.dim() - 1) if t.shape[d] > 1]
    rs = t.stride(lead[-1]) if lead else t.shape[-1]
    if rs < t.shape[-1]:
        raise ValueError("logit row stride is shorter than a row")
    for d in lead:
        if t.stride(d) != rs * math.prod(t.shape[d + 1:-1]):
            raise ValueError("logit rows passed to libeagle must be evenly spaced")
    return C.c_void_p(t.data_ptr()), rs


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


def dtype_code(dt: torch.dtype) -> int:
    if dt == torch.float32:
        return EAGLE_F32
    if dt == torch.bfloat16:
        return EAGLE_BF16
    raise TypeError(f"unsupported dtype {dt}")


# ---------------------------------------------------------------------------
# the C entry points
# ---------------------------------------------------------------------------
def workspace_init(ws: torch.Tensor, stream=None):
    _check(lib().eagle_workspace_init(_ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "eagle_workspace_init")


def read_errors(ws: torch.Tensor, stream=None) -> int:
    bits = C.c_uint32(0)
    _check(lib().eagle_read_errors(_ptr(ws), _stream(stream), C.byref(bits)), "eagle_read_errors")
    return bits.value


def build_tree_workspace_size(p: TreeParams, batch: int) -> int:
    return lib().eagle_build_tree_workspace_size(C.byref(p), batch)


def build_tree(p: TreeParams, batch: int, draft_logits: torch.Tensor, kind: Optional[torch.Tensor],
               tokens, parent, depth, score, src_row, num_nodes, workspace: torch.Tensor, stream=None):
    rows, stride = _rows(draft_logits)
    _check(lib().eagle_build_tree(C.byref(p), batch, rows, dtype_code(draft_logits.dtype),
                                  stride, _ptr(kind), _ptr(tokens), _ptr(parent), _ptr(depth),
                                  _ptr(score), _ptr(src_row), _ptr(num_nodes), _ptr(workspace),
                                  workspace.numel() * workspace.element_size(), _stream(stream)),
           "eagle_build_tree")


def build_tree_mask(p: TreeParams, batch: int, draft_logits: torch.Tensor, kind: Optional[torch.Tensor], prefix_len,
                    tokens, parent, depth, score, src_row, num_nodes, anc_mask, pos, workspace: torch.Tensor,
                    stream=None):
    rows, stride = _rows(draft_logits)
    _check(lib().eagle_build_tree_mask(C.byref(p), batch, rows, dtype_code(draft_logits.dtype), stride, _ptr(kind),
                                       _ptr(prefix_len), _ptr(tokens), _ptr(parent), _ptr(depth), _ptr(score),
                                       _ptr(src_row), _ptr(num_nodes), _ptr(anc_mask), _ptr(pos), _ptr(workspace),
                                       workspace.numel() * workspace.element_size(), _stream(stream)),
           "eagle_build_tree_mask")


def build_tree_mask_noalloc(p: TreeParams, batch: int, draft_logits: torch.Tensor, kind: Optional[torch.Tensor],
                            prefix_len, tokens, parent, depth, score, src_row, num_nodes, anc_mask, pos,
                            device_errors: Optional[torch.Tensor] = None, stream=None):
    """eagle_build_tree_mask on the library's static scratch (no workspace);
    device_errors: optional int32 device tensor of one element."""
    rows, stride = _rows(draft_logits)
    _check(lib().eagle_build_tree_mask_noalloc(C.byref(p), batch, rows, dtype_code(draft_logits.dtype), stride,
                                               _ptr(kind), _ptr(prefix_len), _ptr(tokens), _ptr(parent), _ptr(depth),
                                               _ptr(score), _ptr(src_row), _ptr(num_nodes), _ptr(anc_mask), _ptr(pos),
                                               _ptr(device_errors), _stream(stream)),
           "eagle_build_tree_mask_noalloc")


def build_tree_sampled(p: TreeParams, batch: int, draft_logits: torch.Tensor, child_words, tokens, parent, depth,
                       score, src_row, num_nodes, workspace: torch.Tensor, stream=None):
    """Children drawn from the draft rows; child_words [batch][r_max][children] (int32 bit patterns)."""
    rows, stride = _rows(draft_logits)
    _check(lib().eagle_build_tree_sampled(C.byref(p), batch, rows, dtype_code(draft_logits.dtype), stride,
                                          _ptr(child_words), _ptr(tokens), _ptr(parent), _ptr(depth), _ptr(score),
                                          _ptr(src_row), _ptr(num_nodes), _ptr(workspace),
                                          workspace.numel() * workspace.element_size(), _stream(stream)),
           "eagle_build_tree_sampled")


def build_tree_template(p: TreeParams, batch: int, draft_logits: torch.Tensor, tmpl_parent, tmpl_child, tokens,
                        parent, depth, score, src_row, num_nodes, workspace: torch.Tensor, stream=None):
    """EAGLE-1 static tree from a template (device int32 arrays)."""
    rows, stride = _rows(draft_logits)
    _check(lib().eagle_build_tree_template(C.byref(p), batch, rows, dtype_code(draft_logits.dtype), stride,
                                           tmpl_parent.numel(), _ptr(tmpl_parent), _ptr(tmpl_child), _ptr(tokens),
                                           _ptr(parent), _ptr(depth), _ptr(score), _ptr(src_row), _ptr(num_nodes),
                                           _ptr(workspace), workspace.numel() * workspace.element_size(),
                                           _stream(stream)),
           "eagle_build_tree_template")


def tree_expand(p: TreeParams, batch: int, level: int, level_logits: torch.Tensor, frontier_tokens,
                frontier_parent, frontier_score, workspace: torch.Tensor, stream=None):
    """One level of draft rows ([batch][1 or topk][V]); writes the next frontier."""
    rows, stride = _rows(level_logits)
    _check(lib().eagle_tree_expand(C.byref(p), batch, level, rows, dtype_code(level_logits.dtype), stride,
                                   _ptr(frontier_tokens), _ptr(frontier_parent), _ptr(frontier_score),
                                   _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)),
           "eagle_tree_expand")


def tree_finish(p: TreeParams, batch: int, tokens, parent, depth, score, src_row, num_nodes,
                workspace: torch.Tensor, stream=None):
    _check(lib().eagle_tree_finish(C.byref(p), batch, _ptr(tokens), _ptr(parent), _ptr(depth), _ptr(score),
                                   _ptr(src_row), _ptr(num_nodes), _ptr(workspace),
                                   workspace.numel() * workspace.element_size(), _stream(stream)),
           "eagle_tree_finish")


def tree_mask(batch: int, m_max: int, parent, num_nodes, prefix_len, anc_mask, pos,
              workspace: Optional[torch.Tensor] = None, stream=None):
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().eagle_tree_mask(batch, m_max, _ptr(parent), _ptr(num_nodes), _ptr(prefix_len), _ptr(anc_mask),
                                 _ptr(pos), _ptr(workspace), nbytes, _stream(stream)),
           "eagle_tree_mask")


def tree_attn_workspace_size(a: AttnParams, batch: int) -> int:
    return lib().eagle_tree_attn_workspace_size(C.byref(a), batch)


def tree_attn(a: AttnParams, batch: int, q, k_draft, v_draft, k_cache, v_cache, block_table, prefix_len,
              anc_mask, num_nodes, out, workspace: torch.Tensor, stream=None):
    _check(lib().eagle_tree_attn(C.byref(a), batch, _ptr(q), _ptr(k_draft), _ptr(v_draft), _ptr(k_cache),
                                 _ptr(v_cache), _ptr(block_table), _ptr(prefix_len), _ptr(anc_mask),
                                 _ptr(num_nodes), _ptr(out), _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), _stream(stream)),
           "eagle_tree_attn")


def kv_commit(a: AttnParams, batch: int, k_draft, v_draft, accepted, accept_len, prefix_len, k_cache, v_cache,
              block_table, slot_mapping, prefix_len_out, workspace: torch.Tensor, stream=None):
    """accepted is [batch][max_accept]; prefix_len_out may be prefix_len itself."""
    _check(lib().eagle_kv_commit(C.byref(a), batch, _ptr(k_draft), _ptr(v_draft), _ptr(accepted),
                                 _ptr(accept_len), accepted.shape[-1], _ptr(prefix_len), _ptr(k_cache),
                                 _ptr(v_cache), _ptr(block_table), _ptr(slot_mapping), _ptr(prefix_len_out),
                                 _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)),
           "eagle_kv_commit")


def accept_workspace_size(a: AcceptParams, batch: int) -> int:
    return lib().eagle_accept_workspace_size(C.byref(a), batch)


def accept(a: AcceptParams, batch: int, target_logits: torch.Tensor, tokens, parent, num_nodes,
           rand_words: Optional[torch.Tensor], accepted, accept_len, bonus_token, workspace: torch.Tensor,
           stream=None):
    rows, stride = _rows(target_logits)
    _check(lib().eagle_accept(C.byref(a), batch, rows, dtype_code(target_logits.dtype),
                              stride, _ptr(tokens), _ptr(parent), _ptr(num_nodes),
                              _ptr(rand_words), _ptr(accepted), _ptr(accept_len), _ptr(bonus_token),
                              _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)),
           "eagle_accept")


def accept_rrs_workspace_size(a: AcceptParams, batch: int) -> int:
    return lib().eagle_accept_rrs_workspace_size(C.byref(a), batch)


def accept_rrs(a: AcceptParams, batch: int, target_logits: torch.Tensor, draft_logits: torch.Tensor, tokens, parent,
               src_row, num_nodes, rand_words, accepted, accept_len, bonus_token, workspace: torch.Tensor, stream=None):
    trows, tstride = _rows(target_logits)
    drows, dstride = _rows(draft_logits)
    if draft_logits.dtype != target_logits.dtype:
        raise TypeError("target and draft logits must share a dtype")
    _check(lib().eagle_accept_rrs(C.byref(a), batch, trows, drows, dtype_code(target_logits.dtype), tstride, dstride,
                                  draft_logits.shape[-2], _ptr(tokens), _ptr(parent), _ptr(src_row), _ptr(num_nodes),
                                  _ptr(rand_words), _ptr(accepted), _ptr(accept_len), _ptr(bonus_token),
                                  _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)),
           "eagle_accept_rrs")


def pdraft_prepare(p: PdraftParams, batch: int, tokens, num_nodes, accepted, accept_len, bonus_token, prefix_len,
                   target_hidden, h_shared, input_ids, positions, hidden_src, is_mask, rejected, num_slots,
                   draft_hidden, workspace: torch.Tensor, stream=None):
    _check(lib().eagle_pdraft_prepare(C.byref(p), batch, _ptr(tokens), _ptr(num_nodes), _ptr(accepted),
                                      _ptr(accept_len), _ptr(bonus_token), _ptr(prefix_len), _ptr(target_hidden),
                                      _ptr(h_shared), _ptr(input_ids), _ptr(positions), _ptr(hidden_src),
                                      _ptr(is_mask), _ptr(rejected), _ptr(num_slots), _ptr(draft_hidden),
                                      _ptr(workspace), workspace.numel() * workspace.element_size(),
                                      _stream(stream)),
           "eagle_pdraft_prepare")


# ---------------------------------------------------------------------------
# one verification step with preallocated buffers
# ---------------------------------------------------------------------------
def _workspace(nbytes: int, device) -> torch.Tensor:
    # torch's caching allocator returns 256-byte-aligned blocks
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
    workspace_init(ws)
    return ws


@dataclasses.dataclass
class StepShape:
    batch: int
    vocab: int
    depth: int
    topk: int
    children: int
    m: int
    chain_k: int
    m_max: int
    r_max: int
    max_accept: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    max_blocks: int
    max_prefix: int
    dtype: torch.dtype
    accept_mode: int
    temperature: float


class VerifyStep:
    """Outputs and workspaces of one step; run() enqueues the fused build and
    mask, the attention and the acceptance; commit() the KV commit."""

    def __init__(self, s: StepShape, device="cuda"):
        self.s = s
        dev = torch.device(device)
        B, M = s.batch, s.m_max
        self.tree = TreeParams(s.depth, s.topk, s.children, s.m, s.chain_k, s.vocab, s.m_max, s.r_max)
        self.attn = AttnParams(s.num_q_heads, s.num_kv_heads, s.head_dim, s.m_max, s.block_size, s.max_blocks,
                               s.max_prefix, 0.0, dtype_code(s.dtype))
        self.acc = AcceptParams(s.accept_mode, s.temperature, s.m_max, s.vocab, s.max_accept)
        i32 = dict(dtype=torch.int32, device=dev)
        self.tokens = torch.empty((B, M), **i32)
        self.parent = torch.empty((B, M), **i32)
        self.depth = torch.empty((B, M), **i32)
        self.score = torch.empty((B, M), dtype=torch.float64, device=dev)
        self.src_row = torch.empty((B, M), **i32)
        self.num_nodes = torch.empty((B,), **i32)
        self.anc = torch.empty((B, M), dtype=torch.int64, device=dev)
        self.pos = torch.empty((B, M), **i32)
        self.out = torch.empty((B, M, s.num_q_heads, s.head_dim), dtype=s.dtype, device=dev)
        self.accepted = torch.empty((B, s.max_accept), **i32)
        self.accept_len = torch.empty((B,), **i32)
        self.bonus = torch.empty((B,), **i32)
        self.slot_mapping = torch.empty((B, M), **i32)
        self.ws_tree = _workspace(build_tree_workspace_size(self.tree, B), dev)
        self.ws_mask = _workspace(256, dev)
        self.ws_attn = _workspace(tree_attn_workspace_size(self.attn, B), dev)
        self.ws_acc = _workspace(accept_workspace_size(self.acc, B), dev)
        self.ws_commit = _workspace(256, dev)

    def build(self, draft_logits, kind=None, stream=None):
        build_tree(self.tree, self.s.batch, draft_logits, kind, self.tokens, self.parent, self.depth, self.score,
                   self.src_row, self.num_nodes, self.ws_tree, stream)

    def build_mask(self, draft_logits, kind, prefix_len, stream=None):
        """build() and mask() in one call (one launch fewer)."""
        build_tree_mask(self.tree, self.s.batch, draft_logits, kind, prefix_len, self.tokens, self.parent, self.depth,
                        self.score, self.src_row, self.num_nodes, self.anc, self.pos, self.ws_tree, stream)

    def mask(self, prefix_len, stream=None):
        tree_mask(self.s.batch, self.s.m_max, self.parent, self.num_nodes, prefix_len, self.anc, self.pos,
                  self.ws_mask, stream)

    def attention(self, q, k_draft, v_draft, k_cache, v_cache, block_table, prefix_len, stream=None):
        tree_attn(self.attn, self.s.batch, q, k_draft, v_draft, k_cache, v_cache, block_table, prefix_len,
                  self.anc, self.num_nodes, self.out, self.ws_attn, stream)

    def accept(self, target_logits, rand_words=None, stream=None):
        accept(self.acc, self.s.batch, target_logits, self.tokens, self.parent, self.num_nodes, rand_words,
               self.accepted, self.accept_len, self.bonus, self.ws_acc, stream)

    def commit(self, k_draft, v_draft, prefix_len, k_cache, v_cache, block_table, prefix_len_out=None,
               stream=None):
        """Writes the accepted path's draft K/V into the cache; prefix_len_out
        defaults to prefix_len itself (advanced in place)."""
        kv_commit(self.attn, self.s.batch, k_draft, v_draft, self.accepted, self.accept_len, prefix_len, k_cache,
                  v_cache, block_table, self.slot_mapping,
                  prefix_len if prefix_len_out is None else prefix_len_out, self.ws_commit, stream)

    def run(self, draft_logits, kind, prefix_len, q, k_draft, v_draft, k_cache, v_cache, block_table,
            target_logits, rand_words=None, stream=None):
        self.build_mask(draft_logits, kind, prefix_len, stream)
        self.attention(q, k_draft, v_draft, k_cache, v_cache, block_table, prefix_len, stream)
        self.accept(target_logits, rand_words, stream)

    def errors(self) -> int:
        bits = 0
        for ws in (self.ws_tree, self.ws_mask, self.ws_attn, self.ws_acc, self.ws_commit):
            bits |= read_errors(ws)
        return bits
