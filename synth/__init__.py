"""Seeded synthetic inputs for one EAGLE-2 draft-tree verification step.

This module only draws random numbers and arranges them into the buffers the
step consumes.  It holds none of the method's arithmetic (no softmax, no tree
selection, no attention, no acceptance), so both the CPU oracle and the GPU
path can be fed from it without sharing any computation.

The pages measure with trained draft/target models on text benchmarks
(MT-bench, HumanEval, GSM8K, Alpaca, CNN/DM, Natural Questions, SPEED-Bench).
None of those models or datasets is used: random logits stand in for the
draft and target models, and the five workload shapes below stand in for the
model shapes (EAGLE-2 explainer, section "Implementation", tree depth 6,
expansion 10, m = 60/50/48 for 7B-8B/13B/70B; P-EAGLE in vLLM, section
"Speculative depth efficiency", K = 7 parallel-draft chains).

Layouts (all row-major):
  draft_logits   [B][R_max][V]           fp32 or bf16
  target_logits  [B][m_max + 1][V]       row 0 = root, row i + 1 = tree node i
  q              [B][m_max][Hq][d]
  k_draft/v_draft[B][m_max][Hkv][d]
  contiguous KV  k_cache [B][Hkv][L_max][d],  v_cache [B][Hkv][d][L_max]
  paged KV       k_cache [NB][Hkv][bs][d],    v_cache [NB][Hkv][d][bs]
  block_table    [B][max_blocks]  int32, -1 for unused entries
  rand_words     [B][m_max + 1]   uint32 (stored as int32 bit patterns)
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch

TREE_DYNAMIC = 0
TREE_CHAIN = 1
ACCEPT_GREEDY = 0
ACCEPT_SAMPLE = 1

# independent random streams per workload
_STREAMS = {
    "draft": 0, "target": 1, "q": 2, "kv": 3, "draft_kv": 4,
    "prefix": 5, "blocks": 6, "words": 7, "fresh": 8, "plant": 9,
}


@dataclasses.dataclass
class Workload:
    name: str
    batch: int
    vocab: int
    dtype: torch.dtype            # logits and attention dtype
    draft_sigma: float
    depth: int                    # D: draft levels 1..D
    topk: int                     # k: nodes expanded per depth
    children: int                 # C: children per expanded node
    m: int                        # nodes kept by the rerank (dynamic trees)
    chain_k: int                  # K: chain length for chain sequences (0: none)
    kinds: list                   # per-sequence TREE_DYNAMIC / TREE_CHAIN
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    prefix: object                # int, or (lo, hi) for uniform lengths
    block_size: int               # 0 => contiguous KV
    accept_mode: int
    temperature: float
    target_kind: str              # "iid" or "draft_plus_noise"
    target_sigma: float = 1.0     # noise sd (draft_plus_noise) or iid sd
    poison_tail: bool = False     # NaN in the cache slots past each prefix (last page tail, or contiguous tail)

    @property
    def rows_dynamic(self) -> int:
        return 1 + (self.depth - 1) * self.topk

    @property
    def r_max(self) -> int:
        r = 0
        for kd in self.kinds:
            r = max(r, self.rows_dynamic if kd == TREE_DYNAMIC else self.chain_k)
        return r

    @property
    def m_max(self) -> int:
        r = 0
        for kd in self.kinds:
            r = max(r, self.m if kd == TREE_DYNAMIC else self.chain_k)
        return r

    @property
    def max_accept(self) -> int:
        r = 0
        for kd in self.kinds:
            r = max(r, self.depth if kd == TREE_DYNAMIC else self.chain_k)
        return r

    def nodes(self, b: int) -> int:
        return self.m if self.kinds[b] == TREE_DYNAMIC else self.chain_k


def workload(n: int) -> Workload:
    """The five verification-step workloads, numbered 1..5."""
    if n == 1:
        return Workload("tiny-fp32-v1000-h8x64-L256-m60-greedy", 1, 1000, torch.float32, 2.0,
                        6, 10, 10, 60, 0, [TREE_DYNAMIC], 8, 8, 64, 256, 0,
                        ACCEPT_GREEDY, 1.0, "iid", 2.0)
    if n == 2:
        return Workload("llama2-7b-attn-b1-bf16-h32x128-L2048-v32000-m60-greedy", 1, 32000,
                        torch.bfloat16, 3.0, 6, 10, 10, 60, 0, [TREE_DYNAMIC], 32, 32, 128,
                        2048, 0, ACCEPT_GREEDY, 1.0, "draft_plus_noise")
    if n == 3:
        return Workload("13b-attn-b8-bf16-h40x128-L4096-v32000-m50-rs", 8, 32000,
                        torch.bfloat16, 3.0, 6, 10, 10, 50, 0, [TREE_DYNAMIC] * 8, 40, 40, 128,
                        4096, 0, ACCEPT_SAMPLE, 1.0, "draft_plus_noise")
    if n == 4:
        return Workload("70b-gqa64x8-b16-bf16-L8192-v32000-m48-rs", 16, 32000, torch.bfloat16,
                        3.0, 6, 10, 10, 48, 0, [TREE_DYNAMIC] * 16, 64, 8, 128, 8192, 0,
                        ACCEPT_SAMPLE, 1.0, "draft_plus_noise")
    if n == 5:
        kinds = [TREE_DYNAMIC if b % 2 == 0 else TREE_CHAIN for b in range(64)]
        return Workload("llama3-8b-gqa32x8-b64-paged16-L1k-32k-v128256-tree60+chain7-greedy", 64,
                        128256, torch.bfloat16, 3.0, 6, 10, 10, 60, 7, kinds, 32, 8, 128,
                        (1024, 32768), 16, ACCEPT_GREEDY, 1.0, "draft_plus_noise",
                        poison_tail=True)
    raise ValueError(f"no workload {n}")


def _gen(seed: int, stream: str, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed * 64 + _STREAMS[stream])
    return g


def _normal(shape, sigma, dtype, gen, device, chunk_elems=1 << 26):
    """N(0, sigma^2) drawn in fp32, rounded (RNE) to dtype; chunked to bound memory."""
    out = torch.empty(shape, dtype=dtype, device=device)
    flat = out.view(-1)
    n = flat.numel()
    for s in range(0, n, chunk_elems):
        e = min(n, s + chunk_elems)
        t = torch.randn(e - s, generator=gen, device=device, dtype=torch.float32)
        if sigma != 1.0:
            t.mul_(sigma)
        flat[s:e].copy_(t)
    return out


def draft_logits(w: Workload, seed: int, device="cpu") -> torch.Tensor:
    """[B][R_max][V] draft rows ~ N(0, draft_sigma^2); rows past a sequence's use are also filled."""
    g = _gen(seed, "draft", device)
    return _normal((w.batch, w.r_max, w.vocab), w.draft_sigma, w.dtype, g, device)


def target_logits(w: Workload, seed: int, draft: torch.Tensor, src_row: torch.Tensor,
                  num_nodes: torch.Tensor, device="cpu") -> torch.Tensor:
    """[B][m_max+1][V] target rows.

    "iid": every row ~ N(0, target_sigma^2) (random target argmax).
    "draft_plus_noise": the row of a node that owns a draft row (the root owns
    row 0; an expanded node owns src_row) is that draft row + N(0, 1); any
    other row is a fresh N(0, draft_sigma^2) row + N(0, 1).  src_row comes
    from the tree of the same draft rows and is only used as an index.
    """
    B, M1, V = w.batch, w.m_max + 1, w.vocab
    g = _gen(seed, "target", device)
    if w.target_kind == "iid":
        return _normal((B, M1, V), w.target_sigma, w.dtype, g, device)
    gf = _gen(seed, "fresh", device)
    out = torch.empty((B, M1, V), dtype=w.dtype, device=device)
    src_row = src_row.to("cpu")
    num_nodes = num_nodes.to("cpu")
    for b in range(B):
        for u in range(M1):
            noise = torch.randn(V, generator=g, device=device, dtype=torch.float32)
            if u == 0:
                r = 0
            elif u - 1 < int(num_nodes[b]):
                r = int(src_row[b, u - 1])
            else:
                r = -1
            if r >= 0:
                base = draft[b, r].to(torch.float32)
            else:
                base = torch.randn(V, generator=gf, device=device, dtype=torch.float32) * w.draft_sigma
            out[b, u].copy_(base + noise * w.target_sigma)
    return out


def plant_path(target: torch.Tensor, w: Workload, b: int, path_nodes, tokens, boost=20.0):
    """Add `boost` to the target logit of each planted node's token in its parent's row.

    path_nodes lists tree node indices root-first; the parent row of node
    path_nodes[0] is row 0, of path_nodes[j] it is row path_nodes[j-1] + 1.
    """
    prev_row = 0
    for nd in path_nodes:
        tok = int(tokens[b, nd])
        v = target[b, prev_row, tok].to(torch.float32) + boost
        target[b, prev_row, tok] = v.to(target.dtype)
        prev_row = nd + 1
    return target


def prefix_lengths(w: Workload, seed: int) -> torch.Tensor:
    if isinstance(w.prefix, int):
        return torch.full((w.batch,), w.prefix, dtype=torch.int32)
    lo, hi = w.prefix
    g = _gen(seed, "prefix", "cpu")
    return torch.randint(lo, hi + 1, (w.batch,), generator=g, dtype=torch.int64).to(torch.int32)


@dataclasses.dataclass
class AttnInputs:
    q: torch.Tensor
    k_draft: torch.Tensor
    v_draft: torch.Tensor
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    block_table: Optional[torch.Tensor]
    prefix_len: torch.Tensor
    block_size: int
    max_prefix: int


def attn_inputs(w: Workload, seed: int, device="cpu", prefix_seed: Optional[int] = None) -> AttnInputs:
    """Q, draft K/V and the KV prefix, all N(0,1) in the workload dtype.
    prefix_seed (default: seed) draws the prefix lengths and the block table."""
    B, M, Hq, Hkv, d = w.batch, w.m_max, w.num_q_heads, w.num_kv_heads, w.head_dim
    pseed = seed if prefix_seed is None else prefix_seed
    plen = prefix_lengths(w, pseed)
    q = _normal((B, M, Hq, d), 1.0, w.dtype, _gen(seed, "q", device), device)
    gdk = _gen(seed, "draft_kv", device)
    k_draft = _normal((B, M, Hkv, d), 1.0, w.dtype, gdk, device)
    v_draft = _normal((B, M, Hkv, d), 1.0, w.dtype, gdk, device)
    gkv = _gen(seed, "kv", device)
    if w.block_size == 0:
        # capacity = longest prefix rounded up to 8 keys (16-byte V^T rows in bf16)
        L = (int(plen.max()) + 7) // 8 * 8
        k_cache = _normal((B, Hkv, L, d), 1.0, w.dtype, gkv, device)
        v_cache = _normal((B, Hkv, d, L), 1.0, w.dtype, gkv, device)
        if w.poison_tail:
            for b in range(B):
                used = int(plen[b])
                k_cache[b, :, used:, :] = float("nan")
                v_cache[b, :, :, used:] = float("nan")
        return AttnInputs(q, k_draft, v_draft, k_cache, v_cache, None, plen.to(device), 0, L)
    bs = w.block_size
    nblk = [(int(x) + bs - 1) // bs for x in plen]
    total = sum(nblk)
    maxb = max(nblk)
    gperm = _gen(pseed, "blocks", "cpu")
    perm = torch.randperm(total, generator=gperm).to(torch.int32)
    table = torch.full((B, maxb), -1, dtype=torch.int32)
    o = 0
    for b in range(B):
        table[b, :nblk[b]] = perm[o:o + nblk[b]]
        o += nblk[b]
    k_cache = _normal((total, Hkv, bs, d), 1.0, w.dtype, gkv, device)
    v_cache = _normal((total, Hkv, d, bs), 1.0, w.dtype, gkv, device)
    if w.poison_tail:
        for b in range(B):
            used = int(plen[b]) - (nblk[b] - 1) * bs
            if used < bs:
                blk = int(table[b, nblk[b] - 1])
                k_cache[blk, :, used:, :] = float("nan")
                v_cache[blk, :, :, used:] = float("nan")
    return AttnInputs(q, k_draft, v_draft, k_cache, v_cache, table.to(device), plen.to(device),
                      bs, int(plen.max()))


def plant_draft_keys(attn: AttnInputs, w: Workload, seed: int, gamma: float = 1.5) -> AttnInputs:
    """A copy of `attn` in which the draft keys carry most of every query's
    attention mass, so that which draft keys a query sees changes its output
    by O(1) even over a prefix of 32k keys.

    Per (sequence b, kv head) one direction u is drawn, N(0, 1)^d rescaled to
    |u|^2 = d; every query head of that kv head becomes u + q / 2 and every
    draft key of it gamma * u + k_draft / 2.  At scale 1/sqrt(d) a query then
    scores a draft key near gamma * sqrt(d) (about 17 at d = 128) with a
    spread near 1, and a prefix key N(0, 1.25): the draft keys on a query's
    path hold most of its softmax mass, and the prefix keeps a small share.
    Values are combined in fp32 and rounded (RNE) to the workload dtype.
    """
    B, Hkv, d = w.batch, w.num_kv_heads, w.head_dim
    G = w.num_q_heads // Hkv
    dev = attn.q.device
    g = _gen(seed, "plant", "cpu")
    u = torch.randn((B, Hkv, d), generator=g, dtype=torch.float32)
    u = (u * (math.sqrt(d) / u.norm(dim=-1, keepdim=True))).to(dev)
    uq = u.repeat_interleave(G, dim=1)                               # [B][Hq][d]
    q = (0.5 * attn.q.to(torch.float32) + uq[:, None]).to(w.dtype)
    kd = (0.5 * attn.k_draft.to(torch.float32) + gamma * u[:, None]).to(w.dtype)
    return dataclasses.replace(attn, q=q, k_draft=kd)


def rising_prefix_keys(attn: AttnInputs, w: Workload, seed: int, top: float = 6.0) -> AttnInputs:
    """A copy of `attn` whose prefix scores rise along the prefix, so that an
    online softmax meets a new maximum again and again, also between the two
    halves of one 64-key tile.

    Per (sequence b, kv head) one direction u is drawn, N(0, 1)^d rescaled to
    |u|^2 = d; every query head of that kv head becomes u + q / 2 and the
    prefix key at position p (of L_b) becomes top * (p / L_b) * u + k / 2.  At
    scale 1/sqrt(d) a query then scores key p near top * sqrt(d) * p / L_b (up
    to about 68 at d = 128): the scores climb by tens of natural-log units
    over the prefix.  Values are combined in fp32 and rounded (RNE) to the
    workload dtype; positions past L_b keep whatever they held.
    """
    B, Hkv, d = w.batch, w.num_kv_heads, w.head_dim
    G = w.num_q_heads // Hkv
    dev = attn.q.device
    g = _gen(seed, "plant", "cpu")
    u = torch.randn((B, Hkv, d), generator=g, dtype=torch.float32)
    u = (u * (math.sqrt(d) / u.norm(dim=-1, keepdim=True))).to(dev)
    uq = u.repeat_interleave(G, dim=1)                               # [B][Hq][d]
    q = (0.5 * attn.q.to(torch.float32) + uq[:, None]).to(w.dtype)
    kc = attn.k_cache.clone()
    plen = attn.prefix_len.cpu().tolist()
    for b in range(B):
        L = int(plen[b])
        if L <= 0:
            continue
        coef = (top * torch.arange(L, dtype=torch.float32, device=dev) / L)     # [L]
        add = coef[None, :, None] * u[b][:, None, :]                          # [Hkv][L][d]
        if attn.block_size == 0:
            kc[b, :, :L] = (0.5 * kc[b, :, :L].to(torch.float32) + add).to(w.dtype)
        else:
            bs = attn.block_size
            for i in range((L + bs - 1) // bs):
                blk = int(attn.block_table[b, i])
                n = min(bs, L - i * bs)
                kc[blk, :, :n] = (0.5 * kc[blk, :, :n].to(torch.float32) + add[:, i * bs:i * bs + n]).to(w.dtype)
    return dataclasses.replace(attn, q=q, k_cache=kc)


def rand_words(w: Workload, seed: int, device="cpu") -> torch.Tensor:
    """[B][m_max+1] uniform 32-bit words, held as int32 bit patterns."""
    g = _gen(seed, "words", "cpu")
    x = torch.randint(0, 1 << 32, (w.batch, w.m_max + 1), generator=g, dtype=torch.int64)
    return _u32_as_i32(x).to(device)


def _u32_as_i32(x: torch.Tensor) -> torch.Tensor:
    x = x.clone()
    x[x >= (1 << 31)] -= (1 << 32)
    return x.to(torch.int32)


def kinds_tensor(w: Workload, device="cpu") -> torch.Tensor:
    return torch.tensor(w.kinds, dtype=torch.int32, device=device)


def small_workload(base: int = 2, **over) -> Workload:
    """A reduced copy of a workload (for CPU tests and fast parity cases)."""
    w = dataclasses.replace(workload(base))
    for k, v in over.items():
        setattr(w, k, v)
    if "kinds" not in over and len(w.kinds) != w.batch:
        w.kinds = [w.kinds[b % len(w.kinds)] for b in range(w.batch)]
    return w


def step_dims(w: Workload, attn: AttnInputs) -> dict:
    """Plain dimensions of one step for this workload and its attention inputs."""
    return dict(
        batch=w.batch, vocab=w.vocab, depth=w.depth, topk=w.topk, children=w.children, m=w.m,
        chain_k=w.chain_k, m_max=w.m_max, r_max=w.r_max, max_accept=w.max_accept,
        num_q_heads=w.num_q_heads, num_kv_heads=w.num_kv_heads, head_dim=w.head_dim,
        block_size=attn.block_size,
        max_blocks=0 if attn.block_table is None else int(attn.block_table.shape[1]),
        max_prefix=attn.max_prefix if attn.block_table is None else 0,
        dtype=w.dtype, accept_mode=w.accept_mode, temperature=w.temperature)
