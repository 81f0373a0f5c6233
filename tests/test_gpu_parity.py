"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.  Trees, masks and accepts must be bit-exact; attention
within max-abs 2e-2 (bf16 inputs, fp32 accumulation) or 1e-5 (fp32)."""
import dataclasses

import numpy as np
import pytest
import torch

import eagle_tree_verification_draft_amd as E
import oracle
import synth
from conftest import to_np
from gpu_harness import (BF16_TOL, F32_TOL, assert_accept_equal, assert_tree_equal, check_attn_rows,
                         make_case, oracle_mask, run_gpu, sample_rows, say)

pytestmark = pytest.mark.gpu


REL_L2_TOL = 1e-2   # relative L2 over the checked rows (bf16 inputs, fp32 accumulation)


def _tol(w):
    return F32_TOL if w.dtype == torch.float32 else BF16_TOL


# ---------------------------------------------------------------------------
# the five workloads at full size
# ---------------------------------------------------------------------------
@pytest.fixture(scope="module", params=[1, 2, 3, 4, 5])
def full_case(request):
    n = request.param
    say(f"[full workload {n}] generating inputs")
    w = synth.workload(n)
    c = make_case(w, seed=100 + n)
    say(f"[full workload {n}] running the step on the GPU")
    run_gpu(c)
    yield c
    del c
    torch.cuda.empty_cache()


def test_full_tree(full_case):
    assert_tree_equal(full_case)


def test_full_mask(full_case):
    c = full_case
    anc, pos = oracle_mask(c)
    assert np.array_equal(c.step.anc.cpu().numpy().view(np.uint64), anc)
    assert np.array_equal(c.step.pos.cpu().numpy(), pos)


def test_full_attention(full_case):
    c = full_case
    rng = np.random.default_rng(c.seed)
    nn = c.otree["num_nodes"]
    if int(nn.sum()) * c.w.num_q_heads <= 4096:      # every row
        sel = [(b, i, h) for b in range(c.w.batch) for i in range(int(nn[b])) for h in range(c.w.num_q_heads)]
    else:
        sel = sample_rows(c, 192, rng)
    # every node of sequence 0 for two heads, so every depth and branch is covered
    for i in range(int(c.otree["num_nodes"][0])):
        sel.append((0, i, 0))
        sel.append((0, i, c.w.num_q_heads - 1))
    err, rl2 = check_attn_rows(c, sel, _tol(c.w))
    assert rl2 <= REL_L2_TOL, f"relative L2 error {rl2}"
    say(f"[{c.w.name}] attention max-abs error {err:.3g}, relative L2 {rl2:.3g} over {len(sel)} rows")
    # padding rows are zeros
    nn = c.otree["num_nodes"]
    out = c.step.out.to(torch.float32).cpu().numpy()
    for b in range(c.w.batch):
        assert (out[b, int(nn[b]):] == 0).all()


def test_full_attention_planted(full_case):
    """The full-shape call (same prefix lengths, heads, paging and key
    splits) on planted inputs whose draft keys carry most of the softmax
    mass, so a mistake in the draft tile or the ancestor mask moves the
    output by O(1); every checked row must be within the tolerance and
    within a tenth of its own draft-key gap."""
    c = full_case
    pa = synth.plant_draft_keys(c.attn, c.w, c.seed)
    c.step.attention(pa.q, pa.k_draft, pa.v_draft, pa.k_cache, pa.v_cache, pa.block_table, pa.prefix_len)
    torch.cuda.synchronize()
    rng = np.random.default_rng(c.seed + 1)
    nn = c.otree["num_nodes"]
    sel = sample_rows(c, 128, rng)
    # every node of the first sequence, the first chain and the longest
    # sequence (the most key splits), first and last q head
    plen = c.attn.prefix_len.cpu().numpy()
    seqs = {0, int(np.argmax(plen))}
    if c.w.chain_k and synth.TREE_CHAIN in c.w.kinds:
        seqs.add(c.w.kinds.index(synth.TREE_CHAIN))
    for b in sorted(seqs):
        for i in range(int(nn[b])):
            sel += [(b, i, 0), (b, i, c.w.num_q_heads - 1)]
    err, rl2 = check_attn_rows(c, sel, _tol(c.w), attn=pa, power=0.1)
    assert rl2 <= REL_L2_TOL, f"relative L2 error {rl2}"
    say(f"[{c.w.name}] planted draft keys: attention max-abs error {err:.3g}, relative L2 {rl2:.3g} "
        f"over {len(sel)} rows")
    assert c.step.errors() == 0


def test_full_accept(full_case):
    alen = assert_accept_equal(full_case)
    say(f"[{full_case.w.name}] mean accepted length {alen.mean():.2f}")


def test_full_no_device_errors(full_case):
    assert full_case.step.errors() == 0


# ---------------------------------------------------------------------------
# smaller cases: every code path, ragged sizes, degenerate inputs
# ---------------------------------------------------------------------------
def _small(base, **over):
    w = synth.small_workload(base, **over)
    return w


SMALL = {
    # fp32, vocab not a multiple of the vector width, ragged prefix
    "f32-v1003-L77": lambda: _small(1, vocab=1003, prefix=77),
    # fp32 GQA, head_dim 128, paged with poisoned tails
    "f32-gqa-paged": lambda: _small(1, num_q_heads=8, num_kv_heads=2, head_dim=128, prefix=(1, 300),
                                    block_size=16, batch=3, kinds=[0, 0, 0], poison_tail=True),
    # fp32 kernels by head_dim and cache layout: head_dim 128 contiguous over
    # many key chunks (several rounds of the two key groups, ragged tail);
    # head_dim 64 paged (four key groups) with poisoned tails; empty prefix
    "f32-d128-contig-L1000": lambda: _small(1, num_q_heads=8, num_kv_heads=4, head_dim=128, prefix=(700, 1000),
                                            batch=2, kinds=[0, 0], poison_tail=True),
    "f32-d64-paged": lambda: _small(1, prefix=(1, 900), block_size=16, batch=3, kinds=[0, 0, 0], poison_tail=True),
    "f32-L0": lambda: _small(1, prefix=0, vocab=1000),
    # bf16 contiguous, prefix shorter than one tile, and empty prefix
    "bf16-L13": lambda: _small(2, prefix=13, vocab=5000),
    "bf16-L0": lambda: _small(2, prefix=0, vocab=5000),
    # bf16, many key splits for one sequence (ragged last split)
    "bf16-split-L9000": lambda: _small(2, prefix=9001, vocab=4096, num_q_heads=4, num_kv_heads=4),
    # the same split and merge shapes with planted draft keys (the draft tile
    # rides in the last split and carries most of the mass), few-row and
    # 8-wave kernels, contiguous and paged
    "bf16-split-L9000-planted": lambda: _small(2, prefix=9001, vocab=4096, num_q_heads=4, num_kv_heads=4),
    "bf16-gqa8-split-planted": lambda: _small(4, batch=2, prefix=(6000, 12000), vocab=3000),
    "bf16-paged-split-planted": lambda: _small(5, batch=4, vocab=3000, prefix=(9000, 20000),
                                               kinds=[0, 1, 0, 1]),
    # 8-wave form with 5 and 7 row blocks (rows 20 * 8 = 160, 56 * 4 = 224):
    # the last blocks are computed by key halves on two waves each
    "bf16-gqa8-m20-split-blocks": lambda: _small(4, batch=2, m=20, prefix=(700, 3000), vocab=3000),
    "bf16-paged-m56-split-blocks": lambda: _small(5, batch=3, m=56, vocab=3000, prefix=(300, 2500),
                                                  kinds=[0, 0, 0]),
    # GQA with two row groups (rows = 48 * 8 = 384)
    "bf16-gqa8-rowgroups": lambda: _small(4, batch=2, prefix=700, vocab=3000),
    # prefix scores that climb along the prefix: the softmax reference moves
    # again and again, also between the key halves of one tile (the 8-wave
    # form's per-half rule, contiguous and paged; the key-half form)
    "bf16-gqa8-rising": lambda: _small(4, batch=2, prefix=(700, 2100), vocab=3000),
    "bf16-paged-rising": lambda: _small(5, batch=4, vocab=3000, prefix=(300, 2500)),
    "bf16-keyhalf-rising": lambda: _small(2, batch=2, num_q_heads=8, num_kv_heads=8, prefix=(500, 1500), vocab=3000),
    # paged serving shape with enough long workgroups for the longest-first
    # dispatch table (more than one round of splits of at least 32 tiles)
    "bf16-paged-longest-first": lambda: _small(5, batch=12, vocab=3000, prefix=(1000, 20000),
                                               kinds=[0, 1] * 6, poison_tail=True),
    # two row groups (GQA 8, 384 rows) with the longest-first table and chains:
    # a chain's first row group (56 rows) takes the key-half form and its
    # second (no rows with a node) is zeroed; a tree's groups take the 8-wave form
    "bf16-gqa8-rowgroups-sched-chains": lambda: _small(4, batch=6, vocab=3000, prefix=(3000, 20000),
                                                       kinds=[0, 1] * 3, chain_k=7, block_size=16,
                                                       poison_tail=True),
    # paged, mixed trees and chains, ragged lengths, poisoned tails
    "bf16-paged-mixed": lambda: _small(5, batch=6, vocab=7001, prefix=(1, 5000),
                                       kinds=[0, 1, 0, 1, 1, 0]),
    # contiguous cache, trees and chains in one batch (each workgroup picks the
    # 8-wave or the few-row form by its own sequence's rows), one and many splits
    "bf16-contig-mixed": lambda: _small(5, batch=4, vocab=3000, block_size=0, prefix=(50, 9000),
                                        kinds=[0, 1, 1, 0], poison_tail=True),
    # paged MHA (query rows <= 64: the 4-wave key-half kernel), ragged lengths, poisoned tails
    "bf16-mha-paged16": lambda: _small(2, batch=3, num_q_heads=8, num_kv_heads=8, prefix=(1, 2500),
                                       block_size=16, poison_tail=True, kinds=[0, 0, 0], vocab=3000),
    "bf16-mha-paged32": lambda: _small(2, batch=2, num_q_heads=4, num_kv_heads=4, prefix=(40, 5000),
                                       block_size=32, poison_tail=True, kinds=[0, 0], vocab=3000),
    # contiguous cache with ragged prefixes: short sequences' first tiles are
    # requested past their prefix before its length is known (draft tile among them)
    # (NaN in every cache slot past each prefix: requested, then masked and zeroed)
    "bf16-contig-ragged": lambda: _small(2, batch=4, num_q_heads=8, num_kv_heads=8, prefix=(5, 3000),
                                         kinds=[0, 0, 0, 0], vocab=3000, poison_tail=True),
    "bf16-gqa-contig-ragged": lambda: _small(4, batch=3, prefix=(5, 2000), vocab=3000, poison_tail=True),
    # 65..128 query rows (G = 2): the 4-wave kernel over whole tiles, contiguous and paged
    "bf16-g2-rows120": lambda: _small(2, batch=2, num_q_heads=8, num_kv_heads=4, prefix=(200, 1500),
                                      kinds=[0, 0], vocab=3000),
    "bf16-g2-rows120-paged": lambda: _small(2, batch=2, num_q_heads=8, num_kv_heads=4, prefix=(200, 1500),
                                            block_size=16, poison_tail=True, kinds=[0, 0], vocab=3000),
    # page sizes 8 and 64 (page-major V^T with 1 and 8 chunks per page) and 24
    # (pages that do not tile a 64-key tile: per-key page lookups, swizzled V^T)
    "bf16-paged8": lambda: _small(5, batch=2, vocab=3000, prefix=(30, 1200), block_size=8, poison_tail=True,
                                  kinds=[0, 1]),
    "bf16-paged64": lambda: _small(5, batch=2, vocab=3000, prefix=(30, 1200), block_size=64, poison_tail=True,
                                   kinds=[0, 1]),
    "bf16-paged24": lambda: _small(2, batch=2, num_q_heads=8, num_kv_heads=8, vocab=3000, prefix=(30, 1200),
                                   block_size=24, poison_tail=True, kinds=[0, 0]),
    # sampling at temperature 0.7
    "bf16-rs-T0.7": lambda: dataclasses.replace(_small(3, batch=3, prefix=300, vocab=2000), temperature=0.7),
    # tiny vocabulary: fewer elements than one thread block, exact fallback top-C
    "f32-tiny-vocab": lambda: _small(1, vocab=37, children=16, depth=3, topk=4, m=40, prefix=40),
    # chain only, K = depth 64 is not allowed (m_max <= 64), use K = 64 nodes
    "bf16-chain64": lambda: _small(5, batch=2, kinds=[1, 1], chain_k=64, vocab=3000, prefix=(50, 200)),
    # the largest dynamic trees: m = 64 (a full 64-node draft tile, mask bit
    # 63), GQA 8 (two row groups of 8 blocks); and a wide tree, 16 children per
    # node and 16 expanded per depth (784 candidates, the general-C select)
    "bf16-gqa8-m64": lambda: _small(4, batch=2, m=64, prefix=(300, 2000), vocab=3000),
    "bf16-wide-c16-k16-m64": lambda: _small(5, batch=2, kinds=[0, 0], depth=4, topk=16, children=16, m=64,
                                            vocab=3000, prefix=(100, 1500)),
    # register-held rows (few rows) with heavy ties (sd 0.02), and at 8 vectors per thread
    "bf16-v32000-ties": lambda: _small(2, vocab=32000, draft_sigma=0.02, prefix=100),
    "f32-v32000": lambda: _small(1, vocab=32000, prefix=64),
    # streaming rows (more rows than the register form takes), mixed trees and chains
    "bf16-v16001-stream-mixed": lambda: _small(5, batch=6, vocab=16001, prefix=(50, 300), kinds=[0, 1, 1, 0, 0, 1]),
    # rows too long for registers: streaming kernel (bf16 and fp32, ragged vocab)
    "bf16-stream": lambda: _small(2, batch=2, vocab=70001, prefix=100),
    "bf16-stream-ragged-long": lambda: _small(2, batch=2, vocab=120003, prefix=100),
    "f32-stream": lambda: _small(1, vocab=40003, prefix=64),
    # the largest vocabulary, heavy ties
    "bf16-vmax-ties": lambda: _small(2, vocab=1 << 17, draft_sigma=0.05, prefix=64),
}


@pytest.fixture(scope="module", params=sorted(SMALL))
def small_case(request):
    w = SMALL[request.param]()
    say(f"[small {request.param}] {w}")
    c = make_case(w, seed=7, plant=(w.accept_mode == synth.ACCEPT_GREEDY))
    if request.param.endswith("-planted"):
        c.attn = synth.plant_draft_keys(c.attn, w, c.seed)
    if request.param.endswith("-rising"):
        c.attn = synth.rising_prefix_keys(c.attn, w, c.seed)
    run_gpu(c)
    c.planted_keys = request.param.endswith("-planted")
    return c


def test_separate_build_and_mask_equal_the_fused_call(small_case):
    """The step runs eagle_build_tree_mask; eagle_build_tree followed by
    eagle_tree_mask must give the same outputs bit for bit."""
    c = small_case
    s = c.step
    fused = {k: getattr(s, k).clone() for k in ("tokens", "parent", "depth", "score", "src_row", "num_nodes",
                                                  "anc", "pos")}
    s.build(c.draft, c.kinds)
    s.mask(c.attn.prefix_len)
    torch.cuda.synchronize()
    for k, v in fused.items():
        assert torch.equal(getattr(s, k), v), k


def test_small_all_outputs(small_case):
    c = small_case
    assert_tree_equal(c)
    anc, pos = oracle_mask(c)
    assert np.array_equal(c.step.anc.cpu().numpy().view(np.uint64), anc)
    assert np.array_equal(c.step.pos.cpu().numpy(), pos)
    sel = [(b, i, h) for b in range(c.w.batch) for i in range(int(c.otree["num_nodes"][b]))
           for h in range(c.w.num_q_heads)]
    _, rl2 = check_attn_rows(c, sel, _tol(c.w), power=0.1 if c.planted_keys else None)
    assert rl2 <= REL_L2_TOL, f"relative L2 error {rl2}"
    assert_accept_equal(c)
    assert c.step.errors() == 0


def test_planted_paths_reach_full_depth():
    w = _small(2, batch=2, vocab=6000, prefix=100)
    c = make_case(w, seed=3, plant=True)
    run_gpu(c)
    alen = assert_accept_equal(c)
    # the planted path ends at the deepest selected node
    deepest = [int(c.otree["depth"][b, :int(c.otree["num_nodes"][b])].max()) for b in range(w.batch)]
    assert list(alen) == deepest


def test_heavy_ties_use_exact_fallback():
    # rows of only a few distinct values: thousands of candidates tie at the max
    w = _small(2, batch=1, vocab=8192, prefix=64)
    c = make_case(w, seed=5)
    d = torch.zeros_like(c.draft)
    d[:, :, ::3] = 1.0
    d[:, :, 7::11] = -2.0
    c.draft.copy_(d)
    c.otree = oracle.build_tree(to_np(c.draft), w.depth, w.topk, w.children, w.m, m_max=w.m_max)
    c.step.build(c.draft, c.kinds)
    torch.cuda.synchronize()
    assert_tree_equal(c)


@pytest.mark.parametrize("vocab", [20000, 70000])
def test_weight_bins_and_direct_weights_agree_with_the_oracle(vocab):
    # bf16 rows long enough for the binned weight sum (register form at 20000,
    # streaming form at 70000), planted with values outside the bins' range
    # (zeros, tiny, at and past both range ends, -inf) and rows whose maximum
    # is so large that every binned weight is 0
    w = _small(2, batch=1, vocab=vocab, prefix=64)
    c = make_case(w, seed=7)
    g = torch.Generator().manual_seed(17)
    d = c.draft.float().cpu()
    R, V = d.shape[1], d.shape[2]
    planted = torch.tensor([0.0, -0.0, 1e-6, -1e-6, 2.0 ** -9, -(2.0 ** -9), 2.0 ** -10, 3e-3, 127.0, 128.0,
                            -128.0, 200.0, -300.0, float("-inf")])
    for r in range(R):
        idx = torch.randperm(V, generator=g)[:4 * planted.numel()]
        d[0, r, idx] = planted.repeat(4)
        if r % 5 == 1:
            d[0, r, int(torch.randint(V, (1,), generator=g))] = 400.0
    c.draft.copy_(d.to(c.draft.dtype))
    c.otree = oracle.build_tree(to_np(c.draft), w.depth, w.topk, w.children, w.m, m_max=w.m_max)
    c.step.build(c.draft, c.kinds)
    torch.cuda.synchronize()
    assert_tree_equal(c)


@pytest.mark.parametrize("shape", ["paged-mixed", "gqa8-split-blocks"])
def test_determinism(shape):
    # the paged mix of trees and chains (8-wave and key-half forms), and row
    # groups of 6 blocks (the last two computed by key halves on two waves each)
    if shape == "paged-mixed":
        w = _small(5, batch=4, vocab=9000, prefix=(100, 3000), kinds=[0, 1, 0, 0])
    else:
        w = _small(4, batch=2, vocab=3000, prefix=(1500, 5000))
    c = make_case(w, seed=11)
    outs = []
    for _ in range(10):
        run_gpu(c)
        outs.append([t.clone() for t in (c.step.tokens, c.step.score, c.step.anc, c.step.out, c.step.accepted,
                                         c.step.bonus)])
    for o in outs[1:]:
        for x, y in zip(outs[0], o):
            assert torch.equal(x.view(torch.uint8) if x.dtype == torch.bfloat16 else x,
                               y.view(torch.uint8) if y.dtype == torch.bfloat16 else y)


def test_device_error_bits():
    w = _small(2, batch=2, vocab=4000, prefix=100)
    c = make_case(w, seed=13)
    c.draft[1, 3, 17] = float("nan")
    c.step.build(c.draft, c.kinds)
    torch.cuda.synchronize()
    assert E.read_errors(c.step.ws_tree) & E.DEVERR_NONFINITE_ROW
    # prefix longer than the cache: clamped and reported
    bad = c.attn.prefix_len.clone()
    bad[0] = c.attn.max_prefix + 5
    c.step.mask(bad)
    c.step.attention(c.attn.q, c.attn.k_draft, c.attn.v_draft, c.attn.k_cache, c.attn.v_cache, None, bad)
    torch.cuda.synchronize()
    assert E.read_errors(c.step.ws_attn) & E.DEVERR_PREFIX
    assert E.read_errors(c.step.ws_attn) == 0   # reading clears


# ---------------------------------------------------------------------------
# rejection sampling on the GPU: 10^6 trials, bit-exact and distribution
# ---------------------------------------------------------------------------
def test_rejection_sampling_million_trials():
    import scipy.stats
    V, n = 8, 1_000_000
    rng = np.random.default_rng(21)
    target1 = (rng.standard_normal((1, 4, V)) * 1.5).astype(np.float32)
    tok = np.array([[2, 5, 7]], np.int32)
    par = np.array([[-1, -1, 0]], np.int32)
    words = rng.integers(0, 1 << 32, size=(n, 4), dtype=np.uint64).astype(np.uint32)
    tg = np.ascontiguousarray(np.broadcast_to(target1, (n, 4, V)))
    toks = np.ascontiguousarray(np.broadcast_to(tok, (n, 3)))
    pars = np.ascontiguousarray(np.broadcast_to(par, (n, 3)))
    nn = np.full(n, 3, np.int32)
    o_acc, o_len, o_bon = oracle.accept(1, tg, toks, pars, nn, 2, rand_words=words)
    dev = "cuda"
    a = E.AcceptParams(E.EAGLE_ACCEPT_SAMPLE, 1.0, 3, V, 2)
    ws = torch.empty(E.accept_workspace_size(a, n), dtype=torch.uint8, device=dev)
    E.workspace_init(ws)
    acc = torch.empty((n, 2), dtype=torch.int32, device=dev)
    alen = torch.empty(n, dtype=torch.int32, device=dev)
    bon = torch.empty(n, dtype=torch.int32, device=dev)
    E.accept(a, n, torch.from_numpy(tg).to(dev), torch.from_numpy(toks).to(dev), torch.from_numpy(pars).to(dev),
             torch.from_numpy(nn).to(dev), torch.from_numpy(words.view(np.int32)).to(dev), acc, alen, bon, ws)
    torch.cuda.synchronize()
    assert np.array_equal(acc.cpu().numpy(), o_acc)
    assert np.array_equal(alen.cpu().numpy(), o_len)
    assert np.array_equal(bon.cpu().numpy(), o_bon)
    first = np.where(o_len > 0, tok[0][np.maximum(o_acc[:, 0], 0)], o_bon)
    lf = target1[0, 0]
    p = np.exp(lf.astype(np.float64) - lf.max())
    p /= p.sum()
    chi = scipy.stats.chisquare(np.bincount(first, minlength=V), p * n)
    assert chi.pvalue > 1e-3


def test_graph_replay_matches_eager():
    """The four calls captured into one graph, replayed several times with
    eager work and synchronisations in between; every replay must equal the
    eager result bit for bit (no memset nodes, self-contained workspaces)."""
    w = _small(5, batch=4, vocab=6000, prefix=(100, 4000), kinds=[0, 1, 0, 1])
    c = make_case(w, seed=17)
    run_gpu(c)
    outs = [t.clone() for t in (c.step.tokens, c.step.score, c.step.anc, c.step.pos, c.step.out,
                                c.step.accepted, c.step.accept_len, c.step.bonus)]
    a = c.attn
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        run_gpu(c)
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        c.step.run(c.draft, c.kinds, a.prefix_len, a.q, a.k_draft, a.v_draft, a.k_cache, a.v_cache,
                   a.block_table, c.target, None)
    for rep in range(4):
        for t in (c.step.tokens, c.step.out, c.step.accepted):
            t.zero_()                                   # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        now = (c.step.tokens, c.step.score, c.step.anc, c.step.pos, c.step.out, c.step.accepted,
               c.step.accept_len, c.step.bonus)
        for x, y in zip(outs, now):
            assert torch.equal(x.view(torch.uint8) if x.dtype == torch.bfloat16 else x,
                               y.view(torch.uint8) if y.dtype == torch.bfloat16 else y), f"replay {rep}"
    assert c.step.errors() == 0
