#!/usr/bin/env python3
"""Benchmark of one EAGLE-2 draft-tree verification step on one MI355X.

A step is the whole hot path on one stream: eagle_build_tree (draft-row
softmax statistics, top-C children, expansion, rerank, compaction),
eagle_tree_mask, eagle_tree_attn and eagle_accept, over one batch of
synthetic inputs already resident in HBM.  The headline workload is the
batched serving mix (batch 64, bf16, Llama-3-8B attention shape 32 q / 8 kv
heads x 128, prefixes uniform in 1k-32k in 16-token pages, vocab 128256,
half dynamic trees with m = 60, half K = 7 parallel-draft chains, greedy);
the other four workloads are timed in the same run and reported under
"workloads".  Prints one JSON line.

Inputs: seeded synthetic draft/target logits and Q/K/V (random numbers stand
in for trained models and text benchmarks).  The timed steps rotate over
enough independent input sets to exceed the 256 MB Infinity Cache, so every
step reads its inputs from HBM ("cold"); a warm figure (one set repeated) is
reported beside it.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--config N] [--only]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
MALL_BYTES = 256 << 20


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=5,
                    help="headline workload 1..5 (default 5, the batched serving mix)")
    ap.add_argument("--only", action="store_true", help="time the headline workload only (not the other four)")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the headline's timings of the entry points outside the step")
    ap.add_argument("--sets", type=int, default=0, help="input sets rotated per step (0: enough to exceed the MALL)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="oracle CPU baseline budget for the headline workload (at least one whole step)")
    ap.add_argument("--cpu-seconds-others", type=float, default=5.0,
                    help="oracle CPU baseline budget for each other workload (at least one whole step)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--attn-only", action="store_true", help="time only eagle_tree_attn (for profiling runs)")
    ap.add_argument("--eager", action="store_true", help="time eager launches instead of hipGraph replays")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain fp32 copy kernel (torch.neg) over BYTES, for counter calibration")
    return ap.parse_args()


ATTN_SOURCES = ("eagle_tree_verification_draft_amd/csrc/tree_attn.hip",
                "eagle_tree_verification_draft_amd/csrc/common.h",
                "eagle_tree_verification_draft_amd/csrc/internal.h")


def traffic_note(w):
    """HBM bytes per attention call from the committed counter note for this
    workload (FETCH_SIZE + WRITE_SIZE, copy-calibrated), or None when there is
    no note or the kernel source changed since its counters were taken."""
    from eagle_tree_verification_draft_amd import profiling
    path = os.path.join(ROOT, "profiles", f"tree_attn.{w.name}.traffic.txt")
    if not os.path.exists(path):
        return None, "no counter note for this workload"
    note = profiling.read_note(path)
    srcs = [os.path.join(ROOT, s) for s in note.get("source", "").split(",") if s]
    if not srcs or any(not os.path.exists(s) for s in srcs) or \
            profiling.source_hash(srcs) != note.get("source_sha256"):
        return None, "kernel source changed since the counters were taken"
    return float(note["traffic_bytes_per_call"]), os.path.relpath(path, ROOT)


def mfma_note(w):
    """Counter-derived matrix-core utilisation of the attention kernel from the
    committed note for this workload (rocprofv3 MfmaUtil), or None when there
    is no note or the kernel source changed since its counters were taken."""
    from eagle_tree_verification_draft_amd import profiling
    path = os.path.join(ROOT, "profiles", f"tree_attn.{w.name}.mfma.txt")
    if not os.path.exists(path):
        return None, "no counter note for this workload"
    note = profiling.read_note(path)
    srcs = [os.path.join(ROOT, s) for s in note.get("source", "").split(",") if s]
    if not srcs or any(not os.path.exists(s) for s in srcs) or \
            profiling.source_hash(srcs) != note.get("source_sha256") or "mfma_util" not in note:
        return None, "kernel source changed since the counters were taken"
    return float(note["mfma_util"]), os.path.relpath(path, ROOT)


def copy_calibration(nbytes):
    """A plain copy of known size (read nbytes, write nbytes) for scaling the
    FETCH_SIZE / WRITE_SIZE counters to bytes."""
    import torch
    n = nbytes // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n * 4, "kernel": "torch.neg fp32", "dispatches": 3}), flush=True)


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def attn_algorithmic(w, attn, num_nodes):
    """HBM bytes and flops the attention call must move/do: every prefix K/V
    byte once per kv head, the draft K/V, Q and the output once; flops of
    q.k and p.v over prefix + ancestor keys."""
    import torch
    esz = 4 if w.dtype == torch.float32 else 2
    d, Hq, Hkv = w.head_dim, w.num_q_heads, w.num_kv_heads
    L = attn.prefix_len.to("cpu").to(torch.int64)
    nn = num_nodes.to("cpu").to(torch.int64)
    kv = int(L.sum()) * Hkv * d * 2 * esz
    qo = int(nn.sum()) * Hq * d * esz * 2
    dkv = int(nn.sum()) * Hkv * d * 2 * esz
    flops = 4 * d * Hq * int((nn * L).sum())
    return kv + qo + dkv, flops


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the verification step of one "
              "sequence batch runs on a single GPU, and sharding sequences over GPUs is not implemented",
              file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return

    import torch

    others = [] if args.only else [n for n in (1, 2, 3, 4, 5) if n != args.config]
    head = bench_workload(args.config, args, extras=not args.no_extras,
                          cpu_seconds=args.cpu_seconds)
    subs = {}
    for n in others:
        torch.cuda.empty_cache()
        subs[str(n)] = bench_workload(n, args, extras=False, cpu_seconds=args.cpu_seconds_others)
    out = {
        "metric": "verified tree tokens/s (build+tree-attn+accept), % of HBM/MFMA peak",
        "value": head.pop("value"),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head.pop("ms_per_step"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head.pop("dtype"),
        "data": "synthetic",
        "config": head.pop("config"),
        "roofline": head.pop("roofline"),
        "cpu_baseline": head.pop("cpu_baseline"),
    }
    out.update(head)
    if subs:
        out["workloads"] = subs
    print(json.dumps(out), flush=True)


def bench_workload(n, args, extras, cpu_seconds):
    """One workload: cold step time over rotating input sets (hipGraph
    replays), the attention call's roofline, per-stage times, warm and eager
    figures, and the oracle timed on the host cores.  Returns the fields of
    its JSON line."""
    import numpy as np
    import torch

    import eagle_tree_verification_draft_amd as E
    import synth

    dev = "cuda"
    w = synth.workload(n)
    base_seed = 5000 + 100 * n

    # ---- input sets ----------------------------------------------------
    def make_set(i, step):
        seed = base_seed + i
        draft = synth.draft_logits(w, seed, dev)
        attn = synth.attn_inputs(w, seed, dev, prefix_seed=base_seed)
        step.build(draft, kinds)
        torch.cuda.synchronize()
        target = synth.target_logits(w, seed, draft, step.src_row.cpu(), step.num_nodes.cpu(), dev)
        words = synth.rand_words(w, seed, dev) if w.accept_mode == synth.ACCEPT_SAMPLE else None
        return dict(draft=draft, attn=attn, target=target, words=words)

    kinds = synth.kinds_tensor(w, dev)
    log(f"[bench] workload {w.name}: generating inputs")
    attn0 = synth.attn_inputs(w, base_seed, dev, prefix_seed=base_seed)
    step = E.VerifyStep(E.StepShape(**synth.step_dims(w, attn0)), dev)
    first = dict(draft=synth.draft_logits(w, base_seed, dev), attn=attn0)
    step.build(first["draft"], kinds)
    torch.cuda.synchronize()
    first["target"] = synth.target_logits(w, base_seed, first["draft"], step.src_row.cpu(), step.num_nodes.cpu(), dev)
    first["words"] = synth.rand_words(w, base_seed, dev) if w.accept_mode == synth.ACCEPT_SAMPLE else None
    set_bytes = sum(t.numel() * t.element_size() for t in
                    (first["draft"], first["target"], attn0.q, attn0.k_draft, attn0.v_draft, attn0.k_cache,
                     attn0.v_cache))
    nsets = args.sets or max(2, math.ceil(2 * MALL_BYTES / set_bytes))
    nsets = min(nsets, 64)
    sets = [first] + [make_set(i, step) for i in range(1, nsets)]
    tokens_per_step = int(step.num_nodes.sum().item())
    log(f"[bench] {nsets} input sets of {set_bytes / 1e6:.1f} MB; {tokens_per_step} verified tokens per step")

    def run_step(S, ev=None):
        a = S["attn"]
        if not args.attn_only:
            step.build_mask(S["draft"], kinds, a.prefix_len)
        if ev is not None:
            ev[0].record()
        step.attention(a.q, a.k_draft, a.v_draft, a.k_cache, a.v_cache, a.block_table, a.prefix_len)
        if ev is not None:
            ev[1].record()
        if not args.attn_only:
            step.accept(S["target"], S["words"])

    # ---- one captured graph per input set (the four calls of one step) ----
    graphs = None
    if not args.eager:
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cap):
            for k in range(3):
                run_step(sets[k % nsets])
        torch.cuda.current_stream().wait_stream(cap)
        torch.cuda.synchronize()
        graphs = []
        for S in sets:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                run_step(S)
            graphs.append(g)
        torch.cuda.synchronize()

    def timed_steps(K):
        """K steps (sets rotate), bracketed by device synchronisation."""
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(K):
            if graphs is not None:
                graphs[k % nsets].replay()
            else:
                run_step(sets[k % nsets])
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / K

    # ---- warm-up and the timed region (cold: sets rotate) ----------------
    for k in range(args.warmup):
        if graphs is not None:
            graphs[k % nsets].replay()
        else:
            run_step(sets[k % nsets])
    K = args.steps
    ms_per_step = timed_steps(K)
    eager_ms = ms_per_step if graphs is None else None
    log(f"[bench] timed {K} steps ({'graph replays' if graphs is not None else 'eager'}): "
        f"{ms_per_step * 1e3:.1f} us/step")

    # ---- per-step times (cold, sets rotate): events between the replays --
    step_ev = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    torch.cuda.synchronize()
    step_ev[0].record()
    for k in range(K):
        if graphs is not None:
            graphs[k % nsets].replay()
        else:
            run_step(sets[k % nsets])
        step_ev[k + 1].record()
    torch.cuda.synchronize()
    step_us = np.array([step_ev[k].elapsed_time(step_ev[k + 1]) * 1e3 for k in range(K)])
    pctl = {f"p{q}": round(float(np.percentile(step_us, q)), 2) for q in (10, 50, 90)}

    # accepted draft tokens per sequence, from the last step of input set 0
    run_step(sets[0])
    torch.cuda.synchronize()
    acc_len = step.accept_len.to(torch.float64)
    mean_accepted = float(acc_len.mean().item())

    # ---- eager steps (context), events around each attention call -----
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    torch.cuda.synchronize()
    te0 = time.perf_counter()
    for k in range(K):
        run_step(sets[k % nsets], evs[k])
    torch.cuda.synchronize()
    if eager_ms is None:
        eager_ms = (time.perf_counter() - te0) * 1e3 / K
    attn_eager_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))

    # ---- attention duration: HIP events around graph replays of back-to-back
    # attention calls (one per input set) on the stream they run on ----------
    if graphs is not None:
        ag = torch.cuda.CUDAGraph()
        with torch.cuda.graph(ag):
            for S in sets:
                a = S["attn"]
                step.attention(a.q, a.k_draft, a.v_draft, a.k_cache, a.v_cache, a.block_table, a.prefix_len)
        ag.replay()
        reps = max(1, math.ceil(K / nsets))
        ea, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        ea.record()
        for _ in range(reps):
            ag.replay()
        eb.record()
        torch.cuda.synchronize()
        attn_avg_ms = ea.elapsed_time(eb) / (reps * nsets)
        attn_calls = reps * nsets
    else:
        attn_avg_ms, attn_calls = attn_eager_ms, K
    log(f"[bench] eager {eager_ms * 1e3:.1f} us/step; attention {attn_avg_ms * 1e3:.2f} us/call "
        f"(eager with events {attn_eager_ms * 1e3:.2f})")

    # ---- per-stage breakdown (separate loop, events between the calls) ---
    stage_names = ["build_tree+mask", "tree_attn", "accept"]
    n_stage = min(K, 100)
    sev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(n_stage)]
    for k in range(n_stage):
        S = sets[k % nsets]
        a = S["attn"]
        e = sev[k]
        e[0].record()
        step.build_mask(S["draft"], kinds, a.prefix_len)
        e[1].record()
        step.attention(a.q, a.k_draft, a.v_draft, a.k_cache, a.v_cache, a.block_table, a.prefix_len)
        e[2].record()
        step.accept(S["target"], S["words"])
        e[3].record()
    torch.cuda.synchronize()
    stage_us = {n: float(np.median([sev[k][j].elapsed_time(sev[k][j + 1]) for k in range(n_stage)])) * 1e3
                for j, n in enumerate(stage_names)}

    # ---- warm: one set repeated ------------------------------------------
    for _ in range(5):
        graphs[0].replay() if graphs is not None else run_step(sets[0])
    torch.cuda.synchronize()
    tw0 = time.perf_counter()
    for _ in range(K):
        graphs[0].replay() if graphs is not None else run_step(sets[0])
    torch.cuda.synchronize()
    warm_ms = (time.perf_counter() - tw0) * 1e3 / K

    if extras:
        commit = measure_commit(E, step, w, sets[0], kinds, K)
        log(f"[bench] kv commit {commit['avg_us']:.2f} us/call for {commit['tokens']} tokens")
        expand = measure_expand(E, step, w, sets[0], kinds, K)
        pdraft = measure_pdraft(E, step, w, sets[0], kinds, K)
        policies = measure_policies(E, w, sets[0], kinds, K)
        rrs = measure_rrs(E, w, K)
        log(f"[bench] sampled build {rrs['build_us']:.1f} us, recursive rejection sampling {rrs['accept_us']:.1f} us")
        log(f"[bench] parallel-draft inputs {pdraft['avg_us']:.2f} us/call, {pdraft['hbm_gbs']:.0f} GB/s")
        if expand:
            log(f"[bench] incremental build {expand['total_us']:.1f} us for {expand['levels']} levels + finish")

    errs = step.errors()
    if errs:
        log(f"[bench] WARNING: device error bits {errs:#x}")

    nbytes, flops = attn_algorithmic(w, attn0, step.num_nodes)
    gbs = nbytes / (attn_avg_ms * 1e-3) / 1e9
    tflops = flops / (attn_avg_ms * 1e-3) / 1e12
    mfma_frac = tflops / MFMA_BF16_PEAK_TFLOPS
    # bound: MFMA when the call's arithmetic intensity is past the bf16 ridge
    # (2.5 PFLOP/s / 8 TB/s = 312 flop/B), HBM otherwise
    mfma_bound = w.dtype == torch.bfloat16 and flops / nbytes > MFMA_BF16_PEAK_TFLOPS * 1e3 / HBM_PEAK_GBS
    if mfma_bound:
        bound, achieved, peak, unit = "mfma", tflops, MFMA_BF16_PEAK_TFLOPS, "TFLOP/s"
    else:
        bound, achieved, peak, unit = "hbm", gbs, HBM_PEAK_GBS, "GB/s"
    value = tokens_per_step / (ms_per_step * 1e-3)
    # draft-row bytes the build reads (every row a sequence's tree or chain owns, once)
    esz = 2 if w.dtype == torch.bfloat16 else 4
    build_bytes = sum((w.rows_dynamic if kd == synth.TREE_DYNAMIC else w.chain_k) for kd in w.kinds) * w.vocab * esz
    stage_gbs = {"build_tree+mask": round(build_bytes / (stage_us["build_tree+mask"] * 1e-6) / 1e9, 1),
                 "tree_attn": round(nbytes / (stage_us["tree_attn"] * 1e-6) / 1e9, 1)}
    traffic, traffic_src = traffic_note(w)
    mfma_util, mfma_src = mfma_note(w)

    # ---- the oracle on the host cores (whole steps) ----------------------
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, sets[0], base_seed, tokens_per_step, cpu_seconds)

    out = {
        "value": round(value, 1),
        "ms_per_step": round(ms_per_step, 5),
        "dtype": "bf16" if w.dtype == torch.bfloat16 else "f32",
        "config": {"workload": w.name, "batch": w.batch, "vocab": w.vocab, "depth": w.depth, "topk": w.topk,
                   "m": w.m, "heads": f"{w.num_q_heads}q/{w.num_kv_heads}kv x {w.head_dim}",
                   "prefix": w.prefix if isinstance(w.prefix, int) else list(w.prefix),
                   "kv_layout": "paged16" if w.block_size else "contiguous",
                   "accept": "greedy" if w.accept_mode == synth.ACCEPT_GREEDY else f"sample T={w.temperature}",
                   "input_sets": nsets, "cold": True,
                   "launch": "graph" if graphs is not None else "eager"},
        "roofline": {"kernel": ("k_tree_attn_f32" if w.dtype != torch.bfloat16 else
                                "k_tree_attn_bf16_mixed" if w.m_max * (w.num_q_heads // w.num_kv_heads) > 128
                                else "k_tree_attn_bf16"),
                     "bound": bound, "achieved": round(achieved, 1), "peak": peak, "unit": unit,
                     "frac": round(achieved / peak, 4),
                     "traffic": None if traffic is None else round(traffic),
                     "traffic_source": traffic_src,
                     "call": "eagle_tree_attn (k_attn_schedule when the splits are ordered longest first, "
                             "k_tree_attn_*, k_tree_attn_merge when the keys are split)",
                     "algorithmic_bytes": nbytes, "algorithmic_flops": flops,
                     "avg_us": round(attn_avg_ms * 1e3, 2), "timed_calls": attn_calls,
                     "eager_event_us": round(attn_eager_ms * 1e3, 2),
                     "hbm_gbs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                     "tflops": round(tflops, 2), "mfma_frac": round(mfma_frac, 4),
                     "mfma_frac_is": "algorithmic flops / call time / bf16 dense peak",
                     "mfma_util_counter": mfma_util, "mfma_util_source": mfma_src},
        "cpu_baseline": cpu,
        "stages_us": {k: round(v, 2) for k, v in stage_us.items()},
        "stages_gbs": stage_gbs,
        "stages_bytes": {"build_tree+mask": build_bytes, "tree_attn": nbytes},
        "step_us_percentiles": pctl,
        "mean_accepted_tokens": round(mean_accepted, 3),
        "tau": round(mean_accepted + 1.0, 3),
        "warm": {"ms_per_step": round(warm_ms, 5), "value": round(tokens_per_step / (warm_ms * 1e-3), 1)},
        "launch": "hipGraph replay per step" if graphs is not None else "eager",
        "eager": {"ms_per_step": round(eager_ms, 5), "value": round(tokens_per_step / (eager_ms * 1e-3), 1)},
        "tokens_per_step": tokens_per_step,
        "device": torch.cuda.get_device_name(0),
        "device_errors": errs,
    }
    if extras:
        out.update(kv_commit=commit, tree_expand=expand, pdraft_prepare=pdraft, tree_policies=policies,
                   sampled_rrs=rrs)
    del sets, graphs
    return out




def measure_commit(E, step, w, S, kinds, reps):
    """eagle_kv_commit of input set 0's accepted paths, outside the step: one
    call per replay of a graph of 20 calls, HIP events around the replays.
    The paths are written into a scratch cache of the same layout at
    positions max(prefix_len - max_accept, 0), which lie on assigned pages."""
    import torch
    a = S["attn"]
    step.run(S["draft"], kinds, a.prefix_len, a.q, a.k_draft, a.v_draft, a.k_cache, a.v_cache, a.block_table,
             S["target"], S["words"])
    kc, vc = torch.empty_like(a.k_cache), torch.empty_like(a.v_cache)
    plen = (a.prefix_len - w.max_accept).clamp(min=0).to(torch.int32)
    plo = torch.empty_like(plen)

    def call():
        E.kv_commit(step.attn, w.batch, a.k_draft, a.v_draft, step.accepted, step.accept_len, plen, kc, vc,
                    a.block_table, step.slot_mapping, plo, step.ws_commit)

    per_graph = 20
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(per_graph):
            call()
    g.replay()
    n = max(1, reps // per_graph)
    ea, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ea.record()
    for _ in range(n):
        g.replay()
    eb.record()
    torch.cuda.synchronize()
    us = ea.elapsed_time(eb) * 1e3 / (n * per_graph)
    tokens = int(step.accept_len.sum().item())
    esz = 4 if w.dtype == torch.float32 else 2
    nbytes = tokens * w.num_kv_heads * w.head_dim * esz * 4   # K and V rows read, then written
    assert torch.equal(plo, plen + step.accept_len), "kv commit did not write every accepted token"
    return {"call": "eagle_kv_commit (k_kv_commit)", "avg_us": round(us, 2), "timed_calls": n * per_graph,
            "tokens": tokens, "algorithmic_bytes": nbytes, "hbm_gbs": round(nbytes / (us * 1e-6) / 1e9, 1)}


def measure_rrs(E, w, reps):
    """Children drawn from the draft (depth 4, top 3 expanded, 3 drawn children:
    30 nodes, every one kept) and recursive rejection sampling over them, on
    the workload's batch, vocabulary and dtype: synthetic draft rows N(0, 9),
    target rows = the node's own draft row + N(0, 1).  Graph replays of 10
    calls each, HIP events; mean accepted length."""
    import numpy as np
    import torch
    D, k, C = 4, 3, 3
    B, V = w.batch, w.vocab
    R = 1 + (D - 1) * k
    N = C + (D - 1) * k * C
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    draft = (torch.randn((B, R, V), generator=g, device="cuda") * 3.0).to(w.dtype)
    words_c = torch.randint(-(1 << 31), 1 << 31, (B, R, C), generator=g, device="cuda", dtype=torch.int64).to(torch.int32)
    words = torch.randint(-(1 << 31), 1 << 31, (B, N + 1), generator=g, device="cuda", dtype=torch.int64).to(torch.int32)
    p = E.TreeParams(D, k, C, 1, 0, V, N, R, 0)
    ws_t = torch.empty(max(256, E.build_tree_workspace_size(p, B)), dtype=torch.uint8, device="cuda")
    E.workspace_init(ws_t)
    i32 = dict(dtype=torch.int32, device="cuda")
    tok, par, dep, srow = (torch.empty((B, N), **i32) for _ in range(4))
    score = torch.empty((B, N), dtype=torch.float64, device="cuda")
    nn = torch.empty((B,), **i32)
    E.build_tree_sampled(p, B, draft, words_c, tok, par, dep, score, srow, nn, ws_t)
    torch.cuda.synchronize()
    rows = torch.where(srow >= 0, srow, torch.zeros_like(srow)).long()
    target = torch.empty((B, N + 1, V), dtype=w.dtype, device="cuda")
    target[:, 0] = draft[:, 0]
    target[:, 1:] = torch.gather(draft, 1, rows[:, :, None].expand(B, N, V))
    target = (target.float() + torch.randn(target.shape, generator=g, device="cuda")).to(w.dtype)
    a = E.AcceptParams(E.EAGLE_ACCEPT_SAMPLE, 1.0, N, V, D)
    ws_a = torch.empty(E.accept_rrs_workspace_size(a, B), dtype=torch.uint8, device="cuda")
    E.workspace_init(ws_a)
    acc = torch.empty((B, D), **i32)
    alen = torch.empty((B,), **i32)
    bon = torch.empty((B,), **i32)

    def timed(fn):
        st = torch.cuda.Stream()
        st.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(st):
            fn()
        torch.cuda.current_stream().wait_stream(st)
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            for _ in range(10):
                fn()
        gr.replay()
        n = max(1, reps // 10)
        ea, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        ea.record()
        for _ in range(n):
            gr.replay()
        eb.record()
        torch.cuda.synchronize()
        return ea.elapsed_time(eb) * 1e3 / (n * 10)

    build_us = timed(lambda: E.build_tree_sampled(p, B, draft, words_c, tok, par, dep, score, srow, nn, ws_t))
    accept_us = timed(lambda: E.accept_rrs(a, B, target, draft, tok, par, srow, nn, words, acc, alen, bon, ws_a))
    assert E.read_errors(ws_t) == 0 and E.read_errors(ws_a) == 0, "sampled build or RRS reported device errors"
    return {"tree": f"depth {D}, top {k} expanded, {C} drawn children, {N} nodes", "build_us": round(build_us, 2),
            "accept_us": round(accept_us, 2), "mean_accept_len": round(float(alen.float().mean().item()), 3)}


def measure_policies(E, w, S, kinds, reps):
    """eagle_build_tree under each tree policy on input set 0's draft rows
    (outside the step; m_max 64 so that every policy's tree fits): HIP events
    around replays of a graph of 10 calls.  us per call, and the mean node
    count per sequence."""
    import torch
    out = {}
    B = w.batch
    i32 = dict(dtype=torch.int32, device="cuda")
    bufs = [torch.empty((B, 64), **i32) for _ in range(4)]
    score = torch.empty((B, 64), dtype=torch.float64, device="cuda")
    nn = torch.empty((B,), **i32)
    names = {E.EAGLE_POLICY_EAGLE2: "eagle2", E.EAGLE_POLICY_NO_RERANK: "no_rerank",
             E.EAGLE_POLICY_CONF: "confidence", E.EAGLE_POLICY_CONF_NO_RERANK: "confidence_no_rerank"}
    for pol, name in names.items():
        p = E.TreeParams(w.depth, w.topk, w.children, w.m, w.chain_k, w.vocab, 64, w.r_max, pol)
        if E.build_tree_workspace_size(p, B) == 0:
            out[name] = None   # the tree does not fit
            continue
        ws = torch.empty(E.build_tree_workspace_size(p, B), dtype=torch.uint8, device="cuda")
        E.workspace_init(ws)

        def call():
            E.build_tree(p, B, S["draft"], kinds, bufs[0], bufs[1], bufs[2], score, bufs[3], nn, ws)

        st = torch.cuda.Stream()
        st.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(st):
            call()
        torch.cuda.current_stream().wait_stream(st)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(10):
                call()
        g.replay()
        n = max(1, reps // 10)
        ea, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        ea.record()
        for _ in range(n):
            g.replay()
        eb.record()
        torch.cuda.synchronize()
        assert E.read_errors(ws) == 0, f"tree policy {name} reported device errors"
        out[name] = {"build_us": round(ea.elapsed_time(eb) * 1e3 / (n * 10), 2),
                     "mean_nodes": round(float(nn.float().mean().item()), 2)}
    return out


def measure_pdraft(E, step, w, S, kinds, reps):
    """eagle_pdraft_prepare after input set 0's step (its accepted paths and
    bonus tokens), outside the step: K = 7 parallel-draft slots, hidden size =
    query heads x head_dim, synthetic target hidden states in the workload
    dtype; HIP events around replays of a graph of 20 calls."""
    import torch
    a = S["attn"]
    step.run(S["draft"], kinds, a.prefix_len, a.q, a.k_draft, a.v_draft, a.k_cache, a.v_cache, a.block_table,
             S["target"], S["words"])
    B, M, MA, K = w.batch, w.m_max, w.max_accept, 7
    H = w.num_q_heads * w.head_dim
    Sl = MA + K
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    th = torch.randn((B, M + 1, H), generator=g, device="cuda").to(w.dtype)
    hs = torch.randn((H,), generator=g, device="cuda").to(w.dtype)
    p = E.PdraftParams(M, MA, K, H, w.vocab, E.dtype_code(w.dtype))
    i32 = dict(dtype=torch.int32, device="cuda")
    ids, pos, src = (torch.empty((B, Sl), **i32) for _ in range(3))
    is_mask = torch.empty((B, Sl), dtype=torch.uint8, device="cuda")
    rej = torch.empty((B, M), dtype=torch.uint8, device="cuda")
    nsl = torch.empty((B,), **i32)
    dh = torch.empty((B, Sl, H), dtype=w.dtype, device="cuda")
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    E.workspace_init(ws)

    def call():
        E.pdraft_prepare(p, B, step.tokens, step.num_nodes, step.accepted, step.accept_len, step.bonus, a.prefix_len,
                         th, hs, ids, pos, src, is_mask, rej, nsl, dh, ws)

    per_graph = 20
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        call()
    torch.cuda.current_stream().wait_stream(st)
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        for _ in range(per_graph):
            call()
    gr.replay()
    n = max(1, reps // per_graph)
    ea, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ea.record()
    for _ in range(n):
        gr.replay()
    eb.record()
    torch.cuda.synchronize()
    us = ea.elapsed_time(eb) * 1e3 / (n * per_graph)
    assert E.read_errors(ws) == 0, "parallel-draft preparation reported device errors"
    esz = th.element_size()
    known = int(step.accept_len.sum().item()) + B
    nbytes = (B * Sl + known + 1) * H * esz   # every slot written; each known row and h_shared read once
    return {"call": "eagle_pdraft_prepare (k_pdraft_prepare)", "k_draft": K, "hidden": H, "slots": B * Sl,
            "avg_us": round(us, 2), "timed_calls": n * per_graph, "algorithmic_bytes": nbytes,
            "hbm_gbs": round(nbytes / (us * 1e-6) / 1e9, 1)}


def measure_expand(E, step, w, S, kinds, reps):
    """The incremental build (eagle_tree_expand per level, then
    eagle_tree_finish) over input set 0's draft rows, outside the step: HIP
    events around replays of a graph of one whole build; per-level figures
    from event-timed eager calls.  Dynamic trees only (None otherwise)."""
    import numpy as np
    import torch

    import synth
    if any(kd != synth.TREE_DYNAMIC for kd in w.kinds):
        return None
    B, k, D = w.batch, w.topk, w.depth
    p = E.TreeParams(D, k, w.children, w.m, 0, w.vocab, w.m_max, w.r_max)
    ws = torch.empty(max(256, E.build_tree_workspace_size(p, B)), dtype=torch.uint8, device="cuda")
    E.workspace_init(ws)
    d = S["draft"]
    levels = [d[:, 0:1].contiguous()] + [d[:, 1 + (l - 1) * k:1 + l * k].contiguous() for l in range(1, D)]
    i32 = dict(dtype=torch.int32, device="cuda")
    ft, fp = torch.empty((B, k), **i32), torch.empty((B, k), **i32)
    fs = torch.empty((B, k), dtype=torch.float64, device="cuda")
    t = {n: torch.empty((B, w.m_max), **i32) for n in ("tokens", "parent", "depth", "src_row")}
    t["score"] = torch.empty((B, w.m_max), dtype=torch.float64, device="cuda")
    t["num_nodes"] = torch.empty((B,), **i32)

    def run(ev=None):
        for lv in range(D):
            E.tree_expand(p, B, lv, levels[lv], ft, fp, fs, ws)
            if ev is not None:
                ev[lv + 1].record()
        E.tree_finish(p, B, t["tokens"], t["parent"], t["depth"], t["score"], t["src_row"], t["num_nodes"], ws)
        if ev is not None:
            ev[D + 1].record()

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    g.replay()
    n = max(1, reps)
    ea, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ea.record()
    for _ in range(n):
        g.replay()
    eb.record()
    torch.cuda.synchronize()
    total_us = ea.elapsed_time(eb) * 1e3 / n
    n_ev = min(n, 50)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(D + 2)] for _ in range(n_ev)]
    for e in evs:
        e[0].record()
        run(e)
    torch.cuda.synchronize()
    per = [float(np.median([e[j].elapsed_time(e[j + 1]) for e in evs])) * 1e3 for j in range(D + 1)]
    # the finished tree is the one-shot build's over the same rows
    step.build(S["draft"], kinds)
    torch.cuda.synchronize()
    for name in ("tokens", "parent", "score", "num_nodes"):
        assert torch.equal(t[name], getattr(step, name)), f"incremental build differs in {name}"
    return {"calls": "eagle_tree_expand x depth + eagle_tree_finish", "levels": D,
            "total_us": round(total_us, 2), "per_level_us": [round(x, 2) for x in per[:D]],
            "finish_us": round(per[D], 2), "timed_builds": n}


def cpu_baseline(w, S, seed, tokens_per_step, budget_s):
    """The oracle as it stands, timed on the host cores on the same inputs
    (host copies of input set 0): full steps until the budget is spent."""
    import numpy as np
    import torch

    import oracle
    import synth

    def h(t):
        t = t.detach().to("cpu").contiguous()
        return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()

    a = S["attn"]
    draft, q, kd, vd = h(S["draft"]), h(a.q), h(a.k_draft), h(a.v_draft)
    kc, vc = h(a.k_cache), h(a.v_cache)
    bt = None if a.block_table is None else h(a.block_table)
    plen = h(a.prefix_len)
    words = None if S["words"] is None else h(S["words"])
    # the oracle's own tree defines the target rows it verifies against
    ot = oracle.build_tree(draft, w.depth, w.topk, w.children, w.m, chain_k=w.chain_k, kinds=w.kinds, m_max=w.m_max)
    target = h(synth.target_logits(w, seed, S["draft"].cpu(), torch.from_numpy(ot["src_row"]),
                                   torch.from_numpy(ot["num_nodes"])))
    n_steps, t0 = 0, time.perf_counter()
    while True:
        t = oracle.build_tree(draft, w.depth, w.topk, w.children, w.m, chain_k=w.chain_k, kinds=w.kinds,
                              m_max=w.m_max)
        anc, pos = oracle.tree_mask(t["parent"], t["num_nodes"], plen)
        oracle.tree_attn(q, kd, vd, kc, vc, bt, plen, anc, t["num_nodes"])
        oracle.accept(w.accept_mode, target, t["tokens"], t["parent"], t["num_nodes"], w.max_accept,
                      rand_words=words, T=w.temperature)
        n_steps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or (n_steps >= 1 and el * (n_steps + 1) / n_steps > 3 * budget_s):
            break
    cpu_model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": round(tokens_per_step * n_steps / el, 2), "unit": "tokens/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"{n_steps} full oracle steps (tree build, mask, fp64 attention over every row, accept) "
                      f"on input set 0 in {el:.1f} s",
            "host_cpu": cpu_model or platform.processor(), "nproc": os.cpu_count()}


if __name__ == "__main__":
    main()
