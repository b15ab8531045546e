#!/usr/bin/env python3
"""Decode-step benchmark of indexer-driven sparse attention on one MI355X.

Workload: decode, 4 sequences x 131072 cached tokens, GQA 32 query / 8 KV
heads, head_dim 128, projected rank r=64, top-B = 2048 per KV head (the
1.5625% budget), bf16 caches, seeded synthetic inputs with 64 planted hot
spans of 32 tokens per KV head.

A step is the whole hot path for all sequences and heads of one layer:
scoring preparation + projected-key scoring (one kernel), exact top-B
selection, indexed attention (+ its split merge). Inputs are resident in HBM
before timing starts. Two identical cache instances are alternated step by
step, so no step finds its 2.5 GiB working set in the 256 MB Infinity Cache.

Prints ONE JSON line on stdout; diagnostics go to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse-attn decode steps/s at 128K,B=2048; indexer keys scored/s; % HBM peak"
HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK = 2.5e15   # dense bf16 MFMA flop/s (MI355X)
WORKLOAD = "decode_t128k_b2048"
SCORE_SOURCES = ["indexer_driven_sparse_amd/csrc/score.hip", "indexer_driven_sparse_amd/csrc/common.hpp"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "score_decode_t128k_pmc.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(launch_bytes: int):
    """HBM bytes per scoring launch from the committed rocprofv3 counter runs,
    or None when they are missing or the kernel changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != source_hash(SCORE_SOURCES):
        return None
    return rec.get("traffic_bytes_per_launch")


def to_dev(a, torch):
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def prefill_leg(torch, lsa, synth, runs: int = 5) -> dict:
    """Causal prefill at L=65536 (1 KV head, 8 query heads, r=64, top-2048):
    the fused indexer (scores + per-row exact top-B) and the sparse
    attention over its indices, each the median of `runs` timed calls with
    inputs resident in HBM; sampled rows checked against the oracle."""
    case = synth.workload("prefill_l64k")
    L, Hkv, B, r = case.L, case.Hkv, case.B, case.r
    qd, kd = to_dev(case.q_idx, torch), to_dev(case.k_idx, torch)
    idx = torch.empty(L, Hkv, B, dtype=torch.int32, device="cuda")
    osc = torch.empty(L, Hkv, B, device="cuda")
    ws = torch.empty(lsa.prefill_score_workspace_bytes_for(L, Hkv, r, B), dtype=torch.uint8,
                     device="cuda")
    stream = torch.cuda.current_stream()

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(runs):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) * 1000.0)
        return float(np.median(ts))

    t_idx = timed(lambda: lsa.lsa_index_score(kd, None, q_idx=qd, mode=lsa.MODE_PREFILL_CAUSAL,
                                              topk=B, out_idx=idx, out_score=osc, workspace=ws))
    pairs = int(np.sum(np.arange(1, L + 1, dtype=np.int64))) * Hkv
    flop = 2.0 * r * pairs
    gi = idx.cpu().numpy()
    del ws
    torch.cuda.empty_cache()
    Q, K, V = to_dev(case.Q, torch), to_dev(case.K, torch), to_dev(case.V, torch)
    out = torch.empty(L, case.Hq, case.d, device="cuda")
    lse = torch.empty(L, case.Hq, device="cuda")
    aws = torch.empty(max(16, lsa.lsa_attention_workspace_bytes(Q, K, V, idx, out, lse=lse,
                                                                mode=lsa.MODE_PREFILL_CAUSAL)),
                      dtype=torch.uint8, device="cuda")
    t_att = timed(lambda: lsa.lsa_indexed_attention(Q, K, V, idx, out, lse=lse,
                                                    mode=lsa.MODE_PREFILL_CAUSAL, workspace=aws))
    sel_pairs = int(np.minimum(np.arange(1, L + 1), B).sum()) * case.Hq
    # parity on sampled rows: the oracle's exact top-B (fp64 scores)
    import oracle
    rows = [0, 2047, 2048, 4096, 32768, L - 1] + list(np.random.default_rng(0).integers(2049, L, 10))
    same, ok = 0, 0
    qf = synth.bf16_bits_to_f32(case.q_idx[:, 0]).astype(np.float64)
    kf = synth.bf16_bits_to_f32(case.k_idx[:, 0]).astype(np.float64)
    for i in map(int, rows):
        ref, _ = oracle.prefill_topk(case.q_idx, case.k_idx, B, row_begin=i, row_end=i + 1)
        rv, gv = ref[0, 0], gi[i, 0]
        if np.array_equal(rv, gv):
            same += 1
            ok += 1
            continue
        # a differing set passes only through near-ties at the B-th score
        s = kf[:i + 1] @ qf[i]
        rsel = rv[rv >= 0]
        s_b = s[rsel].min()
        tol = 1e-4 * max(abs(s_b), float(np.sqrt(np.mean(s ** 2))))
        sym = np.setxor1d(rsel, gv[gv >= 0])
        ok += int(len(rsel) == int((gv >= 0).sum()) and np.all(np.abs(s[sym] - s_b) <= tol))
    log(f"prefill: indexer {t_idx:.1f} us, attention {t_att:.1f} us, oracle rows {same}/{len(rows)} "
        f"identical, {ok}/{len(rows)} within the near-tie tolerance")
    # the oracle's indexer on the host, on a bounded sample: 512 of the
    # longest rows (their causal pairs, exact fp64 scores and top-B)
    threads = len(os.sched_getaffinity(0))
    oracle.set_threads(threads)
    r0 = L - 512
    t0 = time.time()
    oracle.prefill_topk(case.q_idx, case.k_idx, B, row_begin=r0, row_end=L)
    el = time.time() - t0
    cpu_pairs = int(np.sum(np.arange(r0 + 1, L + 1, dtype=np.int64))) * Hkv
    cpu = {"value": cpu_pairs / el, "unit": "causal pairs scored and selected/s", "cores": threads,
           "kind": "oracle", "sample": f"rows {r0}..{L - 1} of the same workload ({cpu_pairs} causal pairs, "
                                        f"fp64) in {el:.2f}s"}
    log(f"prefill oracle: {cpu['value']:.3e} pairs/s on {threads} threads")
    # the same inputs with one selection per block of qb tokens
    del idx, osc, aws
    torch.cuda.empty_cache()
    from indexer_driven_sparse_amd import pipeline
    qb = 64
    plan = pipeline.PrefillPlan(L, case.Hq, Hkv, case.d, r, B, query_block=qb)
    t_bidx = timed(lambda: plan.index(qd, kd))
    t_batt = timed(lambda: plan.attend(Q, K, V))
    log(f"prefill, one selection per {qb} tokens: indexer {t_bidx:.1f} us, attention {t_batt:.1f} us")
    block = {"query_block": qb, "indexer_us": t_bidx, "attention_us": t_batt,
             "index_bytes": (L // qb) * Hkv * B * 4,
             "indexer_flop": 2.0 * r * sum(min(L, (b + 1) * qb) for b in range(L // qb)) * Hkv}
    del plan
    torch.cuda.empty_cache()
    return {"workload": "causal prefill, L=65536, 1 KV head / 8 query heads, d=128, r=64, "
                        "top-2048 per row, bf16, sinusoidal position component",
            "indexer_us": t_idx, "indexer_causal_pairs": pairs, "indexer_flop": flop,
            "indexer_mfma_frac": flop / (t_idx * 1e-6) / MFMA_BF16_PEAK,
            "indexer_mfma_peak_tflops": MFMA_BF16_PEAK / 1e12,
            "attention_us": t_att, "attention_selected_pairs": sel_pairs,
            "attention_tflops": sel_pairs * 4.0 * case.d / (t_att * 1e-6) / 1e12,
            # each selected (row, key) gathers one K and one V row of d bf16
            "attention_gather_GBps": sel_pairs // (case.Hq // Hkv) * 2 * case.d * 2 / (t_att * 1e-6) / 1e9,
            "indexer_pairs_per_s": pairs / (t_idx * 1e-6),
            "parity_rows_identical": same, "parity_rows": len(rows),
            "parity_pass": ok == len(rows), "block_shared": block, "cpu_baseline": cpu}


def fp8_leg(torch, lsa, pipeline, case, inst, Q, W, steps: int, warmup: int) -> dict:
    """The headline decode step over an OCP E4M3 projected-key cache (JSSA
    Fig. 10 studies FP8 scoring caches): the same K/V, B and shapes, half
    the scoring bytes. Two cache instances alternate as in the main leg;
    sampled rows are checked against the oracle."""
    N, Hq, Hkv, T, d, r, B = case.N, case.Hq, case.Hkv, case.T, case.d, case.r, case.B
    caches = []
    for K, V, _ in inst:
        k8 = torch.empty(N, Hkv, T, r, dtype=torch.float8_e4m3fn, device="cuda")
        lsa.lsa_project_keys(K, W, k8)
        caches.append((K, V, k8))
    plan = pipeline.DecodePlan(N, Hq, Hkv, T, d, r, B, kidx_dtype=torch.float8_e4m3fn)
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        K, V, k8 = caches[i & 1]
        plan.run(Q, W, k8, K, V)
    torch.cuda.synchronize()
    sampled = set(range(0, steps, 8))
    ev = {i: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for i in sampled}
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for i in range(steps):
        K, V, k8 = caches[i & 1]
        if i in ev:
            ev[i][0].record(stream)
        plan.score(Q, W, k8)
        if i in ev:
            ev[i][1].record(stream)
        plan.select()
        plan.attend(Q, K, V)
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    score_ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in ev.values()]))
    kbytes = N * Hkv * T * r
    step_bytes = kbytes + N * Hkv * B * 2 * d * 2 + N * Hkv * B * 4 + N * Hq * d * 6 + N * Hkv * r * 4
    # parity on sampled rows: the oracle projects those heads to E4M3 itself
    import oracle
    K0, V0, k80 = caches[0]
    plan.run(Q, W, k80, K0, V0)
    torch.cuda.synchronize()
    gidx = plan.idx.cpu().numpy()
    same = 0
    rows = [0, 13, 31]
    for row in rows:
        n, g = divmod(row, Hkv)
        K1, V1 = case.K[n:n + 1, :, g:g + 1], case.V[n:n + 1, :, g:g + 1]
        Q1 = case.Q[n:n + 1, g * case.G:(g + 1) * case.G]
        k1 = oracle.project_keys(K1, case.W, oracle.FP8)
        ref = oracle.decode_step(Q1, case.W, k1, K1, V1, B)
        same += int(np.array_equal(ref["idx"][0, 0], gidx[n, g]))
    log(f"fp8 cache: {ms * 1000:.1f} us/step, scoring {score_ms * 1000:.1f} us, "
        f"oracle rows identical {same}/{len(rows)}")
    return {"workload": "the headline decode step with an OCP E4M3 projected-key cache",
            "ms_per_step": ms, "steps_per_s": 1000.0 / ms,
            "hbm_frac_end_to_end": step_bytes / (ms * 1e-3) / (HBM_PEAK_GBPS * 1e9),
            "algorithmic_bytes_per_step": step_bytes,
            "score_kernel": {"avg_launch_us": score_ms * 1000.0, "bytes_per_launch": kbytes,
                             "achieved_GBps": kbytes / (score_ms * 1e-3) / 1e9},
            "parity_rows_identical": same, "parity_rows": len(rows)}


def _time_us(torch, fn, n: int, warm: int = 10) -> float:
    stream = torch.cuda.current_stream()
    for i in range(warm):
        fn(i)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for i in range(n):
        fn(i)
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / n * 1000.0


def _cold_us(torch, fn, n: int, sweep_mib: int = 512) -> float:
    """Median per-step time with the caches flushed before each step: a
    sweep_mib read-modify-write of a scratch buffer (outside the events)
    evicts the step's inputs from the 256 MB MALL and the L2s."""
    stream = torch.cuda.current_stream()
    scratch = torch.zeros(sweep_mib * (1 << 20) // 4, dtype=torch.float32, device="cuda")
    fn(0)
    ts = []
    for i in range(n):
        scratch.add_(1.0)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn(i)
        b.record(stream)
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b) * 1000.0)
    del scratch
    return float(np.median(ts))


def read_ceiling_leg(torch, lsa, mib: int = 1024, reps: int = 20) -> dict:
    """The achievable streaming-read rate for scale: lsa_stream_read over one
    of two alternating mib-MiB buffers (neither fits the MALL), 16-byte
    nontemporal loads like the scoring stream."""
    n = mib * (1 << 20) // 4
    bufs = [torch.ones(n, dtype=torch.int32, device="cuda") for _ in range(2)]
    sink = torch.zeros(lsa.STREAM_READ_SINK_WORDS, dtype=torch.int32, device="cuda")
    us = _time_us(torch, lambda i: lsa.lsa_stream_read(bufs[i & 1], sink), reps, warm=4)
    del bufs
    torch.cuda.empty_cache()
    gbps = n * 4 / (us * 1e-6) / 1e9
    log(f"read ceiling (lsa_stream_read over {mib} MiB): {gbps:.0f} GB/s")
    return {"kernel": f"lsa_stream_read over {mib} MiB", "GBps": gbps,
            "frac_of_peak": gbps / HBM_PEAK_GBPS}


def hitters_leg(torch, lsa, synth, pipeline, n_warm: int = 1000, n_cold: int = 50) -> dict:
    """The 32K heavy-hitter decode step (1 sequence, GQA 32/8, 1% planted
    positions per KV head, top-1024): warm (back-to-back, its 38 MB working
    set resident in the MALL) and cold (caches flushed before each step);
    every row's set checked against the oracle."""
    case = synth.workload("decode_t32k_hitters")
    N, Hq, Hkv, T, d, r, B = case.N, case.Hq, case.Hkv, case.T, case.d, case.r, case.B
    Q, W = to_dev(case.Q, torch), to_dev(case.W, torch)
    K, V = to_dev(case.K, torch), to_dev(case.V, torch)
    k_idx = torch.empty(N, Hkv, T, r, dtype=torch.bfloat16, device="cuda")
    lsa.lsa_project_keys(K, W, k_idx)
    plan = pipeline.DecodePlan(N, Hq, Hkv, T, d, r, B)
    warm = _time_us(torch, lambda i: plan.run(Q, W, k_idx, K, V), n_warm, warm=50)
    cold = _cold_us(torch, lambda i: plan.run(Q, W, k_idx, K, V), n_cold)
    plan.run(Q, W, k_idx, K, V)
    torch.cuda.synchronize()
    gidx, gout = plan.idx.cpu().numpy(), plan.out.cpu().numpy()
    import oracle
    ref_k = oracle.project_keys(case.K, case.W, oracle.BF16)
    ref = oracle.decode_step(case.Q, case.W, ref_k, case.K, case.V, B)
    same = int(sum(np.array_equal(gidx[0, g], ref["idx"][0, g]) for g in range(Hkv)))
    err = float(np.abs(gout - ref["out"]).max())
    alg = N * Hkv * T * r * 2 + N * Hkv * B * 2 * d * 2 + N * Hkv * B * 4 + N * Hq * d * 6 + N * Hkv * r * 4
    log(f"heavy hitters 32K: warm {warm:.1f} us/step, cold {cold:.1f} us/step, "
        f"oracle rows identical {same}/{Hkv}, max |out err| {err:.2e}")
    return {"workload": "decode, 1 sequence x 32768 cached tokens, GQA 32/8, d=128, r=64, top-1024, "
                        "bf16, 1% planted heavy hitters per KV head",
            "warm_us_per_step": warm, "cold_us_per_step": cold,
            "warm_steps_per_s": 1e6 / warm, "cold_steps_per_s": 1e6 / cold,
            "algorithmic_bytes_per_step": alg,
            "cold_hbm_frac": alg / (cold * 1e-6) / (HBM_PEAK_GBPS * 1e9),
            "parity_rows_identical": same, "parity_rows": Hkv, "max_abs_out_err": err,
            "parity_pass": same == Hkv and err <= 2e-3}


def paged_leg(torch, plan, case, inst, Q, n: int = 200) -> dict:
    """Indexed attention of the headline step through a page-size-1 KV pool
    (the serving layout of LSA-L's configs): every cached row of every
    sequence is scattered into one pool, once in sequence order (identity
    table: the translation's own cost) and once in random order (no DRAM
    locality left between neighbouring positions). Outputs must equal the
    unpaged attention bit for bit."""
    N, Hkv, T, d = case.N, case.Hkv, case.T, case.d
    K, V, _ = inst[0]
    unpaged = _time_us(torch, lambda i: plan.attend(Q, inst[i & 1][0], inst[i & 1][1]), n)
    plan.attend(Q, K, V)
    ref = plan.out.clone()
    res = {"workload": "attention of the headline step, K/V read through a slot table from a "
                       f"pool of {N * T} rows",
           "unpaged_us": unpaged}
    g = torch.Generator().manual_seed(5)
    for kind, rows in (("identity", torch.arange(N * T, dtype=torch.int32)),
                       ("random", torch.randperm(N * T, generator=g).to(torch.int32))):
        rows = rows.cuda()
        pools = []
        for Ki, Vi, _ in inst:
            Kp = torch.empty(N * T, Hkv, d, dtype=Ki.dtype, device="cuda")
            Vp = torch.empty_like(Kp)
            Kp[rows.long()] = Ki.reshape(N * T, Hkv, d)
            Vp[rows.long()] = Vi.reshape(N * T, Hkv, d)
            pools.append((Kp, Vp))
        table = rows.view(N, T)
        us = _time_us(torch, lambda i: plan.attend(Q, pools[i & 1][0], pools[i & 1][1],
                                                   slot_table=table), n)
        plan.attend(Q, pools[0][0], pools[0][1], slot_table=table)
        torch.cuda.synchronize()
        same = bool(torch.equal(plan.out.view(torch.int32), ref.view(torch.int32)))
        res[f"{kind}_table_us"] = us
        res[f"{kind}_equals_unpaged"] = same
        log(f"paged attention ({kind} table): {us:.1f} us vs unpaged {unpaged:.1f} us; "
            f"bit-identical: {same}")
        del pools
    return res


def cross_layer_leg(torch, lsa, pipeline, case, inst, Q, W, steps: int,
                    pattern: str = "FSSS") -> dict:
    """Cross-layer index reuse on a stack of layers of the headline shape:
    the first layer of `pattern` runs the indexer and attention, the shared
    ones attention only on its top-B sets. Every layer has its own caches
    (distinct memory), timed against the same stack with every layer full."""
    N, Hq, Hkv, T, d, r, B = case.N, case.Hq, case.Hkv, case.T, case.d, case.r, case.B
    layers = [(K, V, k) for K, V, k in inst]
    while len(layers) < len(pattern):
        K, V = to_dev(case.K, torch), to_dev(case.V, torch)
        k_idx = torch.empty(N, Hkv, T, r, dtype=torch.bfloat16, device="cuda")
        lsa.lsa_project_keys(K, W, k_idx)
        layers.append((K, V, k_idx))
    args = [(Q, W, k, K, V) for K, V, k in layers[:len(pattern)]]
    res = {"workload": f"{len(pattern)} decode layers of the headline shape, pattern {pattern} "
                       "(F: own indexer, S: reuses the nearest full layer's top-B)"}
    for pat in ("F" * len(pattern), pattern):
        plan = pipeline.CrossLayerPlan(pat, N, Hq, Hkv, T, d, r, B)
        us = _time_us(torch, lambda i: plan.run(args), max(20, steps // 4))
        res["all_full_us" if pat.count("S") == 0 else "reuse_us"] = us
        del plan
    res["speedup"] = res["all_full_us"] / res["reuse_us"]
    log(f"cross-layer {pattern}: {res['reuse_us']:.1f} us per {len(pattern)} layers vs "
        f"{res['all_full_us']:.1f} us all full ({res['speedup']:.2f}x)")
    return res


def hierarchical_leg(torch, lsa, synth, pipeline, steps: int = 200) -> dict:
    """Coarse-to-fine decode at T = 1048576 (1 sequence, GQA 32/8, block 64,
    top-128 blocks, top-2048): warm back-to-back steps (centroid scores,
    block select, candidate scores, token select, attention), and cold steps
    with the caches flushed before each."""
    case = synth.workload("hier_t1m")
    N, Hq, Hkv, T, d, r, B = case.N, case.Hq, case.Hkv, case.T, case.d, case.r, case.B
    blk, Bc = case.block, case.B_coarse
    Q, W = to_dev(case.Q, torch), to_dev(case.W, torch)
    K, V = to_dev(case.K, torch), to_dev(case.V, torch)
    k_idx = torch.empty(N, Hkv, T, r, dtype=torch.bfloat16, device="cuda")
    lsa.lsa_project_keys(K, W, k_idx)
    cent = torch.empty(N, Hkv, T // blk, r, dtype=torch.bfloat16, device="cuda")
    lsa.lsa_build_centroids(k_idx, blk, cent)
    plan = pipeline.HierarchicalPlan(N, Hq, Hkv, T, d, r, B, blk, Bc)
    stream = torch.cuda.current_stream()
    for _ in range(20):
        plan.run(Q, W, k_idx, cent, K, V)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(steps):
        plan.run(Q, W, k_idx, cent, K, V)
    b.record(stream)
    torch.cuda.synchronize()
    us = a.elapsed_time(b) / steps * 1000.0
    cold = _cold_us(torch, lambda i: plan.run(Q, W, k_idx, cent, K, V), 50)
    nb = T // blk
    alg = (N * Hkv * nb * r * 2 + N * Hkv * Bc * blk * r * 2 + N * Hkv * B * 2 * d * 2
           + N * Hkv * (Bc + B) * 4 + N * Hq * d * (2 + 4))
    # planted tokens kept: coarse-to-fine is an approximation -- a span that
    # only grazes a 64-token block barely moves that block's centroid
    sel = plan.idx[0].cpu().numpy()
    hit = sum(int(np.isin(case.planted[g], sel[g]).sum()) for g in range(Hkv))
    tot = sum(len(case.planted[g]) for g in range(Hkv))
    log(f"hierarchical: {us:.1f} us/step warm, {cold:.1f} us/step cold, planted tokens kept {hit}/{tot}")
    return {"workload": "hierarchical decode, 1 sequence x 1048576 tokens, GQA 32/8, d=128, r=64, "
                        "block 64, top-128 blocks, top-2048, bf16, hot spans",
            "us_per_step": us, "steps_per_s": 1e6 / us, "algorithmic_bytes_per_step": alg,
            "hbm_frac": alg / (us * 1e-6) / (HBM_PEAK_GBPS * 1e9),
            "cold_us_per_step": cold, "cold_hbm_frac": alg / (cold * 1e-6) / (HBM_PEAK_GBPS * 1e9),
            "planted_tokens_kept": hit, "planted_tokens": tot}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="wall time budget of the CPU-oracle baseline (0 disables it)")
    ap.add_argument("--no-stages", action="store_true", help="skip the per-stage timing loops")
    ap.add_argument("--no-fp8", action="store_true",
                    help="skip the same decode step over an OCP E4M3 projected-key cache")
    ap.add_argument("--no-hierarchical", action="store_true",
                    help="skip the coarse-to-fine decode leg (T=1048576)")
    ap.add_argument("--no-paged", action="store_true",
                    help="skip the page-size-1 pool attention leg")
    ap.add_argument("--no-cross-layer", action="store_true",
                    help="skip the cross-layer index reuse leg")
    ap.add_argument("--no-hitters", action="store_true",
                    help="skip the 32K heavy-hitter decode leg (warm and cold)")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the causal prefill leg (L=65536 fused indexer + sparse attention)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="finish with three plain device copies of MIB MiB: the reference for "
                         "scaling rocprofv3's FETCH_SIZE / WRITE_SIZE counters to bytes")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the decode path shards "
              "by KV head or sequence with no collective inside the step.", file=sys.stderr)
        return 2

    import torch
    from indexer_driven_sparse_amd import lsa, pipeline, synth

    if not torch.cuda.is_available():
        log("no GPU")
        return 1
    dev_name = torch.cuda.get_device_name(0)
    log(f"device: {dev_name}; library: {lsa.library_path()}")

    t0 = time.time()
    case = synth.workload(WORKLOAD)
    log(f"generated inputs in {time.time() - t0:.1f}s")
    # the record names its inputs: generator seed and a SHA-256 per array
    inputs = {"generator": f"indexer_driven_sparse_amd.synth.workload({WORKLOAD!r})",
              "seed": case.seed, "sha256": {k: hashlib.sha256(np.ascontiguousarray(getattr(case, k)).data).hexdigest()
                                    for k in ("Q", "K", "V", "W")}}
    N, Hq, Hkv, T, d, r, B = case.N, case.Hq, case.Hkv, case.T, case.d, case.r, case.B

    # two cache instances resident in HBM (identical content, distinct memory)
    Q, W = to_dev(case.Q, torch), to_dev(case.W, torch)
    inst = []
    for _ in range(2):
        K, V = to_dev(case.K, torch), to_dev(case.V, torch)
        k_idx = torch.empty(N, Hkv, T, r, dtype=torch.bfloat16, device="cuda")
        lsa.lsa_project_keys(K, W, k_idx)
        inst.append((K, V, k_idx))
    torch.cuda.synchronize()
    plan = pipeline.DecodePlan(N, Hq, Hkv, T, d, r, B)
    stream = torch.cuda.current_stream()

    def step(i):
        K, V, k_idx = inst[i & 1]
        plan.run(Q, W, k_idx, K, V)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed region: K steps; HIP events on the launch stream bracket the
    # scoring launch of every 8th step (an event pair between two kernels
    # costs a few microseconds, so timing every step would slow the step)
    steps = args.steps
    sampled = list(range(0, steps, 8))
    ev_s = {i: torch.cuda.Event(enable_timing=True) for i in sampled}
    ev_e = {i: torch.cuda.Event(enable_timing=True) for i in sampled}
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(steps):
        K, V, k_idx = inst[i & 1]
        if i in ev_s:
            ev_s[i].record(stream)
        plan.score(Q, W, k_idx)
        if i in ev_e:
            ev_e[i].record(stream)
        plan.select()
        plan.attend(Q, K, V)
    end.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / steps
    score_ms = float(np.mean([ev_s[i].elapsed_time(ev_e[i]) for i in sampled]))

    keys = N * Hkv * T
    kidx_bytes = keys * r * 2
    sel_kv_bytes = N * Hkv * B * 2 * d * 2
    step_bytes = kidx_bytes + sel_kv_bytes + N * Hkv * B * 4 + (N * Hq * d * 2 + N * Hq * d * 4 +
                                                                 N * Hkv * r * 4)
    steps_per_s = 1000.0 / ms_per_step
    score_gbps = kidx_bytes / (score_ms * 1e-3) / 1e9

    # the same steps replayed from HIP graphs (one per cache instance): the
    # whole step's launches are submitted at once
    graphs = []
    for k in range(2):
        K_, V_, kidx_ = inst[k]
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            plan.run(Q, W, kidx_, K_, V_)
        graphs.append(g)
    for i in range(args.warmup):
        graphs[i & 1].replay()
    torch.cuda.synchronize()
    ga, gb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ga.record(stream)
    for i in range(steps):
        graphs[i & 1].replay()
    gb.record(stream)
    torch.cuda.synchronize()
    graph_ms = ga.elapsed_time(gb) / steps
    log(f"eager {ms_per_step * 1000:.1f} us/step, graph replay {graph_ms * 1000:.1f} us/step")

    fp8 = None
    if not args.no_fp8:
        fp8 = fp8_leg(torch, lsa, pipeline, case, inst, Q, W, steps, args.warmup)

    paged = None if args.no_paged else paged_leg(torch, plan, case, inst, Q)
    torch.cuda.empty_cache()
    cross = None
    if not args.no_cross_layer:
        cross = cross_layer_leg(torch, lsa, pipeline, case, inst, Q, W, steps)
        torch.cuda.empty_cache()

    stages = None
    if not args.no_stages:
        def time_loop(fn, n=100):
            for i in range(10):
                fn(i)
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for i in range(n):
                fn(i)
            b.record(stream)
            torch.cuda.synchronize()
            return a.elapsed_time(b) / n * 1000.0

        stages = {
            "score_us": time_loop(lambda i: plan.score(Q, W, inst[i & 1][2])),
            "select_us": time_loop(lambda i: plan.select()),
            "attention_us": time_loop(lambda i: plan.attend(Q, inst[i & 1][0], inst[i & 1][1])),
        }
        stages["attended_kv_GBps"] = sel_kv_bytes / (stages["attention_us"] * 1e-6) / 1e9

    # the step's outputs on instance 0, for the parity check in the CPU leg
    step(0)
    torch.cuda.synchronize()
    gpu_idx = plan.idx.cpu().numpy()
    gpu_out = plan.out.cpu().numpy()

    cpu = None
    parity = None
    if args.cpu_seconds > 0:
        import oracle
        threads = len(os.sched_getaffinity(0))
        oracle.set_threads(threads)
        ref_k = oracle.project_keys(case.K, case.W, oracle.BF16)        # setup, untimed
        t0 = time.time()
        n_done = 0
        ref = None
        while n_done == 0 or time.time() - t0 < args.cpu_seconds:
            ref = oracle.decode_step(case.Q, case.W, ref_k, case.K, case.V, B)
            n_done += 1
        el = time.time() - t0
        cpu = {"value": n_done / el, "unit": "steps/s", "cores": threads, "kind": "oracle",
               "sample": f"{n_done} full steps of the same workload (all 32 sequence x KV-head rows, "
                         f"fp64) in {el:.1f}s on {platform.processor() or platform.machine()}",
               "keys_scored_per_s": n_done * keys / el}
        # parity of the timed configuration against the oracle
        same = int(sum(np.array_equal(gpu_idx[n, g], ref["idx"][n, g])
                       for n in range(N) for g in range(Hkv)))
        err = float(np.abs(gpu_out - ref["out"]).max()) if same == N * Hkv else None
        parity = {"rows_identical_sets": same, "rows": N * Hkv, "max_abs_out_err": err,
                  "pass": same == N * Hkv and err is not None and err <= 2e-3}
        log(f"cpu oracle: {cpu['value']:.3f} steps/s on {threads} threads; parity {parity}")

    if args.copy_calibration > 0:
        n_el = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n_el, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: 3 copies of {n_el * 4} bytes")
        del src, dst

    prefill = None
    hier = None
    hitters = None
    ceiling = None
    if not (args.no_prefill and args.no_hierarchical and args.no_hitters and args.no_stages):
        del inst, plan
        torch.cuda.empty_cache()
    if not args.no_stages:
        ceiling = read_ceiling_leg(torch, lsa)
    if not args.no_hitters:
        hitters = hitters_leg(torch, lsa, synth, pipeline)
        torch.cuda.empty_cache()
    if not args.no_hierarchical:
        hier = hierarchical_leg(torch, lsa, synth, pipeline)
        torch.cuda.empty_cache()
    if not args.no_prefill:
        prefill = prefill_leg(torch, lsa, synth)

    traffic = measured_traffic(kidx_bytes)
    line = {
        "metric": METRIC,
        "value": steps_per_s,
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "decode, 4 sequences x 131072 cached tokens, GQA 32/8, d=128, "
                               "r=64, top-B=2048, bf16, 64 hot spans of 32 tokens per KV head",
                   "N": N, "T": T, "Hq": Hq, "Hkv": Hkv, "d": d, "r": r, "B": B,
                   "parallelism": "single GPU"},
        "keys_scored_per_s": keys * steps_per_s,
        "hbm_frac_end_to_end": step_bytes / (ms_per_step * 1e-3) / (HBM_PEAK_GBPS * 1e9),
        "algorithmic_bytes_per_step": step_bytes,
        "roofline": {"kernel": "score_decode_kernel (scoring prep + projected-key scoring)",
                     "bound": "hbm", "achieved": score_gbps, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": score_gbps / HBM_PEAK_GBPS,
                     "avg_launch_us": score_ms * 1000.0,
                     "traffic": traffic},
        "graph_replay": {"ms_per_step": graph_ms, "steps_per_s": 1000.0 / graph_ms,
                         "hbm_frac_end_to_end": step_bytes / (graph_ms * 1e-3) / (HBM_PEAK_GBPS * 1e9)},
        "stages": stages,
        "read_ceiling": ceiling,
        "heavy_hitters_32k": hitters,
        "fp8_cache": fp8,
        "paged_kv": paged,
        "cross_layer": cross,
        "hierarchical": hier,
        "prefill": prefill,
        "cpu_baseline": cpu,
        "parity": parity,
        "inputs": inputs,
        "device": dev_name,
        "rocm": getattr(torch.version, "hip", None),
        "host_cpu": platform.processor() or platform.machine(),
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
