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
SCORE_SOURCES = ["indexer_driven_sparse_amd/csrc/score.hip", "indexer_driven_sparse_amd/csrc/score_body.hpp",
                 "indexer_driven_sparse_amd/csrc/common.hpp"]
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


MFMA_FILE = os.path.join(ROOT, "profiles", "prefill_l64k_mfma_util.json")
PREFILL_SOURCES = ["indexer_driven_sparse_amd/csrc/prefill.hip", "indexer_driven_sparse_amd/csrc/common.hpp"]


def measured_mfma_util():
    """rocprofv3's MfmaUtil of the prefill indexer's kernels from the
    committed counter run, or None when it is missing or the kernels changed
    since."""
    try:
        with open(MFMA_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != source_hash(PREFILL_SOURCES):
        return None
    return rec.get("mfma_util")


def to_dev(a, torch):
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def prefill_leg(torch, lsa, synth, runs: int = 5) -> dict:
    """Causal prefill at L=65536 (1 KV head, 8 query heads, r=64, top-2048):
    the fused indexer (scores + per-row exact top-B; timed without and with
    the optional per-entry scores) and the sparse attention over its
    indices, each the median of `runs` timed calls with inputs resident in
    HBM; sampled rows of both checked against the oracle."""
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

    t_idx_sc = timed(lambda: lsa.lsa_index_score(kd, None, q_idx=qd, mode=lsa.MODE_PREFILL_CAUSAL,
                                                 topk=B, out_idx=idx, out_score=osc, workspace=ws))
    t_idx = timed(lambda: lsa.lsa_index_score(kd, None, q_idx=qd, mode=lsa.MODE_PREFILL_CAUSAL,
                                              topk=B, out_idx=idx, workspace=ws))
    pairs = int(np.sum(np.arange(1, L + 1, dtype=np.int64))) * Hkv
    flop = 2.0 * r * pairs
    gi = idx.cpu().numpy()
    del ws, osc
    torch.cuda.empty_cache()
    Q, K, V = to_dev(case.Q, torch), to_dev(case.K, torch), to_dev(case.V, torch)
    out = torch.empty(L, case.Hq, case.d, device="cuda")
    lse = torch.empty(L, case.Hq, device="cuda")
    aws = torch.empty(max(16, lsa.lsa_attention_workspace_bytes(Q, K, V, idx, out, lse=lse,
                                                                mode=lsa.MODE_PREFILL_CAUSAL)),
                      dtype=torch.uint8, device="cuda")
    t_att = timed(lambda: lsa.lsa_indexed_attention(Q, K, V, idx, out, lse=lse,
                                                    mode=lsa.MODE_PREFILL_CAUSAL, workspace=aws))
    torch.cuda.synchronize()
    go, gl = out.cpu().numpy(), lse.cpu().numpy()
    sel_pairs = int(np.minimum(np.arange(1, L + 1), B).sum()) * case.Hq
    par = oracle_parity_prefill(case, gi, go, gl)
    log(f"prefill: indexer {t_idx:.1f} us ({t_idx_sc:.1f} us with per-entry scores), "
        f"attention {t_att:.1f} us, parity {par}")
    cpu = oracle_baseline_prefill(case)
    # the same inputs with one selection per block of qb tokens
    del idx, aws
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
    ok = par["pass"]
    return {"workload": "causal prefill, L=65536, 1 KV head / 8 query heads, d=128, r=64, "
                        "top-2048 per row, bf16, sinusoidal position component",
            "indexer_us": t_idx if ok else None, "indexer_with_entry_scores_us": t_idx_sc if ok else None,
            "indexer_causal_pairs": pairs, "indexer_flop": flop,
            "indexer_mfma_frac": flop / (t_idx * 1e-6) / MFMA_BF16_PEAK if ok else None,
            "indexer_mfma_peak_tflops": MFMA_BF16_PEAK / 1e12,
            "indexer_mfma_util_counter": measured_mfma_util(),
            "attention_us": t_att if ok else None, "attention_selected_pairs": sel_pairs,
            "attention_tflops": sel_pairs * 4.0 * case.d / (t_att * 1e-6) / 1e12 if ok else None,
            # each selected (row, key) gathers one K and one V row of d bf16
            "attention_gather_GBps": (sel_pairs // (case.Hq // Hkv) * 2 * case.d * 2 / (t_att * 1e-6) / 1e9
                                      if ok else None),
            "indexer_pairs_per_s": pairs / (t_idx * 1e-6) if ok else None,
            "parity": par, "block_shared": block, "cpu_baseline": cpu}


# ---------------------------------------------------------------------------
# oracle legs: same-run parity of every timed configuration, and the CPU
# baseline (the oracle is test infrastructure; only these legs call it)
# ---------------------------------------------------------------------------

def _near_tie_sets(gpu_rows, ref_rows, score_rows):
    """Index sets [rows, B] (ascending, -1 padded) against the oracle's:
    identical, or differing only at positions whose oracle score lies within
    1e-4 * max(|s_B|, rms of the row) of the oracle's B-th score. Returns
    (identical rows, rows passing through near-ties, rows failing)."""
    same, tie, bad = 0, [], []
    for i, (g, r) in enumerate(zip(gpu_rows, ref_rows)):
        gv, rv = g[g >= 0], r[r >= 0]
        if np.array_equal(g, r):
            same += 1
            continue
        sc = score_rows[i]
        ok = len(gv) == len(rv) and (g[len(gv):] == -1).all() and np.all(np.diff(gv) > 0)
        if ok:
            s_b = np.min(sc[rv])
            tol = 1e-4 * max(abs(s_b), float(np.sqrt(np.mean(sc[np.isfinite(sc)] ** 2))))
            ok = bool(np.all(np.abs(sc[np.setxor1d(gv, rv)] - s_b) <= tol))
        (tie if ok else bad).append(i)
    return same, tie, bad


def oracle_parity_decode(case, ref_k, gidx, gout, glse, attn_tol: float = 2e-3) -> dict:
    """Every (sequence, KV head) row of a flat decode step: index set against
    the oracle's exact top-B, then output and lse against the oracle's
    attention over the GPU's own set (the set is checked first)."""
    import oracle
    N, Hkv, B = case.N, case.Hkv, case.B
    ref = oracle.decode_step(case.Q, case.W, ref_k, case.K, case.V, B)
    same, tie, bad = _near_tie_sets(gidx.reshape(N * Hkv, B), ref["idx"].reshape(N * Hkv, B),
                                    list(ref["scores"].reshape(N * Hkv, -1)))
    if tie:
        o, l = oracle.attention(case.Q, case.K, case.V, gidx)
    else:
        o, l = ref["out"], ref["lse"]
    err = float(np.abs(gout - o).max())
    lerr = float(np.abs(glse - l).max())
    return {"rows": N * Hkv, "rows_identical_sets": same, "rows_near_tie_sets": len(tie),
            "rows_failing_sets": len(bad), "max_abs_out_err": err, "max_abs_lse_err": lerr,
            "pass": not bad and err <= attn_tol and lerr <= attn_tol}


def oracle_parity_fp8(case, gidx, gout) -> dict:
    """The E4M3-cache step: the oracle rounds the projected keys to E4M3
    itself, then scores, selects and attends (every row)."""
    import oracle
    ref_k = oracle.project_keys(case.K, case.W, oracle.FP8)
    ref = oracle.decode_step(case.Q, case.W, ref_k, case.K, case.V, case.B)
    N, Hkv, B = case.N, case.Hkv, case.B
    same, tie, bad = _near_tie_sets(gidx.reshape(N * Hkv, B), ref["idx"].reshape(N * Hkv, B),
                                    list(ref["scores"].reshape(N * Hkv, -1)))
    o = oracle.attention(case.Q, case.K, case.V, gidx)[0] if tie else ref["out"]
    err = float(np.abs(gout - o).max())
    return {"rows": N * Hkv, "rows_identical_sets": same, "rows_near_tie_sets": len(tie),
            "rows_failing_sets": len(bad), "max_abs_out_err": err,
            "pass": not bad and err <= 2e-3}


def oracle_parity_prefill(case, gi, go, gl, n_rows: int = 16, n_tokens: int = 16) -> dict:
    """Sampled rows of the L=65536 prefill: the fused indexer's sets against
    the oracle's exact causal top-B, and the per-token attention over the
    GPU's own lists against the oracle's (the cache cut at the token, so
    positions after it are masked)."""
    import oracle
    L, B = case.L, case.B
    rng = np.random.default_rng(0)
    rows = sorted({i for i in [0, 2047, 2048, 4096, 32768, L - 1] if i < L}
                  | {int(x) for x in rng.integers(1, L, n_rows - 6)})
    qf = case.q_idx[:, 0].astype(np.uint32) << 16
    kf = case.k_idx[:, 0].astype(np.uint32) << 16
    qf, kf = qf.view(np.float32).astype(np.float64), kf.view(np.float32).astype(np.float64)
    same, ties, bad = 0, 0, 0
    for i in rows:
        ref, _ = oracle.prefill_topk(case.q_idx, case.k_idx, B, row_begin=i, row_end=i + 1)
        s_full = np.full(L, -np.inf)
        s_full[:i + 1] = kf[:i + 1] @ qf[i]
        a, t, b = _near_tie_sets(gi[i:i + 1, 0], ref[:, 0], [s_full])
        same, ties, bad = same + a, ties + len(t), bad + len(b)
    toks = sorted({i for i in [0, 1, 2047, 2048, 32767, L - 1] if i < L}
                  | {int(x) for x in rng.integers(2, L - 1, n_tokens - 6)})
    err, lerr = 0.0, 0.0
    for i in toks:
        o, l = oracle.attention(case.Q[i:i + 1], case.K[:, :i + 1], case.V[:, :i + 1], gi[i:i + 1])
        err = max(err, float(np.abs(go[i] - o[0]).max()))
        lerr = max(lerr, float(np.abs(gl[i] - l[0]).max()))
    return {"indexer_rows": len(rows), "indexer_rows_identical": same, "indexer_rows_near_tie": ties,
            "indexer_rows_failing": bad, "attention_tokens": len(toks),
            "attention_max_abs_out_err": err, "attention_max_abs_lse_err": lerr,
            "pass": bad == 0 and err <= 2e-3 and lerr <= 2e-3}


def oracle_baseline_prefill(case) -> dict:
    """The oracle's indexer on the host, on a bounded sample: the 512
    longest rows (their causal pairs, exact fp64 scores and top-B)."""
    import oracle
    L, Hkv, B = case.L, case.Hkv, case.B
    threads = len(os.sched_getaffinity(0))
    oracle.set_threads(threads)
    r0 = L - 512
    t0 = time.time()
    oracle.prefill_topk(case.q_idx, case.k_idx, B, row_begin=r0, row_end=L)
    el = time.time() - t0
    cpu_pairs = int(np.sum(np.arange(r0 + 1, L + 1, dtype=np.int64))) * Hkv
    log(f"prefill oracle: {cpu_pairs / el:.3e} pairs/s on {threads} threads")
    return {"value": cpu_pairs / el, "unit": "causal pairs scored and selected/s", "cores": threads,
            "kind": "oracle", "sample": f"rows {r0}..{L - 1} of the same workload ({cpu_pairs} causal "
                                        f"pairs, fp64) in {el:.2f}s"}


def fp8_leg(torch, lsa, pipeline, case, inst, Q, W, steps: int, warmup: int) -> dict:
    """The headline decode step over an OCP E4M3 projected-key cache (JSSA
    Fig. 10 studies FP8 scoring caches): the same K/V, B and shapes, half
    the scoring bytes. Two cache instances alternate as in the main leg;
    every (sequence, KV head) row is checked against the oracle."""
    N, Hq, Hkv, T, d, r, B = case.N, case.Hq, case.Hkv, case.T, case.d, case.r, case.B
    caches = []
    for K, V, _ in inst:
        k8 = torch.empty(N, Hkv, T, r, dtype=torch.float8_e4m3fn, device="cuda")
        lsa.lsa_project_keys(K, W, k8)
        caches.append((K, V, k8))
    plan = pipeline.DecodePlan(N, Hq, Hkv, T, d, r, B, kidx_dtype=torch.float8_e4m3fn)
    us = _windows_us(torch, lambda i: plan.run(Q, W, caches[i & 1][2], caches[i & 1][0],
                                                caches[i & 1][1]), max(steps, 7), warm=warmup)
    score_us = _windows_us(torch, lambda i: plan.score(Q, W, caches[i & 1][2]), 140, warm=10)
    kbytes = N * Hkv * T * r
    step_bytes = kbytes + N * Hkv * B * 2 * d * 2 + N * Hkv * B * 4 + N * Hq * d * 6 + N * Hkv * r * 4
    K0, V0, k80 = caches[0]
    plan.run(Q, W, k80, K0, V0)
    torch.cuda.synchronize()
    par = oracle_parity_fp8(case, plan.idx.cpu().numpy(), plan.out.cpu().numpy())
    log(f"fp8 cache: {us:.1f} us/step, scoring {score_us:.1f} us, parity {par}")
    ok = par["pass"]
    return {"workload": "the headline decode step with an OCP E4M3 projected-key cache",
            "us_per_step": us if ok else None, "steps_per_s": 1e6 / us if ok else None,
            "hbm_frac_end_to_end": step_bytes / (us * 1e-6) / (HBM_PEAK_GBPS * 1e9) if ok else None,
            "algorithmic_bytes_per_step": step_bytes,
            "score_kernel": {"avg_launch_us": score_us, "bytes_per_launch": kbytes,
                             "achieved_GBps": kbytes / (score_us * 1e-6) / 1e9},
            "parity": par}


def _windows_us(torch, fn, n: int, warm: int = 10, windows: int = 7) -> float:
    """Median over `windows` consecutive windows of the per-call time of
    n back-to-back calls fn(i) (HIP events only between windows)."""
    stream = torch.cuda.current_stream()
    for i in range(warm):
        fn(i)
    torch.cuda.synchronize()
    windows = max(1, min(windows, n))
    bounds = [n * w // windows for w in range(windows + 1)]
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(windows + 1)]
    evs[0].record(stream)
    for w in range(windows):
        for i in range(bounds[w], bounds[w + 1]):
            fn(i)
        evs[w + 1].record(stream)
    torch.cuda.synchronize()
    return float(np.median([evs[w].elapsed_time(evs[w + 1]) * 1000.0 / (bounds[w + 1] - bounds[w])
                            for w in range(windows)]))


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
    us = _windows_us(torch, lambda i: lsa.lsa_stream_read(bufs[i & 1], sink), reps, warm=4)
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
    warm = _windows_us(torch, lambda i: plan.run(Q, W, k_idx, K, V), n_warm, warm=50)
    cold = _cold_us(torch, lambda i: plan.run(Q, W, k_idx, K, V), n_cold)
    plan.run(Q, W, k_idx, K, V)
    torch.cuda.synchronize()
    import oracle
    ref_k = oracle.project_keys(case.K, case.W, oracle.BF16)
    par = oracle_parity_decode(case, ref_k, plan.idx.cpu().numpy(), plan.out.cpu().numpy(),
                               plan.lse.cpu().numpy())
    alg = N * Hkv * T * r * 2 + N * Hkv * B * 2 * d * 2 + N * Hkv * B * 4 + N * Hq * d * 6 + N * Hkv * r * 4
    log(f"heavy hitters 32K: warm {warm:.1f} us/step, cold {cold:.1f} us/step, parity {par}")
    ok = par["pass"]
    return {"workload": "decode, 1 sequence x 32768 cached tokens, GQA 32/8, d=128, r=64, top-1024, "
                        "bf16, 1% planted heavy hitters per KV head",
            "warm_us_per_step": warm if ok else None, "cold_us_per_step": cold if ok else None,
            "warm_steps_per_s": 1e6 / warm if ok else None, "cold_steps_per_s": 1e6 / cold if ok else None,
            "algorithmic_bytes_per_step": alg,
            "cold_hbm_frac": alg / (cold * 1e-6) / (HBM_PEAK_GBPS * 1e9) if ok else None,
            "parity": par}


def paged_leg(torch, plan, case, inst, Q, n: int = 200) -> dict:
    """Indexed attention of the headline step through a page-size-1 KV pool
    (the serving layout of LSA-L's configs): every cached row of every
    sequence is scattered into one pool, once in sequence order (identity
    table: the translation's own cost) and once in random order (no DRAM
    locality left between neighbouring positions). Outputs must equal the
    unpaged attention bit for bit."""
    N, Hkv, T, d = case.N, case.Hkv, case.T, case.d
    K, V, _ = inst[0]
    unpaged = _windows_us(torch, lambda i: plan.attend(Q, inst[i & 1][0], inst[i & 1][1]), n)
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
        us = _windows_us(torch, lambda i: plan.attend(Q, pools[i & 1][0], pools[i & 1][1],
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
        us = _windows_us(torch, lambda i: plan.run(args), max(20, steps // 4))
        res["all_full_us" if pat.count("S") == 0 else "reuse_us"] = us
        if pat == pattern:
            # every layer holds a copy of the same cache and query, so every
            # layer's output must equal the first (full) layer's bit for bit
            torch.cuda.synchronize()
            res["layers_equal_full_layer"] = all(
                bool(torch.equal(o.view(torch.int32), plan.out[0].view(torch.int32))) for o in plan.out)
        del plan
    res["speedup"] = res["all_full_us"] / res["reuse_us"]
    log(f"cross-layer {pattern}: {res['reuse_us']:.1f} us per {len(pattern)} layers vs "
        f"{res['all_full_us']:.1f} us all full ({res['speedup']:.2f}x)")
    return res


def oracle_parity_hier(case, gblocks, gidx, gout, glse) -> dict:
    """Coarse-to-fine step, stage by stage: the kept blocks against the
    oracle's top blocks over its centroid scores; the final set against the
    oracle's fine selection over the GPU's kept blocks (and inside them);
    output and lse against the oracle's attention over the GPU's set."""
    import oracle
    N, Hkv, T, B, blk, Bc = case.N, case.Hkv, case.T, case.B, case.block, case.B_coarse
    rows = N * Hkv
    k_idx = oracle.project_keys(case.K, case.W, case.dtype)
    cent = oracle.centroids(k_idx, blk)
    qi = oracle.query_prep(case.Q, Hkv, case.W)
    csc = oracle.scores(qi, cent).reshape(rows, -1)
    rblocks, _, _ = oracle.topk(csc, Bc)
    gb = gblocks.reshape(rows, Bc)
    c_same, c_tie, c_bad = _near_tie_sets(gb, rblocks, list(csc))
    fsc = oracle.scores(qi, k_idx, cand=gblocks, cand_block=blk).reshape(rows, -1)
    ridx, _, _ = oracle.topk(fsc, B, cand=gb, cand_block=blk, n_positions=T)
    pos_scores = []
    inside = True
    gi = gidx.reshape(rows, B)
    for row in range(rows):
        full = np.full(T, -np.inf)
        pos = (gb[row][:, None] * blk + np.arange(blk)[None, :]).reshape(-1)
        full[pos] = fsc[row]
        pos_scores.append(full)
        sel = gi[row][gi[row] >= 0]
        inside &= bool(np.isin(sel // blk, gb[row]).all())
    f_same, f_tie, f_bad = _near_tie_sets(gi, ridx, pos_scores)
    o, l = oracle.attention(case.Q, case.K, case.V, gidx)
    err, lerr = float(np.abs(gout - o).max()), float(np.abs(glse - l).max())
    return {"rows": rows, "coarse_identical": c_same, "coarse_near_tie": len(c_tie),
            "fine_identical": f_same, "fine_near_tie": len(f_tie), "final_inside_kept_blocks": inside,
            "max_abs_out_err": err, "max_abs_lse_err": lerr,
            "pass": not c_bad and not f_bad and inside and err <= 2e-3 and lerr <= 2e-3}


def hierarchical_leg(torch, lsa, synth, pipeline, steps: int = 200) -> dict:
    """Coarse-to-fine decode at T = 1048576 (1 sequence, GQA 32/8, block 64,
    top-128 blocks, top-2048): warm back-to-back steps (centroid scores,
    block select, candidate scores, token select, attention), the same step
    replayed from a HIP graph, and cold steps with the caches flushed before
    each; checked stage by stage against the oracle."""
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
    us = _windows_us(torch, lambda i: plan.run(Q, W, k_idx, cent, K, V), steps, warm=20)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        plan.run(Q, W, k_idx, cent, K, V)
    graph_us = _windows_us(torch, lambda i: g.replay(), steps, warm=20)
    cold = _cold_us(torch, lambda i: plan.run(Q, W, k_idx, cent, K, V), 50)
    plan.run(Q, W, k_idx, cent, K, V)
    torch.cuda.synchronize()
    nb = T // blk
    alg = (N * Hkv * nb * r * 2 + N * Hkv * Bc * blk * r * 2 + N * Hkv * B * 2 * d * 2
           + N * Hkv * (Bc + B) * 4 + N * Hq * d * (2 + 4))
    # planted tokens kept: coarse-to-fine is an approximation -- a span that
    # only grazes a 64-token block barely moves that block's centroid
    sel = plan.idx[0].cpu().numpy()
    hit = sum(int(np.isin(case.planted[g_], sel[g_]).sum()) for g_ in range(Hkv))
    tot = sum(len(case.planted[g_]) for g_ in range(Hkv))
    par = oracle_parity_hier(case, plan.blocks.cpu().numpy(), plan.idx.cpu().numpy(),
                             plan.out.cpu().numpy(), plan.lse.cpu().numpy())
    log(f"hierarchical: {us:.1f} us/step warm, graph replay {graph_us:.1f}, {cold:.1f} cold, "
        f"planted tokens kept {hit}/{tot}, parity {par}")
    ok = par["pass"]
    frac = (lambda t: alg / (t * 1e-6) / (HBM_PEAK_GBPS * 1e9) if ok else None)
    return {"workload": "hierarchical decode, 1 sequence x 1048576 tokens, GQA 32/8, d=128, r=64, "
                        "block 64, top-128 blocks, top-2048, bf16, hot spans",
            "us_per_step": us if ok else None, "steps_per_s": 1e6 / us if ok else None,
            "algorithmic_bytes_per_step": alg, "hbm_frac": frac(us),
            "graph_replay_us_per_step": graph_us if ok else None,
            "cold_us_per_step": cold if ok else None, "cold_hbm_frac": frac(cold),
            "planted_tokens_kept": hit, "planted_tokens": tot, "parity": par}


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

    # timed region: exactly K steps, cut into up to 7 consecutive windows by
    # HIP events on the launch stream (events only between windows, never
    # inside a step); the reported step time is the median window's
    steps = args.steps
    n_win = max(1, min(7, steps))
    bounds = [steps * w // n_win for w in range(n_win + 1)]
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n_win + 1)]
    torch.cuda.synchronize()
    evs[0].record(stream)
    for w in range(n_win):
        for i in range(bounds[w], bounds[w + 1]):
            step(i)
        evs[w + 1].record(stream)
    torch.cuda.synchronize()
    win_ms = [evs[w].elapsed_time(evs[w + 1]) / (bounds[w + 1] - bounds[w]) for w in range(n_win)]
    total_ms = evs[0].elapsed_time(evs[-1])
    ms_per_step = float(np.median(win_ms))
    log(f"timed {steps} steps in {n_win} windows: median {ms_per_step * 1000:.1f} us/step, "
        f"mean {total_ms / steps * 1000:.1f}, windows {[round(x * 1000, 1) for x in win_ms]}")

    # the dominant kernel alone: back-to-back launches of the timed step's
    # scoring part (alternating cache instances), events only around each
    # window of launches; and the plain scoring kernel of the three calls
    step_path = lsa.lsa_step_path(Q, W, inst[0][2], inst[0][0], inst[0][1], plan.idx, plan.out)

    def score_part(i):
        K_, V_, kd_ = inst[i & 1]
        plan.part(lsa.STEP_PART_SCORE, Q, W, kd_, K_, V_)

    def score_window(fn, n):
        a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a_.record(stream)
        for i in range(n):
            fn(i)
        b_.record(stream)
        torch.cuda.synchronize()
        return a_.elapsed_time(b_) / n
    score_window(score_part, 10)
    score_ms = float(np.median([score_window(score_part, 20) for _ in range(7)]))
    plain_fn = lambda i: plan.score(Q, W, inst[i & 1][2])   # noqa: E731
    score_window(plain_fn, 10)
    plain_score_ms = float(np.median([score_window(plain_fn, 20) for _ in range(7)]))
    score_kernel = ("score_emit_kernel (scoring prep, projected-key scoring and the select's candidate lists)"
                    if step_path == "listed" else "score_decode_kernel (scoring prep + projected-key scoring)")
    log(f"timed step path: {step_path}; its scoring launch {score_ms * 1000:.1f} us, "
        f"the plain scoring kernel {plain_score_ms * 1000:.1f} us")

    # the same step as the three separate calls (scoring, select, attention)
    plan3 = pipeline.DecodePlan(N, Hq, Hkv, T, d, r, B, fused=False)
    three_us = _windows_us(torch, lambda i: plan3.run(Q, W, inst[i & 1][2], inst[i & 1][0], inst[i & 1][1]),
                           max(steps, 7), warm=args.warmup)
    # one lsa_decode_step call with LSA_STEP_THREE_CALLS (the select's own
    # collect launch instead of the listing scoring launch)
    plan3f = pipeline.DecodePlan(N, Hq, Hkv, T, d, r, B, three_calls=True)
    three_flag_us = _windows_us(torch, lambda i: plan3f.run(Q, W, inst[i & 1][2], inst[i & 1][0], inst[i & 1][1]),
                                max(steps, 7), warm=args.warmup)
    del plan3f
    log(f"the same call with LSA_STEP_THREE_CALLS: {three_flag_us:.1f} us/step")
    # the opt-in single persistent launch of the same step (LSA_STEP_ONE_LAUNCH):
    # timed the same way, its index sets compared with the timed path's below
    plan1 = pipeline.DecodePlan(N, Hq, Hkv, T, d, r, B, fused=True, one_launch=True)
    one_us = _windows_us(torch, lambda i: plan1.run(Q, W, inst[i & 1][2], inst[i & 1][0], inst[i & 1][1]),
                         max(steps, 7), warm=args.warmup)
    plan1.run(Q, W, inst[0][2], inst[0][0], inst[0][1])
    torch.cuda.synchronize()
    one_idx, one_err = plan1.idx.cpu().numpy(), plan1.step_error()
    one_is = lsa.lsa_step_is_fused(Q, W, inst[0][2], inst[0][0], inst[0][1], plan1.idx, plan1.out,
                                   one_launch=True)
    del plan1
    log(f"the same step as three separate calls: {three_us:.1f} us/step; as one persistent launch "
        f"(opt-in): {one_us:.1f} us/step (runs as one launch: {one_is})")

    keys = N * Hkv * T
    kidx_bytes = keys * r * 2
    sel_kv_bytes = N * Hkv * B * 2 * d * 2
    step_bytes = kidx_bytes + sel_kv_bytes + N * Hkv * B * 4 + (N * Hq * d * 2 + N * Hq * d * 4 +
                                                                 N * Hkv * r * 4)
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
    graph_us = _windows_us(torch, lambda i: graphs[i & 1].replay(), max(steps, 7), warm=args.warmup)
    log(f"eager {ms_per_step * 1000:.1f} us/step, graph replay {graph_us:.1f} us/step")

    # the step's outputs on instance 0, for the same-run parity check
    step(0)
    torch.cuda.synchronize()
    plan_error = plan.step_error()
    gpu_idx = plan.idx.cpu().numpy()
    one_launch = {"us_per_step": one_us, "runs_as_one_launch": bool(one_is),
                  "error_word": int(one_err), "idx_equal_to_timed_step": bool(np.array_equal(one_idx, gpu_idx))}
    gpu_out = plan.out.cpu().numpy()
    gpu_lse = plan.lse.cpu().numpy()

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
        # the timed path's three parts, each in windows of back-to-back launches
        def part_fn(parts):
            return lambda i: plan.part(parts, Q, W, inst[i & 1][2], inst[i & 1][0], inst[i & 1][1])
        stages = {
            "path": step_path,
            "score_us": _windows_us(torch, part_fn(lsa.STEP_PART_SCORE), 140),
            "select_us": _windows_us(torch, part_fn(lsa.STEP_PART_SELECT), 140),
            "attention_us": _windows_us(torch, part_fn(lsa.STEP_PART_ATTEND), 140),
            "three_call_kernels": {
                "score_us": _windows_us(torch, lambda i: plan.score(Q, W, inst[i & 1][2]), 140),
                "select_us": _windows_us(torch, lambda i: plan.select(), 140),
                "attention_us": _windows_us(torch, lambda i: plan.attend(Q, inst[i & 1][0], inst[i & 1][1]),
                                            140)},
        }
        stages["attended_kv_GBps"] = sel_kv_bytes / (stages["attention_us"] * 1e-6) / 1e9

    # the oracle leg: parity of the timed configuration (every row), then
    # the CPU baseline (whole steps of the same workload, about
    # --cpu-seconds of host time)
    import oracle
    threads = len(os.sched_getaffinity(0))
    oracle.set_threads(threads)
    ref_k = oracle.project_keys(case.K, case.W, oracle.BF16)        # setup, untimed
    parity = oracle_parity_decode(case, ref_k, gpu_idx, gpu_out, gpu_lse)
    log(f"parity of the timed step: {parity}")
    cpu = None
    if args.cpu_seconds > 0:
        t0 = time.time()
        n_done = 0
        while n_done == 0 or time.time() - t0 < args.cpu_seconds:
            oracle.decode_step(case.Q, case.W, ref_k, case.K, case.V, B)
            n_done += 1
        el = time.time() - t0
        cpu = {"value": n_done / el, "unit": "steps/s", "cores": threads, "kind": "oracle",
               "sample": f"{n_done} full steps of the same workload (all 32 sequence x KV-head rows, "
                         f"fp64) in {el:.1f}s on {platform.processor() or platform.machine()}",
               "keys_scored_per_s": n_done * keys / el}
        log(f"cpu oracle: {cpu['value']:.3f} steps/s on {threads} threads")

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
        del inst, plan, graphs
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

    # no throughput figure without same-run parity of the timed step
    ok = parity["pass"] and plan_error == 0
    steps_per_s = 1000.0 / ms_per_step if ok else None
    traffic = measured_traffic(kidx_bytes)
    line = {
        "metric": METRIC,
        "value": steps_per_s,
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step if ok else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "decode, 4 sequences x 131072 cached tokens, GQA 32/8, d=128, "
                               "r=64, top-B=2048, bf16, 64 hot spans of 32 tokens per KV head",
                   "N": N, "T": T, "Hq": Hq, "Hkv": Hkv, "d": d, "r": r, "B": B,
                   "parallelism": "single GPU"},
        "timing": {"windows": n_win, "window_us_per_step": [x * 1000.0 for x in win_ms],
                   "mean_us_per_step": total_ms / steps * 1000.0, "reported": "median window"},
        "keys_scored_per_s": keys * steps_per_s if ok else None,
        "hbm_frac_end_to_end": step_bytes / (ms_per_step * 1e-3) / (HBM_PEAK_GBPS * 1e9) if ok else None,
        "algorithmic_bytes_per_step": step_bytes,
        "roofline": {"kernel": score_kernel,
                     "bound": "hbm", "achieved": score_gbps, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": score_gbps / HBM_PEAK_GBPS,
                     "avg_launch_us": score_ms * 1000.0,
                     "launch_timing": "median of 7 windows of 20 back-to-back launches",
                     "traffic": traffic},
        "step_path": step_path,
        "plain_score_kernel_us": plain_score_ms * 1000.0,
        "three_calls_us_per_step": three_us if ok else None,
        "three_calls_flag_us_per_step": three_flag_us if ok else None,
        "one_launch_step": one_launch if ok else None,
        "step_error_word": plan_error,
        "graph_replay": {"us_per_step": graph_us if ok else None,
                         "steps_per_s": 1e6 / graph_us if ok else None,
                         "hbm_frac_end_to_end": (step_bytes / (graph_us * 1e-6) / (HBM_PEAK_GBPS * 1e9)
                                                 if ok else None)},
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
    return 0 if ok else 1


if __name__ == "__main__":
    sys.exit(main())
