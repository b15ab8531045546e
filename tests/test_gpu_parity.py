"""GPU parity: the HIP path, called through the C ABI, against the CPU
oracle on identical seeded inputs. Each test prints the case it runs before
touching the GPU."""
from __future__ import annotations

import math
import os

import numpy as np
import pytest
import torch

import oracle
from indexer_driven_sparse_amd import synth
from tests.helpers import (ATTN_ATOL, LSE_ATOL, assert_scores_close, check_index_sets, decoded,
                           dev, host)

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from indexer_driven_sparse_amd import lsa  # fails loudly without liblsa.so
    globals()["lsa"] = lsa
    oracle.set_threads(min(16, len(os.sched_getaffinity(0))))
    yield


def say(*a):
    print("[case]", *a, flush=True)


def torch_dtype(code):
    return torch.float32 if code == synth.F32 else torch.bfloat16


# --------------------------------------------------------------------------
# setup: projected-key cache and centroids, bit-exact
# --------------------------------------------------------------------------

def test_project_keys_golden_rounding():
    cases = []
    for line in open(os.path.join(GOLDEN, "bf16_rounding.txt")):
        if line.startswith("#") or not line.strip():
            continue
        v, b, _ = line.split(None, 2)
        v = float.fromhex(v)
        if v == 0.0 and math.copysign(1.0, v) < 0:
            continue   # a sum started at +0 never yields -0; the oracle pins this case alone
        cases.append((v, int(b, 16)))
    r = 16
    d = 16
    W = np.zeros((d, r), np.float32)
    want = []
    for j, (v, bits) in enumerate(cases):
        a = np.float32(v)                  # v = a + b exactly, both fp32
        b = np.float32(v - float(a))
        assert float(a) + float(b) == v
        W[0, j], W[1, j] = a, b
        want.append(bits)
    K = np.zeros((1, 1, 1, d), np.float32)
    K[..., 0:2] = 1.0
    say("project golden rounding", len(cases))
    out = torch.empty(1, 1, 1, r, dtype=torch.bfloat16, device="cuda")
    lsa.lsa_project_keys(dev(synth.to_bf16_bits(K)), dev(W), out)
    got = host(out)[0, 0, 0, :len(cases)]
    assert [hex(x) for x in got] == [hex(x) for x in want]


@pytest.mark.parametrize("N,T,Hkv,d,r,dtype,per_head,layout", [
    (1, 4096, 1, 128, 64, synth.F32, False, "tok"),
    (2, 1000, 8, 128, 64, synth.BF16, False, "tok"),
    (1, 777, 2, 64, 32, synth.BF16, True, "head"),
    (1, 100, 3, 256, 128, synth.BF16, False, "tok"),
])
def test_project_keys_bit_exact(N, T, Hkv, d, r, dtype, per_head, layout):
    rng = np.random.default_rng(N * 1000 + T)
    shape = (N, T, Hkv, d) if layout == "tok" else (N, Hkv, T, d)
    Kf = rng.standard_normal(shape).astype(np.float32)
    K = Kf if dtype == synth.F32 else synth.to_bf16_bits(Kf)
    if layout == "head":
        K = K.transpose(0, 2, 1, 3)
    W = (rng.standard_normal((Hkv, d, r) if per_head else (d, r)) / math.sqrt(d)).astype(np.float32)
    say("project", N, T, Hkv, d, r, dtype, per_head, layout)
    ref = oracle.project_keys(K, W, dtype)
    Kd = dev(K if layout == "tok" else np.ascontiguousarray(K.transpose(0, 2, 1, 3)))
    if layout == "head":
        Kd = Kd.permute(0, 2, 1, 3)
    out = torch.empty(N, Hkv, T, r, dtype=torch_dtype(dtype), device="cuda")
    lsa.lsa_project_keys(Kd, dev(W), out)
    np.testing.assert_array_equal(host(out), ref)
    # appending a token range into a larger cache leaves the rest untouched
    cap = torch.full((N, Hkv, T + 5, r), 7.0, dtype=torch_dtype(dtype), device="cuda")
    lsa.lsa_project_keys(Kd, dev(W), cap, tok_begin=T // 2, n_tok=T - T // 2)
    got = host(cap)
    np.testing.assert_array_equal(got[:, :, T // 2:T], ref[:, :, T // 2:])
    assert (decoded(got[:, :, :T // 2]) == 7.0).all() and (decoded(got[:, :, T:]) == 7.0).all()


@pytest.mark.parametrize("T,block,dtype", [(4096, 64, synth.BF16), (1000, 64, synth.BF16),
                                           (333, 16, synth.F32)])
def test_centroids_bit_exact(T, block, dtype):
    rng = np.random.default_rng(T)
    kf = rng.standard_normal((2, 3, T, 64)).astype(np.float32)
    k = kf if dtype == synth.F32 else synth.to_bf16_bits(kf)
    say("centroids", T, block, dtype)
    ref = oracle.centroids(k, block)
    out = torch.empty(ref.shape, dtype=torch_dtype(dtype), device="cuda")
    lsa.lsa_build_centroids(dev(k), block, out)
    np.testing.assert_array_equal(host(out), ref)


# --------------------------------------------------------------------------
# indexer scoring
# --------------------------------------------------------------------------

def _scoring_case(N, Hq, Hkv, T, r, dtype, seed, cap=0):
    case = synth.make_decode_case(N=N, Hq=Hq, Hkv=Hkv, T=T, d=128, r=r, B=16, dtype=dtype, seed=seed)
    k_idx = oracle.project_keys(case.K, case.W, dtype)
    if cap:   # cache allocated for more tokens than are filled
        big = np.zeros((N, Hkv, T + cap, r), k_idx.dtype)
        big[:, :, :T] = k_idx
        k_idx = big
    return case, k_idx


@pytest.mark.parametrize("N,Hq,Hkv,T,r,dtype,cap", [
    (1, 4, 1, 4096, 64, synth.F32, 0),
    (1, 32, 8, 5000, 64, synth.BF16, 0),
    (2, 8, 2, 70001, 64, synth.BF16, 64),
    (3, 6, 3, 333, 32, synth.BF16, 0),
    (1, 2, 1, 1, 64, synth.BF16, 0),
    (1, 8, 1, 2047, 128, synth.BF16, 0),
    (1, 4, 2, 900, 16, synth.F32, 0),
])
def test_decode_scores(N, Hq, Hkv, T, r, dtype, cap):
    case, k_idx = _scoring_case(N, Hq, Hkv, T, r, dtype, seed=T, cap=cap)
    say("scores", N, Hq, Hkv, T, r, dtype, cap)
    q_ref = oracle.query_prep(case.Q, Hkv, case.W)
    kd = dev(k_idx)[:, :, :T]
    ref = oracle.scores(q_ref, k_idx[:, :, :T])
    sc = torch.empty(N, Hkv, T + (4 - T % 4) % 4, device="cuda")[:, :, :T]
    qi = torch.empty(N, Hkv, r, device="cuda")
    lsa.lsa_index_score(kd, sc, q=dev(case.Q), w=dev(case.W), q_idx=qi)
    np.testing.assert_allclose(host(qi), q_ref, rtol=1e-5, atol=1e-5 * np.abs(q_ref).max())
    kdec = decoded(k_idx[:, :, :T]).reshape(N * Hkv, T, r)
    assert_scores_close(host(sc).reshape(N * Hkv, T), ref.reshape(N * Hkv, T),
                        q_ref.reshape(N * Hkv, r), kdec)
    # q_idx supplied directly (the prep skipped)
    qin = torch.from_numpy(q_ref.astype(np.float32)).cuda()
    sc2 = torch.empty(N, Hkv, T + (4 - T % 4) % 4, device="cuda")[:, :, :T]
    lsa.lsa_index_score(kd, sc2, q_idx=qin)
    assert_scores_close(host(sc2).reshape(N * Hkv, T), ref.reshape(N * Hkv, T),
                        q_ref.reshape(N * Hkv, r), kdec)


@pytest.mark.parametrize("cand_block", [1, 64])
def test_decode_scores_candidates(cand_block):
    N, Hq, Hkv, T, r = 2, 8, 2, 3000, 64
    case, k_idx = _scoring_case(N, Hq, Hkv, T, r, synth.BF16, seed=7)
    rng = np.random.default_rng(cand_block)
    nc = 40 if cand_block == 64 else 900
    hi = (T + cand_block - 1) // cand_block
    cand = np.stack([np.sort(rng.choice(hi, nc, replace=False)) for _ in range(N * Hkv)]).astype(np.int32)
    cand[0, -3:] = -1
    cand = cand.reshape(N, Hkv, nc)
    say("scores candidates", cand_block)
    q_ref = oracle.query_prep(case.Q, Hkv, case.W)
    ref = oracle.scores(q_ref, k_idx, cand=cand, cand_block=cand_block)
    n_out = nc * cand_block
    sc = torch.empty(N, Hkv, n_out, device="cuda")
    lsa.lsa_index_score(dev(k_idx), sc, q=dev(case.Q), w=dev(case.W), cand=dev(cand),
                        cand_block=cand_block)
    pos = np.zeros((N * Hkv, n_out), np.int64)
    for i in range(N * Hkv):
        c = cand.reshape(N * Hkv, nc)[i]
        p = np.repeat(c.astype(np.int64) * cand_block, cand_block) + np.tile(np.arange(cand_block), nc)
        pos[i] = np.where((np.repeat(c, cand_block) >= 0) & (p < T), p, 0)
    kdec = decoded(k_idx).reshape(N * Hkv, T, r)
    kg = np.stack([kdec[i, pos[i]] for i in range(N * Hkv)])
    assert_scores_close(host(sc).reshape(N * Hkv, n_out), ref.reshape(N * Hkv, n_out),
                        q_ref.reshape(N * Hkv, r), kg)


# --------------------------------------------------------------------------
# exact top-B selection: identical fp32 scores in, identical sets out
# --------------------------------------------------------------------------

def _run_select(sc32, B, **kw):
    rows, n = sc32.shape
    ld = n + (4 - n % 4) % 4
    buf = torch.full((rows, ld), float("nan"), device="cuda")
    buf[:, :n] = torch.from_numpy(sc32).cuda()
    out = torch.full((rows, B), -7, dtype=torch.int32, device="cuda")
    osc = torch.empty(rows, B, device="cuda")
    cnt = torch.full((rows,), -7, dtype=torch.int32, device="cuda")
    dkw = {k: (dev(v) if isinstance(v, np.ndarray) else v) for k, v in kw.items()}
    lsa.lsa_topk_select(buf[:, :n], B, out, out_score=osc, out_count=cnt, **dkw)
    return host(out), host(osc), host(cnt)


def _assert_select_equal(sc32, B, **kw):
    got, gsc, gcnt = _run_select(sc32, B, **kw)
    okw = dict(kw)
    if "cand" in okw:
        okw["n_positions"] = kw["n_positions"]
    ref, rsc, rcnt = oracle.topk(sc32.astype(np.float64), B, **okw)
    np.testing.assert_array_equal(got, ref)
    np.testing.assert_array_equal(gcnt, rcnt)
    np.testing.assert_array_equal(gsc.astype(np.float64), rsc)


@pytest.mark.parametrize("rows,n,B,kind", [
    (4, 131072, 2048, "normal"),
    (8, 32768, 1024, "normal"),
    (1, 4096, 256, "normal"),
    (3, 5000, 300, "ints"),           # many exact ties
    (2, 1000, 1, "ints"),
    (2, 777, 777, "normal"),          # B == n
    (2, 777, 1000, "normal"),         # B > n
    (2, 20000, 100, "equal"),         # boundary bin larger than the LDS list
    (2, 50000, 9000, "normal"),       # boundary bin with more keys than fit in LDS
    (2, 3001, 64, "special"),         # NaN, +-0, +-inf
    (2, 300000, 2048, "normal"),      # bitmaps in workspace
    (3, 16384, 128, "normal"),        # rows of up to 16384 slots in registers, 16 per thread
    (2, 12000, 3000, "ints"),         # ... with many exact ties
    (2, 8193, 2048, "special"),       # ... one slot past the 8-per-thread rows
    (2, 16384, 16384, "normal"),      # ... every slot taken
])
def test_select_exact(rows, n, B, kind):
    rng = np.random.default_rng(n + B)
    if kind == "normal":
        sc = rng.standard_normal((rows, n)).astype(np.float32)
    elif kind == "ints":
        sc = rng.integers(-20, 20, size=(rows, n)).astype(np.float32)
    elif kind == "equal":
        sc = np.full((rows, n), 1.5, np.float32)
    else:
        sc = rng.choice(np.array([np.nan, 0.0, -0.0, np.inf, -np.inf, 1.0, -1.0], np.float32),
                        size=(rows, n))
    say("select", rows, n, B, kind)
    _assert_select_equal(sc, B)


def test_select_valid_counts_causal_and_candidates():
    rng = np.random.default_rng(11)
    sc = rng.standard_normal((6, 9000)).astype(np.float32)
    say("select n_valid")
    _assert_select_equal(sc, 500, n_valid=np.array([0, 1, 499, 500, 501, 9000], np.int32))
    L = 3000
    scl = rng.standard_normal((L, L)).astype(np.float32)
    say("select causal")
    _assert_select_equal(scl, 700, causal_group=1)
    Hkv = 2
    scl2 = rng.standard_normal((400 * Hkv, 400)).astype(np.float32)
    _assert_select_equal(scl2, 64, causal_group=Hkv)
    say("select candidates, 200 blocks of 64 (rows of 12800 slots in registers)")
    cand16 = np.stack([np.sort(rng.choice(16384, 200, replace=False)) for _ in range(3)]).astype(np.int32)
    cand16[1, -3:] = -1                        # invalid blocks: the row takes the general path
    sc16 = rng.standard_normal((3, 200 * 64)).astype(np.float32)
    _assert_select_equal(sc16, 1500, cand=cand16, cand_block=64, n_positions=16384 * 64 - 20)
    say("select candidates")
    rows, nc, blk = 4, 128, 64
    cand = np.stack([np.sort(rng.choice(16384, nc, replace=False)) for _ in range(rows)]).astype(np.int32)
    cand[1, -5:] = -1
    scc = rng.standard_normal((rows, nc * blk)).astype(np.float32)
    _assert_select_equal(scc, 2048, cand=cand, cand_block=blk, n_positions=16384 * 64 - 100)


def test_select_is_deterministic_and_overwrites_outputs():
    rng = np.random.default_rng(12)
    sc = rng.integers(-5, 5, size=(16, 20000)).astype(np.float32)
    say("select determinism")
    a = _run_select(sc, 1500)
    b = _run_select(sc, 1500)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


# --------------------------------------------------------------------------
# indexed attention on oracle-chosen index sets
# --------------------------------------------------------------------------

def _attn_case(rows, Hq, Hkv, T, d, B, dtype, seed, prefill=False, layout="tok", fill=1.0):
    rng = np.random.default_rng(seed)
    S = 1 if prefill else rows
    q = rng.standard_normal((rows, Hq, d)).astype(np.float32)
    shape = (S, T, Hkv, d) if layout == "tok" else (S, Hkv, T, d)
    K = rng.standard_normal(shape).astype(np.float32)
    V = rng.standard_normal(shape).astype(np.float32)
    if dtype == synth.BF16:
        q, K, V = synth.to_bf16_bits(q), synth.to_bf16_bits(K), synth.to_bf16_bits(V)
    idx = np.full((rows, Hkv, B), -1, np.int32)
    for i in range(rows):
        for g in range(Hkv):
            hi = (i + 1) if prefill else T
            k = min(B, max(0, int(round(fill * min(B, hi)))))
            idx[i, g, :k] = np.sort(rng.choice(hi, k, replace=False))
    return q, K, V, idx


def _run_attention(q, K, V, idx, layout, prefill):
    Kd, Vd = dev(K), dev(V)
    if layout == "head":
        Kd, Vd = Kd.permute(0, 2, 1, 3), Vd.permute(0, 2, 1, 3)
    rows, Hq, d = q.shape
    out = torch.full((rows, Hq, d), float("nan"), device="cuda")
    lse = torch.full((rows, Hq), float("nan"), device="cuda")
    lsa.lsa_indexed_attention(dev(q), Kd, Vd, dev(idx), out, lse=lse,
                              mode=lsa.MODE_PREFILL_CAUSAL if prefill else lsa.MODE_DECODE)
    return host(out), host(lse)


@pytest.mark.parametrize("rows,Hq,Hkv,T,d,B,dtype,prefill,layout,fill", [
    (1, 4, 1, 4096, 128, 256, synth.F32, False, "tok", 1.0),
    (1, 32, 8, 32768, 128, 1024, synth.BF16, False, "tok", 1.0),
    (4, 32, 8, 131072, 128, 2048, synth.BF16, False, "tok", 1.0),
    (3, 8, 2, 5000, 128, 300, synth.BF16, False, "head", 0.7),
    (2, 8, 8, 999, 64, 77, synth.BF16, False, "tok", 0.9),
    (2, 16, 2, 999, 64, 77, synth.F32, False, "tok", 1.0),
    (5, 4, 4, 100, 128, 1, synth.BF16, False, "tok", 1.0),
    (2, 16, 2, 3000, 128, 700, synth.BF16, False, "tok", 0.8),    # G = 8, ragged last split
    (1, 8, 2, 20000, 128, 16384, synth.BF16, False, "tok", 1.0),  # the most splits on matrix cores
    (1, 8, 2, 20000, 128, 16400, synth.BF16, False, "tok", 1.0),  # one split too many: vector path
    (2, 8, 1, 500, 128, 1, synth.BF16, False, "tok", 1.0),       # G = 8, one entry
    (600, 8, 1, 600, 128, 256, synth.BF16, True, "tok", 1.0),
])
def test_attention(rows, Hq, Hkv, T, d, B, dtype, prefill, layout, fill):
    q, K, V, idx = _attn_case(rows, Hq, Hkv, T, d, B, dtype, seed=rows * T + B, prefill=prefill,
                              layout=layout, fill=fill)
    say("attention", rows, Hq, Hkv, T, d, B, dtype, prefill, layout, fill)
    Ko = K if layout == "tok" else K.transpose(0, 2, 1, 3)
    Vo = V if layout == "tok" else V.transpose(0, 2, 1, 3)
    ref, rlse = oracle.attention(q, Ko, Vo, idx, prefill=prefill)
    out, lse = _run_attention(q, K, V, idx, layout, prefill)
    np.testing.assert_allclose(out, ref, rtol=0, atol=ATTN_ATOL)
    np.testing.assert_allclose(lse, rlse, rtol=0, atol=LSE_ATOL)


def test_attention_decode_unaligned_q():
    # q 2 bytes past a 16-byte boundary: decode leaves the matrix-core path
    # (which reads q rows 16 bytes at a time) for the vector one
    rows, Hq, Hkv, T, d, B = 2, 8, 2, 3000, 128, 500
    q, K, V, idx = _attn_case(rows, Hq, Hkv, T, d, B, synth.BF16, seed=11)
    say("attention unaligned q")
    ref, rlse = oracle.attention(q, K, V, idx)
    flat = torch.empty(q.size + 1, dtype=torch.bfloat16, device="cuda")
    qd = flat[1:].view(q.shape)
    qd.copy_(dev(q))
    assert qd.data_ptr() % 16 == 2
    out = torch.full((rows, Hq, d), float("nan"), device="cuda")
    lse = torch.full((rows, Hq), float("nan"), device="cuda")
    lsa.lsa_indexed_attention(qd, dev(K), dev(V), dev(idx), out, lse=lse, mode=lsa.MODE_DECODE)
    np.testing.assert_allclose(host(out), ref, rtol=0, atol=ATTN_ATOL)
    np.testing.assert_allclose(host(lse), rlse, rtol=0, atol=LSE_ATOL)


def test_attention_edge_entries():
    # empty rows, out-of-range and negative entries, full set (B = T = dense)
    rows, Hq, Hkv, T, d, B = 3, 8, 2, 64, 128, 64
    q, K, V, idx = _attn_case(rows, Hq, Hkv, T, d, B, synth.BF16, seed=5)
    idx[0, 0, :] = -1                                 # empty set
    idx[1, 1, ::3] = T + 5                            # beyond the cache: skipped
    idx[1, 0, 1::4] = -9
    idx[2] = np.arange(T)                             # every position
    say("attention edges")
    ref, rlse = oracle.attention(q, K, V, idx)
    out, lse = _run_attention(q, K, V, idx, "tok", False)
    np.testing.assert_allclose(out, ref, rtol=0, atol=ATTN_ATOL)
    assert np.isneginf(lse[0, :4]).all() and (out[0, :4] == 0).all()
    fin = np.isfinite(rlse)
    np.testing.assert_allclose(lse[fin], rlse[fin], rtol=0, atol=LSE_ATOL)


def _paged_pool(K, V, seed, spare=0.25):
    """Scatter a dense [S,T,Hkv,d] cache into a page-size-1 pool with the
    rows in random order; unused pool rows hold NaN, so reading one would
    show. Pool row 0 is always unused: kernels that load a fixed row for a
    skipped entry must keep its NaN out of the result. Returns the pool K/V
    [P,Hkv,d] and the slot table [S,T]."""
    S, T, Hkv, d = K.shape
    rng = np.random.default_rng(seed)
    P = S * T + int(spare * S * T) + 1
    rows = (1 + rng.permutation(P - 1)[: S * T]).astype(np.int32)
    table = rows.reshape(S, T)
    Kp = np.full((P, Hkv, d), np.nan if K.dtype == np.float32 else 0x7fc0, K.dtype)
    Vp = Kp.copy()
    Kp[rows] = K.reshape(S * T, Hkv, d)
    Vp[rows] = V.reshape(S * T, Hkv, d)
    return Kp, Vp, table


@pytest.mark.parametrize("rows,Hq,Hkv,T,d,B,dtype,prefill", [
    (4, 32, 8, 16384, 128, 2048, synth.BF16, False),
    (3, 8, 2, 5000, 128, 300, synth.F32, False),
    (2, 16, 2, 999, 64, 77, synth.BF16, False),
    (600, 8, 1, 600, 128, 256, synth.BF16, True),
])
def test_attention_paged_equals_unpaged(rows, Hq, Hkv, T, d, B, dtype, prefill):
    """Page-size-1 pool: the same rows read through the slot table give the
    unpaged result bit for bit, and the oracle's over the dense cache."""
    q, K, V, idx = _attn_case(rows, Hq, Hkv, T, d, B, dtype, seed=7 * T + B, prefill=prefill,
                              fill=0.9)
    Kp, Vp, table = _paged_pool(K, V, seed=T)
    say("attention paged", rows, Hq, Hkv, T, d, B, dtype, prefill, "pool", Kp.shape[0])
    mode = lsa.MODE_PREFILL_CAUSAL if prefill else lsa.MODE_DECODE
    out_u, lse_u = _run_attention(q, K, V, idx, "tok", prefill)
    out = torch.full((rows, Hq, d), float("nan"), device="cuda")
    lse = torch.full((rows, Hq), float("nan"), device="cuda")
    lsa.lsa_indexed_attention(dev(q), dev(Kp), dev(Vp), dev(idx), out, lse=lse, mode=mode,
                              slot_table=dev(table))
    out, lse = host(out), host(lse)
    assert np.array_equal(out.view(np.uint32), out_u.view(np.uint32))
    assert np.array_equal(lse.view(np.uint32), lse_u.view(np.uint32))
    ref, rlse = oracle.attention(q, K, V, idx, prefill=prefill)
    np.testing.assert_allclose(out, ref, rtol=0, atol=ATTN_ATOL)
    np.testing.assert_allclose(lse, rlse, rtol=0, atol=LSE_ATOL)


def test_attention_paged_stale_slots_are_skipped():
    """Table entries outside the pool (negative, or past its end) are skipped
    like -1 entries of the index list; so are positions >= n_keys, even when
    the table is wider."""
    rows, Hq, Hkv, T, d, B = 3, 8, 2, 512, 128, 128
    q, K, V, idx = _attn_case(rows, Hq, Hkv, T, d, B, synth.BF16, seed=11)
    Kp, Vp, table = _paged_pool(K, V, seed=12)
    wide = np.concatenate([table, np.zeros((rows, 64), np.int32)], axis=1)   # ld = T + 64
    dead = np.zeros((rows, T), bool)
    dead[0, 5::7] = True
    dead[1, 3::11] = True
    wide[:, :T][dead] = np.where(np.arange(dead.sum()) % 2 == 0, -3, Kp.shape[0] + 9)
    idx[2, 0, :4] = [T, T + 1, T + 2, T + 63]                     # inside the table, past n_keys
    idx[2, 0] = np.sort(idx[2, 0])
    expect = idx.copy()
    for i in range(rows):
        for g in range(Hkv):
            e = expect[i, g]
            bad = (e >= T) | ((e >= 0) & dead[i, np.clip(e, 0, T - 1)])
            e[bad] = -1
    say("attention paged stale slots")
    out = torch.full((rows, Hq, d), float("nan"), device="cuda")
    lse = torch.full((rows, Hq), float("nan"), device="cuda")
    lsa.lsa_indexed_attention(dev(q), dev(Kp), dev(Vp), dev(idx), out, lse=lse,
                              slot_table=dev(wide), n_keys=T)
    out, lse = host(out), host(lse)
    ref, rlse = oracle.attention(q, K, V, expect)
    np.testing.assert_allclose(out, ref, rtol=0, atol=ATTN_ATOL)
    np.testing.assert_allclose(lse, rlse, rtol=0, atol=LSE_ATOL)


@pytest.mark.parametrize("rows,B", [(300, 77), (70, 1), (129, 33), (64, 64)])
def test_attention_prefill_matrix_core_edges(rows, B):
    """Prefill with 8 query heads per KV head and d = 128 runs on the matrix
    cores: empty sets, -1 entries inside the list, entries past the cache,
    entries after the row's own token (masked causally), and list lengths
    that are not a multiple of the 32-key chunk."""
    Hq, Hkv, T, d = 8, 1, rows, 128
    q, K, V, idx = _attn_case(rows, Hq, Hkv, T, d, B, synth.BF16, seed=rows + B, prefill=True)
    rng = np.random.default_rng(rows * B)
    idx[0, 0, :] = -1                                         # row 0: empty set
    if B > 2:
        idx[rows // 2, 0, 1] = -1                             # a hole inside a list
        idx[rows - 1, 0, 0] = T + 3                           # past the cache: skipped
    fut = rng.integers(1, rows, size=min(8, rows - 1))        # future positions: masked
    for i in fut:
        idx[i - 1, 0, -1] = min(T - 1, i + 1 + int(rng.integers(0, 5)))
    say("attention prefill matrix cores", rows, B)
    ref, rlse = oracle.attention(q, K, V, idx, prefill=True)
    out, lse = _run_attention(q, K, V, idx, "tok", True)
    np.testing.assert_allclose(out, ref, rtol=0, atol=ATTN_ATOL)
    fin = np.isfinite(rlse)
    assert np.array_equal(np.isneginf(lse), ~fin) and (out[~fin.any(axis=1)] == 0).all()
    np.testing.assert_allclose(lse[fin], rlse[fin], rtol=0, atol=LSE_ATOL)


@pytest.mark.parametrize("L,qb,B", [(1000, 50, 200), (257, 8, 64), (130, 130, 96)])
def test_prefill_block_attention_matrix_core_shapes(L, qb, B):
    """Block-shared selections on the matrix cores (8 heads, d = 128) with
    blocks that are not a multiple of the 16 tokens a workgroup serves, a
    block smaller than that, and a last partial block."""
    Hq, Hkv, d = 8, 1, 128
    rng = np.random.default_rng(L + qb + B)
    q = synth.to_bf16_bits(rng.standard_normal((L, Hq, d)).astype(np.float32))
    K = synth.to_bf16_bits(rng.standard_normal((1, L, Hkv, d)).astype(np.float32))
    V = synth.to_bf16_bits(rng.standard_normal((1, L, Hkv, d)).astype(np.float32))
    nb = (L + qb - 1) // qb
    blk = np.full((nb, Hkv, B), -1, np.int32)
    for b in range(nb):
        hi = min(L, (b + 1) * qb)
        c = min(B, hi)
        blk[b, 0, :c] = np.sort(rng.choice(hi, c, replace=False))
    say("prefill block attention matrix cores", L, qb, B)
    out = torch.full((L, Hq, d), float("nan"), device="cuda")
    lse = torch.full((L, Hq), float("nan"), device="cuda")
    lsa.lsa_indexed_attention(dev(q), dev(K), dev(V), dev(blk), out, lse=lse,
                              mode=lsa.MODE_PREFILL_CAUSAL, query_block=qb)
    ref, rlse = oracle.attention(q, K, V, blk, prefill=True, query_block=qb)
    np.testing.assert_allclose(host(out), ref, rtol=0, atol=ATTN_ATOL)
    np.testing.assert_allclose(host(lse), rlse, rtol=0, atol=LSE_ATOL)
    # the same through a page-size-1 pool: bit-identical
    Kp, Vp, table = _paged_pool(K, V, seed=L)
    out2 = torch.full((L, Hq, d), float("nan"), device="cuda")
    lse2 = torch.full((L, Hq), float("nan"), device="cuda")
    lsa.lsa_indexed_attention(dev(q), dev(Kp), dev(Vp), dev(blk), out2, lse=lse2,
                              mode=lsa.MODE_PREFILL_CAUSAL, query_block=qb, slot_table=dev(table))
    assert torch.equal(out2.view(torch.int32), out.view(torch.int32))
    assert torch.equal(lse2.view(torch.int32), lse.view(torch.int32))


# --------------------------------------------------------------------------
# whole decode step
# --------------------------------------------------------------------------

def gpu_decode_step(case, k_idx_dev):
    from indexer_driven_sparse_amd import pipeline
    res = pipeline.decode_step(dev(case.Q), dev(case.W), k_idx_dev, dev(case.K), dev(case.V), case.B)
    torch.cuda.synchronize()
    return {k: host(v) for k, v in res.items()}


def _compare_step(case, g, ref, rows_sel):
    """Compare GPU step outputs g against oracle outputs ref for the
    (sequence, KV head) rows listed in rows_sel."""
    N, Hkv, G, B = case.N, case.Hkv, case.G, case.B
    gi = g["idx"].reshape(N * Hkv, B)[rows_sel]
    ri = ref["idx"].reshape(-1, B)
    scores = [ref["scores"].reshape(-1, ref["scores"].shape[-1])[j] for j in range(len(rows_sel))]
    diff = check_index_sets(gi, ri, scores, B)
    for j, row in enumerate(rows_sel):
        n, gh = divmod(row, Hkv)
        heads = slice(gh * G, (gh + 1) * G)
        if j in diff:     # tolerated near-tie swap: check the output is right for the GPU's set
            qh = case.Q[n:n + 1]
            o, l = oracle.attention(qh, case.K[n:n + 1], case.V[n:n + 1],
                                    g["idx"].reshape(N, Hkv, B)[n:n + 1])
            want_o, want_l = o[0, heads], l[0, heads]
        else:
            want_o = ref["out"][j]
            want_l = ref["lse"][j]
        np.testing.assert_allclose(g["out"][n, heads], want_o, rtol=0, atol=ATTN_ATOL)
        np.testing.assert_allclose(g["lse"][n, heads], want_l, rtol=0, atol=LSE_ATOL)
    return diff


def _oracle_rows(case, rows_sel, kidx_dtype=None):
    """Oracle decode step for selected (sequence, KV head) rows: project that
    head's keys (stored in kidx_dtype, default the case's dtype), score,
    select, attend. Outputs are stacked per selected row."""
    outs = {"idx": [], "scores": [], "out": [], "lse": []}
    for row in rows_sel:
        n, g = divmod(row, case.Hkv)
        K1 = case.K[n:n + 1, :, g:g + 1]
        V1 = case.V[n:n + 1, :, g:g + 1]
        Q1 = case.Q[n:n + 1, g * case.G:(g + 1) * case.G]
        k1 = oracle.project_keys(K1, case.W, case.dtype if kidx_dtype is None else kidx_dtype)
        r = oracle.decode_step(Q1, case.W, k1, K1, V1, case.B)
        outs["idx"].append(r["idx"][0, 0])
        outs["scores"].append(r["scores"][0, 0])
        outs["out"].append(r["out"][0])
        outs["lse"].append(r["lse"][0])
    return {k: np.stack(v) for k, v in outs.items()}


def test_cross_layer_index_reuse():
    """Layers "FSSFS": full layers run their own indexer; each shared layer
    attends over its own Q/K/V with the top-B sets of the nearest full layer
    before it."""
    from indexer_driven_sparse_amd import pipeline
    pattern = "FSSFS"
    cases = [synth.make_decode_case(N=2, Hq=8, Hkv=2, T=3000, B=256, plant="hitters", seed=40 + i)
             for i in range(len(pattern))]
    c0 = cases[0]
    say("cross-layer reuse", pattern, c0.N, c0.Hq, c0.Hkv, c0.T, c0.B)
    plan = pipeline.CrossLayerPlan(pattern, c0.N, c0.Hq, c0.Hkv, c0.T, c0.d, c0.r, c0.B)
    layers = []
    for i, c in enumerate(cases):
        W = dev(c.W)
        K, V = dev(c.K), dev(c.V)
        k_idx = None
        if pattern[i] == "F":
            k_idx = torch.empty(c.N, c.Hkv, c.T, c.r, dtype=torch.bfloat16, device="cuda")
            lsa.lsa_project_keys(K, W, k_idx)
        layers.append((dev(c.Q), W, k_idx, K, V))
    plan.run(layers)
    torch.cuda.synchronize()
    rows = list(range(c0.N * c0.Hkv))
    sets = {}
    for i, c in enumerate(cases):
        if pattern[i] == "F":
            g = {"idx": host(plan.full[i].idx), "out": host(plan.out[i]), "lse": host(plan.lse[i])}
            _compare_step(c, g, _oracle_rows(c, rows), rows)
            sets[i] = g["idx"]        # checked above against the oracle's sets
        else:
            src = plan.source[i]
            assert src == max(j for j in sets if j < i)
            ref, rlse = oracle.attention(c.Q, c.K, c.V, sets[src])
            np.testing.assert_allclose(host(plan.out[i]), ref, rtol=0, atol=ATTN_ATOL)
            np.testing.assert_allclose(host(plan.lse[i]), rlse, rtol=0, atol=LSE_ATOL)


@pytest.mark.parametrize("name,over", [
    ("decode_t4k_fp32", {}),
    ("decode_t32k_hitters", {}),
    ("decode_t128k_b2048", {"N": 1, "T": 9000}),      # several tiles and a ragged tail
])
def test_decode_step_full(name, over):
    case = synth.workload(name, **over)
    say("decode step", name, over)
    k_idx = oracle.project_keys(case.K, case.W, case.dtype)
    g = gpu_decode_step(case, dev(k_idx))
    rows = list(range(case.N * case.Hkv))
    ref = _oracle_rows(case, rows)
    _compare_step(case, g, ref, rows)


def test_decode_step_headline_workload_every_row():
    """Decode, 4 sequences, T=131072, GQA 32/8, d=128, r=64, B=2048, bf16 --
    the benchmarked workload at full size, in the benchmark's launch shape;
    every one of the 32 (sequence, KV head) rows against the oracle: its
    projected keys, index set, output and lse."""
    case = synth.workload("decode_t128k_b2048")
    say("decode step headline 4x131072 B=2048, every row")
    kd = torch.empty(case.N, case.Hkv, case.T, case.r, dtype=torch.bfloat16, device="cuda")
    lsa.lsa_project_keys(dev(case.K), dev(case.W), kd)
    rows = list(range(case.N * case.Hkv))
    # the GPU-built cache must equal the oracle's on every row
    for row in rows:
        n, gh = divmod(row, case.Hkv)
        ref_k = oracle.project_keys(case.K[n:n + 1, :, gh:gh + 1], case.W, case.dtype)
        np.testing.assert_array_equal(host(kd[n, gh]), ref_k[0, 0])
    g = gpu_decode_step(case, kd)
    ref = _oracle_rows(case, rows)
    _compare_step(case, g, ref, rows)
    # one lsa_decode_step call (the benchmark's path), and the single
    # persistent launch, against the same oracle rows
    from indexer_driven_sparse_amd import pipeline
    for one_launch in (False, True):
        plan = pipeline.DecodePlan(case.N, case.Hq, case.Hkv, case.T, case.d, case.r, case.B,
                                   fused=True, one_launch=one_launch)
        plan.run(dev(case.Q), dev(case.W), kd, dev(case.K), dev(case.V))
        torch.cuda.synchronize()
        assert plan.step_error() == 0
        gf = {"idx": host(plan.idx), "out": host(plan.out), "lse": host(plan.lse)}
        _compare_step(case, gf, ref, rows)


def _fused_vs_three_calls(case, kd, reps=1):
    """The fused lsa_decode_step against the three calls in sequence on the
    same inputs: indices, q_idx and per-entry scores bit for bit (both are
    the exact top-B of the same scores); out and lse over those indices
    within 1e-5 (fp32 attention summed in another order), and against the
    oracle's attention over the same indices within the attention bar.
    Returns the fused plan."""
    from indexer_driven_sparse_amd import pipeline
    N, Hq, Hkv, T, d, r, B = case.N, case.Hq, case.Hkv, case.T, case.d, case.r, case.B
    Q, W, K, V = dev(case.Q), dev(case.W), dev(case.K), dev(case.V)
    ref = pipeline.DecodePlan(N, Hq, Hkv, T, d, r, B, with_idx_scores=True, kidx_dtype=kd.dtype,
                              fused=False)
    ref.run(Q, W, kd, K, V)
    fus = pipeline.DecodePlan(N, Hq, Hkv, T, d, r, B, with_idx_scores=True, kidx_dtype=kd.dtype,
                              fused=True, one_launch=True)
    for _ in range(reps):
        fus.run(Q, W, kd, K, V)
    torch.cuda.synchronize()
    assert fus.step_error() == 0
    for name in ("idx", "q_idx", "idx_scores"):
        a, b = getattr(fus, name), getattr(ref, name)
        assert torch.equal(a.view(torch.int32), b.view(torch.int32)), name
    for name in ("out", "lse"):
        np.testing.assert_allclose(host(getattr(fus, name)), host(getattr(ref, name)), rtol=0, atol=1e-5,
                                   err_msg=name)
    o, l = oracle.attention(case.Q, case.K, case.V, host(fus.idx))
    np.testing.assert_allclose(host(fus.out), o, rtol=0, atol=ATTN_ATOL)
    np.testing.assert_allclose(host(fus.lse), l, rtol=0, atol=LSE_ATOL)
    return fus


@pytest.mark.parametrize("name,over", [
    ("decode_t128k_b2048", {"N": 1, "T": 100000, "B": 1024}),       # 4 splits per row
    ("decode_t128k_b2048", {"N": 3, "Hq": 12, "Hkv": 3, "T": 70000, "B": 512}),  # 9 rows over 8 XCDs
    ("decode_t128k_b2048", {"N": 2, "Hq": 32, "Hkv": 4, "T": 50000, "B": 1500}),  # 8 heads per group, a ragged split
    ("decode_t128k_b2048", {"N": 2, "T": 50000, "B": 256}),         # one split: nothing to merge
    ("decode_t128k_b2048", {"N": 4}),                               # the headline shape
])
def test_decode_step_equals_separate_calls(name, over):
    """lsa_decode_step's default path (the matrix-core attention merging its
    splits in the launch, each row's splits on one XCD) against the separate
    calls lsa_index_score, lsa_topk_select and lsa_indexed_attention (whose
    merge is a kernel of its own): indices, per-entry scores, q_idx, out and
    lse bit for bit; run twice on one workspace, whose control words are
    left zero."""
    from indexer_driven_sparse_amd import pipeline
    case = synth.workload(name, **over)
    say("decode step vs separate calls", name, over)
    N, Hq, Hkv, T, d, r, B = case.N, case.Hq, case.Hkv, case.T, case.d, case.r, case.B
    Q, W, K, V = dev(case.Q), dev(case.W), dev(case.K), dev(case.V)
    kd = torch.empty(N, Hkv, T, r, dtype=torch.bfloat16, device="cuda")
    lsa.lsa_project_keys(K, W, kd)
    ref = pipeline.DecodePlan(N, Hq, Hkv, T, d, r, B, with_idx_scores=True, fused=False)
    ref.run(Q, W, kd, K, V)
    one = pipeline.DecodePlan(N, Hq, Hkv, T, d, r, B, with_idx_scores=True, fused=True)
    for _ in range(2):
        one.run(Q, W, kd, K, V)
    torch.cuda.synchronize()
    assert one.step_error() == 0
    for name_ in ("idx", "q_idx", "idx_scores", "out", "lse"):
        a, b = getattr(one, name_), getattr(ref, name_)
        assert torch.equal(a.view(torch.int32), b.view(torch.int32)), name_
    _assert_step_ctrl_zero(one, N * Hkv)


def _assert_step_ctrl_zero(plan, rows):
    """The step workspace's control words (1024 launch-wide words, then 1024
    per row) are all zero again after a call."""
    ctl = plan.step_ws[:4 * (1024 + 1024 * rows)].view(torch.int32)
    assert int(ctl.abs().sum().item()) == 0


def _sample_slot(gi, row, n):
    """Slot of the listing scoring launch's sample in 64-slot group gi of a
    row: the offset hashed from the group and the row (the rule the step's
    header states), clamped to the row."""
    h = ((gi * 0x9E3779B1) & 0xFFFFFFFF) ^ ((row * 0x85EBCA77) & 0xFFFFFFFF)
    return min(gi * 64 + (((h * 0xC2B2AE3D) & 0xFFFFFFFF) >> 26), n - 1)


def _listed_vs_three_calls(case, kd, reps=2):
    """lsa_decode_step's listing path against LSA_STEP_THREE_CALLS on the
    same inputs: indices, per-entry scores and q_idx bit for bit, out and
    lse bit for bit (the same attention launch); the control words left
    zero after every call. Returns the listing plan."""
    from indexer_driven_sparse_amd import pipeline
    N, Hq, Hkv, T, d, r, B = case.N, case.Hq, case.Hkv, case.T, case.d, case.r, case.B
    Q, W, K, V = dev(case.Q), dev(case.W), dev(case.K), dev(case.V)
    ref = pipeline.DecodePlan(N, Hq, Hkv, T, d, r, B, with_idx_scores=True, kidx_dtype=kd.dtype,
                              three_calls=True)
    ref.run(Q, W, kd, K, V)
    one = pipeline.DecodePlan(N, Hq, Hkv, T, d, r, B, with_idx_scores=True, kidx_dtype=kd.dtype)
    assert lsa.lsa_step_path(Q, W, kd, K, V, one.idx, one.out) == "listed"
    assert lsa.lsa_step_path(Q, W, kd, K, V, one.idx, one.out, three_calls=True) == "three_calls"
    for _ in range(reps):
        one.run(Q, W, kd, K, V)
        torch.cuda.synchronize()
        _assert_step_ctrl_zero(one, N * Hkv)
    for name_ in ("idx", "q_idx", "idx_scores", "out", "lse"):
        a, b = getattr(one, name_), getattr(ref, name_)
        assert torch.equal(a.view(torch.int32), b.view(torch.int32)), name_
    return one


@pytest.mark.parametrize("name,over", [
    ("decode_t128k_b2048", {"N": 4}),                               # the headline shape
    ("decode_t128k_b2048", {"N": 1, "T": 40961, "B": 1024}),        # a ragged last chunk and sample group
    ("decode_t32k_hitters", {}),                                    # chunks of 512 slots
    ("decode_t4k_fp32", {}),                                        # an fp32 cache, one chunk per row
])
def test_decode_step_listed_equals_three_calls(name, over):
    """The default path's scoring launch lists the select's candidates (a
    sampled threshold per row); the result equals the three calls bit for
    bit."""
    case = synth.workload(name, **over)
    say("listed decode step vs three calls", name, over)
    kd = torch.empty(case.N, case.Hkv, case.T, case.r, dtype=torch_dtype(case.dtype), device="cuda")
    lsa.lsa_project_keys(dev(case.K), dev(case.W), kd)
    _listed_vs_three_calls(case, kd)


def test_decode_step_listed_fallbacks():
    """The listing path where its lists cannot settle a row, so the select
    takes the scores: (1) every key of a head equal (each row one big tie:
    every key reaches the threshold, more than the list path takes), whose
    selection is the lowest B positions; (2) keys planted at exactly the
    sampled slots, so the sampled threshold lets fewer than B keys through;
    (3) an fp8 cache. Each equals the three calls bit for bit, and (2) the
    oracle."""
    case = synth.workload("decode_t128k_b2048", N=1, T=40000, B=1024)
    say("listed decode step, constant keys per head")
    K = case.K.copy()
    K[:, :, :, :] = K[:, :1, :, :]
    tie = synth.workload("decode_t128k_b2048", N=1, T=40000, B=1024)
    tie.K = K
    kd = torch.empty(tie.N, tie.Hkv, tie.T, tie.r, dtype=torch.bfloat16, device="cuda")
    lsa.lsa_project_keys(dev(tie.K), dev(tie.W), kd)
    gi = host(_listed_vs_three_calls(tie, kd).idx)
    for g in range(tie.Hkv):
        np.testing.assert_array_equal(gi[0, g], np.arange(tie.B))

    say("listed decode step, keys planted at the sampled slots")
    k_idx = oracle.project_keys(case.K, case.W, case.dtype)
    q_idx = oracle.query_prep(case.Q, case.Hkv, case.W)
    n_groups = (case.T + 63) // 64
    assert n_groups < case.B          # the sample alone cannot reach B
    for g in range(case.Hkv):
        qd = q_idx[0, g] / np.linalg.norm(q_idx[0, g])
        big = synth.to_bf16_bits((6.0 * qd).astype(np.float32))
        for gi_ in range(n_groups):
            k_idx[0, g, _sample_slot(gi_, g, case.T)] = big
    kd = dev(k_idx)
    one = _listed_vs_three_calls(case, kd)
    rows = list(range(case.N * case.Hkv))
    ref = oracle.decode_step(case.Q, case.W, k_idx, case.K, case.V, case.B)
    R = case.N * case.Hkv
    want = {"idx": ref["idx"].reshape(R, case.B), "scores": ref["scores"].reshape(R, case.T),
            "out": ref["out"].reshape(R, case.G, case.d), "lse": ref["lse"].reshape(R, case.G)}
    _compare_step(case, {"idx": host(one.idx), "out": host(one.out), "lse": host(one.lse)}, want, rows)

    say("listed decode step, fp8 cache")
    k8 = torch.empty(case.N, case.Hkv, case.T, case.r, dtype=torch.float8_e4m3fn, device="cuda")
    lsa.lsa_project_keys(dev(case.K), dev(case.W), k8)
    _listed_vs_three_calls(case, k8)


@pytest.mark.parametrize("name,over,kdt", [
    ("decode_t128k_b2048", {"N": 1, "T": 40000, "B": 1024}, torch.float8_e4m3fn),   # 4 pieces per key
    ("decode_t4k_fp32", {}, torch.float32),                                          # 16 pieces per key
    ("decode_t128k_b2048", {"N": 1, "T": 40000, "B": 1024, "r": 128}, torch.bfloat16),  # 16 pieces
])
def test_decode_step_listed_rescored_rows(name, over, kdt):
    """Rows the listing path's lists cannot settle are rescored by the
    select with the scoring arithmetic (the listing launch writes no
    scores): constant keys per head (every key ties, so every row is
    rescored) over each projected-cache layout; indices and per-entry scores
    bit for bit against the three calls, and the lowest B positions."""
    case = synth.workload(name, **over)
    say("listed decode step, rescored rows", name, over, kdt)
    K = case.K.copy()
    K[:, :, :, :] = K[:, :1, :, :]
    case.K = K
    kd = torch.empty(case.N, case.Hkv, case.T, case.r, dtype=kdt, device="cuda")
    lsa.lsa_project_keys(dev(case.K), dev(case.W), kd)
    gi = host(_listed_vs_three_calls(case, kd).idx)
    for g in range(case.Hkv):
        np.testing.assert_array_equal(gi[0, g], np.arange(case.B))


@pytest.mark.parametrize("N,Hq,Hkv,T,B", [(1, 32, 8, 50000, 2048), (4, 32, 8, 20000, 1024), (2, 32, 4, 9000, 1500),
                                        (3, 12, 3, 30000, 256)])
def test_attention_merge_in_launch(N, Hq, Hkv, T, B):
    """lsa_indexed_attention with merge_ctrl (the split partials merged in
    the attention launch) against the same call without it (the merge
    kernel): out and lse bit for bit, twice on the same control words,
    which are left zero; and the no-allocation entry with the same words."""
    case = synth.make_decode_case(N=N, Hq=Hq, Hkv=Hkv, T=T, B=B, dtype=synth.BF16, seed=77)
    say("attention, merge in launch", N, Hq, Hkv, T, B)
    Q, K, V = dev(case.Q), dev(case.K), dev(case.V)
    rng = np.random.default_rng(5)
    idx = np.sort(np.stack([np.stack([rng.choice(T, B, replace=False) for _ in range(Hkv)]) for _ in range(N)]),
                  axis=-1).astype(np.int32)
    idx_d = dev(idx)
    out0 = torch.empty(N, Hq, case.d, device="cuda")
    lse0 = torch.empty(N, Hq, device="cuda")
    lsa.lsa_indexed_attention(Q, K, V, idx_d, out0, lse=lse0)
    ctrl = torch.zeros(lsa.ATTN_MERGE_CTRL_WORDS, dtype=torch.int32, device="cuda")
    for rep in range(2):
        out1 = torch.full_like(out0, 3.0)
        lse1 = torch.full_like(lse0, 3.0)
        lsa.lsa_indexed_attention(Q, K, V, idx_d, out1, lse=lse1, merge_ctrl=ctrl)
        torch.cuda.synchronize()
        assert torch.equal(out1.view(torch.int32), out0.view(torch.int32)), rep
        assert torch.equal(lse1.view(torch.int32), lse0.view(torch.int32)), rep
        assert int(ctrl.abs().sum().item()) == 0, rep
    out2 = torch.full_like(out0, 3.0)
    lsa.lsa_indexed_attention_noalloc(Q, K, V, idx_d, out2, lse=lse1, merge_ctrl=ctrl)
    torch.cuda.synchronize()
    assert torch.equal(out2.view(torch.int32), out0.view(torch.int32))
    assert int(ctrl.abs().sum().item()) == 0
    o, l = oracle.attention(case.Q, case.K, case.V, idx)
    np.testing.assert_allclose(host(out1), o, rtol=0, atol=ATTN_ATOL)
    np.testing.assert_allclose(host(lse1), l, rtol=0, atol=LSE_ATOL)


def test_decode_step_parts_equal_one_call():
    """lsa_decode_step_part: the score, select and attend parts issued one
    at a time (the score part twice, as a timing loop does) equal one
    lsa_decode_step call bit for bit, on the listing and the three-call
    paths."""
    from indexer_driven_sparse_amd import pipeline
    case = synth.workload("decode_t128k_b2048", N=2, T=50000, B=1024)
    say("decode step parts")
    N, Hq, Hkv, T, d, r, B = case.N, case.Hq, case.Hkv, case.T, case.d, case.r, case.B
    Q, W, K, V = dev(case.Q), dev(case.W), dev(case.K), dev(case.V)
    kd = torch.empty(N, Hkv, T, r, dtype=torch.bfloat16, device="cuda")
    lsa.lsa_project_keys(K, W, kd)
    for three in (False, True):
        one = pipeline.DecodePlan(N, Hq, Hkv, T, d, r, B, with_idx_scores=True, three_calls=three)
        one.run(Q, W, kd, K, V)
        parts = pipeline.DecodePlan(N, Hq, Hkv, T, d, r, B, with_idx_scores=True, three_calls=three)
        parts.step(Q, W, kd, K, V)            # allocates the workspace
        parts.idx.fill_(-5)
        parts.out.fill_(7.0)
        kw = dict(workspace=parts.step_ws, lse=parts.lse, q_idx=parts.q_idx, out_score=parts.idx_scores,
                  three_calls=three)
        for p_ in (lsa.STEP_PART_SCORE, lsa.STEP_PART_SCORE, lsa.STEP_PART_SELECT, lsa.STEP_PART_ATTEND):
            lsa.lsa_decode_step_part(p_, Q, W, kd, K, V, parts.idx, parts.out, **kw)
        torch.cuda.synchronize()
        for name_ in ("idx", "q_idx", "idx_scores", "out", "lse"):
            a_, b_ = getattr(parts, name_), getattr(one, name_)
            assert torch.equal(a_.view(torch.int32), b_.view(torch.int32)), (three, name_)
        _assert_step_ctrl_zero(parts, N * Hkv)


@pytest.mark.parametrize("name,over,fused", [
    ("decode_t128k_b2048", {"N": 1, "T": 40000, "B": 1024}, True),    # 8 rows, ragged chunks
    ("decode_t128k_b2048", {"N": 2, "Hq": 24, "Hkv": 6, "T": 20000, "B": 512}, True),  # 12 rows
    ("decode_t128k_b2048", {"N": 1, "T": 40000}, False),           # hints vouch for < B keys
    ("decode_t128k_b2048", {"N": 4}, True),                        # the headline shape
    ("decode_t32k_hitters", {}, True),
    ("decode_t4k_fp32", {}, False),                                # one row: the three calls
])
def test_decode_step_fused_equals_three_calls(name, over, fused):
    case = synth.workload(name, **over)
    say("fused decode step vs three calls", name, over)
    kd = torch.empty(case.N, case.Hkv, case.T, case.r, dtype=torch_dtype(case.dtype), device="cuda")
    lsa.lsa_project_keys(dev(case.K), dev(case.W), kd)
    plan = _fused_vs_three_calls(case, kd, reps=3)
    assert lsa.lsa_step_is_fused(dev(case.Q), dev(case.W), kd, dev(case.K), dev(case.V), plan.idx,
                                 plan.out, one_launch=True) == fused


def test_decode_step_fused_fp8_cache_and_ties():
    """The fused step over an E4M3 projected-key cache, and over a cache in
    which every key of a head is the same (each row one big tie: the hint
    lists overflow and the final selection falls back to the whole row)."""
    case = synth.workload("decode_t128k_b2048", N=1, T=30000, B=896)
    say("fused decode step, fp8 cache")
    k8 = torch.empty(case.N, case.Hkv, case.T, case.r, dtype=torch.float8_e4m3fn, device="cuda")
    lsa.lsa_project_keys(dev(case.K), dev(case.W), k8)
    assert lsa.lsa_step_is_fused(dev(case.Q), dev(case.W), k8, dev(case.K), dev(case.V),
                                 _fused_vs_three_calls(case, k8).idx,
                                 torch.empty(case.N, case.Hq, case.d, device="cuda"), one_launch=True)
    say("fused decode step, constant keys per head")
    K = case.K.copy()
    K[:, :, :, :] = K[:, :1, :, :]
    case.K = K
    kd = torch.empty(case.N, case.Hkv, case.T, case.r, dtype=torch.bfloat16, device="cuda")
    lsa.lsa_project_keys(dev(case.K), dev(case.W), kd)
    fus = _fused_vs_three_calls(case, kd)
    gi = host(fus.idx)
    for g in range(case.Hkv):          # a tie over the whole row keeps the lowest positions
        np.testing.assert_array_equal(gi[0, g], np.arange(case.B))


def test_decode_step_fused_graph_replay():
    """The fused step captured in a HIP graph: every replay (with eager work
    and synchronizations between them, alternating two caches) equals the
    eager call, and the control words come back zero each time."""
    from indexer_driven_sparse_amd import pipeline
    case = synth.workload("decode_t128k_b2048", N=1, T=50000, B=1024)
    say("fused decode step, graph replay")
    N, Hq, Hkv, T, d, r, B = case.N, case.Hq, case.Hkv, case.T, case.d, case.r, case.B
    Q, W, K, V = dev(case.Q), dev(case.W), dev(case.K), dev(case.V)
    caches = []
    for s in (0, 1):
        Kc = K if s == 0 else torch.roll(K, shifts=777, dims=1).contiguous()
        kd = torch.empty(N, Hkv, T, r, dtype=torch.bfloat16, device="cuda")
        lsa.lsa_project_keys(Kc, W, kd)
        caches.append((Kc, kd))
    plan = pipeline.DecodePlan(N, Hq, Hkv, T, d, r, B, fused=True, one_launch=True)
    want = []
    for Kc, kd in caches:
        plan.run(Q, W, kd, Kc, V)
        torch.cuda.synchronize()
        want.append((plan.idx.clone(), plan.out.clone()))
    graphs = []
    for Kc, kd in caches:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            plan.run(Q, W, kd, Kc, V)
        graphs.append(g)
    for i in range(6):
        graphs[i % 2].replay()
        torch.cuda.synchronize()
        wi, wo = want[i % 2]
        assert torch.equal(plan.idx, wi), i
        assert torch.equal(plan.out.view(torch.int32), wo.view(torch.int32)), i
        ctl = plan.step_ws[:256].view(torch.int32)
        assert int(ctl[lsa.STEP_ERROR_WORD]) == 0
        assert int(ctl.abs().sum()) == 0, i      # control words left zero
        plan.out.zero_()


def test_decode_step_budget_T_is_dense_attention():
    case = synth.make_decode_case(N=2, Hq=32, Hkv=8, T=512, B=512, dtype=synth.BF16, seed=21)
    say("decode step B=T")
    k_idx = oracle.project_keys(case.K, case.W, case.dtype)
    g = gpu_decode_step(case, dev(k_idx))
    for n in range(2):
        for gh in range(8):
            np.testing.assert_array_equal(g["idx"][n, gh], np.arange(512))
    # dense attention reference (torch CPU float64), GQA by repeating KV heads
    qt = torch.from_numpy(decoded(case.Q))[:, :, None, :]
    Kt = torch.from_numpy(decoded(case.K)).permute(0, 2, 1, 3).repeat_interleave(4, 1).contiguous()
    Vt = torch.from_numpy(decoded(case.V)).permute(0, 2, 1, 3).repeat_interleave(4, 1).contiguous()
    o = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt)[:, :, 0].numpy()
    np.testing.assert_allclose(g["out"], o, rtol=0, atol=ATTN_ATOL)


# --------------------------------------------------------------------------
# selection hint: speed only, never the result
# --------------------------------------------------------------------------

@pytest.mark.parametrize("name,over", [("decode_t128k_b2048", {"N": 1}),
                                       ("decode_t32k_hitters", {}),
                                       ("decode_t4k_fp32", {})])
def test_select_hint_never_changes_the_result(name, over):
    case = synth.workload(name, **over)
    say("select hint", name, over)
    k_idx = oracle.project_keys(case.K, case.W, case.dtype)
    kd = dev(k_idx)
    N, Hkv, T, B = case.N, case.Hkv, case.T, case.B
    sc = torch.empty(N, Hkv, T + (4 - T % 4) % 4, device="cuda")[:, :, :T]
    count, k = lsa.lsa_score_hint_layout(kd, sc, q=dev(case.Q), w=dev(case.W))
    assert count > 0 and k > 0
    hint = torch.full((N * Hkv, count), 0x12345678, dtype=torch.int32, device="cuda")
    lsa.lsa_index_score(kd, sc, q=dev(case.Q), w=dev(case.W), hint=hint)
    assert not (hint == 0x12345678).any(), "every hint entry is written"
    outs = []
    for h in [hint, None, torch.randint(-2**31, 2**31 - 1, hint.shape, dtype=torch.int32, device="cuda"),
              torch.zeros_like(hint), torch.full_like(hint, -1)]:
        idx = torch.empty(N * Hkv, B, dtype=torch.int32, device="cuda")
        lsa.lsa_topk_select(sc, B, idx, hint=h, hint_k=k)
        outs.append(host(idx))
    for o in outs[1:]:
        np.testing.assert_array_equal(o, outs[0])
    ref, _, _ = oracle.topk(host(sc).reshape(N * Hkv, T).astype(np.float64), B)
    np.testing.assert_array_equal(outs[0], ref)
    # every entry is reached by at least k keys of its row (its group's claim
    # implies this), and the entries together vouch for k*count keys
    keys = host(sc).reshape(N * Hkv, T).view(np.uint32)
    okey = np.sort(np.where(keys & 0x80000000, ~keys, keys | 0x80000000).astype(np.uint32), axis=1)
    hv = host(hint).view(np.uint32)
    r_th = -(-B // k)
    for row in range(N * Hkv):
        reach = T - np.searchsorted(okey[row], hv[row], side="left")
        assert (reach >= k).all()
        if r_th > count:
            continue   # the hints cannot vouch for B keys; the select samples instead
        # the threshold the hints imply keeps at least B keys, and not many more
        t = np.sort(hv[row])[::-1][r_th - 1]
        kept = T - np.searchsorted(okey[row], t, side="left")
        assert B <= kept <= max(8 * B, 2 * B + 4096), (row, kept)


# --------------------------------------------------------------------------
# segmented select (long rows with a hint): edge cases with hand-made hints
# --------------------------------------------------------------------------

def _order_keys(x32: np.ndarray) -> np.ndarray:
    """Order-preserving uint32 keys of float32 scores (-0 as +0, NaN lowest)."""
    u = x32.view(np.uint32).copy()
    u[u == 0x80000000] = 0
    k = np.where(u & 0x80000000, ~u, u | 0x80000000).astype(np.uint32)
    k[np.isnan(x32)] = 0
    return k


def _group_hint(x32: np.ndarray, valid: np.ndarray, k: int, group: int = 128) -> np.ndarray:
    """A valid hint: per disjoint group of `group` slots, the 16-bit prefix of
    the k-th largest valid key (0 where fewer than k are valid)."""
    rows, n = x32.shape
    ng = -(-n // group)
    keys = np.where(valid, _order_keys(x32), 0).astype(np.uint32)
    pad = np.zeros((rows, ng * group), np.uint32)
    pad[:, :n] = keys
    vpad = np.zeros((rows, ng * group), bool)
    vpad[:, :n] = valid
    g = np.sort(pad.reshape(rows, ng, group), axis=2)[:, :, group - k]
    enough = vpad.reshape(rows, ng, group).sum(axis=2) >= k
    return np.where(enough, g & 0xffff0000, 0).astype(np.uint32).view(np.int32)


def _seg_case(kind: str, rows: int, n: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, n)).astype(np.float32)
    if kind == "ties":
        x = (np.round(x * 4) / 4).astype(np.float32)
    elif kind == "recent":
        x[:, -9000:] += 10.0
    elif kind == "special":
        for val in (np.nan, np.inf, -np.inf, -0.0, 0.0):
            pos = rng.choice(n, size=300, replace=False)
            x[np.arange(rows)[:, None], pos[None, :]] = val
    elif kind == "equal":
        x[:] = 1.5
    return x


@pytest.mark.parametrize("kind,rows,n,B,group", [
    ("normal", 6, 40000, 2048, 32), ("normal", 4, 40000, 1, 32), ("normal", 3, 40000, 4096, 32),
    ("normal", 5, 33333, 777, 128), ("ties", 6, 40000, 2048, 32), ("recent", 4, 40000, 2048, 32),
    ("special", 4, 40000, 2048, 32), ("equal", 2, 40000, 2048, 32),
    ("normal", 2, 1000003, 2048, 128)])
def test_segmented_select(kind, rows, n, B, group):
    say("segmented select", kind, rows, n, B, group)
    x = _seg_case(kind, rows, n, seed=n + B)
    k = 4
    hint = _group_hint(x, np.ones_like(x, dtype=bool), k, group)
    assert hint.shape[1] * k >= B   # the hint can vouch for B keys: the segmented path runs
    ld = n + (4 - n % 4) % 4
    sc = torch.empty(rows, ld, device="cuda")[:, :n]
    sc.copy_(torch.from_numpy(x))
    hd = dev(hint)
    idx = torch.empty(rows, B, dtype=torch.int32, device="cuda")
    osc = torch.empty(rows, B, device="cuda")
    cnt = torch.empty(rows, dtype=torch.int32, device="cuda")
    assert lsa.lsa_select_workspace_bytes(sc, B, idx, hint=hd, hint_k=k) >= rows * n * 8
    lsa.lsa_topk_select(sc, B, idx, out_score=osc, out_count=cnt, hint=hd, hint_k=k)
    ref, rs, rc = oracle.topk(x, B)
    np.testing.assert_array_equal(host(idx), ref)
    np.testing.assert_array_equal(host(cnt), rc)
    sel = ref >= 0
    np.testing.assert_array_equal(host(osc)[sel], rs[sel].astype(np.float32))
    # a hint that overshoots (too few keys reach it) or takes everything
    for bad in (np.full_like(hint, np.uint32(0xffff0000).view(np.int32)), np.zeros_like(hint)):
        idx2 = torch.empty_like(idx)
        lsa.lsa_topk_select(sc, B, idx2, hint=dev(bad), hint_k=k)
        np.testing.assert_array_equal(host(idx2), ref)


def test_segmented_select_n_valid():
    rows, n, B, k = 10, 50000, 2048, 4
    say("segmented select n_valid", rows, n, B)
    x = _seg_case("normal", rows, n, seed=7)
    nv = np.array([0, 1, 100, 2048, 2049, 8191, 8192, 9000, 40000, n], np.int32)
    valid = np.arange(n)[None, :] < nv[:, None]
    hint = _group_hint(x, valid, k, 32)
    sc = torch.from_numpy(x).cuda()
    idx = torch.empty(rows, B, dtype=torch.int32, device="cuda")
    cnt = torch.empty(rows, dtype=torch.int32, device="cuda")
    lsa.lsa_topk_select(sc, B, idx, out_count=cnt, n_valid=dev(nv), hint=dev(hint), hint_k=k)
    ref, _, rc = oracle.topk(x, B, n_valid=nv)
    np.testing.assert_array_equal(host(idx), ref)
    np.testing.assert_array_equal(host(cnt), rc)


def test_segmented_select_candidates():
    rows, blk, nb, B, k = 4, 64, 700, 2048, 4
    n = blk * nb
    n_positions = 64 * 1500 - 17
    say("segmented select cand", rows, n, B)
    rng = np.random.default_rng(11)
    # an increasing block list (the contract: slot order is position order), with holes
    cand = np.stack([np.sort(rng.choice(1500, size=nb, replace=False)) for _ in range(rows)])
    cand = cand.astype(np.int32)
    cand[rng.random(cand.shape) < 0.1] = -1
    x = _seg_case("normal", rows, n, seed=12)
    slot = np.arange(n)
    pos = cand[:, slot // blk] * blk + slot % blk
    valid = (cand[:, slot // blk] >= 0) & (pos < n_positions)
    hint = _group_hint(x, valid, k, 32)
    sc = torch.from_numpy(x).cuda()
    idx = torch.empty(rows, B, dtype=torch.int32, device="cuda")
    lsa.lsa_topk_select(sc, B, idx, cand=dev(cand), cand_block=blk, n_positions=n_positions,
                        hint=dev(hint), hint_k=k)
    ref, _, _ = oracle.topk(x, B, cand=cand, cand_block=blk, n_positions=n_positions)
    np.testing.assert_array_equal(host(idx), ref)


# --------------------------------------------------------------------------
# causal prefill indexer: fused top-B == select over the unfused scores,
# and both against the oracle
# --------------------------------------------------------------------------

def _prefill_qk(kind, L, Hkv, seed):
    rng = np.random.default_rng(seed)
    if kind == "c4":
        case = synth.make_prefill_case(L, Hkv=Hkv, seed=seed)
        return case.q_idx, case.k_idx
    if kind == "int":      # integer-valued: exact scores, many exact ties
        q = rng.integers(-3, 4, size=(L, Hkv, 64)).astype(np.float32)
        k = rng.integers(-3, 4, size=(L, Hkv, 64)).astype(np.float32)
        return synth.to_bf16_bits(q), synth.to_bf16_bits(k)
    if kind == "const":    # every key equal: each row is one big tie
        q = rng.standard_normal((L, Hkv, 64)).astype(np.float32)
        k = np.broadcast_to(rng.standard_normal((1, Hkv, 64)).astype(np.float32), (L, Hkv, 64))
        return synth.to_bf16_bits(q), synth.to_bf16_bits(np.ascontiguousarray(k))
    raise KeyError(kind)


def _prefill_fused(qd, kd, B):
    L, Hkv, _ = kd.shape
    idx = torch.empty(L, Hkv, B, dtype=torch.int32, device="cuda")
    osc = torch.empty(L, Hkv, B, device="cuda")
    lsa.lsa_index_score(kd, None, q_idx=qd, mode=lsa.MODE_PREFILL_CAUSAL, topk=B, out_idx=idx,
                        out_score=osc)
    return idx, osc


def _prefill_unfused(qd, kd, B):
    L, Hkv, _ = kd.shape
    sc = torch.empty(L, Hkv, L + (4 - L % 4) % 4, device="cuda")[:, :, :L]
    lsa.lsa_index_score(kd, sc, q_idx=qd, mode=lsa.MODE_PREFILL_CAUSAL)
    idx = torch.empty(L * Hkv, B, dtype=torch.int32, device="cuda")
    osc = torch.empty(L * Hkv, B, device="cuda")
    lsa.lsa_topk_select(sc, B, idx, out_score=osc, causal_group=Hkv)
    return sc, idx.view(L, Hkv, B), osc.view(L, Hkv, B)


def test_prefill_unfused_scores_row_strides():
    # a row's full tiles leave as 16-byte pieces and its last tile (L = 1000
    # ends 8 keys into one) as 4-byte stores; the row stride must keep rows
    # 16-byte aligned, and the scores do not depend on it
    L, Hkv = 1000, 2
    q, k = _prefill_qk("c4", L, Hkv, 21)
    qd, kd = dev(q), dev(k)
    say("prefill unfused scores, row strides", L, Hkv)
    outs = []
    for ld in (L, L + 12):
        sc = torch.full((L, Hkv, ld), float("nan"), device="cuda")[:, :, :L]
        lsa.lsa_index_score(kd, sc, q_idx=qd, mode=lsa.MODE_PREFILL_CAUSAL)
        outs.append(host(sc))
    np.testing.assert_array_equal(outs[0], outs[1])
    tri = np.tril(np.ones((L, L), bool))
    for g in range(Hkv):
        assert np.isneginf(outs[0][:, g][~tri]).all() and np.isfinite(outs[0][:, g][tri]).all()
    odd = torch.empty(L, Hkv, L + 1, device="cuda")[:, :, :L]
    with pytest.raises(lsa.LsaError):
        lsa.lsa_index_score(kd, odd, q_idx=qd, mode=lsa.MODE_PREFILL_CAUSAL)


def _check_prefill_shape(idx, B):
    L = idx.shape[0]
    for i in range(L):
        for g in range(idx.shape[1]):
            row = idx[i, g]
            c = min(B, i + 1)
            assert (row[c:] == -1).all() and (row[:c] >= 0).all() and (row[:c] <= i).all(), (i, g)
            if i + 1 <= B:
                np.testing.assert_array_equal(row[:c], np.arange(i + 1))


@pytest.mark.parametrize("kind,L,Hkv,B", [("c4", 4096, 1, 2048), ("c4", 4096, 2, 2048),
                                          ("c4", 3000, 1, 700), ("c4", 1000, 1, 2048),
                                          ("c4", 777, 2, 1), ("int", 4096, 1, 2048),
                                          ("int", 2500, 2, 333), ("const", 12000, 1, 2048)])
def test_prefill_fused_equals_unfused(kind, L, Hkv, B):
    say("prefill fused vs unfused", kind, L, Hkv, B)
    q, k = _prefill_qk(kind, L, Hkv, seed=L + B)
    qd, kd = dev(q), dev(k)
    idx, osc = _prefill_fused(qd, kd, B)
    sc, idx2, osc2 = _prefill_unfused(qd, kd, B)
    gi, gi2 = host(idx), host(idx2)
    np.testing.assert_array_equal(gi, gi2)
    np.testing.assert_array_equal(host(osc).view(np.uint32) & 0x7fffffff,
                                  host(osc2).view(np.uint32) & 0x7fffffff)
    np.testing.assert_array_equal(host(osc), host(osc2))
    _check_prefill_shape(gi, B)
    if L <= 4096:
        # the scores against the oracle's fp64 ones, and the sets (near ties)
        ref_sc = oracle.prefill_scores(q, k)                       # [L, Hkv, L]
        qf, kf = decoded(q).astype(np.float64), decoded(k).astype(np.float64)
        gsc = host(sc)
        for g in range(Hkv):
            guard = np.abs(qf[:, g]) @ np.abs(kf[:, g]).T
            r_, s_ = ref_sc[:, g], gsc[:, g]
            np.testing.assert_array_equal(np.isneginf(s_), np.isneginf(r_))
            fin = np.isfinite(r_)
            assert np.all(np.abs(s_[fin] - r_[fin]) <= 1e-3 * np.abs(r_[fin]) + 1e-5 * guard[fin])
        ref_idx, _ = oracle.prefill_topk(q, k, B)
        for g in range(Hkv):
            check_index_sets(gi[:, g], ref_idx[:, g], [ref_sc[i, g] for i in range(L)], B)


def test_prefill_fused_sample_overshoot():
    """The per-row threshold comes from a key sample; keys planted at exactly
    the sampled positions make it too high for many rows, which must then
    be recomputed (the redo path) with the same result."""
    L, Hkv, B = 6000, 1, 2048
    say("prefill sample overshoot", L, Hkv, B)
    q, k = _prefill_qk("c4", L, Hkv, seed=5)
    qf = decoded(q).astype(np.float32)
    kf = decoded(k).astype(np.float32)
    # the kernel's sample: per block of 32 rows, m = min(prefix, 1024) keys,
    # one per stratum at a fixed offset
    # the last block of 32 rows samples m = 1024 of its nb = 6000 keys, one
    # per stratum at a fixed offset: plant exactly those
    nb, m = L, 1024
    planted = np.array([kk * nb // m + ((kk * 2654435761) % 2**32 >> 8) % ((kk + 1) * nb // m - kk * nb // m)
                        for kk in range(m)])
    u = qf.mean(axis=(0, 1))
    kf[planted, 0, :] += 6.0 * u / np.linalg.norm(u)
    k = synth.to_bf16_bits(kf)
    qd, kd = dev(q), dev(k)
    idx, osc = _prefill_fused(qd, kd, B)
    _, idx2, osc2 = _prefill_unfused(qd, kd, B)
    np.testing.assert_array_equal(host(idx), host(idx2))
    np.testing.assert_array_equal(host(osc), host(osc2))


def test_prefill_c4_full_size():
    """L = 65536, 1 KV head, B = 2048: every row against select over the
    unfused scores (16 GiB), sampled rows against the oracle."""
    case = synth.workload("prefill_l64k")
    L, Hkv, B = case.L, case.Hkv, case.B
    say("prefill C4 full size", L, Hkv, B)
    qd, kd = dev(case.q_idx), dev(case.k_idx)
    idx, osc = _prefill_fused(qd, kd, B)
    gi = host(idx)
    gs = host(osc)
    del osc
    sc, idx2, _ = _prefill_unfused(qd, kd, B)
    del sc
    np.testing.assert_array_equal(gi, host(idx2))
    del idx2
    torch.cuda.empty_cache()
    rows = [0, 1, 31, 32, 2046, 2047, 2048, 2049, 4095, 4096, 32767, 65534, 65535]
    rows += list(np.random.default_rng(9).integers(2050, L, size=19))
    qf = decoded(case.q_idx).astype(np.float64)
    kf = decoded(case.k_idx).astype(np.float64)
    for i in rows:
        ref, rs = oracle.prefill_topk(case.q_idx, case.k_idx, B, row_begin=i, row_end=i + 1)
        s_full = np.full(L, -np.inf)
        s_full[:i + 1] = kf[:i + 1, 0] @ qf[i, 0]
        check_index_sets(gi[i:i + 1, 0], ref[:, 0], [s_full], B)
        c = min(B, i + 1)
        sel = gi[i, 0, :c]
        guard = np.abs(kf[sel, 0]) @ np.abs(qf[i, 0])
        assert np.all(np.abs(gs[i, 0, :c] - s_full[sel]) <= 1e-3 * np.abs(s_full[sel]) + 1e-5 * guard)
    # structure of every row
    for i in range(0, L, 97):
        c = min(B, i + 1)
        row = gi[i, 0]
        assert (row[c:] == -1).all() and np.all(np.diff(row[:c]) > 0) and row[c - 1] <= i


def test_prefill_attention_c4_full_size_sampled_tokens():
    """L = 65536, 8 query heads on 1 KV head, d = 128, B = 2048: the fused
    indexer's own top-2048 lists feed per-token causal prefill attention in
    the benchmark's launch shape; sampled tokens against the oracle's fp64
    attention over the same lists (positions after the token masked: the
    oracle sees the cache cut at the token)."""
    case = synth.workload("prefill_l64k")
    L, Hkv, B, Hq, d = case.L, case.Hkv, case.B, case.Hq, case.d
    say("prefill attention C4 full size, sampled tokens", L, Hq, Hkv, d, B)
    qd, kd = dev(case.q_idx), dev(case.k_idx)
    idx = torch.empty(L, Hkv, B, dtype=torch.int32, device="cuda")
    lsa.lsa_index_score(kd, None, q_idx=qd, mode=lsa.MODE_PREFILL_CAUSAL, topk=B, out_idx=idx)
    del qd, kd
    torch.cuda.empty_cache()
    Q, K, V = dev(case.Q), dev(case.K), dev(case.V)
    out = torch.empty(L, Hq, d, device="cuda")
    lse = torch.empty(L, Hq, device="cuda")
    lsa.lsa_indexed_attention(Q, K, V, idx, out, lse=lse, mode=lsa.MODE_PREFILL_CAUSAL)
    torch.cuda.synchronize()
    gi, go, gl = host(idx), host(out), host(lse)
    tokens = [0, 1, 2, 31, 32, 2046, 2047, 2048, 2049, 4095, 4096, 32767, 32768, 65534, 65535]
    tokens += sorted(int(t) for t in np.random.default_rng(11).choice(np.arange(3, L - 1), 25,
                                                                       replace=False))
    for i in tokens:
        c = min(B, i + 1)
        row = gi[i, 0]
        assert (row[c:] == -1).all() and (row[:c] >= 0).all() and (row[:c] <= i).all(), i
        o, l = oracle.attention(case.Q[i:i + 1], case.K[:, :i + 1], case.V[:, :i + 1], gi[i:i + 1])
        np.testing.assert_allclose(go[i], o[0], rtol=0, atol=ATTN_ATOL, err_msg=f"token {i}")
        np.testing.assert_allclose(gl[i], l[0], rtol=0, atol=LSE_ATOL, err_msg=f"token {i}")


@pytest.mark.timeout(900)
def test_prefill_c4_every_row_against_the_oracle():
    """L = 65536, B = 2048: every one of the 65536 rows of the fused
    selection against the oracle's exact top-B (fp64 scores), chunk by chunk;
    a differing row passes only through near-ties at its B-th score."""
    case = synth.workload("prefill_l64k")
    L, Hkv, B = case.L, case.Hkv, case.B
    say("prefill C4, every row against the oracle", L, Hkv, B)
    qd, kd = dev(case.q_idx), dev(case.k_idx)
    idx, osc = _prefill_fused(qd, kd, B)
    gi = host(idx)
    del idx, osc
    torch.cuda.empty_cache()
    oracle.set_threads(len(os.sched_getaffinity(0)))
    qf = decoded(case.q_idx).astype(np.float64)
    kf = decoded(case.k_idx).astype(np.float64)
    near_ties = []
    step = 4096
    for r0 in range(0, L, step):
        r1 = min(L, r0 + step)
        ref, _ = oracle.prefill_topk(case.q_idx, case.k_idx, B, row_begin=r0, row_end=r1)
        same = (ref[:, 0] == gi[r0:r1, 0]).all(axis=1)
        for j in np.nonzero(~same)[0]:
            i = r0 + int(j)
            s_full = np.full(L, -np.inf)
            s_full[:i + 1] = kf[:i + 1, 0] @ qf[i, 0]
            near_ties += [i] if check_index_sets(gi[i:i + 1, 0], ref[j:j + 1, 0], [s_full], B) else []
        say(f"  rows {r0}..{r1 - 1}: {int(same.sum())} identical")
    say("  rows differing through near-ties:", len(near_ties), near_ties[:8])
    assert len(near_ties) <= L // 1000


# --------------------------------------------------------------------------
# query-block-shared prefill selection
# --------------------------------------------------------------------------

def _block_select_gpu(qd, kd, B, qb, with_scores=True):
    L, Hkv, _ = kd.shape
    nb = (L + qb - 1) // qb
    sc = None
    if with_scores:
        sc = torch.empty(nb, Hkv, L + (4 - L % 4) % 4, device="cuda")[:, :, :L]
    idx = torch.full((nb, Hkv, B), -7, dtype=torch.int32, device="cuda")
    osc = torch.empty(nb, Hkv, B, device="cuda")
    lsa.lsa_index_score(kd, sc, q_idx=qd, mode=lsa.MODE_PREFILL_CAUSAL, topk=B, out_idx=idx,
                        out_score=osc, query_block=qb)
    return sc, idx, osc


@pytest.mark.parametrize("kind,L,Hkv,qb,B", [("c4", 3000, 1, 64, 512), ("c4", 2500, 2, 16, 300),
                                             ("int", 2000, 1, 32, 256), ("c4", 777, 2, 100, 50),
                                             ("const", 4100, 1, 64, 2048)])
def test_prefill_block_selection(kind, L, Hkv, qb, B):
    """Block scores against the oracle's (fp32 MFMA vs fp64), the selection
    exactly equal to the oracle's top-B over the GPU's own block scores, and
    to the oracle's selection up to near-ties."""
    say("prefill block selection", kind, L, Hkv, qb, B)
    q, k = _prefill_qk(kind, L, Hkv, seed=L + qb)
    qd, kd = dev(q), dev(k)
    sc, idx, osc = _block_select_gpu(qd, kd, B, qb)
    nb = (L + qb - 1) // qb
    gsc = host(sc).reshape(nb * Hkv, L)
    ridx, rsc, rscores = oracle.prefill_block_topk(q, k, B, qb, want_scores=True)
    rscores = rscores.reshape(nb * Hkv, L)
    qf = decoded(q).astype(np.float64)
    kf = decoded(k).astype(np.float64)
    qmax = np.abs(np.concatenate([qf, np.zeros((nb * qb - L, Hkv, qf.shape[2]))])
                  ).reshape(nb, qb, Hkv, -1).max(axis=1).reshape(nb * Hkv, -1)   # bounds |block mean|
    kk = np.broadcast_to(kf.transpose(1, 0, 2)[None], (nb, Hkv, L, kf.shape[2])).reshape(nb * Hkv, L, -1)
    assert_scores_close(gsc, rscores, qmax, kk)
    gi = host(idx).reshape(nb * Hkv, B)
    valid = np.minimum(L, (np.arange(nb * Hkv) // Hkv + 1) * qb).astype(np.int32)
    exact, esc, _ = oracle.topk(gsc, B, n_valid=valid)
    np.testing.assert_array_equal(gi, exact)
    np.testing.assert_array_equal(host(osc).reshape(nb * Hkv, B)[gi >= 0], esc[gi >= 0])
    check_index_sets(gi, ridx.reshape(nb * Hkv, B), list(rscores), B)


@pytest.mark.parametrize("L,Hq,Hkv,d,qb,B", [(1000, 8, 1, 128, 64, 256), (700, 8, 2, 128, 16, 100),
                                             (333, 4, 1, 64, 50, 40)])
def test_prefill_block_attention(L, Hq, Hkv, d, qb, B):
    """Every token attends to its block's selection, masked causally."""
    say("prefill block attention", L, Hq, Hkv, d, qb, B)
    rng = np.random.default_rng(L + qb)
    q = synth.to_bf16_bits(rng.standard_normal((L, Hq, d)).astype(np.float32))
    K = synth.to_bf16_bits(rng.standard_normal((1, L, Hkv, d)).astype(np.float32))
    V = synth.to_bf16_bits(rng.standard_normal((1, L, Hkv, d)).astype(np.float32))
    nb = (L + qb - 1) // qb
    blk = np.full((nb, Hkv, B), -1, np.int32)
    for b in range(nb):
        hi = min(L, (b + 1) * qb)
        for g in range(Hkv):
            c = min(B, hi)
            blk[b, g, :c] = np.sort(rng.choice(hi, c, replace=False))
    out = torch.full((L, Hq, d), float("nan"), device="cuda")
    lse = torch.full((L, Hq), float("nan"), device="cuda")
    lsa.lsa_indexed_attention(dev(q), dev(K), dev(V), dev(blk), out, lse=lse,
                              mode=lsa.MODE_PREFILL_CAUSAL, query_block=qb)
    ref, rlse = oracle.attention(q, K, V, blk, prefill=True, query_block=qb)
    np.testing.assert_allclose(host(out), ref, rtol=0, atol=ATTN_ATOL)
    np.testing.assert_allclose(host(lse), rlse, rtol=0, atol=LSE_ATOL)


def test_prefill_block_c4_full_size():
    """L = 65536, 1 KV head, B = 2048, blocks of 64 tokens: every block row
    against the oracle (near-ties tolerated), exactly against the oracle's
    top-B over the GPU's block scores for sampled rows, and attention of
    sampled tokens through the plan."""
    from indexer_driven_sparse_amd import pipeline
    case = synth.workload("prefill_l64k")
    L, Hkv, B, qb = case.L, case.Hkv, case.B, 64
    say("prefill block C4 full size", L, Hkv, B, qb)
    qd, kd = dev(case.q_idx), dev(case.k_idx)
    plan = pipeline.PrefillPlan(L, case.Hq, Hkv, case.d, case.r, B, query_block=qb)
    Q, K, V = dev(case.Q), dev(case.K), dev(case.V)
    plan.run(qd, kd, Q, K, V)
    torch.cuda.synchronize()
    gi = host(plan.idx).reshape(-1, B)
    nb = L // qb
    ridx, _, rscores = oracle.prefill_block_topk(case.q_idx, case.k_idx, B, qb, want_scores=True)
    diff = check_index_sets(gi, ridx.reshape(nb, B), list(rscores.reshape(nb, L)), B)
    assert len(diff) <= nb // 20, f"{len(diff)} block rows differ by near-ties"
    sc, idx2, _ = _block_select_gpu(qd, kd, B, qb)
    np.testing.assert_array_equal(host(idx2).reshape(-1, B), gi)      # plan == direct call
    rows = [0, 1, 31, 32, 33, 511, 1023]
    gsc = host(sc[rows]).reshape(len(rows), L)
    exact, _, _ = oracle.topk(gsc, B, n_valid=np.minimum(L, (np.array(rows) + 1) * qb).astype(np.int32))
    np.testing.assert_array_equal(gi[rows], exact)
    del sc, idx2
    toks = [0, 63, 64, 127, 2047, 2048, 40000, 65535]
    out, lse = host(plan.out), host(plan.lse)
    for i in toks:
        sel = gi[i // qb]
        sel = np.where((sel >= 0) & (sel <= i), sel, -1).astype(np.int32)[None, None]
        o, l = oracle.attention(case.Q[i:i + 1], case.K, case.V, sel, prefill=False)
        np.testing.assert_allclose(out[i], o[0], rtol=0, atol=ATTN_ATOL)
        np.testing.assert_allclose(lse[i], l[0], rtol=0, atol=LSE_ATOL)


# --------------------------------------------------------------------------
# hierarchical coarse-to-fine decode, stage by stage against the oracle
# --------------------------------------------------------------------------

@pytest.mark.parametrize("T", [131072, 1048576])
def test_hierarchical_decode(T):
    case = synth.workload("hier_t1m", T=T)
    N, Hq, Hkv, d, r, B, blk, Bc = case.N, case.Hq, case.Hkv, case.d, case.r, case.B, case.block, case.B_coarse
    say("hierarchical decode", T, Hkv, blk, Bc, B)
    k_idx = oracle.project_keys(case.K, case.W, case.dtype)          # [N, Hkv, T, r]
    cent = oracle.centroids(k_idx, blk)
    from indexer_driven_sparse_amd import pipeline
    Qd, Wd, Kd, Vd = dev(case.Q), dev(case.W), dev(case.K), dev(case.V)
    kd = dev(k_idx)
    cd = torch.empty(N, Hkv, T // blk, r, dtype=torch.bfloat16, device="cuda")
    lsa.lsa_build_centroids(kd, blk, cd)
    np.testing.assert_array_equal(host(cd), cent)
    plan = pipeline.HierarchicalPlan(N, Hq, Hkv, T, d, r, B, blk, Bc, fused=False)   # the five calls
    plan.run(Qd, Wd, kd, cd, Kd, Vd)
    torch.cuda.synchronize()
    qi = oracle.query_prep(case.Q, Hkv, case.W)
    # coarse: centroid scores, kept blocks
    csc = oracle.scores(qi, cent)
    cq = decoded(cent)
    assert_scores_close(host(plan.coarse).reshape(N * Hkv, -1), csc.reshape(N * Hkv, -1),
                        qi.reshape(N * Hkv, r), cq.reshape(N * Hkv, -1, r))
    gblocks = host(plan.blocks)
    rblocks, _, _ = oracle.topk(csc.reshape(N * Hkv, -1), Bc)
    check_index_sets(gblocks.reshape(N * Hkv, Bc), rblocks, list(csc.reshape(N * Hkv, -1)), Bc)
    # fine, re-anchored on the GPU's blocks
    fsc = oracle.scores(qi, k_idx, cand=gblocks, cand_block=blk)
    ridx, _, _ = oracle.topk(fsc.reshape(N * Hkv, -1), B, cand=gblocks.reshape(N * Hkv, Bc),
                             cand_block=blk, n_positions=T)
    gidx = host(plan.idx).reshape(N * Hkv, B)
    pos_scores = []
    for row in range(N * Hkv):
        full = np.full(T, -np.inf)
        pos = (gblocks.reshape(N * Hkv, Bc)[row][:, None] * blk + np.arange(blk)[None, :]).reshape(-1)
        full[pos] = fsc.reshape(N * Hkv, -1)[row]
        pos_scores.append(full)
        # the final set lies inside the kept blocks
        assert np.isin(gidx[row] // blk, gblocks.reshape(N * Hkv, Bc)[row]).all()
    check_index_sets(gidx, ridx, pos_scores, B)
    # attention, re-anchored on the GPU's index set
    out, lse = oracle.attention(case.Q, case.K, case.V, host(plan.idx))
    np.testing.assert_allclose(host(plan.out), out, rtol=0, atol=ATTN_ATOL)
    np.testing.assert_allclose(host(plan.lse), lse, rtol=0, atol=LSE_ATOL)


# --------------------------------------------------------------------------
# the decode step captured in a HIP graph: every replay equals eager
# --------------------------------------------------------------------------

@pytest.mark.parametrize("nbytes", [16, 4096 * 16 + 48, 64 << 20])
def test_stream_read_reads_every_word(nbytes):
    # the bandwidth reference really reads the whole buffer: its sink words
    # (all overwritten) fold to the XOR of the buffer's words
    rng = np.random.default_rng(nbytes)
    words = rng.integers(-2**31, 2**31, nbytes // 4, dtype=np.int64).astype(np.int32)
    say("stream read", nbytes)
    buf = dev(words)
    sink = torch.full((lsa.STREAM_READ_SINK_WORDS,), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
    lsa.lsa_stream_read(buf, sink)
    assert int(np.bitwise_xor.reduce(host(sink))) == int(np.bitwise_xor.reduce(words))


def test_decode_step_graph_replay():
    from indexer_driven_sparse_amd import pipeline
    case = synth.workload("decode_t32k_hitters")
    say("decode graph replay", case.T)
    Q, W, K, V = dev(case.Q), dev(case.W), dev(case.K), dev(case.V)
    kd = torch.empty(case.N, case.Hkv, case.T, case.r, dtype=torch.bfloat16, device="cuda")
    lsa.lsa_project_keys(K, W, kd)
    plan = pipeline.DecodePlan(case.N, case.Hq, case.Hkv, case.T, case.d, case.r, case.B,
                               with_idx_scores=True)
    plan.run(Q, W, kd, K, V)           # eager, also warms one-time setup
    torch.cuda.synchronize()
    ref = {k: getattr(plan, k).clone() for k in ("idx", "idx_scores", "out", "lse", "q_idx")}
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        plan.run(Q, W, kd, K, V)
    for rep in range(4):
        for t in (plan.idx, plan.out, plan.lse):   # eager work between replays
            t.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in ref.items():
            assert torch.equal(getattr(plan, k), v), (rep, k)


# --------------------------------------------------------------------------
# OCP E4M3 fp8 projected-key cache (JSSA Fig. 10)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("T,per_head", [(1000, False), (4096, True)])
def test_project_keys_fp8_bit_exact(T, per_head):
    rng = np.random.default_rng(T)
    N, Hkv, d, r = 2, 3, 128, 64
    K = synth.to_bf16_bits(rng.standard_normal((N, T, Hkv, d)).astype(np.float32) * 3)
    W = (rng.standard_normal((Hkv, d, r) if per_head else (d, r)) / math.sqrt(d)).astype(np.float32)
    say("project fp8", T, per_head)
    ref = oracle.project_keys(K, W, oracle.FP8)
    out = torch.empty(N, Hkv, T, r, dtype=torch.float8_e4m3fn, device="cuda")
    lsa.lsa_project_keys(dev(K), dev(W), out)
    np.testing.assert_array_equal(host(out), ref)
    # large values saturate at +-448 on both sides
    Wbig = (W * 400).astype(np.float32)
    ref2 = oracle.project_keys(K, Wbig, oracle.FP8)
    lsa.lsa_project_keys(dev(K), dev(Wbig), out)
    np.testing.assert_array_equal(host(out), ref2)
    assert (np.abs(decoded(ref2)) == 448).any()


def test_centroids_fp8_bit_exact():
    rng = np.random.default_rng(8)
    k = oracle.project_keys(synth.to_bf16_bits(rng.standard_normal((2, 1000, 3, 128)).astype(np.float32)),
                            (rng.standard_normal((128, 64)) / 11.3).astype(np.float32), oracle.FP8)
    say("centroids fp8")
    ref = oracle.centroids(k, 64)
    out = torch.empty(2, 3, ref.shape[2], 64, dtype=torch.float8_e4m3fn, device="cuda")
    lsa.lsa_build_centroids(dev(k), 64, out)
    np.testing.assert_array_equal(host(out), ref)


@pytest.mark.parametrize("N,Hq,Hkv,T", [(1, 32, 8, 5000), (2, 8, 2, 70001)])
def test_decode_scores_fp8(N, Hq, Hkv, T):
    case = synth.make_decode_case(N=N, Hq=Hq, Hkv=Hkv, T=T, d=128, r=64, B=16, dtype=synth.BF16,
                                  seed=T + 1)
    k_idx = oracle.project_keys(case.K, case.W, oracle.FP8)
    say("scores fp8", N, Hq, Hkv, T)
    q_ref = oracle.query_prep(case.Q, Hkv, case.W)
    ref = oracle.scores(q_ref, k_idx)
    sc = torch.empty(N, Hkv, T + (4 - T % 4) % 4, device="cuda")[:, :, :T]
    lsa.lsa_index_score(dev(k_idx), sc, q=dev(case.Q), w=dev(case.W))
    assert_scores_close(host(sc).reshape(N * Hkv, T), ref.reshape(N * Hkv, T),
                        q_ref.reshape(N * Hkv, 64), decoded(k_idx).reshape(N * Hkv, T, 64))


@pytest.mark.parametrize("name,over", [("decode_t32k_hitters", {}),
                                       ("decode_t128k_b2048", {"N": 1, "T": 9000})])
def test_decode_step_fp8_cache(name, over):
    case = synth.workload(name, **over)
    say("decode step fp8 cache", name, over)
    k_idx = oracle.project_keys(case.K, case.W, oracle.FP8)
    g = gpu_decode_step(case, dev(k_idx))
    rows = list(range(case.N * case.Hkv))
    ref = _oracle_rows(case, rows, kidx_dtype=oracle.FP8)
    _compare_step(case, g, ref, rows)


@pytest.mark.parametrize("T,ties,kdt,N", [(131072, False, torch.bfloat16, 1), (1048576, False, torch.bfloat16, 1),
                                           (100000, False, torch.bfloat16, 1), (131072, True, torch.bfloat16, 1),
                                           (131072, False, torch.float8_e4m3fn, 1),
                                           (100000, True, torch.float8_e4m3fn, 1),
                                           (60000, False, torch.bfloat16, 3)])
def test_hier_step_equals_separate_calls(T, ties, kdt, N):
    """lsa_hier_decode_step (both stages listed in their scoring launches
    with LSA_STEP_LISTED, as separate calls with LSA_STEP_THREE_CALLS, and
    the default, which picks by row length) against the five separate calls:
    kept blocks, indices, per-entry scores, q_idx, out and lse bit for bit,
    twice on one workspace whose control words are left zero. T=100000 has
    a partial last block; with every key of a head equal every fine row
    ties throughout, so its lists overflow and the select rescores the row
    through the candidate map. The fp8 cases run the E4M3 projected-key
    cache (block summaries in E4M3 as well); N=3 runs several sequences."""
    from indexer_driven_sparse_amd import pipeline
    case = synth.workload("hier_t1m", T=T, N=N)
    say("hierarchical step vs separate calls", T, ties, kdt, N)
    N, Hq, Hkv, d, r, B, blk, Bc = case.N, case.Hq, case.Hkv, case.d, case.r, case.B, case.block, case.B_coarse
    Qd, Wd, Vd = dev(case.Q), dev(case.W), dev(case.V)
    Kd = dev(case.K)
    if ties:
        Kd = Kd[:, :1].expand(N, T, Hkv, d).contiguous()
    kd = torch.empty(N, Hkv, T, r, dtype=kdt, device="cuda")
    lsa.lsa_project_keys(Kd, Wd, kd)
    nb = (T + blk - 1) // blk
    cd = torch.empty(N, Hkv, nb, r, dtype=kdt, device="cuda")
    lsa.lsa_build_centroids(kd, blk, cd)
    ref = pipeline.HierarchicalPlan(N, Hq, Hkv, T, d, r, B, blk, Bc, fused=False, kidx_dtype=kdt)
    ref.run(Qd, Wd, kd, cd, Kd, Vd)
    default_path = "listed" if Bc * blk >= lsa.HIER_LIST_MIN_SLOTS else "three_calls"
    for mode, want_path in (("listed", "listed"), ("three", "three_calls"), ("default", default_path)):
        one = pipeline.HierarchicalPlan(N, Hq, Hkv, T, d, r, B, blk, Bc, three_calls=mode == "three",
                                        listed=mode == "listed", kidx_dtype=kdt)
        assert one.path(Qd, Wd, kd, cd, Kd, Vd) == want_path
        for rep in range(2):
            one.idx.fill_(-9)
            one.out.fill_(5.0)
            one.run(Qd, Wd, kd, cd, Kd, Vd)
            torch.cuda.synchronize()
            for name_ in ("blocks", "idx", "idx_scores", "q_idx", "out", "lse"):
                a_, b_ = getattr(one, name_), getattr(ref, name_)
                assert torch.equal(a_.view(torch.int32), b_.view(torch.int32)), (mode, rep, name_)
            rows = N * Hkv
            ctl = one.step_ws[:4 * (1024 + 1024 * rows)].view(torch.int32)
            assert int(ctl.abs().sum().item()) == 0, (mode, rep)
    if ties:   # a tie over the whole row keeps the lowest positions of the kept blocks
        gi, gb = host(one.idx), host(one.blocks)
        for g in range(Hkv):
            pos = np.sort((gb[0, g][:, None] * blk + np.arange(blk)[None, :]).reshape(-1))
            pos = pos[pos < T]
            np.testing.assert_array_equal(gi[0, g], pos[:B])


def test_hier_step_graph_replay():
    """The one-call hierarchical step captured in HIP graphs (two caches,
    alternating): every replay, with eager work and synchronizations between
    replays, equals the eager call bit for bit, and the workspace's control
    words come back zero each time."""
    from indexer_driven_sparse_amd import pipeline
    case = synth.workload("hier_t1m", T=131072)
    say("hierarchical step, graph replay")
    N, Hq, Hkv, T, d, r, B, blk, Bc = case.N, case.Hq, case.Hkv, case.T, case.d, case.r, case.B, case.block, \
        case.B_coarse
    Qd, Wd, Vd = dev(case.Q), dev(case.W), dev(case.V)
    K0 = dev(case.K)
    caches = []
    for s in (0, 1):
        Kc = K0 if s == 0 else torch.roll(K0, shifts=4099, dims=1).contiguous()
        kd = torch.empty(N, Hkv, T, r, dtype=torch.bfloat16, device="cuda")
        lsa.lsa_project_keys(Kc, Wd, kd)
        cd = torch.empty(N, Hkv, T // blk, r, dtype=torch.bfloat16, device="cuda")
        lsa.lsa_build_centroids(kd, blk, cd)
        caches.append((Kc, kd, cd))
    plan = pipeline.HierarchicalPlan(N, Hq, Hkv, T, d, r, B, blk, Bc)
    names = ("blocks", "idx", "idx_scores", "q_idx", "out", "lse")
    want = []
    for Kc, kd, cd in caches:
        plan.run(Qd, Wd, kd, cd, Kc, Vd)
        torch.cuda.synchronize()
        want.append({k: getattr(plan, k).clone() for k in names})
    assert not torch.equal(want[0]["idx"], want[1]["idx"])   # the two caches select differently
    graphs = []
    for Kc, kd, cd in caches:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            plan.run(Qd, Wd, kd, cd, Kc, Vd)
        graphs.append(g)
    rows = N * Hkv
    for i in range(6):
        for t in (plan.idx, plan.out, plan.lse):   # eager work between replays
            t.fill_(-7)
        torch.cuda.synchronize()
        graphs[i % 2].replay()
        torch.cuda.synchronize()
        for k in names:
            assert torch.equal(getattr(plan, k).view(torch.int32), want[i % 2][k].view(torch.int32)), (i, k)
        ctl = plan.step_ws[:4 * (1024 + 1024 * rows)].view(torch.int32)
        assert int(ctl.abs().sum().item()) == 0, i
