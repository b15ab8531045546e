"""The C ABI on a CPU-only host: the library loads, exports every entry
point include/lsa.h declares, agrees with the binding on descriptor sizes,
and rejects bad arguments during validation -- before any HIP call, so these
calls run without a GPU."""
import ctypes
import os
import re

import pytest

import torch
from indexer_driven_sparse_amd import lsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lsa.h")

INVALID, UNSUPPORTED, WORKSPACE = -1, -2, -3


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^[A-Za-z_][\w \*]*?\b(lsa_\w+)\s*\(", text, re.M)))


def test_header_declares_the_path_calls():
    names = declared_functions()
    for fn in ["lsa_index_score", "lsa_topk_select", "lsa_indexed_attention",
               "lsa_project_keys", "lsa_build_centroids"]:
        assert fn in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(lsa.library_path())
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_descriptor_sizes_and_abi_version():
    lib = lsa._lib()
    for which, cls in lsa.DESCS.items():
        assert lib.lsa_desc_size(which) == ctypes.sizeof(cls)
    assert lib.lsa_desc_size(99) == 0
    assert lsa.abi_version() == 1
    for st in [0, -1, -2, -3, -4, -5, -6]:
        assert lib.lsa_status_str(st)
    assert lib.lsa_status_str(12345) == b"unknown status"


def _score_desc(**kw):
    d = lsa.ScoreDesc()
    d.struct_size = ctypes.sizeof(lsa.ScoreDesc)
    d.mode, d.n_seq, d.n_kv_heads, d.n_keys, d.rank = 0, 1, 2, 100, 64
    d.q_idx = 0x1000
    d.k_idx = 0x2000
    d.k_idx_dtype = lsa.BF16
    d.k_stride_seq, d.k_stride_head, d.k_stride_tok = 2 * 100 * 64, 100 * 64, 64
    d.scores = 0x3000
    d.scores_ld = 100
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def _call_score(d):
    return lsa._lib().lsa_index_score(ctypes.byref(d), None, 0, None)


@pytest.mark.parametrize("field,value,code", [
    ("struct_size", 8, INVALID),
    ("n_kv_heads", 0, INVALID),
    ("n_keys", 0, INVALID),
    ("rank", 48, UNSUPPORTED),            # 96 bytes: not a power of two
    ("rank", 4, UNSUPPORTED),             # 8 bytes: below one 128-bit load
    ("k_idx", 0, INVALID),
    ("k_idx", 0x2008, INVALID),           # misaligned base
    ("k_stride_tok", 60, INVALID),        # row stride not 16-byte multiple / overlapping
    ("k_idx_dtype", 7, UNSUPPORTED),
    ("q_idx", 0, INVALID),                # neither q nor q_idx
    ("scores", 0, INVALID),
    ("scores", 0x3004, INVALID),
    ("scores_ld", 98, INVALID),
    ("scores_ld", 102, INVALID),          # not a multiple of 4
    ("topk", 5, INVALID),                 # fused select is prefill-only
    ("mode", 9, INVALID),
])
def test_score_validation(field, value, code):
    assert _call_score(_score_desc(**{field: value})) == code


def test_score_validation_prep_and_candidates():
    d = _score_desc(q=0x4000, q_dtype=lsa.BF16, n_q_heads=3, head_dim=128, w=0x5000)
    assert _call_score(d) == INVALID                        # Hq % Hkv != 0
    d = _score_desc(q=0x4000, q_dtype=lsa.BF16, n_q_heads=8, head_dim=1024, w=0x5000)
    assert _call_score(d) == UNSUPPORTED                    # d > 512
    d = _score_desc(q=0x4000, q_dtype=lsa.BF16, n_q_heads=8, head_dim=128, w=0)
    assert _call_score(d) == INVALID                        # no W
    d = _score_desc(cand=0x6000, n_cand=4, cand_block=0, cand_ld=4)
    assert _call_score(d) == INVALID
    d = _score_desc(cand=0x6000, n_cand=4, cand_block=64, cand_ld=3)
    assert _call_score(d) == INVALID
    d = _score_desc(cand=0x6000, n_cand=4, cand_block=64, cand_ld=4, scores_ld=252)
    assert _call_score(d) == INVALID                        # 256 slots do not fit
    d = _score_desc(n_seq=40000)
    assert _call_score(d) == UNSUPPORTED                    # rows beyond the grid


def _select_desc(**kw):
    d = lsa.SelectDesc()
    d.struct_size = ctypes.sizeof(lsa.SelectDesc)
    d.rows, d.n, d.topk = 4, 1000, 10
    d.scores, d.scores_ld = 0x1000, 1000
    d.out_idx = 0x2000
    for k, v in kw.items():
        setattr(d, k, v)
    return d


@pytest.mark.parametrize("field,value,code", [
    ("struct_size", 0, INVALID), ("rows", 0, INVALID), ("n", 0, INVALID), ("topk", 0, INVALID),
    ("scores", 0, INVALID), ("scores", 0x1008, INVALID), ("scores_ld", 999, INVALID),
    ("scores_ld", 996, INVALID), ("out_idx", 0, INVALID), ("causal_group", -1, INVALID),
])
def test_select_validation(field, value, code):
    d = _select_desc(**{field: value})
    assert lsa._lib().lsa_topk_select(ctypes.byref(d), None, 0, None) == code


def test_select_validation_combinations_and_workspace():
    lib = lsa._lib()
    d = _select_desc(causal_group=1, n_valid=0x3000)
    assert lib.lsa_topk_select(ctypes.byref(d), None, 0, None) == INVALID
    d = _select_desc(cand=0x3000, cand_block=64, cand_ld=15)          # 1000 slots need 16 entries
    assert lib.lsa_topk_select(ctypes.byref(d), None, 0, None) == INVALID
    big = _select_desc(n=300000, scores_ld=300000)                     # bitmaps go to workspace
    need = lib.lsa_select_workspace_bytes(ctypes.byref(big))
    assert need == 4 * 2 * ((300000 + 31) // 32) * 4
    assert lib.lsa_topk_select(ctypes.byref(big), None, 0, None) == WORKSPACE
    assert lib.lsa_select_workspace_bytes(ctypes.byref(_select_desc())) == 0


def _attn_desc(**kw):
    d = lsa.AttnDesc()
    d.struct_size = ctypes.sizeof(lsa.AttnDesc)
    d.mode, d.rows, d.n_q_heads, d.n_kv_heads, d.head_dim, d.topk, d.n_keys = 0, 4, 32, 8, 128, 2048, 131072
    d.q, d.k, d.v, d.idx, d.out = 0x1000, 0x2000, 0x3000, 0x4000, 0x5000
    d.q_dtype = d.kv_dtype = lsa.BF16
    d.kv_stride_seq, d.kv_stride_tok, d.kv_stride_head = 131072 * 8 * 128, 8 * 128, 128
    for k, v in kw.items():
        setattr(d, k, v)
    return d


@pytest.mark.parametrize("field,value,code", [
    ("struct_size", 1, INVALID), ("mode", 5, INVALID), ("rows", 0, INVALID),
    ("n_q_heads", 30, INVALID), ("n_q_heads", 4, INVALID), ("head_dim", 96, UNSUPPORTED),
    ("n_q_heads", 256, UNSUPPORTED), ("topk", 0, INVALID), ("n_keys", 0, INVALID),
    ("q_dtype", lsa.F32, UNSUPPORTED), ("k", 0, INVALID), ("v", 0x3002, INVALID),
    ("kv_stride_tok", 8 * 128 + 4, INVALID), ("idx", 0, INVALID), ("out", 0, INVALID),
])
def test_attention_validation(field, value, code):
    d = _attn_desc(**{field: value})
    assert lsa._lib().lsa_indexed_attention(ctypes.byref(d), None, 0, None) == code


@pytest.mark.parametrize("kw,code", [
    (dict(slot_table_ld=131071), INVALID),           # narrower than n_keys
    (dict(n_pool_rows=0), INVALID),
    (dict(slot_table=0x6002), INVALID),              # int32 table must be 4-byte aligned
])
def test_attention_paged_validation(kw, code):
    base = dict(slot_table=0x6000, slot_table_ld=131072, n_pool_rows=4 * 131072)
    base.update(kw)
    d = _attn_desc(**base)
    assert lsa._lib().lsa_indexed_attention(ctypes.byref(d), None, 0, None) == code


def test_attention_paged_ignores_seq_stride():
    # a pool has no per-sequence base: a misaligned kv_stride_seq is not looked at
    lib = lsa._lib()
    d = _attn_desc(slot_table=0x6000, slot_table_ld=131072, n_pool_rows=8, kv_stride_seq=3)
    assert lib.lsa_indexed_attention(ctypes.byref(d), None, 0, None) == WORKSPACE
    u = _attn_desc(kv_stride_seq=3)
    assert lib.lsa_indexed_attention(ctypes.byref(u), None, 0, None) == INVALID


def test_attention_workspace_sizing():
    lib = lsa._lib()
    d = _attn_desc()
    need = lib.lsa_attention_workspace_bytes(ctypes.byref(d))
    assert need > 0 and need % (4 * (128 + 2)) == 0
    assert lib.lsa_indexed_attention(ctypes.byref(d), None, 0, None) == WORKSPACE
    assert lib.lsa_indexed_attention(ctypes.byref(d), ctypes.c_void_p(0x10000), need - 16, None) == WORKSPACE
    p = _attn_desc(mode=1, rows=65536, n_q_heads=8, n_kv_heads=1, topk=2048, n_keys=65536)
    assert lib.lsa_attention_workspace_bytes(ctypes.byref(p)) == 0   # one split per query row


def test_setup_validation():
    lib = lsa._lib()
    d = lsa.ProjectDesc()
    d.struct_size = ctypes.sizeof(lsa.ProjectDesc)
    d.n_seq, d.n_kv_heads, d.head_dim, d.rank, d.n_tok = 1, 1, 128, 64, 10
    d.k, d.w, d.out = 0x1000, 0x2000, 0x3000
    d.rank = 48
    assert lib.lsa_project_keys(ctypes.byref(d), None) == UNSUPPORTED
    d.rank, d.head_dim = 64, 600
    assert lib.lsa_project_keys(ctypes.byref(d), None) == UNSUPPORTED
    d.head_dim, d.tok_begin = 128, -1
    assert lib.lsa_project_keys(ctypes.byref(d), None) == INVALID
    c = lsa.CentroidDesc()
    c.struct_size = ctypes.sizeof(lsa.CentroidDesc)
    c.n_seq, c.n_kv_heads, c.n_keys, c.rank, c.block = 1, 1, 64, 64, 0
    c.in_, c.out = 0x1000, 0x2000
    assert lib.lsa_build_centroids(ctypes.byref(c), None) == INVALID


def test_stream_read_validation():
    lib = lsa._lib()
    assert lib.lsa_stream_read(None, 1024, 0x2000, None) == INVALID
    assert lib.lsa_stream_read(0x1000, 1024, None, None) == INVALID
    assert lib.lsa_stream_read(0x1000, 0, 0x2000, None) == INVALID
    assert lib.lsa_stream_read(0x1000, 1000, 0x2000, None) == INVALID     # not a multiple of 16
    assert lib.lsa_stream_read(0x1008, 1024, 0x2000, None) == INVALID     # misaligned buffer
    assert lib.lsa_stream_read(0x1000, 1024, 0x2002, None) == INVALID     # misaligned sink


def test_binding_raises_on_bad_arguments():
    import torch
    k = torch.zeros(1, 1, 8, 48, dtype=torch.bfloat16)
    s = torch.zeros(1, 1, 8)
    with pytest.raises(lsa.LsaError) as e:
        lsa.lsa_index_score(k, s, q_idx=torch.zeros(1, 1, 48), stream=0)
    assert e.value.status == UNSUPPORTED


def test_hint_validation_and_layout():
    lib = lsa._lib()
    d = _score_desc(hint=0x7002, hint_ld=4)           # misaligned
    assert _call_score(d) == INVALID
    d = _score_desc(hint=0x7000, hint_ld=0)           # too short for the layout
    assert _call_score(d) == INVALID
    c, k = ctypes.c_int32(0), ctypes.c_int32(0)
    assert lib.lsa_score_hint_layout(ctypes.byref(_score_desc()), ctypes.byref(c), ctypes.byref(k)) == 0
    assert c.value >= 1 and k.value >= 1
    count, kk = lsa.score_hint_layout_for(4, 8, 131072)
    assert count * kk * 32 == 131072          # one key vouched per 32 slots
    s = _select_desc(hint=0x5000, hint_count=0, hint_k=4, hint_ld=8)
    assert lib.lsa_topk_select(ctypes.byref(s), None, 0, None) == INVALID
    s = _select_desc(hint=0x5000, hint_count=8, hint_k=0, hint_ld=8)
    assert lib.lsa_topk_select(ctypes.byref(s), None, 0, None) == INVALID
    s = _select_desc(hint=0x5000, hint_count=8, hint_k=4, hint_ld=7)
    assert lib.lsa_topk_select(ctypes.byref(s), None, 0, None) == INVALID


def _prefill_desc(**kw):
    d = lsa.ScoreDesc()
    d.struct_size = ctypes.sizeof(lsa.ScoreDesc)
    d.mode, d.n_seq, d.n_kv_heads, d.n_keys, d.rank = lsa.MODE_PREFILL_CAUSAL, 1, 1, 65536, 64
    d.q_idx = 0x1000
    d.k_idx = 0x2000
    d.k_idx_dtype = lsa.BF16
    d.k_stride_head, d.k_stride_tok = 64, 64
    d.topk = 2048
    d.out_idx = 0x3000
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def test_prefill_fused_workspace_and_limits():
    lib = lsa._lib()
    ws = lib.lsa_score_workspace_bytes(ctypes.byref(_prefill_desc()))
    # candidate sub-lists (8 x 1024 pairs per row) dominate: 64 KiB per row
    assert ws >= 65536 * 8 * 1024 * 8
    assert lib.lsa_score_workspace_bytes(ctypes.byref(_prefill_desc(n_keys=4096))) < ws
    assert lsa.prefill_score_workspace_bytes_for(65536, 1, 64, 2048) == ws
    # the workspace check comes after validation: a valid fused call without
    # one is a workspace error (no HIP call is made)
    assert _call_score(_prefill_desc()) == WORKSPACE


@pytest.mark.parametrize("field,value,code", [
    ("rank", 32, UNSUPPORTED),              # the MFMA path is built for r = 64
    ("topk", 4097, UNSUPPORTED),            # candidates would not fit the sub-lists
    ("n_keys", 262145, UNSUPPORTED),        # bitmaps beyond LDS
    ("k_stride_tok", 68, INVALID),          # rows must stay 16-byte aligned
    ("k_idx", 0x2008, INVALID),
    ("q_idx", 0x1008, INVALID),
    ("k_idx_dtype", lsa.F32, UNSUPPORTED),
    ("out_idx", 0, INVALID),
    ("topk", -1, INVALID),
    ("n_seq", 2, INVALID),
])
def test_prefill_fused_validation(field, value, code):
    assert _call_score(_prefill_desc(**{field: value})) == code


def test_cross_layer_plan_sources():
    # host logic only: which full layer's selection each layer attends with
    from indexer_driven_sparse_amd import pipeline
    p = pipeline.CrossLayerPlan("FSSFS", 2, 8, 2, 3000, 128, 64, 256, device="cpu")
    assert p.source == [0, 0, 0, 3, 3] and sorted(p.full) == [0, 3]
    assert p.out[0] is p.full[0].out and p.out[1] is not p.out[2]
    for bad in ("", "SF", "FX"):
        with pytest.raises(ValueError):
            pipeline.CrossLayerPlan(bad, 2, 8, 2, 3000, 128, 64, 256, device="cpu")


def test_query_block_validation_and_workspace():
    lib = lsa._lib()
    pre = dict(mode=1, n_seq=1, n_kv_heads=1, n_keys=65536, k_stride_seq=0, k_stride_head=64,
               k_stride_tok=64, scores=0, scores_ld=0, topk=2048, out_idx=0x7000)
    assert _call_score(_score_desc(**pre, query_block=-1)) == INVALID
    assert _call_score(_score_desc(**pre, query_block=64, k_idx_dtype=lsa.F32)) == UNSUPPORTED
    assert _call_score(_score_desc(**dict(pre, out_idx=0), query_block=64)) == INVALID
    assert _call_score(_score_desc(query_block=2)) == INVALID          # decode has no blocks
    d = _score_desc(**pre, query_block=64)
    need = lib.lsa_score_workspace_bytes(ctypes.byref(d))
    assert need >= 1024 * 65536 * 4 + 1024 * 64 * 2                    # block scores + queries
    assert _call_score(d) == WORKSPACE
    # with a caller score buffer the workspace holds no scores
    e = _score_desc(**dict(pre, scores=0x9000, scores_ld=65536), query_block=64)
    assert 0 < lib.lsa_score_workspace_bytes(ctypes.byref(e)) < 1024 * 65536 * 4
    # scores only (topk 0) need the caller's buffer
    assert _call_score(_score_desc(**dict(pre, topk=0, out_idx=0), query_block=64)) == INVALID
    s = _select_desc(causal_group=1, causal_block=-2)
    assert lib.lsa_topk_select(ctypes.byref(s), None, 0, None) == INVALID
    a = _attn_desc(query_block=2)                                       # decode rows are not blocked
    assert lib.lsa_indexed_attention(ctypes.byref(a), None, 0, None) == INVALID
    a = _attn_desc(query_block=-1, mode=1)
    assert lib.lsa_indexed_attention(ctypes.byref(a), None, 0, None) == INVALID


def test_binding_rejects_buffers_the_kernels_would_overrun():
    """The C ABI takes bare pointers, so the binding checks every tensor's
    dtype, contiguity and shape before building a descriptor: each case
    below would otherwise make a kernel read or write past a buffer."""
    import torch
    rows, Hq, Hkv, T, d, B = 2, 8, 2, 64, 128, 16
    q = torch.zeros(rows, Hq, d, dtype=torch.bfloat16)
    k = torch.zeros(rows, T, Hkv, d, dtype=torch.bfloat16)
    idx = torch.zeros(rows, Hkv, B, dtype=torch.int32)
    out = torch.zeros(rows, Hq, d)
    lse = torch.zeros(rows, Hq)
    bad_attn = [
        dict(k=torch.zeros(rows, T, Hkv, 64, dtype=torch.bfloat16),
             v=torch.zeros(rows, T, Hkv, 64, dtype=torch.bfloat16)),     # head dim differs from q
        dict(idx=idx.long()),                                             # int64 index lists
        dict(out=out.to(torch.bfloat16)),                                 # kernels write fp32
        dict(lse=torch.zeros(1)),                                         # too short
        dict(lse=torch.zeros(rows, Hq, dtype=torch.float64)),             # wrong dtype
        dict(lse=torch.zeros(Hq, rows).t()),                              # not contiguous
        dict(v=k.to(torch.float32)),                                      # k and v differ in dtype
        dict(q=q[0]),                                                     # not [rows,Hq,d]
    ]
    for over in bad_attn:
        kw = dict(q=q, k=k, v=k.clone(), idx=idx, out=out, lse=lse)
        kw.update(over)
        with pytest.raises(ValueError):
            lsa._attn_desc(kw["q"], kw["k"], kw["v"], kw["idx"], kw["out"], kw["lse"],
                           lsa.MODE_DECODE, 0.0)
    lsa._attn_desc(q, k, k.clone(), idx, out, lse, lsa.MODE_DECODE, 0.0)   # the good case builds

    N, r = 2, 64
    kx = torch.zeros(N, Hkv, T, r, dtype=torch.bfloat16)
    sc = torch.zeros(N, Hkv, T)
    qi = torch.zeros(N, Hkv, r)
    bad_score = [
        dict(scores=sc.to(torch.bfloat16)),                               # kernels write fp32
        dict(q_idx=qi.to(torch.bfloat16)),                                # decode q_idx is fp32
        dict(q=torch.zeros(N, Hq, d), w=torch.zeros(d, r, dtype=torch.float64)),
        dict(hint=torch.zeros(1, 4, dtype=torch.int32)),                  # too few hint rows
    ]
    for over in bad_score:
        kw = dict(scores=sc, q_idx=qi)
        kw.update(over)
        with pytest.raises(ValueError):
            lsa._score_desc(kx, kw["scores"], kw.get("q"), kw.get("w"), kw.get("q_idx"), None, 1,
                            lsa.MODE_DECODE, 0, None, None, kw.get("hint"))
    L = 128
    kp = torch.zeros(L, 1, r, dtype=torch.bfloat16)
    qp = torch.zeros(L, 1, r, dtype=torch.bfloat16)
    for over in [dict(out_idx=torch.zeros(L, 1, B, dtype=torch.int64)),
                 dict(out_score=torch.zeros(L, 1, B, dtype=torch.bfloat16)),
                 dict(q_idx=qp.float())]:
        kw = dict(out_idx=torch.zeros(L, 1, B, dtype=torch.int32), out_score=None, q_idx=qp)
        kw.update(over)
        with pytest.raises(ValueError):
            lsa._score_desc(kp, None, None, None, kw["q_idx"], None, 1, lsa.MODE_PREFILL_CAUSAL, B,
                            kw["out_idx"], kw["out_score"])

    scs = torch.zeros(4, 100)
    oi = torch.zeros(4, B, dtype=torch.int32)
    bad_sel = [
        dict(scores=scs.double()),
        dict(out_score=torch.zeros(4, B, dtype=torch.bfloat16)),
        dict(out_count=torch.zeros(4, dtype=torch.int64)),
        dict(n_valid=torch.zeros(4, dtype=torch.int64)),
        dict(cand=torch.zeros(4, 100, dtype=torch.int64)),
        dict(hint=torch.zeros(4, 2, dtype=torch.float32), hint_k=4),
    ]
    for over in bad_sel:
        kw = dict(scores=scs, out_score=None, out_count=None, n_valid=None, cand=None, hint=None,
                  hint_k=0)
        kw.update(over)
        with pytest.raises(ValueError):
            lsa._select_desc(kw["scores"], B, oi, None, kw["out_score"], kw["out_count"],
                             kw["n_valid"], 0, kw["cand"], 1, 100, kw["hint"], kw["hint_k"])

    with pytest.raises(ValueError):
        lsa.lsa_project_keys(k, torch.zeros(d, r, dtype=torch.float64),
                             torch.zeros(rows, Hkv, T, r, dtype=torch.bfloat16), stream=0)


def test_noalloc_attention_rejects_shapes_beyond_its_scratch():
    """The no-allocation attention call validates like lsa_indexed_attention
    and refuses, before touching the device, any shape whose partials would
    not fit its static scratch."""
    lib = lsa._lib()
    SCRATCH_LIMIT = -6
    # the headline decode shape (4 x 8 rows, 8 splits) fits
    assert lib.lsa_attention_workspace_bytes(ctypes.byref(_attn_desc())) <= lsa.NOALLOC_SCRATCH_BYTES
    # decode, 4096 sequences x 8 KV heads x 4 query heads, B = 2048: 8 splits
    # of fp32 partials (130 floats per head) = 133 MB > 4 MiB
    big = _attn_desc(rows=4096, n_q_heads=32, n_kv_heads=8, head_dim=128, topk=2048,
                     n_keys=131072, q_dtype=lsa.BF16, kv_dtype=lsa.BF16)
    need = lib.lsa_attention_workspace_bytes(ctypes.byref(big))
    assert need > lsa.NOALLOC_SCRATCH_BYTES
    assert lib.lsa_indexed_attention_noalloc(ctypes.byref(big), None) == SCRATCH_LIMIT
    bad = _attn_desc(rows=0)
    assert lib.lsa_indexed_attention_noalloc(ctypes.byref(bad), None) == INVALID


def test_step_plan_flags_and_one_launch_conditions():
    """lsa_decode_step's planner (host only): the one persistent launch only
    with LSA_STEP_ONE_LAUNCH, B a multiple of 32 and out_idx on a 128-byte
    line; unknown flag bits are rejected."""
    lib = lsa._lib()
    N, Hq, Hkv, T, d, r = 1, 32, 8, 40000, 128, 64
    bf = dict(dtype=torch.bfloat16)
    q = torch.empty(N, Hq, d, **bf)
    w = torch.empty(d, r, dtype=torch.float32)
    kd = torch.empty(N, Hkv, T, r, **bf)
    k = torch.empty(N, T, Hkv, d, **bf)
    v = torch.empty(N, T, Hkv, d, **bf)
    out = torch.empty(N, Hq, d, dtype=torch.float32)

    def fused(B, one_launch, shift=0):
        buf = torch.empty(N * Hkv * B + 64, dtype=torch.int32)
        base = (-buf.data_ptr() // 4) % 32 + shift    # element offset of a 128-byte line (+ shift)
        idx = buf[base:base + N * Hkv * B].view(N, Hkv, B)
        return lsa.lsa_step_is_fused(q, w, kd, k, v, idx, out, one_launch=one_launch)

    assert not fused(1024, False)
    assert fused(1024, True)
    assert not fused(1000, True)                # B not a multiple of 32
    assert not fused(1024, True, shift=1)       # selected positions off a 128-byte line
    idx = torch.empty(N, Hkv, 1024, dtype=torch.int32)
    d_ = lsa._step_desc(q, w, kd, k, v, idx, out, None, None, None, 0.0, True)
    assert lib.lsa_step_workspace_bytes(ctypes.byref(d_)) > 0
    d_.flags = 4
    assert lib.lsa_step_workspace_bytes(ctypes.byref(d_)) == 0
    assert lib.lsa_step_is_fused(ctypes.byref(d_)) == -1
    assert lib.lsa_step_path(ctypes.byref(d_)) == -1


def test_step_plan_listed_path_conditions():
    """lsa_decode_step's planner (host only): the default path lists the
    select's candidates in the scoring launch where the sampled threshold
    is useful (B well below T); LSA_STEP_THREE_CALLS, the one launch and
    budgets near T take the other paths; the listing path's workspace
    holds its samples, lists and metadata."""
    N, Hq, Hkv, d, r = 1, 32, 8, 128, 64
    bf = dict(dtype=torch.bfloat16)

    def path(T, B, kd_dtype=torch.bfloat16, **kw):
        q = torch.empty(N, Hq, d, **bf)
        w = torch.empty(d, r, dtype=torch.float32)
        kd = torch.empty(N, Hkv, T, r, dtype=kd_dtype)
        k = torch.empty(N, T, Hkv, d, **bf)
        out = torch.empty(N, Hq, d, dtype=torch.float32)
        buf = torch.empty(N * Hkv * B + 64, dtype=torch.int32)
        base = (-buf.data_ptr() // 4) % 32          # positions on a 128-byte line (the one launch needs it)
        idx = buf[base:base + N * Hkv * B].view(N, Hkv, B)
        return (lsa.lsa_step_path(q, w, kd, k, k, idx, out, **kw),
                lsa.lsa_step_workspace_bytes(q, w, kd, k, k, idx, out, **kw))

    p_list, ws_list = path(131072, 2048)
    p_three, ws_three = path(131072, 2048, three_calls=True)
    assert (p_list, p_three) == ("listed", "three_calls")
    # samples (one key per 64 slots), metadata and 8-byte list entries of
    # each row's 32 chunks on top of the three calls' workspace
    assert ws_list >= ws_three + N * Hkv * 32 * 8192 * 8
    assert path(131072, 2048, one_launch=True)[0] == "one_launch"
    assert path(40000, 1024)[0] == "listed"
    assert path(40000, 1024, kd_dtype=torch.float8_e4m3fn)[0] == "listed"
    assert path(4096, 256, kd_dtype=torch.float32)[0] == "listed"
    assert path(512, 512)[0] == "three_calls"              # B = T: nothing to select
    assert path(8192, 4096)[0] == "three_calls"            # half the row: the sample cannot help
    assert path(131072, 8192)[0] == "three_calls"          # more listed keys than the list path takes


def test_step_parts_argument_checks():
    """lsa_decode_step_part rejects parts outside 1..7 and the one-launch
    path (which has no parts) before any HIP call."""
    lib = lsa._lib()
    N, Hq, Hkv, T, d, r, B = 1, 32, 8, 131072, 128, 64, 2048
    bf = dict(dtype=torch.bfloat16)
    q = torch.empty(N, Hq, d, **bf)
    w = torch.empty(d, r, dtype=torch.float32)
    kd = torch.empty(N, Hkv, T, r, **bf)
    k = torch.empty(N, T, Hkv, d, **bf)
    out = torch.empty(N, Hq, d, dtype=torch.float32)
    buf = torch.empty(N * Hkv * B + 64, dtype=torch.int32)
    base = (-buf.data_ptr() // 4) % 32
    idx = buf[base:base + N * Hkv * B].view(N, Hkv, B)
    ws = torch.empty(16, dtype=torch.uint8)
    for parts in (0, 8, -1):
        d_ = lsa._step_desc(q, w, kd, k, k, idx, out, None, None, None, 0.0)
        assert lib.lsa_decode_step_part(ctypes.byref(d_), parts, ws.data_ptr(), 16, None) == -1   # LSA_ERR_INVALID_ARG
    d_ = lsa._step_desc(q, w, kd, k, k, idx, out, None, None, None, 0.0, True)
    assert lib.lsa_decode_step_part(ctypes.byref(d_), 1, ws.data_ptr(), 16, None) == -2   # LSA_ERR_UNSUPPORTED


def test_binding_rejects_bad_hierarchical_step_buffers():
    """lsa_hier_decode_step's descriptor: every output the step writes is
    checked for dtype, contiguity and exact shape (out_blocks against
    n_blocks_kept), and the inputs against one another, before any call."""
    import torch
    N, Hq, Hkv, T, d, r, B, blk, Bc = 1, 8, 2, 1024, 128, 64, 64, 64, 4
    nb = T // blk
    q = torch.zeros(N, Hq, d, dtype=torch.bfloat16)
    w = torch.zeros(d, r)
    kx = torch.zeros(N, Hkv, T, r, dtype=torch.bfloat16)
    cent = torch.zeros(N, Hkv, nb, r, dtype=torch.bfloat16)
    k = torch.zeros(N, T, Hkv, d, dtype=torch.bfloat16)
    good = dict(q=q, w=w, k_idx=kx, centroids=cent, k=k, v=k.clone(), n_blocks_kept=Bc,
                out_blocks=torch.zeros(N, Hkv, Bc, dtype=torch.int32),
                out_idx=torch.zeros(N, Hkv, B, dtype=torch.int32), out=torch.zeros(N, Hq, d),
                lse=torch.zeros(N, Hq), q_idx=torch.zeros(N, Hkv, r), out_score=torch.zeros(N, Hkv, B))

    def build(kw):
        return lsa._hier_desc(kw["q"], kw["w"], kw["k_idx"], kw["centroids"], kw["k"], kw["v"], blk,
                              kw["n_blocks_kept"], kw["out_blocks"], kw["out_idx"], kw["out"], kw["lse"],
                              kw["q_idx"], kw["out_score"], 0.0, False)

    d0 = build(good)   # the good case builds
    assert (d0.n_keys, d0.topk, d0.block, d0.n_blocks_kept) == (T, B, blk, Bc)
    bad = [
        dict(out_blocks=torch.zeros(N, Hkv, Bc - 1, dtype=torch.int32)),   # fewer slots than blocks kept
        dict(n_blocks_kept=Bc + 1),                                         # the same, the other way
        dict(out_blocks=torch.zeros(N, Hkv, Bc, dtype=torch.int64)),
        dict(out_idx=torch.zeros(N, Hkv, B, dtype=torch.int64)),
        dict(out=torch.zeros(N, Hq, d, dtype=torch.bfloat16)),              # kernels write fp32
        dict(lse=torch.zeros(N, Hq + 1)),
        dict(q_idx=torch.zeros(N, Hkv, r, dtype=torch.bfloat16)),
        dict(out_score=torch.zeros(N, Hkv, B - 1)),
        dict(centroids=torch.zeros(N, Hkv, nb - 1, r, dtype=torch.bfloat16)),   # a block short
        dict(centroids=torch.zeros(N, Hkv, nb, r, dtype=torch.float32)),        # not k_idx's dtype
        dict(v=torch.zeros(N, T, Hkv, d, dtype=torch.float32)),                  # k and v differ
        dict(w=torch.zeros(d, r, dtype=torch.float64)),
        dict(k=torch.zeros(N, T, Hkv, 64, dtype=torch.bfloat16),
             v=torch.zeros(N, T, Hkv, 64, dtype=torch.bfloat16)),              # head dim differs from q
    ]
    for over in bad:
        kw = dict(good)
        kw.update(over)
        with pytest.raises(ValueError):
            build(kw)


def test_hier_step_path_choice():
    """lsa_hier_step_path (host-only planning, no device work): the default
    runs the fine stage as separate calls on rows shorter than
    LSA_HIER_LIST_MIN_SLOTS and lists it on longer ones; LSA_STEP_LISTED and
    LSA_STEP_THREE_CALLS force a path; both together are invalid."""
    import ctypes as c
    import torch
    N, Hq, Hkv, T, d, r, B, blk = 1, 32, 8, 131072, 128, 64, 2048, 64
    q = torch.zeros(N, Hq, d, dtype=torch.bfloat16)
    w = torch.zeros(d, r)
    kx = torch.zeros(N, Hkv, T, r, dtype=torch.bfloat16)
    cent = torch.zeros(N, Hkv, T // blk, r, dtype=torch.bfloat16)
    k = torch.zeros(N, T, Hkv, d, dtype=torch.bfloat16)
    oi = torch.zeros(N, Hkv, B, dtype=torch.int32)
    out = torch.zeros(N, Hq, d)
    assert lsa.HIER_LIST_MIN_SLOTS == 32768
    cases = [(False, False, 128, 0), (True, False, 128, 0), (False, True, 128, 1),
             (False, False, 512, 1), (True, False, 512, 0), (True, True, 128, -1)]
    for three, listed, kept, want in cases:
        dd = lsa._hier_desc(q, w, kx, cent, k, k, blk, kept, None, oi, out, None, None, None, 0.0, three, listed)
        assert lsa._lib().lsa_hier_step_path(c.byref(dd)) == want, (three, listed, kept)


def test_step_paths_and_flags_on_the_host():
    """lsa_step_path (host-only planning): the flat decode step takes the
    listing path by default at the headline shape, the three calls with
    LSA_STEP_THREE_CALLS, and rejects flags it does not know, including
    the hierarchical step's LSA_STEP_LISTED."""
    import ctypes as c
    import torch
    N, Hq, Hkv, T, d, r, B = 4, 32, 8, 131072, 128, 64, 2048
    q = torch.zeros(N, Hq, d, dtype=torch.bfloat16)
    w = torch.zeros(d, r)
    kx = torch.zeros(N, Hkv, T, r, dtype=torch.bfloat16)
    k = torch.zeros(N, T, Hkv, d, dtype=torch.bfloat16)
    oi = torch.zeros(N, Hkv, B, dtype=torch.int32)
    out = torch.zeros(N, Hq, d)
    lib = lsa._lib()
    dd = lsa._step_desc(q, w, kx, k, k, oi, out, None, None, None, 0.0)
    assert lib.lsa_step_path(c.byref(dd)) == 1                     # listed
    dd = lsa._step_desc(q, w, kx, k, k, oi, out, None, None, None, 0.0, three_calls=True)
    assert lib.lsa_step_path(c.byref(dd)) == 0                     # three calls
    for bad in (lsa.STEP_LISTED, 8, 1 << 20):
        dd = lsa._step_desc(q, w, kx, k, k, oi, out, None, None, None, 0.0)
        dd.flags = bad
        assert lib.lsa_step_path(c.byref(dd)) == -1, bad
