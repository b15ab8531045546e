"""The C ABI on a CPU-only host: the library loads, exports every entry
point include/lsa.h declares, agrees with the binding on descriptor sizes,
and rejects bad arguments during validation -- before any HIP call, so these
calls run without a GPU."""
import ctypes
import os
import re

import pytest

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
    for st in [0, -1, -2, -3, -4, -5]:
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
