"""Thin ctypes binding of liblsa.so (include/lsa.h).

Argument marshalling only: every step of the path runs in the HIP kernels of
liblsa.so. torch supplies device memory and the stream; tensors are passed as
raw device pointers plus sizes and element strides. Importing this module
loads the library and fails loudly if it is missing -- there is no fallback.

The function names match the C entry points. Query head h belongs to KV
head h // (Hq // Hkv).
"""
from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblsa.so")

F32 = 0
BF16 = 1
FP8_E4M3 = 2     # OCP E4M3 (torch.float8_e4m3fn): projected-key caches only
MODE_DECODE = 0
MODE_PREFILL_CAUSAL = 1

STATUS = {0: "LSA_OK", -1: "LSA_ERR_INVALID_ARG", -2: "LSA_ERR_UNSUPPORTED",
          -3: "LSA_ERR_WORKSPACE", -4: "LSA_ERR_NO_DEVICE_CODE", -5: "LSA_ERR_HIP",
          -6: "LSA_ERR_SCRATCH_LIMIT"}
NOALLOC_SCRATCH_BYTES = 4 << 20     # LSA_NOALLOC_SCRATCH_BYTES


class LsaError(RuntimeError):
    def __init__(self, fn: str, status: int, hip: int = 0):
        self.status = status
        self.hip_error = hip
        msg = f"{fn}: {STATUS.get(status, status)} ({_lib().lsa_status_str(status).decode()})"
        if status == -5:
            msg += f", HIP error {hip}"
        super().__init__(msg)


_c = ctypes
_U32, _I32, _I64, _P, _F = _c.c_uint32, _c.c_int32, _c.c_int64, _c.c_void_p, _c.c_float


class ScoreDesc(_c.Structure):
    _fields_ = [("struct_size", _U32), ("mode", _I32), ("n_seq", _I32), ("n_kv_heads", _I32),
                ("n_keys", _I32), ("rank", _I32),
                ("q_idx", _P), ("q", _P), ("q_dtype", _I32), ("n_q_heads", _I32),
                ("head_dim", _I32), ("w_per_head", _I32), ("w", _P),
                ("k_idx", _P), ("k_idx_dtype", _I32), ("reserved0", _I32),
                ("k_stride_seq", _I64), ("k_stride_head", _I64), ("k_stride_tok", _I64),
                ("cand", _P), ("n_cand", _I32), ("cand_block", _I32), ("cand_ld", _I64),
                ("scores", _P), ("scores_ld", _I64),
                ("topk", _I32), ("query_block", _I32), ("out_idx", _P), ("out_score", _P),
                ("hint", _P), ("hint_ld", _I64)]


class SelectDesc(_c.Structure):
    _fields_ = [("struct_size", _U32), ("rows", _I32), ("n", _I32), ("topk", _I32),
                ("scores", _P), ("scores_ld", _I64), ("n_valid", _P),
                ("causal_group", _I32), ("cand_block", _I32), ("cand", _P), ("cand_ld", _I64),
                ("n_positions", _I32), ("causal_block", _I32),
                ("out_idx", _P), ("out_score", _P), ("out_count", _P),
                ("hint", _P), ("hint_ld", _I64), ("hint_count", _I32), ("hint_k", _I32)]


class AttnDesc(_c.Structure):
    _fields_ = [("struct_size", _U32), ("mode", _I32), ("rows", _I32), ("n_q_heads", _I32),
                ("n_kv_heads", _I32), ("head_dim", _I32), ("topk", _I32), ("n_keys", _I32),
                ("q", _P), ("q_dtype", _I32), ("kv_dtype", _I32), ("k", _P), ("v", _P),
                ("kv_stride_seq", _I64), ("kv_stride_tok", _I64), ("kv_stride_head", _I64),
                ("idx", _P), ("scale", _F), ("query_block", _I32), ("out", _P), ("lse", _P),
                ("slot_table", _P), ("slot_table_ld", _I64), ("n_pool_rows", _I32),
                ("reserved1", _I32), ("merge_ctrl", _P)]

ATTN_MERGE_CTRL_WORDS = 1024   # lsa_attn_desc.merge_ctrl: zeroed int32 words for the in-launch merge


class ProjectDesc(_c.Structure):
    _fields_ = [("struct_size", _U32), ("n_seq", _I32), ("n_kv_heads", _I32), ("head_dim", _I32),
                ("rank", _I32), ("tok_begin", _I32), ("n_tok", _I32), ("k_dtype", _I32),
                ("k", _P), ("k_stride_seq", _I64), ("k_stride_tok", _I64), ("k_stride_head", _I64),
                ("w", _P), ("w_per_head", _I32), ("out_dtype", _I32), ("out", _P),
                ("out_stride_seq", _I64), ("out_stride_head", _I64), ("out_stride_tok", _I64)]


class CentroidDesc(_c.Structure):
    _fields_ = [("struct_size", _U32), ("n_seq", _I32), ("n_kv_heads", _I32), ("n_keys", _I32),
                ("rank", _I32), ("block", _I32), ("dtype", _I32), ("in_", _P),
                ("in_stride_seq", _I64), ("in_stride_head", _I64), ("in_stride_tok", _I64),
                ("out", _P), ("out_stride_seq", _I64), ("out_stride_head", _I64),
                ("out_stride_blk", _I64)]


class StepDesc(_c.Structure):
    _fields_ = [("struct_size", _U32), ("n_seq", _I32), ("n_q_heads", _I32), ("n_kv_heads", _I32),
                ("head_dim", _I32), ("rank", _I32), ("n_keys", _I32), ("topk", _I32),
                ("q", _P), ("q_dtype", _I32), ("w_per_head", _I32), ("w", _P),
                ("k_idx", _P), ("k_idx_dtype", _I32), ("kv_dtype", _I32),
                ("k_stride_seq", _I64), ("k_stride_head", _I64), ("k_stride_tok", _I64),
                ("k", _P), ("v", _P),
                ("kv_stride_seq", _I64), ("kv_stride_tok", _I64), ("kv_stride_head", _I64),
                ("scale", _F), ("flags", _I32),
                ("q_idx", _P), ("out_idx", _P), ("out_score", _P), ("out", _P), ("lse", _P)]


class HierStepDesc(_c.Structure):
    _fields_ = [("struct_size", _U32), ("n_seq", _I32), ("n_q_heads", _I32), ("n_kv_heads", _I32),
                ("head_dim", _I32), ("rank", _I32), ("n_keys", _I32), ("topk", _I32),
                ("block", _I32), ("n_blocks_kept", _I32),
                ("q", _P), ("q_dtype", _I32), ("w_per_head", _I32), ("w", _P),
                ("k_idx", _P), ("k_idx_dtype", _I32), ("kv_dtype", _I32),
                ("k_stride_seq", _I64), ("k_stride_head", _I64), ("k_stride_tok", _I64),
                ("centroids", _P), ("c_stride_seq", _I64), ("c_stride_head", _I64), ("c_stride_blk", _I64),
                ("k", _P), ("v", _P),
                ("kv_stride_seq", _I64), ("kv_stride_tok", _I64), ("kv_stride_head", _I64),
                ("scale", _F), ("flags", _I32),
                ("q_idx", _P), ("out_blocks", _P), ("out_idx", _P), ("out_score", _P), ("out", _P),
                ("lse", _P)]


DESCS = {0: ScoreDesc, 1: SelectDesc, 2: AttnDesc, 3: ProjectDesc, 4: CentroidDesc, 5: StepDesc,
         6: HierStepDesc}

_SIGS = {
    "lsa_index_score": (_I32, [_P, _P, _c.c_size_t, _P]),
    "lsa_topk_select": (_I32, [_P, _P, _c.c_size_t, _P]),
    "lsa_indexed_attention": (_I32, [_P, _P, _c.c_size_t, _P]),
    "lsa_indexed_attention_noalloc": (_I32, [_P, _P]),
    "lsa_project_keys": (_I32, [_P, _P]),
    "lsa_build_centroids": (_I32, [_P, _P]),
    "lsa_score_workspace_bytes": (_c.c_size_t, [_P]),
    "lsa_score_hint_layout": (_I32, [_P, _P, _P]),
    "lsa_select_workspace_bytes": (_c.c_size_t, [_P]),
    "lsa_attention_workspace_bytes": (_c.c_size_t, [_P]),
    "lsa_stream_read": (_I32, [_P, _c.c_size_t, _P, _P]),
    "lsa_decode_step": (_I32, [_P, _P, _c.c_size_t, _P]),
    "lsa_step_workspace_bytes": (_c.c_size_t, [_P]),
    "lsa_step_is_fused": (_I32, [_P]),
    "lsa_step_path": (_I32, [_P]),
    "lsa_decode_step_part": (_I32, [_P, _I32, _P, _c.c_size_t, _P]),
    "lsa_hier_decode_step": (_I32, [_P, _P, _c.c_size_t, _P]),
    "lsa_hier_step_workspace_bytes": (_c.c_size_t, [_P]),
    "lsa_hier_step_path": (_I32, [_P]),
    "lsa_status_str": (_c.c_char_p, [_I32]),
    "lsa_last_hip_error": (_I32, []),
    "lsa_abi_version": (_I32, []),
    "lsa_desc_size": (_c.c_size_t, [_I32]),
}

_handle = None


def _lib():
    global _handle
    if _handle is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError(f"liblsa.so is not built ({_LIB_PATH}); run "
                              "`python -m indexer_driven_sparse_amd.build`")
        lib = _c.CDLL(_LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        for which, cls in DESCS.items():
            if lib.lsa_desc_size(which) != _c.sizeof(cls):
                raise ImportError(f"liblsa.so descriptor {cls.__name__} has size "
                                  f"{lib.lsa_desc_size(which)}, binding expects {_c.sizeof(cls)}")
        _handle = lib
    return _handle


def library_path() -> str:
    _lib()
    return _LIB_PATH


def abi_version() -> int:
    return int(_lib().lsa_abi_version())


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------

def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float8_e4m3fn:
        return FP8_E4M3
    raise TypeError(f"liblsa takes float32, bfloat16 or float8_e4m3fn tensors, got {t.dtype}")


def _ptr(t) -> int | None:
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        return int(t)
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _rows2d(t: torch.Tensor, rows: int, name: str) -> int:
    """Leading dimension of `t` read as `rows` evenly spaced rows of its last
    dimension (e.g. [N, Hkv, n] with any row spacing that is uniform)."""
    if t.stride(-1) != 1:
        raise ValueError(f"{name}: innermost dimension must be contiguous")
    if t.dim() == 1:
        ld = t.shape[0]
    else:
        ld = t.stride(-2)
        span = ld
        for dim in range(t.dim() - 2, -1, -1):
            if t.shape[dim] > 1 and t.stride(dim) != span:
                raise ValueError(f"{name}: rows must be evenly spaced")
            span *= t.shape[dim]
    if t.numel() // t.shape[-1] != rows:
        raise ValueError(f"{name}: expected {rows} rows, got {t.numel() // t.shape[-1]}")
    return ld


def _need(t, name: str, dtype=None, shape=None) -> None:
    """The binding is the only layer that sees tensor sizes (the C ABI takes
    bare pointers), so it checks what the kernels will read or write:
    dtype, contiguity and exact shape."""
    if t is None:
        return
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _check(fn: str, rc: int) -> None:
    if rc != 0:
        raise LsaError(fn, rc, int(_lib().lsa_last_hip_error()))


def _workspace(need: int, workspace, device):
    if need == 0:
        return None, 0
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    return workspace, workspace.numel() * workspace.element_size()


# ---------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------

def _score_desc(k_idx, scores, q, w, q_idx, cand, cand_block, mode, topk, out_idx, out_score,
                hint=None, query_block=0):
    d = ScoreDesc()
    d.struct_size = _c.sizeof(ScoreDesc)
    d.mode = mode
    d.k_idx = _ptr(k_idx)
    d.k_idx_dtype = _dt(k_idx)
    if mode == MODE_DECODE:
        N, Hkv, T, r = k_idx.shape
        d.k_stride_seq, d.k_stride_head, d.k_stride_tok = k_idx.stride(0), k_idx.stride(1), k_idx.stride(2)
    else:
        L, Hkv, r = k_idx.shape
        N, T = 1, L
        d.k_stride_seq, d.k_stride_head, d.k_stride_tok = 0, k_idx.stride(1), k_idx.stride(0)
    if k_idx.stride(-1) != 1:
        raise ValueError("k_idx: innermost dimension must be contiguous")
    d.n_seq, d.n_kv_heads, d.n_keys, d.rank = N, Hkv, T, r
    qb = max(1, int(query_block))
    n_rows = (T + qb - 1) // qb          # prefill rows: tokens, or blocks of qb tokens
    if q is not None and mode != MODE_DECODE:
        raise ValueError("q (the fused scoring prep) is a decode input")
    if q is not None and (q.dim() != 3 or q.shape[0] != N or not q.is_contiguous()):
        raise ValueError("q must be contiguous [N,Hq,d]")
    if w is not None and w.dtype != torch.float32:
        raise ValueError("w must be float32")
    if q_idx is not None and q_idx.dtype != (torch.float32 if mode == MODE_DECODE else k_idx.dtype):
        raise ValueError("q_idx must be float32 (decode) or k_idx's dtype (prefill)")
    if scores is not None and scores.dtype != torch.float32:
        raise ValueError("scores must be float32")
    if out_idx is not None and out_idx.dtype != torch.int32:
        raise ValueError("out_idx must be int32")
    if out_score is not None and out_score.dtype != torch.float32:
        raise ValueError("out_score must be float32")
    if q is not None and (w is None or w.shape[-1] != r or w.shape[-2] != q.shape[2]
                          or not w.is_contiguous() or (w.dim() == 3 and w.shape[0] != Hkv)):
        raise ValueError("w must be contiguous [d,r] or [Hkv,d,r]")
    if q_idx is not None and (not q_idx.is_contiguous() or tuple(q_idx.shape) !=
                              ((N, Hkv, r) if mode == MODE_DECODE else (T, Hkv, r))):
        raise ValueError("q_idx must be contiguous [N,Hkv,r] (decode) or [L,Hkv,r] (prefill)")
    if cand is not None and (not cand.is_contiguous() or cand.dtype != torch.int32
                             or tuple(cand.shape[:-1]) != (N, Hkv)):
        raise ValueError("cand must be contiguous int32 [N,Hkv,n_cand]")
    if out_idx is not None and (not out_idx.is_contiguous() or out_idx.numel() != n_rows * Hkv * topk):
        raise ValueError("out_idx must be contiguous [rows,Hkv,B] (rows = L, or ceil(L/query_block))")
    if out_score is not None and (not out_score.is_contiguous() or
                                  out_score.numel() != n_rows * Hkv * topk):
        raise ValueError("out_score must be contiguous [rows,Hkv,B]")
    if q is not None:
        d.q = _ptr(q)
        d.q_dtype = _dt(q)
        d.n_q_heads, d.head_dim = q.shape[1], q.shape[2]
        d.w = _ptr(w)
        d.w_per_head = 1 if w.dim() == 3 else 0
    d.q_idx = _ptr(q_idx)
    if cand is not None:
        d.cand = _ptr(cand)
        d.n_cand = cand.shape[-1]
        d.cand_block = cand_block
        d.cand_ld = cand.stride(-2) if cand.dim() >= 2 else cand.shape[-1]
    if scores is not None:
        d.scores = _ptr(scores)
        d.scores_ld = _rows2d(scores, N * Hkv if mode == MODE_DECODE else n_rows * Hkv, "scores")
    d.topk = topk
    d.query_block = int(query_block)
    d.out_idx = _ptr(out_idx)
    d.out_score = _ptr(out_score)
    if hint is not None:
        if hint.dtype != torch.int32 or not hint.is_contiguous():
            raise ValueError("hint must be a contiguous int32 (bit pattern uint32) tensor")
        if hint.numel() // max(1, hint.shape[-1]) != N * Hkv:
            raise ValueError("hint must be [N*Hkv, hint_ld]")
        d.hint = _ptr(hint)
        d.hint_ld = hint.shape[-1]
    return d


def lsa_score_hint_layout(k_idx, scores, *, q=None, w=None, q_idx=None, cand=None,
                          cand_block=1):
    """(entries per row, keys per entry) of the selection hint a decode
    lsa_index_score call with these arguments writes."""
    d = _score_desc(k_idx, scores, q, w, q_idx, cand, cand_block, MODE_DECODE, 0, None, None)
    c, k = _c.c_int32(0), _c.c_int32(0)
    _lib().lsa_score_hint_layout(_c.byref(d), _c.byref(c), _c.byref(k))
    return int(c.value), int(k.value)


def lsa_index_score(k_idx: torch.Tensor, scores: torch.Tensor | None, *, q=None, w=None,
                    q_idx=None, cand=None, cand_block: int = 1, mode: int = MODE_DECODE,
                    topk: int = 0, out_idx=None, out_score=None, hint=None, workspace=None,
                    stream=None, query_block: int = 0) -> None:
    """Indexer scores. Decode: k_idx [N,Hkv,T,r] (any strides, r contiguous);
    either q [N,Hq,d] with w [d,r] / [Hkv,d,r] (prep fused; q_idx, if given,
    receives fp32 [N,Hkv,r]) or q_idx fp32 [N,Hkv,r]; optional cand
    [N,Hkv,nc] int32 with cand_block; scores fp32 [N,Hkv,n_out].
    Prefill: k_idx [L,Hkv,r], q_idx [L,Hkv,r]; topk=0 writes scores
    [L,Hkv,L]; topk=B fills out_idx [L,Hkv,B] (and out_score).
    Prefill with query_block=qb > 1: one selection per block of qb tokens
    (rows ceil(L/qb)): scores [nb,Hkv,L] and/or out_idx [nb,Hkv,B]."""
    d = _score_desc(k_idx, scores, q, w, q_idx, cand, cand_block, mode, topk, out_idx, out_score,
                    hint, query_block)
    lib = _lib()
    ws, wsb = _workspace(lib.lsa_score_workspace_bytes(_c.byref(d)), workspace, k_idx.device)
    _check("lsa_index_score", lib.lsa_index_score(_c.byref(d), _ptr(ws), wsb, _stream(stream)))


def lsa_score_workspace_bytes(k_idx, scores, *, q=None, w=None, q_idx=None, cand=None,
                              cand_block=1, mode=MODE_DECODE, topk=0, out_idx=None,
                              out_score=None, query_block: int = 0) -> int:
    d = _score_desc(k_idx, scores, q, w, q_idx, cand, cand_block, mode, topk, out_idx, out_score,
                    None, query_block)
    return int(_lib().lsa_score_workspace_bytes(_c.byref(d)))


def _select_desc(scores, topk, out_idx, n, out_score, out_count, n_valid, causal_group, cand,
                 cand_block, n_positions, hint=None, hint_k=0, causal_block=0):
    if scores.dtype != torch.float32:
        raise ValueError("scores must be float32")
    rows = scores.numel() // scores.shape[-1]
    if not out_idx.is_contiguous() or out_idx.numel() != rows * topk or out_idx.dtype != torch.int32:
        raise ValueError("out_idx must be contiguous int32 [rows, B]")
    if out_score is not None and (not out_score.is_contiguous() or out_score.numel() != rows * topk
                                  or out_score.dtype != torch.float32):
        raise ValueError("out_score must be contiguous float32 [rows, B]")
    if out_count is not None and (not out_count.is_contiguous() or out_count.numel() != rows
                                  or out_count.dtype != torch.int32):
        raise ValueError("out_count must be contiguous int32 [rows]")
    if n_valid is not None and (not n_valid.is_contiguous() or n_valid.numel() != rows
                                or n_valid.dtype != torch.int32):
        raise ValueError("n_valid must be contiguous int32 [rows]")
    if cand is not None and cand.dtype != torch.int32:
        raise ValueError("cand must be int32")
    if hint is not None and hint.dtype != torch.int32:
        raise ValueError("hint must be int32 (bit pattern uint32)")
    if n is not None and n > scores.shape[-1]:
        raise ValueError("n exceeds the row length")
    if cand is not None and (not cand.is_contiguous() or cand.numel() // cand.shape[-1] != rows
                             or cand.shape[-1] * cand_block < (scores.shape[-1] if n is None else n)):
        raise ValueError("cand must be contiguous [rows, n_cand] covering every slot")
    d = SelectDesc()
    d.struct_size = _c.sizeof(SelectDesc)
    d.rows = rows
    d.n = scores.shape[-1] if n is None else n
    d.topk = topk
    d.scores = _ptr(scores)
    d.scores_ld = _rows2d(scores, rows, "scores")
    d.n_valid = _ptr(n_valid)
    d.causal_group = causal_group
    d.causal_block = causal_block
    if cand is not None:
        d.cand = _ptr(cand)
        d.cand_block = cand_block
        d.cand_ld = cand.shape[-1]
        d.n_positions = n_positions
    d.out_idx = _ptr(out_idx)
    d.out_score = _ptr(out_score)
    d.out_count = _ptr(out_count)
    if hint is not None:
        if not hint.is_contiguous() or hint.numel() // hint.shape[-1] != rows:
            raise ValueError("hint must be contiguous [rows, hint_count]")
        d.hint = _ptr(hint)
        d.hint_ld = hint.shape[-1]
        d.hint_count = hint.shape[-1]
        d.hint_k = hint_k
    return d


def lsa_topk_select(scores: torch.Tensor, topk: int, out_idx: torch.Tensor, *, n=None,
                    out_score=None, out_count=None, n_valid=None, causal_group: int = 0,
                    cand=None, cand_block: int = 1, n_positions: int = 0, hint=None,
                    hint_k: int = 0, workspace=None, stream=None, causal_block: int = 0) -> None:
    """Exact top-B per row of scores [..., n] (rows evenly spaced): ascending
    positions in out_idx [rows, B], -1 padded. hint/hint_k: the selection
    hint of the scoring call (speed only, never the result). causal_group k:
    row i has (i//k + 1) * max(1, causal_block) valid slots."""
    d = _select_desc(scores, topk, out_idx, n, out_score, out_count, n_valid, causal_group, cand,
                     cand_block, n_positions, hint, hint_k, causal_block)
    lib = _lib()
    ws, wsb = _workspace(lib.lsa_select_workspace_bytes(_c.byref(d)), workspace, scores.device)
    _check("lsa_topk_select", lib.lsa_topk_select(_c.byref(d), _ptr(ws), wsb, _stream(stream)))


def lsa_select_workspace_bytes(scores, topk, out_idx, *, n=None, n_valid=None, causal_group=0,
                               cand=None, cand_block=1, n_positions=0, hint=None,
                               hint_k: int = 0) -> int:
    d = _select_desc(scores, topk, out_idx, n, None, None, n_valid, causal_group, cand, cand_block,
                     n_positions, hint, hint_k)
    return int(_lib().lsa_select_workspace_bytes(_c.byref(d)))


def _attn_desc(q, k, v, idx, out, lse, mode, scale, slot_table=None, n_keys=None,
               query_block=0, merge_ctrl=None):
    if q.dim() != 3:
        raise ValueError("q must be [rows,Hq,d]")
    rows, Hq, hd = q.shape
    if k.stride() != v.stride() or k.shape != v.shape or k.dtype != v.dtype:
        raise ValueError("k and v must share shape, strides and dtype")
    if k.shape[-1] != hd:
        raise ValueError(f"k/v head dim {k.shape[-1]} differs from q's {hd}")
    if idx.dtype != torch.int32:
        raise ValueError("idx must be int32")
    _need(out, "out", torch.float32)
    _need(lse, "lse", torch.float32, (rows, Hq))
    if slot_table is None:
        S, T, Hkv, _ = k.shape
        strides = (k.stride(0), k.stride(1), k.stride(2))
    else:
        if k.dim() != 3:
            raise ValueError("a paged K/V pool is [pool_rows, Hkv, d]")
        if slot_table.dtype != torch.int32 or slot_table.dim() != 2 or slot_table.stride(1) != 1:
            raise ValueError("slot_table must be int32 [n_seq, ld] with unit inner stride")
        P, Hkv, _ = k.shape
        S = slot_table.shape[0]
        T = slot_table.shape[1] if n_keys is None else int(n_keys)
        if T > slot_table.shape[1]:
            raise ValueError("n_keys exceeds the slot table's width")
        strides = (0, k.stride(0), k.stride(1))
    if mode == MODE_DECODE and S < rows:
        raise ValueError(f"decode reads sequence `row` of k/v: {S} sequences < {rows} rows")
    if not q.is_contiguous() or not idx.is_contiguous() or not out.is_contiguous():
        raise ValueError("q, idx and out must be contiguous")
    qb = max(1, int(query_block))
    if tuple(idx.shape[:-1]) != ((rows + qb - 1) // qb, Hkv) or tuple(out.shape) != (rows, Hq, hd):
        raise ValueError("idx must be [ceil(rows/query_block),Hkv,B] and out [rows,Hq,d]")
    d = AttnDesc()
    d.struct_size = _c.sizeof(AttnDesc)
    d.mode = mode
    d.rows, d.n_q_heads, d.n_kv_heads, d.head_dim = rows, Hq, Hkv, hd
    d.topk = idx.shape[-1]
    d.n_keys = T
    d.q = _ptr(q)
    d.q_dtype = _dt(q)
    d.kv_dtype = _dt(k)
    d.k, d.v = _ptr(k), _ptr(v)
    d.kv_stride_seq, d.kv_stride_tok, d.kv_stride_head = strides
    d.idx = _ptr(idx)
    d.scale = scale
    d.query_block = int(query_block)
    d.out = _ptr(out)
    d.lse = _ptr(lse)
    if slot_table is not None:
        d.slot_table = _ptr(slot_table)
        d.slot_table_ld = slot_table.stride(0)
        d.n_pool_rows = k.shape[0]
    if merge_ctrl is not None:
        if (merge_ctrl.device != q.device or not merge_ctrl.is_contiguous()
                or merge_ctrl.numel() * merge_ctrl.element_size() < 4 * ATTN_MERGE_CTRL_WORDS):
            raise ValueError(f"merge_ctrl must be {ATTN_MERGE_CTRL_WORDS} contiguous zeroed 32-bit words "
                             "on q's device")
        d.merge_ctrl = _ptr(merge_ctrl)
    return d


def lsa_indexed_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, idx: torch.Tensor,
                          out: torch.Tensor, *, lse=None, mode: int = MODE_DECODE,
                          scale: float = 0.0, workspace=None, stream=None,
                          slot_table=None, n_keys=None, query_block: int = 0, merge_ctrl=None) -> None:
    """q [rows,Hq,d]; k, v [S,T,Hkv,d] viewed through their strides (same for
    both); idx [rows,Hkv,B] int32; out fp32 [rows,Hq,d]; lse fp32 [rows,Hq].
    Paged: k, v are a pool [P,Hkv,d] and slot_table int32 [S, ld] maps
    (sequence, position) to a pool row; n_keys defaults to the table width.
    Prefill is causal; query_block=qb > 1 shares idx row i//qb among tokens.
    merge_ctrl: ATTN_MERGE_CTRL_WORDS zeroed int32 words, for the split
    merge inside the attention launch (bf16 decode on the matrix cores)."""
    d = _attn_desc(q, k, v, idx, out, lse, mode, scale, slot_table, n_keys, query_block, merge_ctrl)
    lib = _lib()
    ws, wsb = _workspace(lib.lsa_attention_workspace_bytes(_c.byref(d)), workspace, q.device)
    _check("lsa_indexed_attention",
           lib.lsa_indexed_attention(_c.byref(d), _ptr(ws), wsb, _stream(stream)))


def lsa_indexed_attention_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                                  idx: torch.Tensor, out: torch.Tensor, *, lse=None,
                                  mode: int = MODE_DECODE, scale: float = 0.0, stream=None,
                                  slot_table=None, n_keys=None, query_block: int = 0,
                                  merge_ctrl=None) -> None:
    """lsa_indexed_attention with its split partials in the library's static
    per-GPU scratch (NOALLOC_SCRATCH_BYTES): no workspace, no allocation --
    for callers that cannot allocate. Same arguments and bit-identical
    results; a shape needing more scratch raises LsaError
    (LSA_ERR_SCRATCH_LIMIT). Calls overlapping in time on one GPU race."""
    d = _attn_desc(q, k, v, idx, out, lse, mode, scale, slot_table, n_keys, query_block, merge_ctrl)
    _check("lsa_indexed_attention_noalloc",
           _lib().lsa_indexed_attention_noalloc(_c.byref(d), _stream(stream)))


def lsa_attention_workspace_bytes(q, k, v, idx, out, *, lse=None, mode=MODE_DECODE,
                                  scale=0.0, slot_table=None, n_keys=None,
                                  query_block: int = 0, merge_ctrl=None) -> int:
    d = _attn_desc(q, k, v, idx, out, lse, mode, scale, slot_table, n_keys, query_block, merge_ctrl)
    return int(_lib().lsa_attention_workspace_bytes(_c.byref(d)))


def attention_workspace_bytes_for(rows: int, Hq: int, Hkv: int, d: int, B: int, T: int,
                                  kv_dtype: int = BF16, mode: int = MODE_DECODE,
                                  merge_in_launch: bool = False) -> int:
    """Workspace lsa_indexed_attention needs for a shape (no tensors needed:
    the size depends on the shape only); merge_in_launch: with merge_ctrl."""
    dd = AttnDesc()
    if merge_in_launch:
        dd.merge_ctrl = 256                              # placeholder: sizing never dereferences
    dd.struct_size = _c.sizeof(AttnDesc)
    dd.mode, dd.rows, dd.n_q_heads, dd.n_kv_heads, dd.head_dim, dd.topk, dd.n_keys = \
        mode, rows, Hq, Hkv, d, B, T
    dd.q = dd.k = dd.v = dd.idx = dd.out = 256          # placeholders: sizing never dereferences
    dd.q_dtype = dd.kv_dtype = kv_dtype
    dd.kv_stride_seq, dd.kv_stride_tok, dd.kv_stride_head = T * Hkv * d, Hkv * d, d
    return int(_lib().lsa_attention_workspace_bytes(_c.byref(dd)))


def score_hint_layout_for(N: int, Hkv: int, n_out: int, r: int = 64, dtype: int = BF16):
    """(entries per row, keys per entry) of the selection hint written by a
    decode scoring call over n_out slots per row (shape only)."""
    dd = ScoreDesc()
    dd.struct_size = _c.sizeof(ScoreDesc)
    dd.mode, dd.n_seq, dd.n_kv_heads, dd.n_keys, dd.rank = MODE_DECODE, N, Hkv, n_out, r
    dd.q_idx = dd.k_idx = dd.scores = 256          # placeholders: sizing never dereferences
    dd.k_idx_dtype = dtype
    dd.k_stride_tok, dd.k_stride_head, dd.k_stride_seq = r, n_out * r, Hkv * n_out * r
    dd.scores_ld = (n_out + 3) // 4 * 4
    c, k = _c.c_int32(0), _c.c_int32(0)
    _lib().lsa_score_hint_layout(_c.byref(dd), _c.byref(c), _c.byref(k))
    return int(c.value), int(k.value)


def prefill_score_workspace_bytes_for(L: int, Hkv: int, r: int, B: int,
                                      query_block: int = 0) -> int:
    """Workspace of the fused causal prefill indexer (bf16, [L,Hkv,r]); with
    query_block > 1, of the block-shared selection (scores in workspace)."""
    dd = ScoreDesc()
    dd.struct_size = _c.sizeof(ScoreDesc)
    dd.mode, dd.n_seq, dd.n_kv_heads, dd.n_keys, dd.rank = MODE_PREFILL_CAUSAL, 1, Hkv, L, r
    dd.q_idx = dd.k_idx = dd.out_idx = 256
    dd.k_idx_dtype = BF16
    dd.k_stride_head, dd.k_stride_tok = r, Hkv * r
    dd.topk = B
    dd.query_block = query_block
    return int(_lib().lsa_score_workspace_bytes(_c.byref(dd)))


STEP_ONE_LAUNCH = 1   # lsa_step_desc.flags: the one persistent launch where the shape allows
STEP_THREE_CALLS = 2  # lsa_step_desc.flags: the three calls, with the select's own collect launch
STEP_LISTED = 4       # lsa_hier_step_desc.flags: both stages' listing launches wherever the shape allows
HIER_LIST_MIN_SLOTS = 32768   # row length from which lsa_hier_decode_step lists a stage by default


def _step_desc(q, w, k_idx, k, v, out_idx, out, lse, q_idx, out_score, scale, one_launch=False,
               three_calls=False):
    if q.dim() != 3 or not q.is_contiguous():
        raise ValueError("q must be contiguous [N,Hq,d]")
    N, Hq, hd = q.shape
    if k_idx.dim() != 4 or k_idx.stride(-1) != 1:
        raise ValueError("k_idx must be [N,Hkv,T,r] with r contiguous")
    _, Hkv, T, r = k_idx.shape
    if k_idx.shape[0] != N:
        raise ValueError("k_idx must hold the N sequences of q")
    if k.dim() != 4 or k.shape != v.shape or k.stride() != v.stride() or k.dtype != v.dtype:
        raise ValueError("k and v must share shape [N,T,Hkv,d], strides and dtype")
    if k.shape[0] < N or k.shape[1] != T or k.shape[2] != Hkv or k.shape[3] != hd:
        raise ValueError("k/v must be [N,T,Hkv,d] matching q and k_idx")
    if w.dtype != torch.float32 or not w.is_contiguous() or w.shape[-1] != r or w.shape[-2] != hd \
            or (w.dim() == 3 and w.shape[0] != Hkv):
        raise ValueError("w must be contiguous float32 [d,r] or [Hkv,d,r]")
    B = out_idx.shape[-1]
    _need(out_idx, "out_idx", torch.int32, (N, Hkv, B))
    _need(out, "out", torch.float32, (N, Hq, hd))
    _need(lse, "lse", torch.float32, (N, Hq))
    _need(q_idx, "q_idx", torch.float32, (N, Hkv, r))
    _need(out_score, "out_score", torch.float32, (N, Hkv, B))
    d = StepDesc()
    d.struct_size = _c.sizeof(StepDesc)
    d.n_seq, d.n_q_heads, d.n_kv_heads, d.head_dim, d.rank, d.n_keys, d.topk = N, Hq, Hkv, hd, r, T, B
    d.q, d.q_dtype = _ptr(q), _dt(q)
    d.w, d.w_per_head = _ptr(w), 1 if w.dim() == 3 else 0
    d.k_idx, d.k_idx_dtype = _ptr(k_idx), _dt(k_idx)
    d.k_stride_seq, d.k_stride_head, d.k_stride_tok = k_idx.stride(0), k_idx.stride(1), k_idx.stride(2)
    d.k, d.v, d.kv_dtype = _ptr(k), _ptr(v), _dt(k)
    d.kv_stride_seq, d.kv_stride_tok, d.kv_stride_head = k.stride(0), k.stride(1), k.stride(2)
    d.scale = scale
    d.flags = (STEP_ONE_LAUNCH if one_launch else 0) | (STEP_THREE_CALLS if three_calls else 0)
    d.q_idx, d.out_idx, d.out_score, d.out, d.lse = (_ptr(q_idx), _ptr(out_idx), _ptr(out_score),
                                                     _ptr(out), _ptr(lse))
    return d


def lsa_decode_step(q, w, k_idx, k, v, out_idx, out, *, lse=None, q_idx=None, out_score=None,
                    scale: float = 0.0, workspace=None, stream=None, one_launch: bool = False,
                    three_calls: bool = False) -> None:
    """One whole flat decode step (scoring prep, scores, exact top-B, indexed
    attention): q [N,Hq,d], w [d,r] fp32, k_idx [N,Hkv,T,r], k/v [N,T,Hkv,d];
    out_idx int32 [N,Hkv,B], out fp32 [N,Hq,d]. workspace: uint8 of at least
    lsa_step_workspace_bytes, all zero before its first use (the call leaves
    its control words zero); allocated zeroed here when not given.
    one_launch: the single persistent launch where the shape allows it;
    three_calls: the three calls with the select's own collect launch."""
    d = _step_desc(q, w, k_idx, k, v, out_idx, out, lse, q_idx, out_score, scale, one_launch, three_calls)
    lib = _lib()
    need = lib.lsa_step_workspace_bytes(_c.byref(d))
    if need == 0:
        _check("lsa_decode_step", lib.lsa_decode_step(_c.byref(d), None, 0, _stream(stream)))
    if workspace is None:
        workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)
    wsb = workspace.numel() * workspace.element_size()
    _check("lsa_decode_step", lib.lsa_decode_step(_c.byref(d), _ptr(workspace), wsb, _stream(stream)))


STEP_PART_SCORE, STEP_PART_SELECT, STEP_PART_ATTEND, STEP_PART_ALL = 1, 2, 4, 7


def lsa_decode_step_part(parts: int, q, w, k_idx, k, v, out_idx, out, *, workspace, lse=None,
                         q_idx=None, out_score=None, scale: float = 0.0, stream=None,
                         three_calls: bool = False) -> None:
    """The default decode step's launches named in `parts` (an OR of
    STEP_PART_SCORE, STEP_PART_SELECT, STEP_PART_ATTEND), issued as
    lsa_decode_step issues them; workspace as for lsa_decode_step."""
    d = _step_desc(q, w, k_idx, k, v, out_idx, out, lse, q_idx, out_score, scale, False, three_calls)
    wsb = workspace.numel() * workspace.element_size()
    _check("lsa_decode_step_part",
           _lib().lsa_decode_step_part(_c.byref(d), int(parts), _ptr(workspace), wsb, _stream(stream)))


def lsa_step_workspace_bytes(q, w, k_idx, k, v, out_idx, out, *, lse=None, q_idx=None,
                             out_score=None, scale: float = 0.0, one_launch: bool = False,
                             three_calls: bool = False) -> int:
    d = _step_desc(q, w, k_idx, k, v, out_idx, out, lse, q_idx, out_score, scale, one_launch, three_calls)
    return int(_lib().lsa_step_workspace_bytes(_c.byref(d)))


def lsa_step_is_fused(q, w, k_idx, k, v, out_idx, out, **kw) -> bool:
    """Whether the step (shape and one_launch flag) runs as one persistent launch."""
    d = _step_desc(q, w, k_idx, k, v, out_idx, out, kw.get("lse"), kw.get("q_idx"),
                   kw.get("out_score"), kw.get("scale", 0.0), kw.get("one_launch", False),
                   kw.get("three_calls", False))
    return int(_lib().lsa_step_is_fused(_c.byref(d))) == 1


STEP_PATHS = {0: "three_calls", 1: "listed", 2: "one_launch"}


def lsa_step_path(q, w, k_idx, k, v, out_idx, out, **kw) -> str:
    """Which path the step takes for this shape and these flags:
    'three_calls', 'listed' (the scoring launch lists the select's
    candidates) or 'one_launch'."""
    d = _step_desc(q, w, k_idx, k, v, out_idx, out, kw.get("lse"), kw.get("q_idx"),
                   kw.get("out_score"), kw.get("scale", 0.0), kw.get("one_launch", False),
                   kw.get("three_calls", False))
    code = int(_lib().lsa_step_path(_c.byref(d)))
    if code < 0:
        raise ValueError("lsa_step_path: invalid step descriptor")
    return STEP_PATHS[code]


STEP_ERROR_WORD = 9    # 32-bit word index of the step workspace's error word


def lsa_project_keys(k: torch.Tensor, w: torch.Tensor, out: torch.Tensor, *, tok_begin: int = 0,
                     n_tok: int | None = None, stream=None) -> None:
    """out[n,g,t,:] = round(k[n,t,g,:] . w) for t in [tok_begin, tok_begin+n_tok).
    k [N,T,Hkv,d] (strided), w [d,r] / [Hkv,d,r] fp32, out [N,Hkv,T',r]."""
    N, T, Hkv, hd = k.shape
    d = ProjectDesc()
    d.struct_size = _c.sizeof(ProjectDesc)
    d.n_seq, d.n_kv_heads, d.head_dim, d.rank = N, Hkv, hd, w.shape[-1]
    d.tok_begin = tok_begin
    d.n_tok = T - tok_begin if n_tok is None else n_tok
    if tok_begin < 0 or tok_begin + d.n_tok > T or tok_begin + d.n_tok > out.shape[2]:
        raise ValueError("token range outside k or out")
    if tuple(out.shape[:2]) != (N, Hkv) or out.shape[3] != w.shape[-1] or w.shape[-2] != hd:
        raise ValueError("out must be [N,Hkv,T,r] and w [d,r] or [Hkv,d,r]")
    if w.dtype != torch.float32 or not w.is_contiguous() or (w.dim() == 3 and w.shape[0] != Hkv):
        raise ValueError("w must be contiguous float32 [d,r] or [Hkv,d,r]")
    if out.stride(-1) != 1 or k.stride(-1) != 1:
        raise ValueError("k and out must be contiguous in their last dimension")
    d.k_dtype = _dt(k)
    d.k = _ptr(k)
    d.k_stride_seq, d.k_stride_tok, d.k_stride_head = k.stride(0), k.stride(1), k.stride(2)
    d.w = _ptr(w)
    d.w_per_head = 1 if w.dim() == 3 else 0
    d.out_dtype = _dt(out)
    d.out = _ptr(out)
    d.out_stride_seq, d.out_stride_head, d.out_stride_tok = out.stride(0), out.stride(1), out.stride(2)
    _check("lsa_project_keys", _lib().lsa_project_keys(_c.byref(d), _stream(stream)))


STREAM_READ_SINK_WORDS = 8192


def lsa_stream_read(buf: torch.Tensor, sink: torch.Tensor, *, stream=None) -> None:
    """Measurement helper: stream the bytes of a contiguous device tensor
    (16-byte aligned, size a multiple of 16). sink: int32
    [STREAM_READ_SINK_WORDS], overwritten; the XOR of its words is the XOR
    of every 32-bit word of buf."""
    if not buf.is_contiguous() or sink.dtype != torch.int32 or sink.numel() < STREAM_READ_SINK_WORDS:
        raise ValueError("lsa_stream_read: contiguous buf and an int32 sink of "
                         f"{STREAM_READ_SINK_WORDS} words are required")
    nbytes = buf.numel() * buf.element_size()
    _check("lsa_stream_read", _lib().lsa_stream_read(_ptr(buf), nbytes, _ptr(sink), _stream(stream)))


def lsa_build_centroids(k_idx: torch.Tensor, block: int, out: torch.Tensor, *, stream=None) -> None:
    """out[n,g,b,:] = round(mean of k_idx[n,g,t,:] over block b). k_idx
    [N,Hkv,T,r], out [N,Hkv,ceil(T/block),r], same dtype."""
    N, Hkv, T, r = k_idx.shape
    d = CentroidDesc()
    d.struct_size = _c.sizeof(CentroidDesc)
    d.n_seq, d.n_kv_heads, d.n_keys, d.rank, d.block = N, Hkv, T, r, block
    d.dtype = _dt(k_idx)
    if out.dtype != k_idx.dtype or tuple(out.shape) != (N, Hkv, (T + block - 1) // block, r):
        raise ValueError("out must be [N,Hkv,ceil(T/block),r] in k_idx's dtype")
    d.in_ = _ptr(k_idx)
    d.in_stride_seq, d.in_stride_head, d.in_stride_tok = k_idx.stride(0), k_idx.stride(1), k_idx.stride(2)
    d.out = _ptr(out)
    d.out_stride_seq, d.out_stride_head, d.out_stride_blk = out.stride(0), out.stride(1), out.stride(2)
    _check("lsa_build_centroids", _lib().lsa_build_centroids(_c.byref(d), _stream(stream)))


def _hier_desc(q, w, k_idx, centroids, k, v, block, n_blocks_kept, out_blocks, out_idx, out, lse, q_idx,
               out_score, scale, three_calls, listed=False):
    if q.dim() != 3 or not q.is_contiguous():
        raise ValueError("q must be contiguous [N,Hq,d]")
    N, Hq, hd = q.shape
    if k_idx.dim() != 4 or k_idx.stride(-1) != 1 or k_idx.shape[0] != N:
        raise ValueError("k_idx must be [N,Hkv,T,r] with r contiguous")
    _, Hkv, T, r = k_idx.shape
    nb = (T + block - 1) // block
    if (centroids.dim() != 4 or centroids.stride(-1) != 1 or tuple(centroids.shape) != (N, Hkv, nb, r)
            or centroids.dtype != k_idx.dtype):
        raise ValueError("centroids must be [N,Hkv,ceil(T/block),r] in k_idx's dtype, r contiguous")
    if k.dim() != 4 or k.shape != v.shape or k.stride() != v.stride() or k.dtype != v.dtype:
        raise ValueError("k and v must share shape [N,T,Hkv,d], strides and dtype")
    if k.shape[0] < N or k.shape[1] != T or k.shape[2] != Hkv or k.shape[3] != hd:
        raise ValueError("k/v must be [N,T,Hkv,d] matching q and k_idx")
    if w.dtype != torch.float32 or not w.is_contiguous() or w.shape[-1] != r or w.shape[-2] != hd \
            or (w.dim() == 3 and w.shape[0] != Hkv):
        raise ValueError("w must be contiguous float32 [d,r] or [Hkv,d,r]")
    B = out_idx.shape[-1]
    _need(out_idx, "out_idx", torch.int32, (N, Hkv, B))
    _need(out_blocks, "out_blocks", torch.int32, (N, Hkv, n_blocks_kept))
    _need(out, "out", torch.float32, (N, Hq, hd))
    _need(lse, "lse", torch.float32, (N, Hq))
    _need(q_idx, "q_idx", torch.float32, (N, Hkv, r))
    _need(out_score, "out_score", torch.float32, (N, Hkv, B))
    d = HierStepDesc()
    d.struct_size = _c.sizeof(HierStepDesc)
    d.n_seq, d.n_q_heads, d.n_kv_heads, d.head_dim, d.rank, d.n_keys, d.topk = N, Hq, Hkv, hd, r, T, B
    d.block, d.n_blocks_kept = block, n_blocks_kept
    d.q, d.q_dtype = _ptr(q), _dt(q)
    d.w, d.w_per_head = _ptr(w), 1 if w.dim() == 3 else 0
    d.k_idx, d.k_idx_dtype = _ptr(k_idx), _dt(k_idx)
    d.k_stride_seq, d.k_stride_head, d.k_stride_tok = k_idx.stride(0), k_idx.stride(1), k_idx.stride(2)
    d.centroids = _ptr(centroids)
    d.c_stride_seq, d.c_stride_head, d.c_stride_blk = centroids.stride(0), centroids.stride(1), centroids.stride(2)
    d.k, d.v, d.kv_dtype = _ptr(k), _ptr(v), _dt(k)
    d.kv_stride_seq, d.kv_stride_tok, d.kv_stride_head = k.stride(0), k.stride(1), k.stride(2)
    d.scale = scale
    d.flags = (STEP_THREE_CALLS if three_calls else 0) | (STEP_LISTED if listed else 0)
    d.q_idx, d.out_blocks, d.out_idx, d.out_score, d.out, d.lse = (
        _ptr(q_idx), _ptr(out_blocks), _ptr(out_idx), _ptr(out_score), _ptr(out), _ptr(lse))
    return d


def lsa_hier_decode_step(q, w, k_idx, centroids, k, v, block: int, n_blocks_kept: int, out_idx, out, *,
                         out_blocks=None, lse=None, q_idx=None, out_score=None, scale: float = 0.0,
                         workspace=None, stream=None, three_calls: bool = False,
                         listed: bool = False) -> None:
    """One coarse-to-fine decode step: centroids [N,Hkv,ceil(T/block),r]
    scored and the n_blocks_kept best blocks kept, their tokens scored and
    the top B (= out_idx.shape[-1]) attended. out_blocks int32
    [N,Hkv,n_blocks_kept] optional. workspace: uint8 of at least
    lsa_hier_step_workspace_bytes, all zero before its first use (allocated
    zeroed here when not given). three_calls: the fine stage as the
    separate scoring and select calls in both stages (by default a stage
    runs them when its rows hold fewer than 32768 slots); listed: both
    stages' listing launches wherever the shape allows."""
    d = _hier_desc(q, w, k_idx, centroids, k, v, block, n_blocks_kept, out_blocks, out_idx, out, lse, q_idx,
                   out_score, scale, three_calls, listed)
    lib = _lib()
    need = lib.lsa_hier_step_workspace_bytes(_c.byref(d))
    if need == 0:
        _check("lsa_hier_decode_step", lib.lsa_hier_decode_step(_c.byref(d), None, 0, _stream(stream)))
    if workspace is None:
        workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)
    wsb = workspace.numel() * workspace.element_size()
    _check("lsa_hier_decode_step", lib.lsa_hier_decode_step(_c.byref(d), _ptr(workspace), wsb, _stream(stream)))


def lsa_hier_step_workspace_bytes(q, w, k_idx, centroids, k, v, block: int, n_blocks_kept: int, out_idx,
                                  out, *, out_blocks=None, lse=None, q_idx=None, out_score=None,
                                  scale: float = 0.0, three_calls: bool = False, listed: bool = False) -> int:
    d = _hier_desc(q, w, k_idx, centroids, k, v, block, n_blocks_kept, out_blocks, out_idx, out, lse, q_idx,
                   out_score, scale, three_calls, listed)
    return int(_lib().lsa_hier_step_workspace_bytes(_c.byref(d)))


def lsa_hier_step_path(q, w, k_idx, centroids, k, v, block: int, n_blocks_kept: int, out_idx, out,
                       **kw) -> str:
    """'listed' or 'three_calls': how the step runs its fine stage."""
    d = _hier_desc(q, w, k_idx, centroids, k, v, block, n_blocks_kept, kw.get("out_blocks"), out_idx, out,
                   kw.get("lse"), kw.get("q_idx"), kw.get("out_score"), kw.get("scale", 0.0),
                   kw.get("three_calls", False), kw.get("listed", False))
    code = int(_lib().lsa_hier_step_path(_c.byref(d)))
    if code < 0:
        raise ValueError("lsa_hier_step_path: invalid descriptor")
    return STEP_PATHS[code]
