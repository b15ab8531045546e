"""numpy front end of the CPU oracle (test infrastructure, never the product).

Arrays: fp32 tensors are ``numpy.float32``; bf16 tensors are ``numpy.uint16``
holding the raw bf16 bits; OCP E4M3 fp8 tensors are ``numpy.uint8`` holding
the raw bits. Every computation happens in ``lsa_oracle.c`` in
double precision; results come back as ``numpy.float64`` except where the
method stores a value (projected keys, centroids), which come back in the
storage dtype.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

F32 = 0
BF16 = 1
FP8 = 2      # OCP E4M3 ("FN": no infinities, max 448)

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lsa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liblsa_oracle.so")
_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int
_L = ctypes.c_int64
_D = ctypes.c_double

_SIGS = {
    "lsa_ref_round_bf16": (ctypes.c_uint16, [_D]),
    "lsa_ref_round_fp8": (ctypes.c_uint8, [_D]),
    "lsa_ref_decode_fp8": (_D, [ctypes.c_uint8]),
    "lsa_ref_set_threads": (None, [_I]),
    "lsa_ref_get_threads": (_I, []),
    "lsa_ref_project_keys": (_I, [_P, _I, _L, _L, _L, _I, _I, _I, _I, _P, _I, _I, _P, _I]),
    "lsa_ref_centroids": (_I, [_P, _I, _I, _I, _I, _I, _I, _P]),
    "lsa_ref_query_prep": (_I, [_P, _I, _I, _I, _I, _I, _P, _I, _I, _P]),
    "lsa_ref_scores": (_I, [_P, _I, _I, _I, _P, _I, _L, _L, _L, _I, _P, _I, _I, _L, _P, _L]),
    "lsa_ref_topk": (_I, [_P, _I, _I, _L, _P, _I, _P, _I, _L, _I, _I, _P, _P, _P]),
    "lsa_ref_prefill_topk": (_I, [_P, _P, _I, _I, _I, _I, _I, _I, _I, _P, _P]),
    "lsa_ref_prefill_scores": (_I, [_P, _P, _I, _I, _I, _I, _P, _L]),
    "lsa_ref_prefill_block_topk": (_I, [_P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _P, _L]),
    "lsa_ref_attention": (_I, [_I, _I, _I, _I, _I, _I, _P, _I, _P, _P, _I, _L, _L, _L, _I, _P, _I,
                               _D, _P, _P]),
}


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (OpenMP) into oracle/liblsa_oracle.so."""
    stale = not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)
    if force or stale:
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
             "-Wno-unused-parameter", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _get():
    global _lib
    if _lib is None:
        # LSA_ORACLE_LIB names another build of lsa_oracle.c (the sanitizer
        # test loads one built with AddressSanitizer and UBSan)
        path = os.environ.get("LSA_ORACLE_LIB")
        if not path:
            path = build()
        lib = ctypes.CDLL(path)
        for name, (res, args) in _SIGS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def set_threads(n: int) -> None:
    _get().lsa_ref_set_threads(int(n))


def get_threads() -> int:
    return int(_get().lsa_ref_get_threads())


def round_bf16(x: float) -> int:
    """Bits of the bf16 nearest to the double x (ties to even)."""
    return int(_get().lsa_ref_round_bf16(float(x)))


def round_fp8(x: float) -> int:
    """Bits of the E4M3 value nearest to the double x (ties to even,
    saturating at +-448, NaN to 0x7F)."""
    return int(_get().lsa_ref_round_fp8(float(x)))


def decode_fp8(b: int) -> float:
    """Exact value of the E4M3 bit pattern b."""
    return float(_get().lsa_ref_decode_fp8(int(b)))


_STORE = {F32: np.float32, BF16: np.uint16, FP8: np.uint8}


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.uint8:
        return FP8
    raise TypeError(f"oracle takes float32, uint16 (bf16 bits) or uint8 (E4M3 bits) arrays, "
                    f"got {a.dtype}")


def _estrides(a: np.ndarray):
    st = [s // a.itemsize for s in a.strides]
    if a.strides[-1] != a.itemsize:
        raise ValueError("innermost dimension must be contiguous")
    return st


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (rc={rc})")


def project_keys(K: np.ndarray, W: np.ndarray, out_dtype: int = BF16) -> np.ndarray:
    """k_idx[n,g,t,:] = K[n,t,g,:] . W, stored as out_dtype (setup of the
    projected-key cache, JSSA Fig. 1). K is [N,T,Hkv,d] (any strides, d
    contiguous); W is [d,r] or [Hkv,d,r] fp32. Returns [N,Hkv,T,r]."""
    N, T, Hkv, d = K.shape
    W = np.ascontiguousarray(W, dtype=np.float32)
    r = W.shape[-1]
    s = _estrides(K)
    out = np.empty((N, Hkv, T, r), dtype=_STORE[out_dtype])
    _check(_get().lsa_ref_project_keys(_ptr(K), _dtype_code(K), s[0], s[1], s[2], N, T, Hkv, d,
                                       _ptr(W), int(W.ndim == 3), r, _ptr(out), out_dtype),
           "project_keys")
    return out


def centroids(k_idx: np.ndarray, block: int) -> np.ndarray:
    """Mean projected key of each block of `block` tokens (LongCat abstract,
    item 3: coarse summaries). k_idx [N,Hkv,T,r] -> [N,Hkv,ceil(T/block),r]."""
    k_idx = np.ascontiguousarray(k_idx)
    N, Hkv, T, r = k_idx.shape
    nb = (T + block - 1) // block
    out = np.empty((N, Hkv, nb, r), dtype=k_idx.dtype)
    _check(_get().lsa_ref_centroids(_ptr(k_idx), _dtype_code(k_idx), N, Hkv, T, r, block, _ptr(out)),
           "centroids")
    return out


def query_prep(Q: np.ndarray, Hkv: int, W: np.ndarray) -> np.ndarray:
    """q_idx[n,g] = mean of the group's query heads, projected by W (JSSA
    Fig. 1; Fig. 9 'scoring preparation'). Q [N,Hq,d] -> float64 [N,Hkv,r]."""
    Q = np.ascontiguousarray(Q)
    N, Hq, d = Q.shape
    W = np.ascontiguousarray(W, dtype=np.float32)
    r = W.shape[-1]
    out = np.empty((N, Hkv, r), dtype=np.float64)
    _check(_get().lsa_ref_query_prep(_ptr(Q), _dtype_code(Q), N, Hq, Hkv, d, _ptr(W),
                                     int(W.ndim == 3), r, _ptr(out)), "query_prep")
    return out


def scores(q_idx: np.ndarray, k_idx: np.ndarray, cand: np.ndarray | None = None,
           cand_block: int = 1) -> np.ndarray:
    """Indexer scores (JSSA Fig. 1): q_idx [N,Hkv,r] (float64) against the
    projected-key cache k_idx [N,Hkv,T,r]. With cand [N,Hkv,nc] int32 only the
    candidate slots are scored (cand_block tokens per entry; the fine pass of
    hierarchical indexing, LongCat abstract item 3). Returns float64
    [N,Hkv,n_out]; slots that map to no token score -inf."""
    q_idx = np.ascontiguousarray(q_idx, dtype=np.float64)
    N, Hkv, T, r = k_idx.shape
    s = _estrides(k_idx)
    if cand is not None:
        cand = np.ascontiguousarray(cand, dtype=np.int32).reshape(N * Hkv, -1)
        nc = cand.shape[1]
        n_out = nc * cand_block
    else:
        nc, n_out = 0, T
    out = np.empty((N, Hkv, n_out), dtype=np.float64)
    _check(_get().lsa_ref_scores(_ptr(q_idx), N, Hkv, r, _ptr(k_idx), _dtype_code(k_idx),
                                 s[0], s[1], s[2], T, _ptr(cand), nc, cand_block, nc,
                                 _ptr(out), n_out), "scores")
    return out


def topk(sc: np.ndarray, B: int, n_valid: np.ndarray | None = None, causal_group: int = 0,
         cand: np.ndarray | None = None, cand_block: int = 1, n_positions: int | None = None):
    """Exact top-B per row (JSSA Fig. 1) under the order (score desc,
    position asc), NaN last. sc [rows,n] (float64, or float32 which is
    widened exactly). Returns (idx int32 [rows,B] ascending, -1 padded;
    score float64 [rows,B]; count int32 [rows])."""
    sc = np.ascontiguousarray(sc, dtype=np.float64)
    rows, n = sc.shape
    nv = None if n_valid is None else np.ascontiguousarray(n_valid, dtype=np.int32)
    if cand is not None:
        cand = np.ascontiguousarray(cand, dtype=np.int32).reshape(rows, -1)
        if n_positions is None:
            raise ValueError("n_positions is required with a candidate list")
    idx = np.empty((rows, B), dtype=np.int32)
    osc = np.empty((rows, B), dtype=np.float64)
    cnt = np.empty((rows,), dtype=np.int32)
    _check(_get().lsa_ref_topk(_ptr(sc), rows, n, n, _ptr(nv), causal_group, _ptr(cand),
                               cand_block, 0 if cand is None else cand.shape[1],
                               n if n_positions is None else n_positions, B,
                               _ptr(idx), _ptr(osc), _ptr(cnt)), "topk")
    return idx, osc, cnt


def prefill_topk(q_idx: np.ndarray, k_idx: np.ndarray, B: int, row_begin: int = 0,
                 row_end: int | None = None):
    """Causal prefill indexer (LongCat abstract: O(L^2) indexer scoring): for
    query rows [row_begin,row_end) and each KV head, the top-B of
    q_idx[i,g] . k_idx[j,g] over j <= i. q_idx/k_idx [L,Hkv,r] (same dtype).
    Returns (idx int32 [rows,Hkv,B], score float64 [rows,Hkv,B])."""
    q_idx = np.ascontiguousarray(q_idx)
    k_idx = np.ascontiguousarray(k_idx)
    if q_idx.dtype != k_idx.dtype:
        raise TypeError("q_idx and k_idx must share a dtype")
    L, Hkv, r = k_idx.shape
    if row_end is None:
        row_end = L
    if not 0 <= row_begin <= row_end <= L or q_idx.shape != k_idx.shape:
        raise ValueError(f"rows [{row_begin}, {row_end}) must lie in [0, {L}] and q_idx match k_idx")
    nr = row_end - row_begin
    idx = np.empty((nr, Hkv, B), dtype=np.int32)
    osc = np.empty((nr, Hkv, B), dtype=np.float64)
    _check(_get().lsa_ref_prefill_topk(_ptr(q_idx), _ptr(k_idx), _dtype_code(k_idx), L, Hkv, r,
                                       row_begin, row_end, B, _ptr(idx), _ptr(osc)),
           "prefill_topk")
    return idx, osc


def prefill_block_topk(q_idx: np.ndarray, k_idx: np.ndarray, B: int, query_block: int,
                       want_scores: bool = False):
    """Query-block-shared prefill selection (the query_block_size option
    named on the LSA-L reproduction page; its meaning is a reading): tokens
    form blocks of query_block; block b scores k_idx[j] for j <
    min(L,(b+1)*query_block) with the block's mean q_idx, stored in the
    q_idx dtype, and keeps the top-B (B = 0: scores only). Returns (idx
    int32 [nb,Hkv,B], score float64 [nb,Hkv,B], scores float64 [nb,Hkv,L]
    with -inf past the block's prefix, or None)."""
    q_idx = np.ascontiguousarray(q_idx)
    k_idx = np.ascontiguousarray(k_idx)
    if q_idx.dtype != k_idx.dtype:
        raise TypeError("q_idx and k_idx must share a dtype")
    L, Hkv, r = k_idx.shape
    nb = (L + query_block - 1) // query_block
    idx = np.empty((nb, Hkv, max(B, 1)), dtype=np.int32)
    osc = np.empty((nb, Hkv, max(B, 1)), dtype=np.float64)
    sc = np.empty((nb, Hkv, L), dtype=np.float64) if (want_scores or B == 0) else None
    _check(_get().lsa_ref_prefill_block_topk(_ptr(q_idx), _ptr(k_idx), _dtype_code(k_idx), L, Hkv,
                                             r, int(query_block), int(B), _ptr(idx), _ptr(osc),
                                             _ptr(sc), L), "prefill_block_topk")
    return idx[..., :B], osc[..., :B], sc


def prefill_scores(q_idx: np.ndarray, k_idx: np.ndarray) -> np.ndarray:
    """Full causal indexer score matrix for small L: [L,Hkv,L] float64, -inf
    above the diagonal."""
    q_idx = np.ascontiguousarray(q_idx)
    k_idx = np.ascontiguousarray(k_idx)
    L, Hkv, r = k_idx.shape
    out = np.empty((L, Hkv, L), dtype=np.float64)
    _check(_get().lsa_ref_prefill_scores(_ptr(q_idx), _ptr(k_idx), _dtype_code(k_idx), L, Hkv, r,
                                         _ptr(out), L), "prefill_scores")
    return out


def attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, idx: np.ndarray,
              prefill: bool = False, scale: float | None = None, query_block: int = 1):
    """Indexed attention (JSSA Fig. 1 and Key contributions): each query head
    attends over its KV head's selected positions, read from the standard
    GQA cache. q [rows,Hq,d]; K, V [S,T,Hkv,d] with identical strides (d
    contiguous); idx [ceil(rows/query_block),Hkv,B] int32, -1 (or anything
    outside [0,T)) skipped. Decode: row n reads sequence n. Prefill: every
    row reads sequence 0, causally (positions after the row are skipped),
    and row i uses index row i // query_block. Returns (out float64
    [rows,Hq,d], lse float64 [rows,Hq])."""
    q = np.ascontiguousarray(q)
    rows, Hq, d = q.shape
    S, T, Hkv, _ = K.shape
    if K.strides != V.strides or K.dtype != V.dtype:
        raise ValueError("K and V must share dtype and strides")
    s = _estrides(K)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    B = idx.shape[-1]
    out = np.empty((rows, Hq, d), dtype=np.float64)
    lse = np.empty((rows, Hq), dtype=np.float64)
    _check(_get().lsa_ref_attention(1 if prefill else 0, rows, Hq, Hkv, d, B, _ptr(q),
                                    _dtype_code(q), _ptr(K), _ptr(V), _dtype_code(K),
                                    s[0], s[1], s[2], T, _ptr(idx), int(query_block),
                                    0.0 if scale is None else float(scale),
                                    _ptr(out), _ptr(lse)), "attention")
    return out, lse


def decode_step(Q: np.ndarray, W: np.ndarray, k_idx: np.ndarray, K: np.ndarray,
                V: np.ndarray, B: int) -> dict:
    """One flat decode step, JSSA Fig. 1 in its order: scoring preparation,
    candidate scoring, top-B selection, indexed attention."""
    Hkv = k_idx.shape[1]
    qi = query_prep(Q, Hkv, W)
    sc = scores(qi, k_idx)
    N, _, T = sc.shape
    idx, isc, cnt = topk(sc.reshape(N * Hkv, T), B)
    out, lse = attention(Q, K, V, idx.reshape(N, Hkv, B))
    return {"q_idx": qi, "scores": sc, "idx": idx.reshape(N, Hkv, B),
            "idx_scores": isc.reshape(N, Hkv, B), "out": out, "lse": lse}


def hierarchical_decode_step(Q: np.ndarray, W: np.ndarray, k_idx: np.ndarray,
                             cent: np.ndarray, K: np.ndarray, V: np.ndarray, block: int,
                             B_coarse: int, B: int) -> dict:
    """Coarse-to-fine decode (LongCat abstract item 3): score the block
    centroids, keep the top B_coarse blocks, score only their tokens, keep
    the top-B positions, attend (JSSA Fig. 1)."""
    N, Hkv, T, r = k_idx.shape
    nb = cent.shape[2]
    qi = query_prep(Q, Hkv, W)
    csc = scores(qi, cent)
    blocks, bsc, _ = topk(csc.reshape(N * Hkv, nb), B_coarse)
    blocks = blocks.reshape(N, Hkv, B_coarse)
    fsc = scores(qi, k_idx, cand=blocks, cand_block=block)
    idx, isc, cnt = topk(fsc.reshape(N * Hkv, -1), B, cand=blocks.reshape(N * Hkv, B_coarse),
                         cand_block=block, n_positions=T)
    out, lse = attention(Q, K, V, idx.reshape(N, Hkv, B))
    return {"q_idx": qi, "coarse_scores": csc, "blocks": blocks, "fine_scores": fsc,
            "idx": idx.reshape(N, Hkv, B), "idx_scores": isc.reshape(N, Hkv, B),
            "out": out, "lse": lse}
