"""The hot path as a sequence of liblsa calls.

Flat decode step (JSSA, "Joint Subspace Sparse Attention for Efficient
Long-Context Decoding", Fig. 1 and the Fig. 9 stages):
    lsa_index_score        scoring preparation fused with candidate scoring
    lsa_topk_select        top-B per (sequence, KV head)
    lsa_indexed_attention  the group's heads attend to those B positions
Hierarchical decode step (LongCat Sparse Attention abstract, item 3): score
block centroids, keep the top blocks, score only their tokens, keep the
top-B, attend. Causal prefill (LongCat abstract, O(L^2) indexer): causal
scores + per-row top-B, then per-query indexed attention.

Plans preallocate every buffer and workspace once, so `run` allocates
nothing and can be captured in a HIP graph. All arithmetic happens in
liblsa's kernels; this module only sequences calls and holds buffers.
"""
from __future__ import annotations

import torch

from . import lsa


def _code(dtype) -> int:
    if dtype == torch.float8_e4m3fn:
        return lsa.FP8_E4M3
    return lsa.BF16 if dtype == torch.bfloat16 else lsa.F32


def _ld4(n: int) -> int:
    return (n + 3) // 4 * 4


def _select_ws(scores, B, idx, device, **kw):
    need = lsa.lsa_select_workspace_bytes(scores, B, idx, **kw)
    return torch.empty(max(need, 16), dtype=torch.uint8, device=device)


class DecodePlan:
    """Buffers for one flat decode step of N sequences with T cached tokens
    (K/V in kv_dtype; the projected-key cache in kidx_dtype, default the
    same; torch.float8_e4m3fn selects the OCP E4M3 cache)."""

    def __init__(self, N: int, Hq: int, Hkv: int, T: int, d: int, r: int, B: int,
                 device="cuda", kv_dtype=torch.bfloat16, with_idx_scores: bool = False,
                 kidx_dtype=None, fused: bool = True, one_launch: bool = False,
                 three_calls: bool = False):
        self.N, self.Hq, self.Hkv, self.T, self.d, self.r, self.B = N, Hq, Hkv, T, d, r, B
        self.with_idx_scores = with_idx_scores
        self.fused = fused
        self.one_launch = one_launch
        self.three_calls = three_calls
        self.step_ws = None
        f32 = dict(dtype=torch.float32, device=device)
        self.scores = torch.empty(N, Hkv, _ld4(T), **f32)[:, :, :T]
        self.q_idx = torch.empty(N, Hkv, r, **f32)
        self.idx = torch.empty(N, Hkv, B, dtype=torch.int32, device=device)
        self.idx_scores = torch.empty(N, Hkv, B, **f32)
        self.out = torch.empty(N, Hq, d, **f32)
        self.lse = torch.empty(N, Hq, **f32)
        # selection hint written by the scoring kernel, read by the select
        kidx_code = _code(kv_dtype if kidx_dtype is None else kidx_dtype)
        self.hint_count, self.hint_k = lsa.score_hint_layout_for(N, Hkv, T, r, kidx_code)
        self.hint = torch.empty(N * Hkv, max(1, self.hint_count), dtype=torch.int32, device=device)
        # attention and select workspaces, sized by the library for this shape
        need = lsa.attention_workspace_bytes_for(N, Hq, Hkv, d, B, T, _code(kv_dtype))
        self.attn_ws = torch.empty(max(need, 16), dtype=torch.uint8, device=device)
        self.sel_ws = _select_ws(self.scores, B, self.idx, device,
                                 hint=self.hint if self.hint_count else None, hint_k=self.hint_k)

    def score(self, q, w, k_idx, stream=None):
        lsa.lsa_index_score(k_idx, self.scores, q=q, w=w, q_idx=self.q_idx,
                            hint=self.hint if self.hint_count else None, stream=stream)

    def select(self, stream=None):
        lsa.lsa_topk_select(self.scores, self.B, self.idx,
                            out_score=self.idx_scores if self.with_idx_scores else None,
                            hint=self.hint if self.hint_count else None, hint_k=self.hint_k,
                            workspace=self.sel_ws, stream=stream)

    def attend(self, q, k, v, stream=None, *, out=None, lse=None, slot_table=None):
        """Attention over this plan's selection; out/lse default to the
        plan's buffers. With slot_table, k and v are a page-size-1 pool."""
        lsa.lsa_indexed_attention(q, k, v, self.idx, self.out if out is None else out,
                                  lse=self.lse if lse is None else lse, workspace=self.attn_ws,
                                  stream=stream, slot_table=slot_table,
                                  n_keys=self.T if slot_table is not None else None)

    def step(self, q, w, k_idx, k, v, stream=None):
        """The whole step through one lsa_decode_step call (with one_launch,
        the single persistent launch where the shape allows it)."""
        if self.step_ws is None:
            need = lsa.lsa_step_workspace_bytes(q, w, k_idx, k, v, self.idx, self.out, lse=self.lse,
                                                q_idx=self.q_idx, one_launch=self.one_launch,
                                                three_calls=self.three_calls)
            self.step_ws = torch.zeros(max(need, 16), dtype=torch.uint8, device=q.device)
        lsa.lsa_decode_step(q, w, k_idx, k, v, self.idx, self.out, lse=self.lse, q_idx=self.q_idx,
                            out_score=self.idx_scores if self.with_idx_scores else None,
                            workspace=self.step_ws, stream=stream, one_launch=self.one_launch,
                            three_calls=self.three_calls)

    def part(self, parts, q, w, k_idx, k, v, stream=None):
        """Some of the launches of step() (lsa_decode_step_part: an OR of
        lsa.STEP_PART_SCORE, _SELECT, _ATTEND), on this plan's workspace;
        step() must have run once (it allocates the workspace)."""
        lsa.lsa_decode_step_part(parts, q, w, k_idx, k, v, self.idx, self.out, workspace=self.step_ws,
                                 lse=self.lse, q_idx=self.q_idx,
                                 out_score=self.idx_scores if self.with_idx_scores else None,
                                 stream=stream, three_calls=self.three_calls)

    def step_error(self) -> int:
        """The step workspace's error word (0 when every call was clean)."""
        if self.step_ws is None:
            return 0
        return int(self.step_ws[:64].view(torch.int32)[lsa.STEP_ERROR_WORD].item())

    def run(self, q, w, k_idx, k, v, stream=None, slot_table=None):
        if self.fused and slot_table is None:
            self.step(q, w, k_idx, k, v, stream)
            return self
        self.score(q, w, k_idx, stream)
        self.select(stream)
        self.attend(q, k, v, stream, slot_table=slot_table)
        return self


def decode_step(q, w, k_idx, k, v, B, stream=None) -> dict:
    """One flat decode step; returns the step's buffers (device tensors)."""
    N, Hkv, T, r = k_idx.shape
    plan = DecodePlan(N, q.shape[1], Hkv, T, q.shape[2], r, B, device=q.device, kv_dtype=k.dtype,
                      with_idx_scores=True, kidx_dtype=k_idx.dtype, fused=False)
    plan.run(q, w, k_idx, k, v, stream)
    return {"q_idx": plan.q_idx, "scores": plan.scores, "idx": plan.idx,
            "idx_scores": plan.idx_scores, "out": plan.out, "lse": plan.lse}


class CrossLayerPlan:
    """Cross-layer index reuse over a stack of decode layers (LongCat Sparse
    Attention abstract, item 2; IndexCache and "You Only Index Once" in the
    related-paper list): `pattern` names each layer "F" (full: runs its own
    indexer, a1-a3, then attention) or "S" (shared: attention only, on the
    top-B sets of the nearest full layer before it). The first layer must be
    full. Every layer has its own Q, K, V and outputs; only full layers need
    a projected-key cache and W."""

    def __init__(self, pattern: str, N: int, Hq: int, Hkv: int, T: int, d: int, r: int, B: int,
                 device="cuda", kv_dtype=torch.bfloat16, kidx_dtype=None):
        if not pattern or pattern[0] != "F" or set(pattern) - {"F", "S"}:
            raise ValueError("pattern is a string of 'F'/'S' starting with 'F'")
        self.pattern = pattern
        self.source = []                 # layer -> the full layer whose selection it uses
        self.full = {}                   # full layer -> its DecodePlan
        for i, c in enumerate(pattern):
            if c == "F":
                self.full[i] = DecodePlan(N, Hq, Hkv, T, d, r, B, device=device, kv_dtype=kv_dtype,
                                          kidx_dtype=kidx_dtype)
            self.source.append(i if c == "F" else self.source[-1])
        f32 = dict(dtype=torch.float32, device=device)
        self.out = [self.full[i].out if c == "F" else torch.empty(N, Hq, d, **f32)
                    for i, c in enumerate(pattern)]
        self.lse = [self.full[i].lse if c == "F" else torch.empty(N, Hq, **f32)
                    for i, c in enumerate(pattern)]

    def layer(self, i, q, w, k_idx, k, v, stream=None):
        """Layer i's sparse attention; w and k_idx are read by full layers only."""
        if self.pattern[i] == "F":
            self.full[i].run(q, w, k_idx, k, v, stream)
        else:
            self.full[self.source[i]].attend(q, k, v, stream, out=self.out[i], lse=self.lse[i])

    def run(self, layers, stream=None):
        """layers: one (q, w, k_idx, k, v) per layer, in order."""
        for i, (q, w, k_idx, k, v) in enumerate(layers):
            self.layer(i, q, w, k_idx, k, v, stream)
        return self


class HierarchicalPlan:
    """Buffers for one coarse-to-fine decode step: n_blocks centroids per
    (sequence, KV head), B_coarse kept blocks of `block` tokens, top-B."""

    def __init__(self, N: int, Hq: int, Hkv: int, T: int, d: int, r: int, B: int, block: int,
                 B_coarse: int, device="cuda", kv_dtype=torch.bfloat16, kidx_dtype=None,
                 fused: bool = True, three_calls: bool = False, listed: bool = False):
        self.N, self.Hq, self.Hkv, self.T, self.d, self.r = N, Hq, Hkv, T, d, r
        self.B, self.block, self.B_coarse = B, block, B_coarse
        self.fused, self.three_calls, self.listed = fused, three_calls, listed
        self.step_ws = None
        self.n_blocks = (T + block - 1) // block
        f32 = dict(dtype=torch.float32, device=device)
        self.q_idx = torch.empty(N, Hkv, r, **f32)
        self.coarse = torch.empty(N, Hkv, _ld4(self.n_blocks), **f32)[:, :, :self.n_blocks]
        self.blocks = torch.empty(N, Hkv, B_coarse, dtype=torch.int32, device=device)
        self.n_fine = B_coarse * block
        self.fine = torch.empty(N, Hkv, _ld4(self.n_fine), **f32)[:, :, :self.n_fine]
        self.idx = torch.empty(N, Hkv, B, dtype=torch.int32, device=device)
        self.idx_scores = torch.empty(N, Hkv, B, **f32)
        self.out = torch.empty(N, Hq, d, **f32)
        self.lse = torch.empty(N, Hq, **f32)
        # the attention merges its splits in its own launch (zeroed control words)
        need = lsa.attention_workspace_bytes_for(N, Hq, Hkv, d, B, T, _code(kv_dtype), merge_in_launch=True)
        self.attn_ws = torch.empty(max(need, 16), dtype=torch.uint8, device=device)
        self.attn_ctrl = torch.zeros(lsa.ATTN_MERGE_CTRL_WORDS, dtype=torch.int32, device=device)
        code = _code(kv_dtype if kidx_dtype is None else kidx_dtype)
        self.hc_count, self.hint_k = lsa.score_hint_layout_for(N, Hkv, self.n_blocks, r, code)
        self.hf_count, _ = lsa.score_hint_layout_for(N, Hkv, self.n_fine, r, code)
        self.hint_c = torch.empty(N * Hkv, max(1, self.hc_count), dtype=torch.int32, device=device)
        self.hint_f = torch.empty(N * Hkv, max(1, self.hf_count), dtype=torch.int32, device=device)
        self.ws_c = _select_ws(self.coarse, B_coarse, self.blocks, device, hint=self.hint_c,
                               hint_k=self.hint_k)
        self.ws_f = _select_ws(self.fine, B, self.idx, device, cand=self.blocks, cand_block=block,
                               n_positions=T, hint=self.hint_f, hint_k=self.hint_k)

    def step(self, q, w, k_idx, centroids, k, v, stream=None):
        """The whole step through one lsa_hier_decode_step call."""
        kw = dict(out_blocks=self.blocks, lse=self.lse, q_idx=self.q_idx, out_score=self.idx_scores,
                  three_calls=self.three_calls, listed=self.listed)
        if self.step_ws is None:
            need = lsa.lsa_hier_step_workspace_bytes(q, w, k_idx, centroids, k, v, self.block, self.B_coarse,
                                                     self.idx, self.out, **kw)
            self.step_ws = torch.zeros(max(need, 16), dtype=torch.uint8, device=q.device)
        lsa.lsa_hier_decode_step(q, w, k_idx, centroids, k, v, self.block, self.B_coarse, self.idx, self.out,
                                 workspace=self.step_ws, stream=stream, **kw)

    def path(self, q, w, k_idx, centroids, k, v) -> str:
        return lsa.lsa_hier_step_path(q, w, k_idx, centroids, k, v, self.block, self.B_coarse, self.idx,
                                      self.out, out_blocks=self.blocks, three_calls=self.three_calls,
                                      listed=self.listed)

    def run(self, q, w, k_idx, centroids, k, v, stream=None):
        if self.fused:
            self.step(q, w, k_idx, centroids, k, v, stream)
            return self
        # coarse: score every block summary, keep the top B_coarse blocks
        lsa.lsa_index_score(centroids, self.coarse, q=q, w=w, q_idx=self.q_idx, hint=self.hint_c,
                            stream=stream)
        lsa.lsa_topk_select(self.coarse, self.B_coarse, self.blocks, hint=self.hint_c,
                            hint_k=self.hint_k, workspace=self.ws_c, stream=stream)
        # fine: score only the kept blocks' tokens, keep the top-B positions
        lsa.lsa_index_score(k_idx, self.fine, q_idx=self.q_idx, cand=self.blocks,
                            cand_block=self.block, hint=self.hint_f, stream=stream)
        lsa.lsa_topk_select(self.fine, self.B, self.idx, out_score=self.idx_scores,
                            cand=self.blocks, cand_block=self.block, n_positions=self.T,
                            hint=self.hint_f, hint_k=self.hint_k, workspace=self.ws_f,
                            stream=stream)
        lsa.lsa_indexed_attention(q, k, v, self.idx, self.out, lse=self.lse,
                                  workspace=self.attn_ws, stream=stream, merge_ctrl=self.attn_ctrl)
        return self


class PrefillPlan:
    """Buffers for causal prefill of one sequence of L tokens: per query row
    the top-B keys of its causal prefix, then indexed attention. With
    query_block = qb > 1 one selection serves each block of qb tokens (the
    block's mean query scores the keys its last token sees) and every token
    of the block attends to it causally."""

    def __init__(self, L: int, Hq: int, Hkv: int, d: int, r: int, B: int, device="cuda",
                 fused: bool = True, query_block: int = 1):
        self.L, self.Hq, self.Hkv, self.d, self.r, self.B = L, Hq, Hkv, d, r, B
        self.fused = fused
        self.query_block = qb = max(1, query_block)
        nsel = (L + qb - 1) // qb
        self.idx = torch.empty(nsel, Hkv, B, dtype=torch.int32, device=device)
        self.idx_scores = torch.empty(nsel, Hkv, B, dtype=torch.float32, device=device)
        self.out = torch.empty(L, Hq, d, dtype=torch.float32, device=device)
        self.lse = torch.empty(L, Hq, dtype=torch.float32, device=device)
        self.scores = None
        self.score_ws = None
        if qb > 1:
            # block queries, block scores and the select live in the workspace
            self.fused = True
            need = lsa.prefill_score_workspace_bytes_for(L, Hkv, r, B, query_block=qb)
            self.score_ws = torch.empty(max(need, 16), dtype=torch.uint8, device=device)
        elif fused:
            need = lsa.prefill_score_workspace_bytes_for(L, Hkv, r, B)
            self.score_ws = torch.empty(max(need, 16), dtype=torch.uint8, device=device)
        else:
            self.scores = torch.empty(L, Hkv, _ld4(L), dtype=torch.float32, device=device)[:, :, :L]

    def index(self, q_idx, k_idx, stream=None):
        if self.fused:
            lsa.lsa_index_score(k_idx, None, q_idx=q_idx, mode=lsa.MODE_PREFILL_CAUSAL,
                                topk=self.B, out_idx=self.idx, out_score=self.idx_scores,
                                workspace=self.score_ws, stream=stream,
                                query_block=self.query_block)
        else:
            lsa.lsa_index_score(k_idx, self.scores, q_idx=q_idx, mode=lsa.MODE_PREFILL_CAUSAL,
                                stream=stream)
            lsa.lsa_topk_select(self.scores, self.B, self.idx.view(self.L * self.Hkv, self.B),
                                out_score=self.idx_scores.view(self.L * self.Hkv, self.B),
                                causal_group=self.Hkv, stream=stream)

    def attend(self, q, k, v, stream=None):
        lsa.lsa_indexed_attention(q, k, v, self.idx, self.out, lse=self.lse,
                                  mode=lsa.MODE_PREFILL_CAUSAL, stream=stream,
                                  query_block=self.query_block)

    def run(self, q_idx, k_idx, q, k, v, stream=None):
        self.index(q_idx, k_idx, stream)
        self.attend(q, k, v, stream)
        return self
