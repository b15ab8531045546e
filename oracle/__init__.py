"""CPU oracle for indexer-driven sparse attention (test infrastructure).

This package is the plain, slow, obviously correct reference that the GPU
library is checked against. It is NOT part of the product: only the tests,
the package smoke check and the benchmark's CPU-baseline leg may import it,
and the GPU library never calls it. It shares no code with the GPU path: the
arithmetic lives in ``lsa_oracle.c`` (double precision throughout) and this
module only marshals numpy arrays into it.

Sources it follows (cited per function):
  * JSSA -- "Joint Subspace Sparse Attention for Efficient Long-Context
    Decoding", Fig. 1 (mean query heads score a projected-key cache, top-B
    positions per KV head, the group's heads attend to them) and Key
    contributions (per-KV-head index sets in the standard GQA cache layout).
  * LongCat -- "LongCat Sparse Attention: Taming the Lightning via
    Streaming-aware Hierarchical Cross-Layer Indexing", abstract (O(L^2)
    causal indexer scoring; item 3, hierarchical coarse-to-fine indexing).
  * The LSA-L reproduction page ("Their 42x decode speedup never compiled on
    my GPU"): the query_block_size option of its sparse-attention call, read
    as one selection per block of query tokens.
"""
from .oracle import (  # noqa: F401
    BF16,
    F32,
    FP8,
    decode_fp8,
    round_fp8,
    attention,
    build,
    centroids,
    decode_step,
    hierarchical_decode_step,
    prefill_block_topk,
    prefill_scores,
    prefill_topk,
    project_keys,
    query_prep,
    round_bf16,
    scores,
    set_threads,
    get_threads,
    topk,
)
