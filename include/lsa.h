/*
 * lsa.h -- C ABI of liblsa: indexer-driven sparse attention on AMD MI355X
 * (gfx950, CDNA4).
 *
 * The hot path has three calls, in this order for one decode step:
 *
 *   lsa_index_score        a cheap indexer scores every cached key: the mean
 *                          of a KV head's query heads, projected to r dims,
 *                          dotted with a projected-key cache (JSSA Fig. 1;
 *                          Fig. 9 "scoring preparation" and "candidate
 *                          scoring"). Also the causal prefill indexer (LongCat
 *                          Sparse Attention abstract: O(L^2) indexer scoring)
 *                          and the fine pass of coarse-to-fine indexing
 *                          (same abstract, item 3).
 *   lsa_topk_select        exact top-B positions per row, lowest position on
 *                          ties (JSSA Fig. 1; Fig. 9 "top-B selection").
 *   lsa_indexed_attention  every query head of a GQA group attends only to
 *                          its KV head's selected positions, read in place
 *                          from the standard KV-cache layout with no gathered
 *                          copy (JSSA Key contributions; Fig. 6).
 *
 * Setup calls (outside the step): lsa_project_keys builds or appends to the
 * projected-key cache, lsa_build_centroids builds the block summaries the
 * coarse pass scores.
 *
 * Sources: JSSA = "Joint Subspace Sparse Attention for Efficient
 * Long-Context Decoding"; LongCat = "LongCat Sparse Attention: Taming the
 * Lightning via Streaming-aware Hierarchical Cross-Layer Indexing".
 *
 * Conventions for every call:
 *   - Tensor pointers are DEVICE pointers owned by the caller. The library
 *     never allocates, frees, synchronises or reads back to the host.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream of the current device) and can be captured in a HIP graph.
 *   - Every argument is validated BEFORE anything is launched; on any error
 *     nothing is launched and no output is touched.
 *   - Outputs are fully overwritten (padding included); callers never clear
 *     them first. Identical inputs give bit-identical outputs.
 *   - Strides are in ELEMENTS. Rows read with 128-bit loads need a 16-byte
 *     aligned base and row strides that are multiples of 16 bytes;
 *     misalignment is rejected (there is no slow path).
 *   - Query head h belongs to KV head h / (Hq / Hkv).
 *   - Reentrant and thread-safe; the only global state is a per-device cache
 *     of "is this a gfx950" answers and, for lsa_indexed_attention_noalloc,
 *     one static scratch buffer per device (and its looked-up address).
 *   - Return value: LSA_OK (0) or a negative lsa_status. After LSA_ERR_HIP,
 *     lsa_last_hip_error() gives the HIP error code (thread-local).
 */
#ifndef LSA_H_
#define LSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LSA_ABI_VERSION 1

/* Storage dtypes. */
/* Storage dtypes. LSA_FP8_E4M3 is the OCP 8-bit float E4M3 ("FN": no
 * infinities, largest finite 448, NaN 0x7f/0xff), accepted for the
 * projected-key cache only: decode scoring's k_idx, the output of
 * lsa_project_keys and the block centroids (JSSA Fig. 10 studies FP8
 * projected-key caches; the format is a reading). Values are rounded to it
 * once from the exact fp64 sum, to nearest-even, saturating at +-448. */
enum { LSA_F32 = 0, LSA_BF16 = 1, LSA_FP8_E4M3 = 2 };

/* Status codes. */
enum {
  LSA_OK = 0,
  LSA_ERR_INVALID_ARG = -1,    /* null/misaligned pointer, bad size or stride */
  LSA_ERR_UNSUPPORTED = -2,    /* valid but not built: dtype combo, r, d, G */
  LSA_ERR_WORKSPACE = -3,      /* workspace missing or smaller than required */
  LSA_ERR_NO_DEVICE_CODE = -4, /* current device is not gfx950 */
  LSA_ERR_HIP = -5,            /* a HIP call failed; see lsa_last_hip_error */
  LSA_ERR_SCRATCH_LIMIT = -6   /* the shape needs more than the static scratch (noalloc calls) */
};

/* Modes. Decode: a row is one (sequence, KV head). Prefill: a row is one
 * (query token, KV head) of a single sequence, row index i*Hkv + g. */
enum { LSA_MODE_DECODE = 0, LSA_MODE_PREFILL_CAUSAL = 1 };

/* ------------------------------------------------------------------------ */
/* lsa_index_score                                                          */
/* ------------------------------------------------------------------------ */
/*
 * Decode (JSSA Fig. 1): for row (n, g)
 *     q_idx[n,g,:] = ( (1/G) sum_{i<G} q[n, g*G+i, :] ) . W          (prep)
 *     scores[row, s] = q_idx[n,g,:] . k_idx[n, g, pos(s), :]          (scoring)
 *   pos(s) = s for s < n_keys when cand is NULL. With cand, slot s covers
 *   token cand[row, s / cand_block] * cand_block + s % cand_block
 *   (cand_block = 1: a position list; cand_block > 1: block ids, the fine
 *   pass of coarse-to-fine indexing, LongCat abstract item 3); n_cand *
 *   cand_block slots are written and a slot whose entry is negative or
 *   whose token is >= n_keys scores -inf. Candidate lists must be strictly
 *   increasing per row (lsa_topk_select breaks ties in slot order).
 *   The prep runs inside the scoring kernel when `q` is given (then q_idx,
 *   if not NULL, receives the fp32 q_idx); otherwise q_idx [N,Hkv,r] fp32
 *   is read.
 *
 * Prefill (LongCat abstract: the indexer's O(L^2) causal scoring):
 *     S[i,g,j] = q_idx[i,g,:] . k_idx[j,g,:] for j <= i (n_seq must be 1,
 *   q_idx [L,Hkv,r] in k_idx_dtype, k_idx read through its strides). With
 *   topk == 0 the full rows are written to scores ([L*Hkv, scores_ld], -inf
 *   above the diagonal). With topk = B > 0 the selection is fused into the
 *   scoring and no score matrix is written: out_idx [L,Hkv,B] gets exactly
 *   what lsa_topk_select would give on the causal rows, and out_score (if
 *   not NULL) the matching scores. Needs workspace
 *   (lsa_score_workspace_bytes).
 *
 * Query-block-shared prefill (query_block = qb > 1; the query_block_size
 *   option of LSA-L's sparse-attention call, "Their 42x decode speedup
 *   never compiled on my GPU", section "The failure that decided the
 *   verdict"; its meaning there is not spelled out, this is the reading):
 *   tokens form nb = ceil(L/qb) blocks. Block b's query is the mean of
 *   q_idx over its tokens [b*qb, min(L,(b+1)*qb)), taken exactly and
 *   rounded once to bf16 (nearest-even); it scores keys j < min(L,(b+1)*qb)
 *   (those its last token sees). Rows are (block, KV head), row b*Hkv + g.
 *   topk == 0: scores [nb*Hkv, scores_ld], -inf past the block's keys.
 *   topk = B > 0: out_idx [nb,Hkv,B] (+ out_score) is lsa_topk_select over
 *   those rows; scores, if given, also receive the block scores, else they
 *   live in the workspace. bf16, r = 64 only. Attention then shares each
 *   block's set among its tokens (lsa_attn_desc.query_block).
 *
 * Accumulation is fp32 over exact products of the stored values.
 *
 * Selection hint (decode, optional): with `hint` set, the call also writes
 * hint_count entries per row (lsa_score_hint_layout) at hint[row*hint_ld].
 * Each entry is an order key (the 32-bit key under which larger scores rank
 * higher) that at least hint_k of the row's scores reach, over disjoint slot
 * groups. lsa_topk_select uses it to skip its sampling pass; it never
 * changes a result, only how fast the select gets there.
 */
typedef struct lsa_score_desc {
  uint32_t struct_size;      /* sizeof(lsa_score_desc) */
  int32_t mode;              /* LSA_MODE_* */
  int32_t n_seq;             /* N (decode); 1 (prefill) */
  int32_t n_kv_heads;        /* Hkv >= 1 */
  int32_t n_keys;            /* T cached positions (decode); L (prefill) */
  int32_t rank;              /* r; r * element size in {16,32,64,128,256} bytes */

  void* q_idx;               /* see above */
  const void* q;             /* decode prep input [N,Hq,d] contiguous, or NULL */
  int32_t q_dtype;           /* LSA_F32 / LSA_BF16 */
  int32_t n_q_heads;         /* Hq, a multiple of Hkv (with q) */
  int32_t head_dim;          /* d <= 512 (with q) */
  int32_t w_per_head;        /* 0: w is [d,r]; 1: w is [Hkv,d,r] */
  const float* w;            /* fp32 projection (with q) */

  const void* k_idx;         /* projected-key cache, innermost r contiguous */
  int32_t k_idx_dtype;       /* LSA_F32 / LSA_BF16; decode also LSA_FP8_E4M3 */
  int32_t reserved0;
  int64_t k_stride_seq;      /* decode: between sequences */
  int64_t k_stride_head;     /* between KV heads */
  int64_t k_stride_tok;      /* between positions */

  const int32_t* cand;       /* decode candidate list [N*Hkv, cand_ld] or NULL */
  int32_t n_cand;
  int32_t cand_block;        /* >= 1 */
  int64_t cand_ld;

  float* scores;             /* fp32 [rows, scores_ld] */
  int64_t scores_ld;

  int32_t topk;              /* prefill fused selection budget B, or 0 */
  int32_t query_block;       /* prefill: 0 or 1 per token; qb > 1 one selection per qb tokens */
  int32_t* out_idx;          /* prefill fused: [L,Hkv,B] ascending, -1 padded */
  float* out_score;          /* prefill fused: [L,Hkv,B] or NULL */

  uint32_t* hint;            /* decode: optional selection hint [rows, hint_ld] */
  int64_t hint_ld;
} lsa_score_desc;

int lsa_index_score(const lsa_score_desc* desc, void* workspace, size_t workspace_bytes,
                    void* stream);
size_t lsa_score_workspace_bytes(const lsa_score_desc* desc);
/* Hint entries per row and keys each entry vouches for, for a decode
 * descriptor (0 / 0 when the descriptor is invalid or not decode). */
int lsa_score_hint_layout(const lsa_score_desc* desc, int32_t* count_per_row, int32_t* k);

/* ------------------------------------------------------------------------ */
/* lsa_topk_select                                                          */
/* ------------------------------------------------------------------------ */
/*
 * Per row, the min(B, #valid) valid slots that come first in the order
 * (higher score first; equal scores -- +0 and -0 are equal -- to the lower
 * slot; NaN after every number), i.e. the top-B token positions of JSSA
 * Fig. 1 with lowest-index tie-break. Their positions are written in
 * ascending order to out_idx[row, 0..count), then -1 up to B.
 *
 * Valid slots: s < n_valid[row] (all n when n_valid is NULL); with
 * causal_group = k > 0, s < min(n, row / k + 1) instead (causal prefill rows
 * i*Hkv + g use k = Hkv). With cand, slot s maps to a token as in
 * lsa_index_score and is valid only if that token is in [0, n_positions);
 * the map must be increasing so slot order is position order.
 *
 * out_score[row, j] (optional) is the score of out_idx[row, j], -inf for
 * padding; out_count[row] (optional) is the number selected. Exact integer
 * work on order-preserving 32-bit keys of the fp32 scores: the result does
 * not depend on launch shape. Rows longer than 262144 slots use workspace.
 *
 * hint (optional): the selection hint lsa_index_score wrote with the same
 * scores (hint_count entries per row, each vouching for hint_k keys). Any
 * hint -- even a stale or wrong one -- gives the same, exact result: the
 * select verifies what the hint implies and falls back when it fails.
 */
typedef struct lsa_select_desc {
  uint32_t struct_size;      /* sizeof(lsa_select_desc) */
  int32_t rows;
  int32_t n;                 /* slots per row */
  int32_t topk;              /* B >= 1 */
  const float* scores;       /* [rows, scores_ld] */
  int64_t scores_ld;
  const int32_t* n_valid;    /* [rows] or NULL */
  int32_t causal_group;      /* 0 or k > 0 */
  int32_t cand_block;        /* >= 1 (with cand) */
  const int32_t* cand;       /* [rows, cand_ld] or NULL */
  int64_t cand_ld;
  int32_t n_positions;       /* with cand: tokens >= n_positions are invalid */
  int32_t causal_block;      /* with causal_group k: row r has (r/k + 1) * max(1, causal_block) valid */
  int32_t* out_idx;          /* [rows, B] */
  float* out_score;          /* [rows, B] or NULL */
  int32_t* out_count;        /* [rows] or NULL */
  const uint32_t* hint;      /* [rows, hint_ld] or NULL */
  int64_t hint_ld;
  int32_t hint_count;        /* entries per row */
  int32_t hint_k;            /* keys each entry vouches for */
} lsa_select_desc;

int lsa_topk_select(const lsa_select_desc* desc, void* workspace, size_t workspace_bytes,
                    void* stream);
size_t lsa_select_workspace_bytes(const lsa_select_desc* desc);

/* ------------------------------------------------------------------------ */
/* lsa_indexed_attention                                                    */
/* ------------------------------------------------------------------------ */
/*
 * For each row and query head h (KV head g = h / G):
 *     z_t = scale * q[row,h,:] . K[seq, t, g, :]      for t in idx[row,g,:]
 *     out[row,h,:] = sum_t softmax(z)_t V[seq, t, g, :]
 *     lse[row,h]   = log sum_t exp(z_t)
 * Entries outside [0, n_keys) (e.g. the -1 padding) are skipped; an empty
 * set gives out = 0 and lse = -inf. Decode: seq = row. Prefill: seq = 0 for
 * every row, and causal: entries after the row's own token are skipped.
 * Prefill with query_block = qb > 1: idx is [ceil(rows/qb), Hkv, B] and
 * row i reads index row i / qb (a selection shared by qb tokens), each
 * token still masked causally. K and V rows are read in place through their strides (the
 * standard [N,T,Hkv,d] cache, or [N,Hkv,T,d]); nothing is gathered into a
 * copy (JSSA Key contributions; Fig. 6). Online softmax with fp32
 * accumulation; idx entries of one row must be distinct. Long index lists
 * are split across workgroups and merged by log-sum-exp, which needs
 * workspace (lsa_attention_workspace_bytes; it depends on the shape and
 * dtypes only, not on pointer values). Decode in bf16 with head_dim 128 and
 * 4 or 8 query heads per KV head runs on the matrix cores when q is 16-byte
 * aligned; p then enters the P.V product as two bf16 terms (about 2^-17
 * relative). Every other case runs on the vector units.
 *
 * Paged KV (page size 1, the KV-pool setting of LSA-L's serving configs,
 * "Their 42x decode speedup never compiled on my GPU", section "What their
 * numbers claim"): when slot_table is non-NULL,
 * K and V are one pool of n_pool_rows rows, row p of KV head g at
 * k + p*kv_stride_tok + g*kv_stride_head (kv_stride_seq is ignored), and
 * position t of sequence seq lives in pool row slot_table[seq*slot_table_ld
 * + t] for t < n_keys. A position outside [0, n_keys) or a pool row outside
 * [0, n_pool_rows) is skipped like the -1 padding, so a stale table entry
 * never reads outside the pool. The table is read once per selected entry,
 * where the index list is staged; the K/V loads are the unpaged ones, and
 * the result equals unpaged attention over K'[seq,t] = pool[table[seq,t]]
 * bit for bit. slot_table: int32 [n_seq, slot_table_ld], device memory
 * owned by the caller, slot_table_ld >= n_keys.
 */
typedef struct lsa_attn_desc {
  uint32_t struct_size;      /* sizeof(lsa_attn_desc) */
  int32_t mode;              /* LSA_MODE_* */
  int32_t rows;              /* N (decode) or L (prefill) */
  int32_t n_q_heads;         /* Hq */
  int32_t n_kv_heads;        /* Hkv; G = Hq/Hkv in {1,2,4,8,16} */
  int32_t head_dim;          /* d in {64, 128} */
  int32_t topk;              /* B >= 1: entries per (row, KV head) */
  int32_t n_keys;            /* T */
  const void* q;             /* [rows,Hq,d] contiguous, q_dtype */
  int32_t q_dtype;
  int32_t kv_dtype;          /* K and V share dtype and strides */
  const void* k;
  const void* v;
  int64_t kv_stride_seq;
  int64_t kv_stride_tok;
  int64_t kv_stride_head;
  const int32_t* idx;        /* [rows, Hkv, B] int32 */
  float scale;               /* <= 0: 1/sqrt(d) */
  int32_t query_block;       /* prefill: 0/1, or qb > 1: row i reads idx row i / qb */
  float* out;                /* fp32 [rows,Hq,d] */
  float* lse;                /* fp32 [rows,Hq] or NULL */
  const int32_t* slot_table; /* NULL (unpaged) or [n_seq, slot_table_ld] */
  int64_t slot_table_ld;     /* >= n_keys when slot_table is set */
  int32_t n_pool_rows;       /* >= 1 when slot_table is set */
  int32_t reserved1;
  uint32_t* merge_ctrl;      /* NULL, or LSA_ATTN_MERGE_CTRL_WORDS zeroed device words (below) */
} lsa_attn_desc;

/* merge_ctrl: with it set, decode on the matrix cores (bf16, head_dim 128,
 * G = 4 or 8, q 16-byte aligned, at most 1000 (sequence, KV head) rows)
 * merges its split partials inside the attention launch, as
 * lsa_decode_step's attention does: each row's splits are placed on one
 * XCD through per-XCD queues in these words, and the row's last split to
 * finish merges them (the same arithmetic, in the same order, as the merge
 * kernel, so the results are identical bit for bit). The words must be
 * zero before the first call that uses them; every call leaves them zero.
 * Two calls that share the words must not overlap in time. The workspace
 * (lsa_attention_workspace_bytes of the same descriptor) then holds the
 * partials on whole 128-byte lines. Other shapes ignore it. */
#define LSA_ATTN_MERGE_CTRL_WORDS 1024

int lsa_indexed_attention(const lsa_attn_desc* desc, void* workspace, size_t workspace_bytes,
                          void* stream);
size_t lsa_attention_workspace_bytes(const lsa_attn_desc* desc);

/*
 * lsa_indexed_attention_noalloc: lsa_indexed_attention with no workspace
 * argument, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation).
 * The split partials live in a static device buffer of
 * LSA_NOALLOC_SCRATCH_BYTES that each GPU the library runs on holds until
 * the process ends; the call itself allocates and frees nothing.
 *   - Same descriptor, semantics and outputs as lsa_indexed_attention (the
 *     same kernels; results are bit-identical).
 *   - A shape whose lsa_attention_workspace_bytes exceeds
 *     LSA_NOALLOC_SCRATCH_BYTES is rejected with LSA_ERR_SCRATCH_LIMIT
 *     before anything is launched. 4 MiB holds the partials of decode with
 *     up to 252 (sequence, KV head) rows of 4 query heads at B = 2048 and
 *     head_dim 128 (16640 bytes per row); the 4 x 8-row step at that shape
 *     needs 1.06 MB.
 *   - Every call on one GPU shares that GPU's buffer, which keeps the last
 *     call's contents: calls ordered on one stream are safe; calls that
 *     overlap in time on one GPU (other streams, other threads) race. No
 *     part of the buffer needs to start at zero: a call writes every
 *     partial it reads.
 *   - The first call on a device, with that device current, looks up the
 *     device's copy of the buffer (hipGetSymbolAddress) and keeps it.
 */
#define LSA_NOALLOC_SCRATCH_BYTES (4u << 20)
int lsa_indexed_attention_noalloc(const lsa_attn_desc* desc, void* stream);

/* ------------------------------------------------------------------------ */
/* lsa_decode_step                                                          */
/* ------------------------------------------------------------------------ */
/*
 * One whole flat decode step (JSSA Fig. 1, the four stages of Fig. 9): for
 * every (sequence, KV head) row, the scoring preparation, the projected-key
 * scores, the exact top-B selection and the indexed attention. The results
 * are exactly those of the sequence
 *     lsa_index_score   (decode, q and w given, selection hint on)
 *     lsa_topk_select   (with that hint)
 *     lsa_indexed_attention
 * on the same arguments: out_idx (and q_idx, out_score) bit-identical,
 * out / lse within the attention's own rounding. By default the call runs
 * those three calls in sequence with two changes that keep the results bit
 * for bit:
 *   - where the shape allows it (a bf16, fp8 or fp32 projected-key cache of
 *     4, 8 or 16 sixteen-byte pieces per key, B < T, a sample rank k, below,
 *     of at most half the sample and 64 k <= 6553), the scoring launch also
 *     does the select's collect, so no collect launch runs: each chunk of a
 *     row first scores its share of a sample of the row (one key in each
 *     group of 64 slots, at an offset hashed from the group and the row);
 *     after its stream it reads the whole row's sample, takes as threshold
 *     the 16-bit key prefix of the sample's k-th largest key,
 *     k = ceil(mu + 3.5 sqrt(mu) + 6) with mu = (samples) B / T, and lists
 *     its keys at or above the threshold; no hint is computed. The select then
 *     refines the lists, or, where they hold fewer than B keys or more than
 *     its list path takes (or a chunk found the sample incomplete), selects from
 *     the scores, which are written in full as before (the sample decides
 *     speed, never the result). lsa_step_path tells which path a shape takes;
 *   - the matrix-core decode attention merges its splits within its own
 *     launch (each row's splits on one XCD, the last to finish merging
 *     them).
 * The control words at the workspace head make both possible. With flags =
 * LSA_STEP_THREE_CALLS the call runs the three calls exactly as listed,
 * with the select's own collect launch.
 * With flags = LSA_STEP_ONE_LAUNCH, shapes
 * with a bf16 or fp8 projected-key cache of 64 or 128 bytes per key, head
 * dim 128, 1, 2, 4 or 8 query heads per KV head, B a multiple of 32 that
 * the scoring hints vouch for (T >= 32 B), at most 32 chunks of 4096 keys
 * per row and out_idx on a 128-byte boundary run instead as one persistent
 * launch: each (sequence, KV head) row is cut into chunks of 4096 keys, one
 * workgroup per chunk, all of a row's workgroups on one XCD (its L2 carries
 * the row's hand-offs); the chunk's scorer keeps its scores in LDS, the
 * row's last scorer derives the threshold from the hints, every chunk lists
 * its keys above it, the row's last lister selects the exact top B, every
 * chunk attends over its share of the selection and the last one merges
 * the partials. Either way the call is asynchronous on `stream`, allocates
 * nothing and takes one workspace (lsa_step_workspace_bytes, for the same
 * flags) that holds the scores, hints, lists, attention partials and, at
 * its head, the persistent launch's control words.
 * Workspace contract: the workspace must be all zero before the first call
 * that uses it (allocate it zeroed, or clear it once); every call leaves
 * the control words zero again, except the 32-bit error word at byte
 * offset 36, which stays set once a call of the persistent launch gives
 * up an internal wait (bit 0) or finds a row listing fewer than B keys
 * above its threshold (bit 1, which the kernel's own hints rule out); the
 * outputs of such a call are not valid. Two calls that share a workspace
 * must not overlap in time.
 */
typedef struct lsa_step_desc {
  uint32_t struct_size;      /* sizeof(lsa_step_desc) */
  int32_t n_seq;             /* N */
  int32_t n_q_heads;         /* Hq, a multiple of Hkv */
  int32_t n_kv_heads;        /* Hkv */
  int32_t head_dim;          /* d */
  int32_t rank;              /* r */
  int32_t n_keys;            /* T cached positions */
  int32_t topk;              /* B >= 1 */
  const void* q;             /* [N,Hq,d] contiguous, q_dtype (LSA_F32 / LSA_BF16) */
  int32_t q_dtype;
  int32_t w_per_head;        /* 0: w is [d,r]; 1: w is [Hkv,d,r] */
  const float* w;            /* fp32 projection */
  const void* k_idx;         /* projected-key cache [N,Hkv,T,r], innermost r contiguous */
  int32_t k_idx_dtype;       /* LSA_F32 / LSA_BF16 / LSA_FP8_E4M3 */
  int32_t kv_dtype;          /* dtype of K and V (= q_dtype) */
  int64_t k_stride_seq;      /* projected-key cache strides (elements) */
  int64_t k_stride_head;
  int64_t k_stride_tok;
  const void* k;             /* K cache, default [N,T,Hkv,d], through its strides */
  const void* v;             /* V cache, same strides */
  int64_t kv_stride_seq;
  int64_t kv_stride_tok;
  int64_t kv_stride_head;
  float scale;               /* <= 0: 1/sqrt(d) */
  int32_t flags;             /* 0, LSA_STEP_ONE_LAUNCH or LSA_STEP_THREE_CALLS */
  float* q_idx;              /* optional out: fp32 [N,Hkv,r] */
  int32_t* out_idx;          /* [N,Hkv,B] ascending positions, -1 padded */
  float* out_score;          /* optional out: fp32 [N,Hkv,B] */
  float* out;                /* fp32 [N,Hq,d] */
  float* lse;                /* optional out: fp32 [N,Hq] */
} lsa_step_desc;

/* flags: run the one-launch kernel (scoring, selection and attention in a
 * single persistent launch) where the shape allows it; without the flag the
 * step always runs the three calls. */
#define LSA_STEP_ONE_LAUNCH 1
/* flags: run the three calls exactly as listed above, with the select's own
 * collect launch, instead of the default path's listing scoring launch. */
#define LSA_STEP_THREE_CALLS 2

int lsa_decode_step(const lsa_step_desc* desc, void* workspace, size_t workspace_bytes, void* stream);
size_t lsa_step_workspace_bytes(const lsa_step_desc* desc);

/* The launches of lsa_decode_step's default path one group at a time:
 * `parts` is a nonzero OR of the flags below, and the call issues the named
 * parts, in order, exactly as lsa_decode_step issues them (the same
 * descriptor, flags and workspace). Calling SCORE, SELECT and ATTEND in
 * that order on one stream equals one lsa_decode_step call, bit for bit. A
 * caller may put its own work between the parts, or time one part alone
 * (a part may be repeated: each call of SCORE leaves the workspace's control
 * words zero again). Reads and writes: SCORE the scores, q_idx, lists and
 * samples in the workspace; SELECT those, writing out_idx / out_score;
 * ATTEND out_idx, writing out / lse. Returns LSA_ERR_UNSUPPORTED for a
 * descriptor that runs as the one persistent launch (it has no parts), and
 * LSA_ERR_INVALID_ARG for parts outside 1..7. */
#define LSA_STEP_PART_SCORE 1    /* scoring prep and scores (with the select's lists where listed) */
#define LSA_STEP_PART_SELECT 2   /* exact top-B (the collect and the row select, or the row select) */
#define LSA_STEP_PART_ATTEND 4   /* indexed attention, splits merged in the launch */
#define LSA_STEP_PART_ALL 7
int lsa_decode_step_part(const lsa_step_desc* desc, int parts, void* workspace, size_t workspace_bytes,
                         void* stream);
/* 1 when the descriptor (its shape and flags) runs as the one persistent
 * launch, 0 when it runs the three calls in sequence, -1 when the
 * descriptor is invalid. */
int lsa_step_is_fused(const lsa_step_desc* desc);
/* The path a descriptor (its shape and flags) runs: LSA_STEP_PATH_*, or -1
 * when the descriptor is invalid. */
#define LSA_STEP_PATH_THREE_CALLS 0
#define LSA_STEP_PATH_LISTED 1
#define LSA_STEP_PATH_ONE_LAUNCH 2
int lsa_step_path(const lsa_step_desc* desc);

/* ------------------------------------------------------------------------ */
/* lsa_hier_decode_step                                                     */
/* ------------------------------------------------------------------------ */
/*
 * One whole coarse-to-fine decode step (LongCat Sparse Attention abstract,
 * hierarchical indexing; JSSA Fig. 1 for the scoring and attention): for
 * every (sequence, KV head) row, the block summaries (centroids, from
 * lsa_build_centroids) are scored with the row's q_idx (the scoring prep
 * runs here), the n_blocks_kept best blocks are kept, every token of the
 * kept blocks is scored and the exact top-B of those tokens is attended.
 * The results are exactly those of the sequence
 *     lsa_index_score   (decode over the centroids, q and w given, hint on)
 *     lsa_topk_select   (top n_blocks_kept blocks, that hint)
 *     lsa_index_score   (decode over the kept blocks' tokens: cand = the
 *                        blocks, cand_block = block, q_idx from the first)
 *     lsa_topk_select   (top B, the same candidate map, n_positions = T)
 *     lsa_indexed_attention
 * on the same arguments: out_blocks, out_idx, q_idx, out_score bit-identical,
 * out / lse within the attention's own rounding. The attention merges its
 * splits in its own launch. Each stage (coarse over the block summaries,
 * fine over the kept blocks' tokens, through the candidate map) runs either
 * as its two separate calls or as one scoring launch that lists its
 * select's candidates (the listing path of lsa_decode_step) followed by the
 * select over the lists. By default a stage lists when its rows hold at
 * least LSA_HIER_LIST_MIN_SLOTS slots and the shape allows it; on shorter
 * rows the separate calls were measured faster (56.8 us per step at 16384
 * summaries and 128 blocks of 64, against 59.0 with the fine stage listed
 * and 64.7 with both). flags = LSA_STEP_THREE_CALLS always runs the separate
 * calls; LSA_STEP_LISTED lists both stages wherever the shape allows it.
 * Asynchronous on `stream`; allocates nothing; one workspace
 * (lsa_hier_step_workspace_bytes, same descriptor), all zero before its
 * first use; every call leaves its control words zero again. Two calls
 * sharing a workspace must not overlap in time. Returns the LSA_ERR_* code
 * of the first of the calls above that rejects its part of the descriptor.
 */
typedef struct lsa_hier_step_desc {
  uint32_t struct_size;      /* sizeof(lsa_hier_step_desc) */
  int32_t n_seq;             /* N */
  int32_t n_q_heads;         /* Hq, a multiple of Hkv */
  int32_t n_kv_heads;        /* Hkv */
  int32_t head_dim;          /* d */
  int32_t rank;              /* r */
  int32_t n_keys;            /* T cached positions */
  int32_t topk;              /* B */
  int32_t block;             /* tokens per block */
  int32_t n_blocks_kept;     /* blocks kept per row (B_coarse) */
  const void* q;             /* [N,Hq,d] contiguous, q_dtype */
  int32_t q_dtype;
  int32_t w_per_head;        /* 0: w is [d,r]; 1: w is [Hkv,d,r] */
  const float* w;
  const void* k_idx;         /* projected-key cache [N,Hkv,T,r] through its strides */
  int32_t k_idx_dtype;
  int32_t kv_dtype;          /* dtype of K and V (= q_dtype) */
  int64_t k_stride_seq, k_stride_head, k_stride_tok;
  const void* centroids;     /* [N,Hkv,ceil(T/block),r], k_idx_dtype, through its strides */
  int64_t c_stride_seq, c_stride_head, c_stride_blk;
  const void* k;             /* K cache [N,T,Hkv,d] through its strides */
  const void* v;             /* V cache, same strides */
  int64_t kv_stride_seq, kv_stride_tok, kv_stride_head;
  float scale;               /* <= 0: 1/sqrt(d) */
  int32_t flags;             /* 0, LSA_STEP_THREE_CALLS or LSA_STEP_LISTED */
  float* q_idx;              /* optional out: fp32 [N,Hkv,r] */
  int32_t* out_blocks;       /* optional out: [N,Hkv,n_blocks_kept] ascending block numbers */
  int32_t* out_idx;          /* [N,Hkv,B] ascending positions, -1 padded */
  float* out_score;          /* optional out: fp32 [N,Hkv,B] */
  float* out;                /* fp32 [N,Hq,d] */
  float* lse;                /* optional out: fp32 [N,Hq] */
} lsa_hier_step_desc;

/* flags of lsa_hier_decode_step: both stages' listing launches wherever
 * the shape allows them, whatever the row length */
#define LSA_STEP_LISTED 4
/* row length (slots: summaries for the coarse stage, n_blocks_kept * block
 * for the fine stage) from which the default path lists a stage */
#define LSA_HIER_LIST_MIN_SLOTS 32768

int lsa_hier_decode_step(const lsa_hier_step_desc* desc, void* workspace, size_t workspace_bytes,
                         void* stream);
size_t lsa_hier_step_workspace_bytes(const lsa_hier_step_desc* desc);
/* LSA_STEP_PATH_LISTED when the fine stage lists its candidates in the
 * scoring launch, LSA_STEP_PATH_THREE_CALLS when it runs the separate calls,
 * -1 for an invalid descriptor (the coarse stage follows the same rule on
 * its own row length). */
int lsa_hier_step_path(const lsa_hier_step_desc* desc);

/* ------------------------------------------------------------------------ */
/* Setup calls                                                              */
/* ------------------------------------------------------------------------ */
/*
 * lsa_project_keys: out[n,g,t,:] = round(K[n,t,g,:] . W) for tokens t in
 * [tok_begin, tok_begin + n_tok) -- building the projected-key cache, or
 * appending the newest token's projected key (JSSA Fig. 9 calls the key
 * projection negligible). The sum is exact-product fp64, rounded once to
 * out_dtype (round to nearest even), so the result equals a double-precision
 * reference bit for bit.
 */
typedef struct lsa_project_desc {
  uint32_t struct_size;      /* sizeof(lsa_project_desc) */
  int32_t n_seq;
  int32_t n_kv_heads;
  int32_t head_dim;          /* d <= 512 */
  int32_t rank;              /* r <= 256 */
  int32_t tok_begin;
  int32_t n_tok;
  int32_t k_dtype;           /* LSA_F32 / LSA_BF16 */
  const void* k;             /* K cache, innermost d contiguous */
  int64_t k_stride_seq;
  int64_t k_stride_tok;
  int64_t k_stride_head;
  const float* w;            /* [d,r] or [Hkv,d,r] fp32 */
  int32_t w_per_head;
  int32_t out_dtype;         /* LSA_F32 / LSA_BF16 / LSA_FP8_E4M3 */
  void* out;                 /* projected-key cache, innermost r contiguous */
  int64_t out_stride_seq;
  int64_t out_stride_head;
  int64_t out_stride_tok;
} lsa_project_desc;

int lsa_project_keys(const lsa_project_desc* desc, void* stream);

/*
 * lsa_build_centroids: out[n,g,b,:] = round(mean of in[n,g,t,:] over the
 * tokens t of block b), blocks of `block` tokens, a partial last block
 * averaged over its tokens -- the block summaries scored by the coarse pass
 * of hierarchical indexing (LongCat abstract item 3). fp64 sum, one rounding.
 */
typedef struct lsa_centroid_desc {
  uint32_t struct_size;      /* sizeof(lsa_centroid_desc) */
  int32_t n_seq;
  int32_t n_kv_heads;
  int32_t n_keys;            /* T */
  int32_t rank;              /* r <= 256 */
  int32_t block;             /* >= 1 */
  int32_t dtype;             /* of both in and out: LSA_F32 / LSA_BF16 / LSA_FP8_E4M3 */
  const void* in;            /* projected-key cache */
  int64_t in_stride_seq;
  int64_t in_stride_head;
  int64_t in_stride_tok;
  void* out;                 /* [.., ceil(T/block), r] */
  int64_t out_stride_seq;
  int64_t out_stride_head;
  int64_t out_stride_blk;
} lsa_centroid_desc;

int lsa_build_centroids(const lsa_centroid_desc* desc, void* stream);

/* ------------------------------------------------------------------------ */
/* lsa_stream_read (measurement)                                            */
/* ------------------------------------------------------------------------ */
/*
 * A plain streaming read of `bytes` bytes at `buf`: the achievable HBM read
 * bandwidth on this part, the reference beside the published peak for the
 * memory-bound calls above (the scoring stream of lsa_index_score reads its
 * projected-key cache the same way: 16-byte nontemporal loads). Not part of
 * the method. buf: device memory, 16-byte aligned; bytes: a positive
 * multiple of 16. sink: LSA_STREAM_READ_SINK_WORDS device uint32 words,
 * all overwritten; the XOR of them all is the XOR of every 32-bit word of
 * the buffer (which keeps the loads alive and makes the read checkable).
 * Errors: LSA_ERR_INVALID_ARG for a null or misaligned pointer or a bad
 * size.
 */
#define LSA_STREAM_READ_SINK_WORDS 8192
int lsa_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream);

/* ------------------------------------------------------------------------ */
/* Helpers                                                                  */
/* ------------------------------------------------------------------------ */
const char* lsa_status_str(int status);   /* static string, never NULL */
int lsa_last_hip_error(void);             /* HIP error of this thread's last LSA_ERR_HIP */
int lsa_abi_version(void);                /* LSA_ABI_VERSION */
/* sizeof of a descriptor, for bindings: 0 score, 1 select, 2 attention,
 * 3 project, 4 centroid, 5 step, 6 hierarchical step; 0 for anything else. */
size_t lsa_desc_size(int which);

#ifdef __cplusplus
}
#endif

#endif /* LSA_H_ */
