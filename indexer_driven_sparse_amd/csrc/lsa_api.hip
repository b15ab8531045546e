// C ABI of liblsa: argument validation, launch planning and dispatch.
// Every check runs before the first HIP call of an entry point, so a
// rejected call launches nothing and touches no output.
#include <algorithm>
#include <atomic>
#include <climits>
#include <cmath>
#include <cstring>

#include "lsa.h"
#include "kernels.hpp"

namespace {

thread_local int g_last_hip = 0;

int hip_fail(hipError_t e) {
  g_last_hip = (int)e;
  return LSA_ERR_HIP;
}

bool al16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// The MFMA prefill paths read q_idx / k_idx rows as 16-byte fragments.
bool mfma_rows_ok(const lsa_score_desc* d) {
  return al16(d->k_idx) && al16(d->q_idx) && d->k_stride_tok % 8 == 0 && d->k_stride_head % 8 == 0;
}
// Bytes per element of a storage dtype (0: unknown).
int esize(int dtype) {
  return dtype == LSA_BF16 ? 2 : dtype == LSA_F32 ? 4 : dtype == LSA_FP8_E4M3 ? 1 : 0;
}
// fp32 / bf16 only (queries, K/V, projection inputs, prefill caches).
int esize_wide(int dtype) { return dtype == LSA_FP8_E4M3 ? 0 : esize(dtype); }
bool pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }
bool strides16(int es, int64_t a, int64_t b, int64_t c) {
  return a >= 0 && b >= 0 && c >= 0 && (a * es) % 16 == 0 && (b * es) % 16 == 0 && (c * es) % 16 == 0;
}

// gfx950 check, cached per device (the library's only global state).
constexpr int kMaxDevices = 64;
std::atomic<int> g_device_state[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other

int check_device() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev < 0 || dev >= kMaxDevices) return LSA_ERR_NO_DEVICE_CODE;
  int st = g_device_state[dev].load(std::memory_order_acquire);
  if (st == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return hip_fail(e);
    st = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_device_state[dev].store(st, std::memory_order_release);
  }
  return st == 1 ? LSA_OK : LSA_ERR_NO_DEVICE_CODE;
}

// XCD count of the current device, cached per device (0 when unknown).
std::atomic<int> g_device_xccs[kMaxDevices];

int device_xccs() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  int n = g_device_xccs[dev].load(std::memory_order_acquire);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess) return 0;
    g_device_xccs[dev].store(n, std::memory_order_release);
  }
  return n;
}

#define LSA_TRY(expr)              \
  do {                             \
    int _rc = (expr);              \
    if (_rc != LSA_OK) return _rc; \
  } while (0)

// ---------------------------------------------------------------------------
// lsa_index_score
// ---------------------------------------------------------------------------
size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Query-block-shared prefill: workspace = block queries | block scores (when
// the caller gives none) | the select's own workspace.
struct BlockWs {
  uint16_t* qbar;
  float* scores;
  int64_t ld;
  void* sel;
};
size_t block_prefill_layout(const lsa_score_desc* d, void* base, BlockWs* w) {
  const int qb = d->query_block;
  const int nb = (d->n_keys + qb - 1) / qb;
  const int rows = nb * d->n_kv_heads;
  size_t off = align256((size_t)rows * d->rank * 2);
  const int64_t ld = d->scores ? d->scores_ld : ((int64_t)d->n_keys + 3) / 4 * 4;
  const size_t sc_off = off;
  if (!d->scores) off += align256((size_t)rows * ld * sizeof(float));
  const size_t sel_off = off;
  if (d->topk > 0) off += lsa::select_workspace(rows, d->n_keys, d->topk, false);
  if (w) {
    char* b = (char*)base;
    w->qbar = (uint16_t*)b;
    w->scores = d->scores ? d->scores : (float*)(b + sc_off);
    w->ld = ld;
    w->sel = b + sel_off;
  }
  return off;
}

int64_t score_slots(const lsa_score_desc* d) {
  if (d->mode == LSA_MODE_DECODE && d->cand) return (int64_t)d->n_cand * d->cand_block;
  return d->n_keys;
}

int validate_score(const lsa_score_desc* d, size_t* ws_need) {
  if (!d || d->struct_size != sizeof(lsa_score_desc)) return LSA_ERR_INVALID_ARG;
  *ws_need = 0;
  const int ke = esize(d->k_idx_dtype);
  if (ke == 0) return LSA_ERR_UNSUPPORTED;
  if (d->n_kv_heads < 1 || d->n_keys < 1 || d->rank < 1) return LSA_ERR_INVALID_ARG;
  const int64_t rbytes = (int64_t)d->rank * ke;
  if (!pow2(rbytes) || rbytes < 16 || rbytes > 256) return LSA_ERR_UNSUPPORTED;
  if (!d->k_idx || !al16(d->k_idx)) return LSA_ERR_INVALID_ARG;
  if (!strides16(ke, d->k_stride_seq, d->k_stride_head, d->k_stride_tok)) return LSA_ERR_INVALID_ARG;
  if (d->k_stride_tok < d->rank) return LSA_ERR_INVALID_ARG;
  if (d->mode == LSA_MODE_DECODE) {
    if (d->n_seq < 1) return LSA_ERR_INVALID_ARG;
    const int64_t rows = (int64_t)d->n_seq * d->n_kv_heads;
    if (rows > 65535) return LSA_ERR_UNSUPPORTED;
    if (d->q) {
      if (esize_wide(d->q_dtype) == 0) return LSA_ERR_UNSUPPORTED;
      if (d->n_q_heads < d->n_kv_heads || d->n_q_heads % d->n_kv_heads != 0) return LSA_ERR_INVALID_ARG;
      if (d->head_dim < 1 || d->head_dim > 512) return LSA_ERR_UNSUPPORTED;
      if (!d->w) return LSA_ERR_INVALID_ARG;
      if (d->w_per_head != 0 && d->w_per_head != 1) return LSA_ERR_INVALID_ARG;
    } else if (!d->q_idx) {
      return LSA_ERR_INVALID_ARG;
    }
    if (d->cand) {
      if (d->n_cand < 1 || d->cand_block < 1 || d->cand_ld < d->n_cand) return LSA_ERR_INVALID_ARG;
      if ((int64_t)d->n_cand * d->cand_block > INT_MAX) return LSA_ERR_UNSUPPORTED;
    }
    if (!d->scores || !al16(d->scores) || d->scores_ld % 4 != 0 || d->scores_ld < score_slots(d))
      return LSA_ERR_INVALID_ARG;
    if (d->topk != 0 || d->out_idx || d->out_score || d->query_block > 1) return LSA_ERR_INVALID_ARG;
    if (d->hint && (((uintptr_t)d->hint & 3u) || d->hint_ld < lsa::score_hint_count((int)score_slots(d), d->k_idx_dtype)))
      return LSA_ERR_INVALID_ARG;
    return LSA_OK;
  }
  if (d->mode == LSA_MODE_PREFILL_CAUSAL) {
    if (d->n_seq != 1 || !d->q_idx || d->q || d->cand || d->hint) return LSA_ERR_INVALID_ARG;
    if (esize_wide(d->k_idx_dtype) == 0) return LSA_ERR_UNSUPPORTED;
    if (!al16(d->q_idx)) return LSA_ERR_INVALID_ARG;
    if (d->topk < 0 || d->query_block < 0) return LSA_ERR_INVALID_ARG;
    if (d->query_block > 1) {
      if (d->k_idx_dtype != LSA_BF16 || !lsa::prefill_mfma_scores_supported(d->rank) || !mfma_rows_ok(d))
        return LSA_ERR_UNSUPPORTED;
      const int nb = (d->n_keys + d->query_block - 1) / d->query_block;
      if ((d->n_keys + 31) / 32 > 65535 || ((int64_t)nb * d->n_kv_heads + 31) / 32 > 65535)
        return LSA_ERR_UNSUPPORTED;
      if (d->scores && (!al16(d->scores) || d->scores_ld % 4 != 0 || d->scores_ld < d->n_keys))
        return LSA_ERR_INVALID_ARG;
      if (d->topk == 0 && (!d->scores || d->out_idx || d->out_score)) return LSA_ERR_INVALID_ARG;
      if (d->topk > 0 && !d->out_idx) return LSA_ERR_INVALID_ARG;
      *ws_need = block_prefill_layout(d, nullptr, nullptr);
      return LSA_OK;
    }
    if (d->topk == 0) {
      const bool mfma = d->k_idx_dtype == LSA_BF16 && lsa::prefill_mfma_scores_supported(d->rank) &&
                        mfma_rows_ok(d);
      if (!mfma && (int64_t)d->n_keys * d->n_kv_heads > 65535) return LSA_ERR_UNSUPPORTED;
      if (mfma && (d->n_keys + 31) / 32 > 65535) return LSA_ERR_UNSUPPORTED;
      if (!d->scores || !al16(d->scores) || d->scores_ld % 4 != 0 || d->scores_ld < d->n_keys)
        return LSA_ERR_INVALID_ARG;
      return LSA_OK;
    }
    if (!d->out_idx) return LSA_ERR_INVALID_ARG;
    if (d->k_idx_dtype != LSA_BF16 || !lsa::prefill_topk_supported(d->n_keys, d->rank, d->topk) ||
        !mfma_rows_ok(d))
      return LSA_ERR_UNSUPPORTED;
    *ws_need = lsa::prefill_topk_workspace(d->n_keys, d->n_kv_heads, d->topk);
    return LSA_OK;
  }
  return LSA_ERR_INVALID_ARG;
}

// ---------------------------------------------------------------------------
// lsa_topk_select
// ---------------------------------------------------------------------------
int validate_select(const lsa_select_desc* d, size_t* ws_need) {
  if (!d || d->struct_size != sizeof(lsa_select_desc)) return LSA_ERR_INVALID_ARG;
  if (d->rows < 1 || d->n < 1 || d->topk < 1) return LSA_ERR_INVALID_ARG;
  if (!d->scores || !al16(d->scores) || d->scores_ld % 4 != 0 || d->scores_ld < d->n)
    return LSA_ERR_INVALID_ARG;
  if (!d->out_idx) return LSA_ERR_INVALID_ARG;
  if (d->causal_group < 0 || (d->causal_group > 0 && d->n_valid) || d->causal_block < 0)
    return LSA_ERR_INVALID_ARG;
  if (d->cand) {
    if (d->cand_block < 1 || d->n_positions < 0) return LSA_ERR_INVALID_ARG;
    if (d->cand_ld < ((int64_t)d->n + d->cand_block - 1) / d->cand_block) return LSA_ERR_INVALID_ARG;
  }
  if (d->hint && (d->hint_count < 1 || d->hint_k < 1 || d->hint_ld < d->hint_count ||
                  ((uintptr_t)d->hint & 3u)))
    return LSA_ERR_INVALID_ARG;
  const bool hint_usable = d->hint && (int64_t)d->hint_count * d->hint_k >= d->topk;
  *ws_need = lsa::select_workspace(d->rows, d->n, d->topk, hint_usable);
  return LSA_OK;
}

// ---------------------------------------------------------------------------
// lsa_indexed_attention
// Decode shapes the matrix cores take: bf16, d = 128, G = 4 or 8, and a
// grid of 512-thread workgroups under 2^32 threads. The launch also wants
// q 16-byte aligned (its rows are read 16 bytes at a time); the workspace
// is sized for either path, so it depends on the shape alone.
bool decode_mfma_shape(const lsa_attn_desc* d) {
  if (d->mode != LSA_MODE_DECODE) return false;
  const int G = d->n_q_heads / d->n_kv_heads;
  if (!lsa::attention_decode_mfma_supported(G, d->head_dim, d->topk, d->kv_dtype == LSA_BF16)) return false;
  const int64_t splits = (d->topk + lsa::kDecodeSplit - 1) / lsa::kDecodeSplit;
  return (int64_t)d->rows * d->n_kv_heads * splits < (int64_t{1} << 23);
}

// ---------------------------------------------------------------------------
int validate_attn(const lsa_attn_desc* d, size_t* ws_need) {
  if (!d || d->struct_size != sizeof(lsa_attn_desc)) return LSA_ERR_INVALID_ARG;
  if (d->mode != LSA_MODE_DECODE && d->mode != LSA_MODE_PREFILL_CAUSAL) return LSA_ERR_INVALID_ARG;
  if (d->rows < 1 || d->n_kv_heads < 1 || d->n_q_heads < d->n_kv_heads || d->topk < 1 || d->n_keys < 1)
    return LSA_ERR_INVALID_ARG;
  if (d->n_q_heads % d->n_kv_heads != 0) return LSA_ERR_INVALID_ARG;
  const int G = d->n_q_heads / d->n_kv_heads;
  if (!lsa::attention_supported(G, d->head_dim)) return LSA_ERR_UNSUPPORTED;
  const int ke = esize_wide(d->kv_dtype);
  if (ke == 0 || d->q_dtype != d->kv_dtype) return LSA_ERR_UNSUPPORTED;
  if (!d->q || !d->k || !d->v || !d->idx || !d->out) return LSA_ERR_INVALID_ARG;
  if (!al16(d->k) || !al16(d->v)) return LSA_ERR_INVALID_ARG;
  const bool paged = d->slot_table != nullptr;
  if (!strides16(ke, paged ? 0 : d->kv_stride_seq, d->kv_stride_tok, d->kv_stride_head))
    return LSA_ERR_INVALID_ARG;
  if (paged && (d->n_pool_rows < 1 || d->slot_table_ld < d->n_keys || (uintptr_t)d->slot_table % 4 != 0))
    return LSA_ERR_INVALID_ARG;
  if (d->query_block < 0 || (d->query_block > 1 && d->mode != LSA_MODE_PREFILL_CAUSAL))
    return LSA_ERR_INVALID_ARG;
  int sp, kps;
  lsa::attention_plan(d->rows, d->n_kv_heads, G, d->head_dim, d->topk, false, &sp, &kps);
  if ((int64_t)d->rows * d->n_kv_heads * sp > INT_MAX) return LSA_ERR_UNSUPPORTED;
  size_t need = lsa::attention_workspace(d->rows, d->n_kv_heads, G, d->head_dim, d->topk, false);
  if (decode_mfma_shape(d)) {
    need = std::max(need, lsa::attention_workspace(d->rows, d->n_kv_heads, G, d->head_dim, d->topk, true));
    if (d->merge_ctrl) {   // the in-launch merge keeps each split partial on whole 128-byte lines
      int sp2 = 1, kps2 = 0;
      lsa::attention_plan(d->rows, d->n_kv_heads, G, d->head_dim, d->topk, true, &sp2, &kps2);
      need = std::max(need, (size_t)d->rows * d->n_kv_heads * sp2 * lsa::decode_partial_stride(G) * sizeof(float));
    }
  }
  if (d->merge_ctrl && (uintptr_t)d->merge_ctrl % 4 != 0) return LSA_ERR_INVALID_ARG;
  *ws_need = need;
  return LSA_OK;
}

int check_ws(void* ws, size_t have, size_t need) {
  if (need == 0) return LSA_OK;
  if (!ws || have < need || !al16(ws)) return LSA_ERR_WORKSPACE;
  return LSA_OK;
}

// Launch an attention call whose descriptor has been validated; ws holds
// the split partials (the caller's workspace, or the static scratch).
// ctrl/nxcc: the decode step's zeroed control words and the XCD count; with
// them the matrix-core decode path merges its splits in the launch.
int run_attention(const lsa_attn_desc* d, void* ws, void* stream, uint32_t* ctrl = nullptr, int nxcc = 0) {
  lsa::AttnArgs a{};
  a.q = d->q;
  a.k = d->k;
  a.v = d->v;
  const bool paged = d->slot_table != nullptr;
  a.s_seq = paged ? 0 : d->kv_stride_seq;   // a pool has no per-sequence base
  a.s_tok = d->kv_stride_tok;
  a.s_head = d->kv_stride_head;
  a.slot = d->slot_table;
  a.slot_ld = paged ? d->slot_table_ld : 0;
  a.n_rows_kv = paged ? d->n_pool_rows : d->n_keys;
  a.idx = d->idx;
  a.rows = d->rows;
  a.Hq = d->n_q_heads;
  a.Hkv = d->n_kv_heads;
  a.d = d->head_dim;
  a.B = d->topk;
  a.T = d->n_keys;
  a.prefill = d->mode == LSA_MODE_PREFILL_CAUSAL;
  a.qblk = d->query_block > 1 ? d->query_block : 1;
  const float scale = d->scale > 0.f ? d->scale : 1.0f / std::sqrt((float)d->head_dim);
  a.scale_log2 = scale * 1.4426950408889634f;
  a.out = d->out;
  a.lse = d->lse;
  a.partial = (float*)ws;
  const bool mfma_decode = decode_mfma_shape(d) && al16(d->q);
  lsa::attention_plan(d->rows, d->n_kv_heads, a.Hq / a.Hkv, a.d, a.B, mfma_decode, &a.splits,
                      &a.keys_per_split);
  hipError_t e;
  if (mfma_decode && ctrl != nullptr && nxcc >= 1 && nxcc <= 8 && (int64_t)d->rows * d->n_kv_heads <= 1000) {
    a.ctrl = ctrl;
    a.nxcc = nxcc;
  }
  if (mfma_decode)
    e = lsa::launch_attention_decode_mfma(a, (hipStream_t)stream);
  else if (lsa::attention_mfma_supported(a, d->kv_dtype == LSA_BF16))
    e = lsa::launch_attention_mfma(a, (hipStream_t)stream);
  else
    e = lsa::launch_attention(a, d->q_dtype == LSA_BF16, d->kv_dtype == LSA_BF16, (hipStream_t)stream);
  return e == hipSuccess ? LSA_OK : hip_fail(e);
}

}  // namespace

namespace {

// ---------------------------------------------------------------------------
// lsa_decode_step: the three calls' descriptors, built from one step
// descriptor, and the workspace layout they share.
// ---------------------------------------------------------------------------
struct StepPlan {
  lsa_score_desc score;
  lsa_select_desc select;
  lsa_attn_desc attn;
  bool fused;
  bool listed;                 // the scoring launch lists the select's candidates
  int rows, wpr;
  int list_rank, list_chunk, list_wpr;
  int64_t s_ld;
  size_t off_samples, off_lmeta, off_lists2, off_qidx;
  size_t off_scores, off_hint, off_sel, off_attn;           // three calls
  size_t off_lists, off_meta, off_partial;                  // fused
  size_t total;
  size_t sel_bytes, attn_bytes;
};

int plan_step(const lsa_step_desc* d, StepPlan* p) {
  if (!d || d->struct_size != sizeof(lsa_step_desc)) return LSA_ERR_INVALID_ARG;
  if (d->n_seq < 1 || d->n_kv_heads < 1 || d->n_keys < 1 || d->topk < 1) return LSA_ERR_INVALID_ARG;
  if (d->flags & ~(LSA_STEP_ONE_LAUNCH | LSA_STEP_THREE_CALLS)) return LSA_ERR_INVALID_ARG;
  const int64_t rows = (int64_t)d->n_seq * d->n_kv_heads;
  if (rows > 65535) return LSA_ERR_UNSUPPORTED;
  const int64_t ld = ((int64_t)d->n_keys + 31) / 32 * 32;   // rows of whole 128-byte lines
  const int hint_count = lsa::score_hint_count(d->n_keys, d->k_idx_dtype);
  const int hint_ld = (hint_count + 31) / 32 * 32;   // rows of whole 128-byte lines
  const size_t ctrl_bytes = align256((size_t)lsa::step_ctrl_words((int)rows) * 4);
  p->rows = (int)rows;
  p->off_scores = ctrl_bytes;
  p->off_hint = p->off_scores + align256((size_t)rows * ld * sizeof(float));
  p->off_sel = p->off_hint + align256((size_t)rows * hint_ld * sizeof(uint32_t));

  lsa_score_desc& sd = p->score;
  std::memset(&sd, 0, sizeof(sd));
  sd.struct_size = sizeof(sd);
  sd.mode = LSA_MODE_DECODE;
  sd.n_seq = d->n_seq;
  sd.n_kv_heads = d->n_kv_heads;
  sd.n_keys = d->n_keys;
  sd.rank = d->rank;
  sd.q_idx = d->q_idx;
  sd.q = d->q;
  sd.q_dtype = d->q_dtype;
  sd.n_q_heads = d->n_q_heads;
  sd.head_dim = d->head_dim;
  sd.w_per_head = d->w_per_head;
  sd.w = d->w;
  sd.k_idx = d->k_idx;
  sd.k_idx_dtype = d->k_idx_dtype;
  sd.k_stride_seq = d->k_stride_seq;
  sd.k_stride_head = d->k_stride_head;
  sd.k_stride_tok = d->k_stride_tok;
  sd.scores = (float*)(uintptr_t)(p->off_scores + 256);   // placeholders: validation checks alignment only
  sd.scores_ld = ld;
  sd.hint = (uint32_t*)(uintptr_t)(p->off_hint + 256);
  sd.hint_ld = hint_ld;
  if (!d->q) return LSA_ERR_INVALID_ARG;
  size_t need = 0;
  LSA_TRY(validate_score(&sd, &need));

  lsa_select_desc& se = p->select;
  std::memset(&se, 0, sizeof(se));
  se.struct_size = sizeof(se);
  se.rows = (int)rows;
  se.n = d->n_keys;
  se.topk = d->topk;
  se.scores = sd.scores;
  se.scores_ld = ld;
  se.cand_block = 1;
  se.out_idx = d->out_idx;
  se.out_score = d->out_score;
  se.hint = sd.hint;
  se.hint_ld = hint_ld;
  se.hint_count = hint_count;
  se.hint_k = lsa::score_hint_k(d->k_idx_dtype);
  LSA_TRY(validate_select(&se, &p->sel_bytes));

  lsa_attn_desc& at = p->attn;
  std::memset(&at, 0, sizeof(at));
  at.struct_size = sizeof(at);
  at.mode = LSA_MODE_DECODE;
  at.rows = d->n_seq;
  at.n_q_heads = d->n_q_heads;
  at.n_kv_heads = d->n_kv_heads;
  at.head_dim = d->head_dim;
  at.topk = d->topk;
  at.n_keys = d->n_keys;
  at.q = d->q;
  at.q_dtype = d->q_dtype;
  at.kv_dtype = d->kv_dtype;
  at.k = d->k;
  at.v = d->v;
  at.kv_stride_seq = d->kv_stride_seq;
  at.kv_stride_tok = d->kv_stride_tok;
  at.kv_stride_head = d->kv_stride_head;
  at.idx = d->out_idx;
  at.scale = d->scale;
  at.out = d->out;
  at.lse = d->lse;
  LSA_TRY(validate_attn(&at, &p->attn_bytes));
  {   // the in-launch merge keeps each split partial on whole 128-byte lines
    const int Gq = d->n_q_heads / d->n_kv_heads;
    int sp = 1, kps = 0;
    lsa::attention_plan((int)rows / d->n_kv_heads, d->n_kv_heads, Gq, d->head_dim, d->topk, true, &sp, &kps);
    p->attn_bytes = std::max(p->attn_bytes, (size_t)rows * sp * lsa::decode_partial_stride(Gq) * sizeof(float));
  }

  p->off_attn = p->off_sel + align256(p->sel_bytes);
  p->total = p->off_attn + p->attn_bytes;
  const int G = d->n_q_heads / d->n_kv_heads;
  p->fused = (d->flags & LSA_STEP_ONE_LAUNCH) &&
             lsa::decode_step_supported((int)rows, d->n_keys, d->topk, d->rank, d->k_idx_dtype, d->kv_dtype,
                                        G, d->head_dim, hint_count, se.hint_k) &&
             ((uintptr_t)d->out_idx & 127u) == 0;
  if (p->fused) {
    const int chunk = lsa::step_chunk_slots();
    p->wpr = (d->n_keys + chunk - 1) / chunk;
    const size_t parts = (size_t)rows * p->wpr;
    p->off_lists = p->off_sel;
    p->off_meta = p->off_lists + align256(parts * chunk * sizeof(int2));
    p->off_partial = p->off_meta + align256(parts * lsa::step_meta_stride() * sizeof(int4));
    const size_t fused_total = p->off_partial + parts * lsa::step_partial_stride(G) * sizeof(float);
    p->total = std::max(p->total, fused_total);
  }
  // default path: the scoring launch also lists each chunk's candidates,
  // and the select runs over those lists (no separate collect launch)
  p->listed = false;
  if (!p->fused && !(d->flags & LSA_STEP_THREE_CALLS)) {
    const int k = lsa::score_emit_rank(d->n_keys, (int)rows, d->topk, d->rank, d->k_idx_dtype,
                                       lsa::select_list_stride(), lsa::select_list_max_segments(),
                                       lsa::select_list_max());
    if (k > 0) {
      p->listed = true;
      p->list_rank = k;
      p->list_chunk = lsa::score_chunk_slots(d->n_keys, (int)rows, d->k_idx_dtype);
      p->list_wpr = (d->n_keys + p->list_chunk - 1) / p->list_chunk;
      p->s_ld = ((int64_t)lsa::score_emit_samples(d->n_keys) + 63) / 64 * 64;
      p->off_samples = align256(p->total);
      p->off_lmeta = p->off_samples + align256((size_t)rows * p->s_ld * sizeof(uint32_t));
      p->off_lists2 = p->off_lmeta + align256((size_t)rows * p->list_wpr * sizeof(int4));
      p->off_qidx = p->off_lists2 + align256((size_t)rows * p->list_wpr * lsa::select_list_stride() * sizeof(int2));
      p->total = p->off_qidx + (size_t)rows * d->rank * sizeof(float);
    }
  }
  return LSA_OK;
}

// Points the plan's descriptors at the workspace.
void bind_step(StepPlan* p, void* ws) {
  char* b = (char*)ws;
  p->score.scores = (float*)(b + p->off_scores);
  p->score.hint = (uint32_t*)(b + p->off_hint);
  p->select.scores = p->score.scores;
  p->select.hint = p->score.hint;
}

}  // namespace

// ---------------------------------------------------------------------------
// Static scratch of lsa_indexed_attention_noalloc: each GPU the library runs
// on holds one copy until the process ends. Host code never uses this name
// as an address (on the host it is only a stand-in for the device symbol);
// it uses the per-device pointer that scratch_ptr looks up once.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[LSA_NOALLOC_SCRATCH_BYTES];

namespace {

std::atomic<void*> g_scratch[kMaxDevices];   // device address of `scratch`, per device

// The current device's copy of `scratch`, looked up on the first call on
// that device (with it current) and kept.
int scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev < 0 || dev >= kMaxDevices) return LSA_ERR_NO_DEVICE_CODE;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e);
    if (p == nullptr || !al16(p)) return LSA_ERR_HIP;
    g_scratch[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return LSA_OK;
}

}  // namespace

extern "C" {

int lsa_index_score(const lsa_score_desc* d, void* ws, size_t ws_bytes, void* stream) {
  size_t need = 0;
  LSA_TRY(validate_score(d, &need));
  LSA_TRY(check_ws(ws, ws_bytes, need));
  LSA_TRY(check_device());
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if (d->mode == LSA_MODE_DECODE) {
    lsa::ScoreDecodeArgs a{};
    a.k_idx = d->k_idx;
    a.ks_seq = d->k_stride_seq;
    a.ks_head = d->k_stride_head;
    a.ks_tok = d->k_stride_tok;
    a.Hkv = d->n_kv_heads;
    a.T = d->n_keys;
    a.r = d->rank;
    a.q = d->q;
    a.q_idx_in = d->q ? nullptr : (const float*)d->q_idx;
    a.q_idx_out = d->q ? (float*)d->q_idx : nullptr;
    a.q_bf16 = d->q_dtype == LSA_BF16;
    a.Hq = d->n_q_heads;
    a.d = d->head_dim;
    a.w_per_head = d->w_per_head;
    a.w = d->w;
    a.cand = d->cand;
    a.cand_ld = d->cand_ld;
    a.cand_block = d->cand_block;
    a.n_out = (int)score_slots(d);
    a.scores = d->scores;
    a.scores_ld = d->scores_ld;
    const int rows = d->n_seq * d->n_kv_heads;
    a.chunk = lsa::score_chunk_slots(a.n_out, rows, d->k_idx_dtype);
    a.hint = d->hint;
    a.hint_ld = d->hint_ld;
    e = lsa::launch_score_decode(a, rows, d->k_idx_dtype, s);
  } else if (d->query_block > 1) {
    // one selection per block of query tokens: block queries, block scores
    // through the same MFMA tiles, then the select with a block-causal rule
    BlockWs w;
    block_prefill_layout(d, ws, &w);
    const int qb = d->query_block;
    const int nb = (d->n_keys + qb - 1) / qb;
    const int rows = nb * d->n_kv_heads;
    e = lsa::launch_block_queries((const uint16_t*)d->q_idx, d->n_keys, d->n_kv_heads, qb, w.qbar, s);
    if (e == hipSuccess) {
      lsa::PrefillTopkArgs a{};
      a.q_idx = w.qbar;
      a.k_idx = (const uint16_t*)d->k_idx;
      a.ks_head = d->k_stride_head;
      a.ks_tok = d->k_stride_tok;
      a.L = d->n_keys;
      a.Hkv = d->n_kv_heads;
      a.r = d->rank;
      a.Lq = nb;
      a.qblk = qb;
      e = lsa::launch_prefill_scores_mfma(a, w.scores, w.ld, s);
    }
    if (e == hipSuccess && d->topk > 0) {
      lsa::SelectArgs sa{};
      sa.scores = w.scores;
      sa.scores_ld = w.ld;
      sa.n = d->n_keys;
      sa.B = d->topk;
      sa.causal_group = d->n_kv_heads;
      sa.causal_block = qb;
      sa.cand_block = 1;
      sa.out_idx = d->out_idx;
      sa.out_score = d->out_score;
      lsa::select_bind_workspace(sa, rows, w.sel);
      e = lsa::launch_select(sa, rows, s);
    }
  } else if (d->topk == 0 && d->k_idx_dtype == LSA_BF16 &&
             lsa::prefill_mfma_scores_supported(d->rank) && mfma_rows_ok(d)) {
    lsa::PrefillTopkArgs a{};
    a.q_idx = (const uint16_t*)d->q_idx;
    a.k_idx = (const uint16_t*)d->k_idx;
    a.ks_head = d->k_stride_head;
    a.ks_tok = d->k_stride_tok;
    a.L = d->n_keys;
    a.Hkv = d->n_kv_heads;
    a.r = d->rank;
    a.Lq = d->n_keys;
    a.qblk = 1;
    e = lsa::launch_prefill_scores_mfma(a, d->scores, d->scores_ld, s);
  } else if (d->topk == 0) {
    lsa::ScorePrefillArgs a{};
    a.q_idx = d->q_idx;
    a.k_idx = d->k_idx;
    a.ks_head = d->k_stride_head;
    a.ks_tok = d->k_stride_tok;
    a.L = d->n_keys;
    a.Hkv = d->n_kv_heads;
    a.r = d->rank;
    a.scores = d->scores;
    a.scores_ld = d->scores_ld;
    e = lsa::launch_score_prefill(a, d->k_idx_dtype == LSA_BF16, s);
  } else {
    lsa::PrefillTopkArgs a{};
    a.q_idx = (const uint16_t*)d->q_idx;
    a.k_idx = (const uint16_t*)d->k_idx;
    a.ks_head = d->k_stride_head;
    a.ks_tok = d->k_stride_tok;
    a.L = d->n_keys;
    a.Hkv = d->n_kv_heads;
    a.r = d->rank;
    a.B = d->topk;
    a.Lq = d->n_keys;
    a.qblk = 1;
    a.out_idx = d->out_idx;
    a.out_score = d->out_score;
    a.ws = ws;
    a.ws_bytes = ws_bytes;
    e = lsa::launch_prefill_topk(a, s);
  }
  return e == hipSuccess ? LSA_OK : hip_fail(e);
}

size_t lsa_score_workspace_bytes(const lsa_score_desc* d) {
  size_t need = 0;
  return validate_score(d, &need) == LSA_OK ? need : 0;
}

int lsa_score_hint_layout(const lsa_score_desc* d, int32_t* count_per_row, int32_t* k) {
  size_t need = 0;
  int32_t c = 0, kk = 0;
  if (d && d->struct_size == sizeof(lsa_score_desc) && d->mode == LSA_MODE_DECODE) {
    lsa_score_desc probe = *d;
    probe.hint = nullptr;   // the layout does not depend on the hint buffer itself
    if (validate_score(&probe, &need) == LSA_OK) {
      c = lsa::score_hint_count((int)score_slots(d), d->k_idx_dtype);
      kk = lsa::score_hint_k(d->k_idx_dtype);
    }
  }
  if (count_per_row) *count_per_row = c;
  if (k) *k = kk;
  return c > 0 ? LSA_OK : LSA_ERR_INVALID_ARG;
}

int lsa_topk_select(const lsa_select_desc* d, void* ws, size_t ws_bytes, void* stream) {
  size_t need = 0;
  LSA_TRY(validate_select(d, &need));
  LSA_TRY(check_ws(ws, ws_bytes, need));
  LSA_TRY(check_device());
  lsa::SelectArgs a{};
  a.scores = d->scores;
  a.scores_ld = d->scores_ld;
  a.n = d->n;
  a.B = d->topk;
  a.n_valid = d->n_valid;
  a.causal_group = d->causal_group;
  a.causal_block = d->causal_block > 1 ? d->causal_block : 1;
  a.cand = d->cand;
  a.cand_ld = d->cand_ld;
  a.cand_block = d->cand ? d->cand_block : 1;
  a.n_positions = d->n_positions;
  a.out_idx = d->out_idx;
  a.out_score = d->out_score;
  a.out_count = d->out_count;
  a.hint = d->hint;
  a.hint_ld = d->hint_ld;
  a.hint_count = d->hint ? d->hint_count : 0;
  a.hint_k = d->hint ? d->hint_k : 0;
  lsa::select_bind_workspace(a, d->rows, ws);
  hipError_t e = lsa::launch_select(a, d->rows, (hipStream_t)stream);
  return e == hipSuccess ? LSA_OK : hip_fail(e);
}

size_t lsa_select_workspace_bytes(const lsa_select_desc* d) {
  size_t need = 0;
  return validate_select(d, &need) == LSA_OK ? need : 0;
}

int lsa_indexed_attention(const lsa_attn_desc* d, void* ws, size_t ws_bytes, void* stream) {
  size_t need = 0;
  LSA_TRY(validate_attn(d, &need));
  LSA_TRY(check_ws(ws, ws_bytes, need));
  LSA_TRY(check_device());
  return d->merge_ctrl ? run_attention(d, ws, stream, d->merge_ctrl, device_xccs()) : run_attention(d, ws, stream);
}

int lsa_indexed_attention_noalloc(const lsa_attn_desc* d, void* stream) {
  size_t need = 0;
  LSA_TRY(validate_attn(d, &need));
  if (need > LSA_NOALLOC_SCRATCH_BYTES) return LSA_ERR_SCRATCH_LIMIT;
  LSA_TRY(check_device());
  void* ws = nullptr;
  LSA_TRY(scratch_ptr(&ws));
  return d->merge_ctrl ? run_attention(d, ws, stream, d->merge_ctrl, device_xccs()) : run_attention(d, ws, stream);
}

namespace {

// ---------------------------------------------------------------------------
// lsa_hier_decode_step: the five calls' descriptors and their workspace.
// ---------------------------------------------------------------------------
struct HierPlan {
  lsa_score_desc cs, fs;          // coarse and fine scoring
  lsa_select_desc csel, fsel;     // coarse and fine selection
  lsa_attn_desc attn;
  int rows, nb, n_fine;
  bool listed;                    // the fine scoring launch lists its select's candidates
  int list_rank, list_chunk, list_wpr;
  int64_t s_ld;
  bool clisted;                   // the coarse scoring launch lists its select's candidates
  int clist_rank, clist_chunk, clist_wpr;
  int64_t cs_ld;
  size_t off_cscore, off_chint, off_csel, off_blocks, off_qidx, off_fscore, off_fhint, off_fsel;
  size_t off_samples, off_lmeta, off_lists, off_attn, total;
  size_t off_csamples, off_cmeta, off_clists;
  size_t csel_bytes, fsel_bytes, attn_bytes;
};

lsa_score_desc decode_score_desc(const lsa_hier_step_desc* d) {
  lsa_score_desc sd;
  std::memset(&sd, 0, sizeof(sd));
  sd.struct_size = sizeof(sd);
  sd.mode = LSA_MODE_DECODE;
  sd.n_seq = d->n_seq;
  sd.n_kv_heads = d->n_kv_heads;
  sd.rank = d->rank;
  sd.k_idx_dtype = d->k_idx_dtype;
  return sd;
}

int plan_hier(const lsa_hier_step_desc* d, HierPlan* p) {
  if (!d || d->struct_size != sizeof(lsa_hier_step_desc)) return LSA_ERR_INVALID_ARG;
  if (d->n_seq < 1 || d->n_kv_heads < 1 || d->n_keys < 1 || d->topk < 1 || d->block < 1 ||
      d->n_blocks_kept < 1 || !d->q || !d->centroids)
    return LSA_ERR_INVALID_ARG;
  if ((d->flags & ~(LSA_STEP_THREE_CALLS | LSA_STEP_LISTED)) ||
      (d->flags & (LSA_STEP_THREE_CALLS | LSA_STEP_LISTED)) == (LSA_STEP_THREE_CALLS | LSA_STEP_LISTED))
    return LSA_ERR_INVALID_ARG;
  const int64_t rows = (int64_t)d->n_seq * d->n_kv_heads;
  if (rows > 65535) return LSA_ERR_UNSUPPORTED;
  const int64_t nb = ((int64_t)d->n_keys + d->block - 1) / d->block;
  if (d->n_blocks_kept > nb || (int64_t)d->n_blocks_kept * d->block > INT_MAX) return LSA_ERR_INVALID_ARG;
  p->rows = (int)rows;
  p->nb = (int)nb;
  p->n_fine = d->n_blocks_kept * d->block;
  const int dt = d->k_idx_dtype;
  auto ld32 = [](int64_t n) { return (n + 31) / 32 * 32; };   // rows of whole 128-byte lines
  size_t off = align256((size_t)lsa::step_ctrl_words((int)rows) * 4);
  // placeholders (offset + 256): validation checks alignment only; bind_hier sets the addresses
  auto at = [](size_t o) { return (void*)(uintptr_t)(o + 256); };

  // coarse: score every block summary, keep the n_blocks_kept best blocks
  lsa_score_desc& cs = p->cs;
  cs = decode_score_desc(d);
  cs.n_keys = p->nb;
  cs.q = d->q;
  cs.q_dtype = d->q_dtype;
  cs.n_q_heads = d->n_q_heads;
  cs.head_dim = d->head_dim;
  cs.w_per_head = d->w_per_head;
  cs.w = d->w;
  cs.k_idx = d->centroids;
  cs.k_stride_seq = d->c_stride_seq;
  cs.k_stride_head = d->c_stride_head;
  cs.k_stride_tok = d->c_stride_blk;
  p->off_qidx = off;
  off = align256(off + (size_t)rows * d->rank * sizeof(float));
  cs.q_idx = at(p->off_qidx);
  p->off_cscore = off;
  cs.scores_ld = ld32(p->nb);
  off = align256(off + (size_t)rows * cs.scores_ld * sizeof(float));
  cs.scores = (float*)at(p->off_cscore);
  const int chint = lsa::score_hint_count(p->nb, dt);
  p->off_chint = off;
  cs.hint_ld = ld32(chint);
  off = align256(off + (size_t)rows * cs.hint_ld * sizeof(uint32_t));
  cs.hint = (uint32_t*)at(p->off_chint);
  size_t need = 0;
  LSA_TRY(validate_score(&cs, &need));

  lsa_select_desc& csel = p->csel;
  std::memset(&csel, 0, sizeof(csel));
  csel.struct_size = sizeof(csel);
  csel.rows = (int)rows;
  csel.n = p->nb;
  csel.topk = d->n_blocks_kept;
  csel.scores = cs.scores;
  csel.scores_ld = cs.scores_ld;
  csel.cand_block = 1;
  p->off_blocks = off;
  off = align256(off + (size_t)rows * d->n_blocks_kept * sizeof(int32_t));
  csel.out_idx = (int32_t*)at(p->off_blocks);
  csel.hint = cs.hint;
  csel.hint_ld = cs.hint_ld;
  csel.hint_count = chint;
  csel.hint_k = lsa::score_hint_k(dt);
  LSA_TRY(validate_select(&csel, &p->csel_bytes));
  p->off_csel = off;
  off = align256(off + p->csel_bytes);

  // the coarse stage's listing launch over the block summaries, by the
  // same rule as the fine stage's: by default only for rows of at least
  // LSA_HIER_LIST_MIN_SLOTS slots (16384 summaries per row with 128 kept:
  // 62.6 us per step listed against 56.8 for the separate calls)
  p->clisted = false;
  const bool want_clist = (d->flags & LSA_STEP_LISTED) ||
                          (!(d->flags & LSA_STEP_THREE_CALLS) && p->nb >= LSA_HIER_LIST_MIN_SLOTS);
  if (want_clist && p->nb <= lsa::kSelectLdsMaxSlots) {
    const int k = lsa::score_emit_rank(p->nb, (int)rows, d->n_blocks_kept, d->rank, dt, lsa::select_list_stride(),
                                       lsa::select_list_max_segments(), lsa::select_list_max());
    if (k > 0) {
      p->clisted = true;
      p->clist_rank = k;
      p->clist_chunk = lsa::score_chunk_slots(p->nb, (int)rows, dt);
      p->clist_wpr = (p->nb + p->clist_chunk - 1) / p->clist_chunk;
      p->cs_ld = ((int64_t)lsa::score_emit_samples(p->nb) + 63) / 64 * 64;
      p->off_csamples = off;
      off = align256(off + (size_t)rows * p->cs_ld * sizeof(uint32_t));
      p->off_cmeta = off;
      off = align256(off + (size_t)rows * p->clist_wpr * sizeof(int4));
      p->off_clists = off;
      off = align256(off + (size_t)rows * p->clist_wpr * lsa::select_list_stride() * sizeof(int2));
    }
  }

  // fine: score the kept blocks' tokens, keep the top B
  lsa_score_desc& fs = p->fs;
  fs = decode_score_desc(d);
  fs.n_keys = d->n_keys;
  fs.q_idx = cs.q_idx;   // q_idx from the coarse call
  fs.k_idx = d->k_idx;
  fs.k_stride_seq = d->k_stride_seq;
  fs.k_stride_head = d->k_stride_head;
  fs.k_stride_tok = d->k_stride_tok;
  fs.cand = csel.out_idx;
  fs.n_cand = d->n_blocks_kept;
  fs.cand_block = d->block;
  fs.cand_ld = d->n_blocks_kept;
  p->off_fscore = off;
  fs.scores_ld = ld32(p->n_fine);
  off = align256(off + (size_t)rows * fs.scores_ld * sizeof(float));
  fs.scores = (float*)at(p->off_fscore);
  const int fhint = lsa::score_hint_count(p->n_fine, dt);
  p->off_fhint = off;
  fs.hint_ld = ld32(fhint);
  off = align256(off + (size_t)rows * fs.hint_ld * sizeof(uint32_t));
  fs.hint = (uint32_t*)at(p->off_fhint);
  LSA_TRY(validate_score(&fs, &need));

  lsa_select_desc& fsel = p->fsel;
  std::memset(&fsel, 0, sizeof(fsel));
  fsel.struct_size = sizeof(fsel);
  fsel.rows = (int)rows;
  fsel.n = p->n_fine;
  fsel.topk = d->topk;
  fsel.scores = fs.scores;
  fsel.scores_ld = fs.scores_ld;
  fsel.cand = fs.cand;
  fsel.cand_ld = fs.cand_ld;
  fsel.cand_block = d->block;
  fsel.n_positions = d->n_keys;
  fsel.out_idx = d->out_idx;
  fsel.out_score = d->out_score;
  fsel.hint = fs.hint;
  fsel.hint_ld = fs.hint_ld;
  fsel.hint_count = fhint;
  fsel.hint_k = lsa::score_hint_k(dt);
  LSA_TRY(validate_select(&fsel, &p->fsel_bytes));
  p->off_fsel = off;
  off = align256(off + p->fsel_bytes);

  // the fine stage's listing launch, where the shape allows it: by default
  // only for rows of at least LSA_HIER_LIST_MIN_SLOTS slots (on shorter rows
  // the separate scoring and select calls were measured faster)
  p->listed = false;
  const bool want_list = (d->flags & LSA_STEP_LISTED) ||
                         (!(d->flags & LSA_STEP_THREE_CALLS) && p->n_fine >= LSA_HIER_LIST_MIN_SLOTS);
  if (want_list) {
    const int k = lsa::score_emit_rank(p->n_fine, (int)rows, d->topk, d->rank, dt, lsa::select_list_stride(),
                                       lsa::select_list_max_segments(), lsa::select_list_max());
    if (k > 0) {
      p->listed = true;
      p->list_rank = k;
      p->list_chunk = lsa::score_chunk_slots(p->n_fine, (int)rows, dt);
      p->list_wpr = (p->n_fine + p->list_chunk - 1) / p->list_chunk;
      p->s_ld = ((int64_t)lsa::score_emit_samples(p->n_fine) + 63) / 64 * 64;
      p->off_samples = off;
      off = align256(off + (size_t)rows * p->s_ld * sizeof(uint32_t));
      p->off_lmeta = off;
      off = align256(off + (size_t)rows * p->list_wpr * sizeof(int4));
      p->off_lists = off;
      off = align256(off + (size_t)rows * p->list_wpr * lsa::select_list_stride() * sizeof(int2));
    }
  }

  // attention over the selection, its splits merged in the launch
  lsa_attn_desc& at_ = p->attn;
  std::memset(&at_, 0, sizeof(at_));
  at_.struct_size = sizeof(at_);
  at_.mode = LSA_MODE_DECODE;
  at_.rows = d->n_seq;
  at_.n_q_heads = d->n_q_heads;
  at_.n_kv_heads = d->n_kv_heads;
  at_.head_dim = d->head_dim;
  at_.topk = d->topk;
  at_.n_keys = d->n_keys;
  at_.q = d->q;
  at_.q_dtype = d->q_dtype;
  at_.kv_dtype = d->kv_dtype;
  at_.k = d->k;
  at_.v = d->v;
  at_.kv_stride_seq = d->kv_stride_seq;
  at_.kv_stride_tok = d->kv_stride_tok;
  at_.kv_stride_head = d->kv_stride_head;
  at_.idx = d->out_idx;
  at_.scale = d->scale;
  at_.out = d->out;
  at_.lse = d->lse;
  at_.merge_ctrl = (uint32_t*)at(0);
  LSA_TRY(validate_attn(&at_, &p->attn_bytes));
  p->off_attn = off;
  p->total = off + p->attn_bytes;
  return LSA_OK;
}

// Points the plan's descriptors at the workspace (and the caller's optional outputs).
void bind_hier(HierPlan* p, const lsa_hier_step_desc* d, void* ws) {
  char* b = (char*)ws;
  float* q_idx = d->q_idx ? d->q_idx : (float*)(b + p->off_qidx);
  int32_t* blocks = d->out_blocks ? d->out_blocks : (int32_t*)(b + p->off_blocks);
  p->cs.q_idx = q_idx;
  p->cs.scores = (float*)(b + p->off_cscore);
  p->cs.hint = (uint32_t*)(b + p->off_chint);
  p->csel.scores = p->cs.scores;
  p->csel.hint = p->cs.hint;
  p->csel.out_idx = blocks;
  p->fs.q_idx = q_idx;
  p->fs.cand = blocks;
  p->fs.scores = (float*)(b + p->off_fscore);
  p->fs.hint = (uint32_t*)(b + p->off_fhint);
  p->fsel.scores = p->fs.scores;
  p->fsel.hint = p->fs.hint;
  p->fsel.cand = blocks;
  p->attn.merge_ctrl = (uint32_t*)b;
}

int run_hier(const lsa_hier_step_desc* d, HierPlan& p, char* b, hipStream_t s) {
  void* stream = (void*)s;
  if (p.clisted) {
    // coarse: the scoring prep and the block-summary scores in one launch
    // that lists the block select's candidates; the select takes the lists
    // (a row they do not settle is rescored from q_idx and the summaries)
    float* q_idx = (float*)p.cs.q_idx;
    lsa::ScoreDecodeArgs sc{};
    sc.k_idx = d->centroids;
    sc.ks_seq = d->c_stride_seq;
    sc.ks_head = d->c_stride_head;
    sc.ks_tok = d->c_stride_blk;
    sc.Hkv = d->n_kv_heads;
    sc.T = p.nb;
    sc.r = d->rank;
    sc.q = d->q;
    sc.q_idx_out = q_idx;
    sc.q_bf16 = d->q_dtype == LSA_BF16;
    sc.Hq = d->n_q_heads;
    sc.d = d->head_dim;
    sc.w_per_head = d->w_per_head;
    sc.w = d->w;
    sc.cand_block = 1;
    sc.n_out = p.nb;
    sc.scores = nullptr;   // the lists carry the scores the select needs
    sc.scores_ld = p.cs.scores_ld;
    sc.chunk = p.clist_chunk;
    lsa::ScoreEmitArgs e{};
    e.samples = (uint32_t*)(b + p.off_csamples);
    e.s_ld = p.cs_ld;
    e.k_rank = p.clist_rank;
    e.wpr = p.clist_wpr;
    e.ctrl = (uint32_t*)b + lsa::step_ctrl_row0();   // shared with the fine launch: each leaves them zero
    e.ctrl_stride = lsa::step_ctrl_per_row();
    e.lists = (int2*)(b + p.off_clists);
    e.list_stride = lsa::select_list_stride();
    e.meta = (int4*)(b + p.off_cmeta);
    e.no_list = lsa::select_list_max() + 1;
    hipError_t err = lsa::launch_score_emit(sc, e, p.rows, d->k_idx_dtype, s);
    if (err != hipSuccess) return hip_fail(err);
    lsa::SelectArgs a{};
    a.scores = p.cs.scores;   // the rescoring fallback's rows
    a.scores_ld = p.cs.scores_ld;
    a.n = p.nb;
    a.B = d->n_blocks_kept;
    a.cand_block = 1;
    a.out_idx = p.csel.out_idx;
    a.seg_list = e.lists;
    a.seg_meta = e.meta;
    a.nseg = p.clist_wpr;
    a.rs_k_idx = d->centroids;
    a.rs_ks_seq = d->c_stride_seq;
    a.rs_ks_head = d->c_stride_head;
    a.rs_ks_tok = d->c_stride_blk;
    a.rs_q_idx = q_idx;
    a.rs_r = d->rank;
    a.rs_dt = d->k_idx_dtype;
    a.rs_Hkv = d->n_kv_heads;
    err = lsa::launch_select_lists(a, p.rows, s);
    if (err != hipSuccess) return hip_fail(err);
  } else {
    LSA_TRY(lsa_index_score(&p.cs, nullptr, 0, stream));
    LSA_TRY(lsa_topk_select(&p.csel, b + p.off_csel, p.csel_bytes, stream));
  }
  if (p.listed) {
    lsa::ScoreDecodeArgs sc{};
    sc.k_idx = d->k_idx;
    sc.ks_seq = d->k_stride_seq;
    sc.ks_head = d->k_stride_head;
    sc.ks_tok = d->k_stride_tok;
    sc.Hkv = d->n_kv_heads;
    sc.T = d->n_keys;
    sc.r = d->rank;
    sc.q_idx_in = (const float*)p.fs.q_idx;
    sc.cand = p.fs.cand;
    sc.cand_ld = p.fs.cand_ld;
    sc.cand_block = d->block;
    sc.n_out = p.n_fine;
    sc.scores = nullptr;   // the lists carry the scores the select needs
    sc.scores_ld = p.fs.scores_ld;
    sc.chunk = p.list_chunk;
    lsa::ScoreEmitArgs e{};
    e.samples = (uint32_t*)(b + p.off_samples);
    e.s_ld = p.s_ld;
    e.k_rank = p.list_rank;
    e.wpr = p.list_wpr;
    e.ctrl = (uint32_t*)b + lsa::step_ctrl_row0();   // one word per row: finished chunks
    e.ctrl_stride = lsa::step_ctrl_per_row();
    e.lists = (int2*)(b + p.off_lists);
    e.list_stride = lsa::select_list_stride();
    e.meta = (int4*)(b + p.off_lmeta);
    e.no_list = lsa::select_list_max() + 1;
    hipError_t err = lsa::launch_score_emit(sc, e, p.rows, d->k_idx_dtype, s);
    if (err != hipSuccess) return hip_fail(err);
    lsa::SelectArgs a{};
    a.scores = p.fs.scores;
    a.scores_ld = p.fs.scores_ld;
    a.n = p.n_fine;
    a.B = d->topk;
    a.cand = p.fs.cand;
    a.cand_ld = p.fs.cand_ld;
    a.cand_block = d->block;
    a.n_positions = d->n_keys;
    a.out_idx = d->out_idx;
    a.out_score = d->out_score;
    a.gbitmap = p.n_fine > lsa::kSelectLdsMaxSlots ? (uint32_t*)(b + p.off_fsel) : nullptr;
    a.seg_list = e.lists;
    a.seg_meta = e.meta;
    a.nseg = p.list_wpr;
    a.rs_k_idx = d->k_idx;   // a row the lists do not settle is rescored
    a.rs_ks_seq = d->k_stride_seq;
    a.rs_ks_head = d->k_stride_head;
    a.rs_ks_tok = d->k_stride_tok;
    a.rs_q_idx = (const float*)p.fs.q_idx;
    a.rs_r = d->rank;
    a.rs_dt = d->k_idx_dtype;
    a.rs_Hkv = d->n_kv_heads;
    err = lsa::launch_select_lists(a, p.rows, s);
    if (err != hipSuccess) return hip_fail(err);
  } else {
    LSA_TRY(lsa_index_score(&p.fs, nullptr, 0, stream));
    LSA_TRY(lsa_topk_select(&p.fsel, b + p.off_fsel, p.fsel_bytes, stream));
  }
  return run_attention(&p.attn, p.attn_bytes ? b + p.off_attn : nullptr, stream, p.attn.merge_ctrl,
                       device_xccs());
}

}  // namespace

namespace {

// The default path's launches, those named in `parts`, in order.
int run_step_parts(const lsa_step_desc* d, StepPlan& p, char* b, hipStream_t s, int parts) {
  void* stream = (void*)s;
  if (p.listed) {
    // q_idx: the caller's buffer, or the workspace's (the select's fallback reads it)
    float* q_idx = d->q_idx ? d->q_idx : (float*)(b + p.off_qidx);
    lsa::ScoreDecodeArgs sc{};
    sc.k_idx = d->k_idx;
    sc.ks_seq = d->k_stride_seq;
    sc.ks_head = d->k_stride_head;
    sc.ks_tok = d->k_stride_tok;
    sc.Hkv = d->n_kv_heads;
    sc.T = d->n_keys;
    sc.r = d->rank;
    sc.q = d->q;
    sc.q_idx_out = q_idx;
    sc.q_bf16 = d->q_dtype == LSA_BF16;
    sc.Hq = d->n_q_heads;
    sc.d = d->head_dim;
    sc.w_per_head = d->w_per_head;
    sc.w = d->w;
    sc.cand_block = 1;
    sc.n_out = d->n_keys;
    sc.scores = nullptr;   // the lists carry the scores the select needs
    sc.scores_ld = p.score.scores_ld;
    sc.chunk = p.list_chunk;
    lsa::ScoreEmitArgs e{};
    e.samples = (uint32_t*)(b + p.off_samples);
    e.s_ld = p.s_ld;
    e.k_rank = p.list_rank;
    e.wpr = p.list_wpr;
    e.ctrl = (uint32_t*)b + lsa::step_ctrl_row0();   // one word per row: finished chunks
    e.ctrl_stride = lsa::step_ctrl_per_row();
    e.lists = (int2*)(b + p.off_lists2);
    e.list_stride = lsa::select_list_stride();
    e.meta = (int4*)(b + p.off_lmeta);
    e.no_list = lsa::select_list_max() + 1;
    if (parts & LSA_STEP_PART_SCORE) {
      const hipError_t err = lsa::launch_score_emit(sc, e, p.rows, d->k_idx_dtype, s);
      if (err != hipSuccess) return hip_fail(err);
    }
    lsa::SelectArgs a{};
    a.scores = p.score.scores;
    a.scores_ld = p.score.scores_ld;
    a.n = d->n_keys;
    a.B = d->topk;
    a.cand_block = 1;
    a.out_idx = d->out_idx;
    a.out_score = d->out_score;
    // bitmaps of rows too long for LDS lead the select workspace
    a.gbitmap = d->n_keys > lsa::kSelectLdsMaxSlots ? (uint32_t*)(b + p.off_sel) : nullptr;
    a.seg_list = e.lists;
    a.seg_meta = e.meta;
    a.nseg = p.list_wpr;
    a.rs_k_idx = d->k_idx;   // a row the lists do not settle is rescored
    a.rs_ks_seq = d->k_stride_seq;
    a.rs_ks_head = d->k_stride_head;
    a.rs_ks_tok = d->k_stride_tok;
    a.rs_q_idx = q_idx;
    a.rs_r = d->rank;
    a.rs_dt = d->k_idx_dtype;
    a.rs_Hkv = d->n_kv_heads;
    if (parts & LSA_STEP_PART_SELECT) {
      const hipError_t err = lsa::launch_select_lists(a, p.rows, s);
      if (err != hipSuccess) return hip_fail(err);
    }
  } else {
    if (parts & LSA_STEP_PART_SCORE) LSA_TRY(lsa_index_score(&p.score, nullptr, 0, stream));
    if (parts & LSA_STEP_PART_SELECT) LSA_TRY(lsa_topk_select(&p.select, b + p.off_sel, p.sel_bytes, stream));
  }
  if (parts & LSA_STEP_PART_ATTEND)
    return run_attention(&p.attn, p.attn_bytes ? b + p.off_attn : nullptr, stream, (uint32_t*)b, device_xccs());
  return LSA_OK;
}

}  // namespace

int lsa_decode_step(const lsa_step_desc* d, void* ws, size_t ws_bytes, void* stream) {
  StepPlan p;
  LSA_TRY(plan_step(d, &p));
  LSA_TRY(check_ws(ws, ws_bytes, p.total));
  LSA_TRY(check_device());
  bind_step(&p, ws);
  char* b = (char*)ws;
  hipStream_t s = (hipStream_t)stream;
  const int nxcc = p.fused ? device_xccs() : 0;
  if (nxcc >= 1 && nxcc <= 8) {
    lsa::StepArgs a{};
    lsa::ScoreDecodeArgs& sc = a.sc;
    sc.k_idx = d->k_idx;
    sc.ks_seq = d->k_stride_seq;
    sc.ks_head = d->k_stride_head;
    sc.ks_tok = d->k_stride_tok;
    sc.Hkv = d->n_kv_heads;
    sc.T = d->n_keys;
    sc.r = d->rank;
    sc.q = d->q;
    sc.q_idx_out = d->q_idx;
    sc.q_bf16 = d->q_dtype == LSA_BF16;
    sc.Hq = d->n_q_heads;
    sc.d = d->head_dim;
    sc.w_per_head = d->w_per_head;
    sc.w = d->w;
    sc.cand_block = 1;
    sc.n_out = d->n_keys;
    sc.scores = p.score.scores;
    sc.scores_ld = p.score.scores_ld;
    sc.hint = p.score.hint;
    sc.hint_ld = p.score.hint_ld;
    a.B = d->topk;
    a.hint_count = p.select.hint_count;
    a.hint_k = p.select.hint_k;
    a.lists = (int2*)(b + p.off_lists);
    a.meta = (int4*)(b + p.off_meta);
    a.out_idx = d->out_idx;
    a.out_score = d->out_score;
    a.q = d->q;
    a.k = d->k;
    a.v = d->v;
    a.kv_s_seq = d->kv_stride_seq;
    a.kv_s_tok = d->kv_stride_tok;
    a.kv_s_head = d->kv_stride_head;
    a.kv_bf16 = d->kv_dtype == LSA_BF16;
    a.Hq = d->n_q_heads;
    a.Hkv = d->n_kv_heads;
    a.T = d->n_keys;
    const float scale = d->scale > 0.f ? d->scale : 1.0f / std::sqrt((float)d->head_dim);
    a.scale_log2 = scale * 1.4426950408889634f;
    a.out = d->out;
    a.lse = d->lse;
    a.partial = (float*)(b + p.off_partial);
    a.ctrl = (uint32_t*)b;
    a.rows = p.rows;
    a.wpr = p.wpr;
    a.nxcc = nxcc;
    hipError_t e = lsa::launch_decode_step(a, d->k_idx_dtype, s);
    return e == hipSuccess ? LSA_OK : hip_fail(e);
  }
  return run_step_parts(d, p, b, s, LSA_STEP_PART_ALL);
}


int lsa_decode_step_part(const lsa_step_desc* d, int parts, void* ws, size_t ws_bytes, void* stream) {
  if (parts < 1 || parts > LSA_STEP_PART_ALL) return LSA_ERR_INVALID_ARG;
  StepPlan p;
  LSA_TRY(plan_step(d, &p));
  if (p.fused) return LSA_ERR_UNSUPPORTED;   // the one launch has no parts
  LSA_TRY(check_ws(ws, ws_bytes, p.total));
  LSA_TRY(check_device());
  bind_step(&p, ws);
  return run_step_parts(d, p, (char*)ws, (hipStream_t)stream, parts);
}

size_t lsa_step_workspace_bytes(const lsa_step_desc* d) {
  StepPlan p;
  return plan_step(d, &p) == LSA_OK ? p.total : 0;
}

int lsa_step_is_fused(const lsa_step_desc* d) {
  StepPlan p;
  return plan_step(d, &p) == LSA_OK ? (p.fused ? 1 : 0) : -1;
}

int lsa_step_path(const lsa_step_desc* d) {
  StepPlan p;
  if (plan_step(d, &p) != LSA_OK) return -1;
  return p.fused ? LSA_STEP_PATH_ONE_LAUNCH : p.listed ? LSA_STEP_PATH_LISTED : LSA_STEP_PATH_THREE_CALLS;
}

int lsa_hier_decode_step(const lsa_hier_step_desc* d, void* ws, size_t ws_bytes, void* stream) {
  HierPlan p;
  LSA_TRY(plan_hier(d, &p));
  LSA_TRY(check_ws(ws, ws_bytes, p.total));
  LSA_TRY(check_device());
  bind_hier(&p, d, ws);
  return run_hier(d, p, (char*)ws, (hipStream_t)stream);
}

size_t lsa_hier_step_workspace_bytes(const lsa_hier_step_desc* d) {
  HierPlan p;
  return plan_hier(d, &p) == LSA_OK ? p.total : 0;
}

int lsa_hier_step_path(const lsa_hier_step_desc* d) {
  HierPlan p;
  if (plan_hier(d, &p) != LSA_OK) return -1;
  return p.listed ? LSA_STEP_PATH_LISTED : LSA_STEP_PATH_THREE_CALLS;
}

size_t lsa_attention_workspace_bytes(const lsa_attn_desc* d) {
  size_t need = 0;
  return validate_attn(d, &need) == LSA_OK ? need : 0;
}

int lsa_project_keys(const lsa_project_desc* d, void* stream) {
  if (!d || d->struct_size != sizeof(lsa_project_desc)) return LSA_ERR_INVALID_ARG;
  if (esize_wide(d->k_dtype) == 0 || esize(d->out_dtype) == 0) return LSA_ERR_UNSUPPORTED;
  if (d->n_seq < 1 || d->n_kv_heads < 1 || d->head_dim < 1 || d->tok_begin < 0 || d->n_tok < 0)
    return LSA_ERR_INVALID_ARG;
  if (d->head_dim > 512 || !pow2(d->rank) || d->rank > 256) return LSA_ERR_UNSUPPORTED;
  if (d->n_seq > 65535 || d->n_kv_heads > 65535) return LSA_ERR_UNSUPPORTED;
  if (!d->k || !d->w || !d->out) return LSA_ERR_INVALID_ARG;
  if (d->w_per_head != 0 && d->w_per_head != 1) return LSA_ERR_INVALID_ARG;
  if (d->k_stride_seq < 0 || d->k_stride_tok < 0 || d->k_stride_head < 0 || d->out_stride_seq < 0 ||
      d->out_stride_head < 0 || d->out_stride_tok < 0)
    return LSA_ERR_INVALID_ARG;
  LSA_TRY(check_device());
  lsa::ProjectArgs a{};
  a.k = d->k;
  a.ks_seq = d->k_stride_seq;
  a.ks_tok = d->k_stride_tok;
  a.ks_head = d->k_stride_head;
  a.w = d->w;
  a.w_per_head = d->w_per_head;
  a.out = d->out;
  a.os_seq = d->out_stride_seq;
  a.os_head = d->out_stride_head;
  a.os_tok = d->out_stride_tok;
  a.N = d->n_seq;
  a.Hkv = d->n_kv_heads;
  a.d = d->head_dim;
  a.r = d->rank;
  a.tok_begin = d->tok_begin;
  a.n_tok = d->n_tok;
  hipError_t e = lsa::launch_project(a, d->k_dtype == LSA_BF16, d->out_dtype, (hipStream_t)stream);
  return e == hipSuccess ? LSA_OK : hip_fail(e);
}

int lsa_build_centroids(const lsa_centroid_desc* d, void* stream) {
  if (!d || d->struct_size != sizeof(lsa_centroid_desc)) return LSA_ERR_INVALID_ARG;
  if (esize(d->dtype) == 0) return LSA_ERR_UNSUPPORTED;
  if (d->n_seq < 1 || d->n_kv_heads < 1 || d->n_keys < 1 || d->rank < 1 || d->block < 1)
    return LSA_ERR_INVALID_ARG;
  if (d->n_seq > 65535 || d->n_kv_heads > 65535) return LSA_ERR_UNSUPPORTED;
  if (!d->in || !d->out) return LSA_ERR_INVALID_ARG;
  if (d->in_stride_seq < 0 || d->in_stride_head < 0 || d->in_stride_tok < 0 || d->out_stride_seq < 0 ||
      d->out_stride_head < 0 || d->out_stride_blk < 0)
    return LSA_ERR_INVALID_ARG;
  LSA_TRY(check_device());
  lsa::CentroidArgs a{};
  a.in = d->in;
  a.is_seq = d->in_stride_seq;
  a.is_head = d->in_stride_head;
  a.is_tok = d->in_stride_tok;
  a.out = d->out;
  a.os_seq = d->out_stride_seq;
  a.os_head = d->out_stride_head;
  a.os_blk = d->out_stride_blk;
  a.N = d->n_seq;
  a.Hkv = d->n_kv_heads;
  a.T = d->n_keys;
  a.r = d->rank;
  a.block = d->block;
  hipError_t e = lsa::launch_centroids(a, d->dtype, (hipStream_t)stream);
  return e == hipSuccess ? LSA_OK : hip_fail(e);
}

static_assert(lsa::kStreamReadBlocks == LSA_STREAM_READ_SINK_WORDS, "one sink word per workgroup");

int lsa_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
  if (!buf || !sink || bytes == 0 || bytes % 16 != 0 || !al16(buf) || (uintptr_t)sink % 4 != 0)
    return LSA_ERR_INVALID_ARG;
  LSA_TRY(check_device());
  hipError_t e = lsa::launch_stream_read(buf, bytes, sink, (hipStream_t)stream);
  return e == hipSuccess ? LSA_OK : hip_fail(e);
}

const char* lsa_status_str(int status) {
  switch (status) {
    case LSA_OK: return "ok";
    case LSA_ERR_INVALID_ARG: return "invalid argument";
    case LSA_ERR_UNSUPPORTED: return "unsupported configuration";
    case LSA_ERR_WORKSPACE: return "workspace missing or too small";
    case LSA_ERR_NO_DEVICE_CODE: return "current device is not gfx950";
    case LSA_ERR_HIP: return "HIP error";
    case LSA_ERR_SCRATCH_LIMIT: return "needs more scratch than the static buffer holds";
  }
  return "unknown status";
}

int lsa_last_hip_error(void) { return g_last_hip; }

int lsa_abi_version(void) { return LSA_ABI_VERSION; }

size_t lsa_desc_size(int which) {
  switch (which) {
    case 0: return sizeof(lsa_score_desc);
    case 1: return sizeof(lsa_select_desc);
    case 2: return sizeof(lsa_attn_desc);
    case 3: return sizeof(lsa_project_desc);
    case 4: return sizeof(lsa_centroid_desc);
    case 5: return sizeof(lsa_step_desc);
    case 6: return sizeof(lsa_hier_step_desc);
  }
  return 0;
}

}  // extern "C"
