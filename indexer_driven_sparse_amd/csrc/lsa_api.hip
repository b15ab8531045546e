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
  if (decode_mfma_shape(d))
    need = std::max(need, lsa::attention_workspace(d->rows, d->n_kv_heads, G, d->head_dim, d->topk, true));
  *ws_need = need;
  return LSA_OK;
}

int check_ws(void* ws, size_t have, size_t need) {
  if (need == 0) return LSA_OK;
  if (!ws || have < need || !al16(ws)) return LSA_ERR_WORKSPACE;
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
  if (mfma_decode)
    e = lsa::launch_attention_decode_mfma(a, (hipStream_t)stream);
  else if (lsa::attention_mfma_supported(a, d->kv_dtype == LSA_BF16))
    e = lsa::launch_attention_mfma(a, (hipStream_t)stream);
  else
    e = lsa::launch_attention(a, d->q_dtype == LSA_BF16, d->kv_dtype == LSA_BF16, (hipStream_t)stream);
  return e == hipSuccess ? LSA_OK : hip_fail(e);
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
  }
  return 0;
}

}  // extern "C"
