// Internal launch interface between the C ABI layer (lsa_api.hip) and the
// kernel translation units. Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lsa {

// ----- indexer scoring -----------------------------------------------------
struct ScoreDecodeArgs {
  const void* k_idx;
  int64_t ks_seq, ks_head, ks_tok;   // elements
  int Hkv, T, r;
  const float* q_idx_in;             // [rows, r] fp32 (when q == nullptr)
  float* q_idx_out;                  // optional fp32 output of the prep
  const void* q;                     // [N,Hq,d] (prep input) or nullptr
  int q_bf16, Hq, d, w_per_head;
  const float* w;
  const int32_t* cand;               // nullptr: slots are positions
  int64_t cand_ld;
  int cand_block;
  int n_out;                         // slots per row
  float* scores;
  int64_t scores_ld;
  int chunk;                         // slots per workgroup, multiple of the step
  uint32_t* hint;                    // optional selection hint [rows, hint_ld] (see below)
  int64_t hint_ld;
};
int score_chunk_slots(int n_out, int rows, int k_dt);
// Selection hint of the decode scoring kernel: the row is cut into groups
// of slots (one wave's loads of one loop step, 64 slots per group in flight;
// the count depends on the cache dtype); for each group the hint is the
// largest 16-bit order-key prefix p (as p << 16) that at least
// score_hint_k of the group's keys reach. Groups are numbered in slot order
// of their first slot, four per step.
int score_hint_count(int n_out, int k_dt);   // hint entries per row
int score_hint_k(int k_dt);                 // keys each hint vouches for
hipError_t launch_score_decode(const ScoreDecodeArgs& a, int rows, int k_dt, hipStream_t s);

// Decode scoring that also lists each chunk's candidates for the row
// select (the decode step's collect, done in the scoring launch). Every
// chunk first scores a sample of its row -- slot 64*i + j(i) for each
// 64-slot group i, j(i) in [0, 64) a fixed hash of i and the row -- and
// writes each sample key's 16-bit prefix, marked, to the row's sample
// entries. After its stream every chunk reads all of the row's entries and
// takes as threshold t_lo the 16-bit prefix (as p << 16) of the k_rank-th
// largest; it lists its slots whose keys reach t_lo, in slot order, as
// (score bits, slot) pairs, with {count, max key, t_lo, 0} in its meta
// word: what the row select's list path reads. A chunk that finds an
// entry not yet written lists nothing and writes count = no_list (more than
// the select takes), sending the row to the select's path over the scores,
// which the select then recomputes (SelectArgs::rs_*): the kernel writes
// no scores, only q_idx (q_idx_out, which it needs). No chunk waits for
// another. samples: zero before the first launch; ctrl: per
// row one zeroed word at ctrl + row * ctrl_stride (the count of finished
// chunks). The row's last chunk out zeroes both again.
struct ScoreEmitArgs {
  uint32_t* samples;                 // [rows, s_ld] sample keys
  int64_t s_ld;
  int k_rank;
  int wpr;                           // chunks per row
  uint32_t* ctrl;
  int64_t ctrl_stride;
  int2* lists;                       // [rows, wpr, list_stride]
  int list_stride;
  int4* meta;                        // [rows, wpr]
  int no_list;
};
// Whether a decode step of this shape can use launch_score_emit, and the
// sample rank it takes (0: not supported).
int score_emit_rank(int n_out, int rows, int B, int r, int k_dt, int seg_cap, int max_segs, int max_listed);
int score_emit_samples(int n_out);   // sample keys per row (s_ld is at least this)
hipError_t launch_score_emit(const ScoreDecodeArgs& a, const ScoreEmitArgs& e, int rows, int k_dt,
                             hipStream_t s);

struct ScorePrefillArgs {
  const void* q_idx;                 // [L, Hkv, r] (contiguous rows of r)
  const void* k_idx;
  int64_t ks_head, ks_tok;
  int L, Hkv, r;
  float* scores;
  int64_t scores_ld;
};
hipError_t launch_score_prefill(const ScorePrefillArgs& a, bool bf16, hipStream_t s);

// Fused causal prefill indexer + exact top-B.
struct PrefillTopkArgs {
  const uint16_t* q_idx;             // [Lq, Hkv, r] bf16
  const uint16_t* k_idx;
  int64_t ks_head, ks_tok;
  int L, Hkv, r, B;
  int Lq, qblk;                      // query rows and tokens per row: row i sees keys
                                     // j < min(L, (i+1)*qblk); the fused path needs Lq = L, qblk = 1
  int32_t* out_idx;                  // [L, Hkv, B]
  float* out_score;                  // or nullptr
  void* ws;
  size_t ws_bytes;
};
size_t prefill_topk_workspace(int L, int Hkv, int B);
hipError_t launch_prefill_topk(const PrefillTopkArgs& a, hipStream_t s);
bool prefill_topk_supported(int L, int r, int B);
// Unfused causal scores through the same MFMA tiles as the fused path
// (bf16, r = 64, 16-byte aligned rows); ScorePrefillArgs' VALU kernel
// serves the other cases.
bool prefill_mfma_scores_supported(int r);
hipError_t launch_prefill_scores_mfma(const PrefillTopkArgs& a, float* scores, int64_t ld,
                                      hipStream_t s);
// Block queries for query-block-shared prefill: out[b,g,:] = bf16 of the
// exact mean of q_idx[i,g,:] over the block's tokens (r = 64).
hipError_t launch_block_queries(const uint16_t* q_idx, int L, int Hkv, int qblk, uint16_t* out,
                                hipStream_t s);

// ----- exact top-B selection -----------------------------------------------
struct SelectArgs {
  const float* scores;
  int64_t scores_ld;
  int n, B;
  const int32_t* n_valid;
  int causal_group;
  int causal_block;                  // with causal_group: (row/group + 1) * causal_block valid
  const int32_t* cand;
  int64_t cand_ld;
  int cand_block, n_positions;
  int32_t* out_idx;
  float* out_score;
  int32_t* out_count;
  uint32_t* gbitmap;                 // workspace bitmaps for long rows, or nullptr
  const uint32_t* hint;              // optional: per row hint_count keys, each reached by
  int64_t hint_ld;                   //   at least hint_k of the row's valid keys
  int hint_count, hint_k;
  // segmented collect (long rows with a hint): per (row, segment) a list of
  // (score bits, slot) pairs in slot order and its {count, max key, t_lo}
  int2* seg_list;
  int4* seg_meta;
  int nseg;
  // Lists from the listing scoring launch, which writes no scores: where
  // the lists do not settle a row, the row's scores are first recomputed
  // into `scores` with the scoring kernels' arithmetic (rs_k_idx set; 4, 8
  // or 16 sixteen-byte pieces per key)
  const void* rs_k_idx;
  int64_t rs_ks_seq, rs_ks_head, rs_ks_tok;   // elements
  const float* rs_q_idx;                      // [rows, rs_r]
  int rs_r, rs_dt, rs_Hkv;
};
constexpr int kSelectLdsMaxSlots = 262144;
// Workspace of a select: bitmaps of rows longer than kSelectLdsMaxSlots,
// then the segment lists when the segmented collect applies.
size_t select_workspace(int rows, int n, int B, bool hint_usable);
// Segments of the segmented collect for a row of n slots (0: not used).
int select_segments(int n, int B, bool hint_usable);
// Points gbitmap / seg_meta / seg_list into ws (select_workspace bytes) and
// sets nseg; needs n, B and the hint fields set.
void select_bind_workspace(SelectArgs& a, int rows, void* ws);
hipError_t launch_select(const SelectArgs& a, int rows, hipStream_t s);
// The row select alone over lists already collected (seg_list / seg_meta /
// nseg set, kSeg entries per segment of seg_list): what launch_select runs
// after its own collect.
hipError_t launch_select_lists(const SelectArgs& a, int rows, hipStream_t s);
int select_list_stride();            // entries per segment of seg_list
int select_list_max();               // most listed entries the list path takes
int select_list_max_segments();      // most segments per row the list path takes

// ----- fused decode step (scoring, selection and attention in one launch) -----
// Control words at the head of the step workspace: [8] the count of finished
// workgroups, [9] an error word (bit 0: a wait gave up), then six counters
// and flags per row. Zero before the first launch; each launch leaves them
// zero again, except the error word.
struct StepArgs {
  ScoreDecodeArgs sc;                // scoring of every row (prep fused, hints on)
  int B;
  int hint_count, hint_k;
  int2* lists;                       // [rows, wpr, step_chunk_slots()] (score bits, slot)
  int4* meta;                        // [rows, wpr, step_meta_stride()] {count, max key, t_lo, 0}
  int32_t* out_idx;                  // [rows, B]
  float* out_score;                  // [rows, B] or nullptr
  const void* q;                     // attention: [N,Hq,d]
  const void* k;
  const void* v;
  int64_t kv_s_seq, kv_s_tok, kv_s_head;
  int kv_bf16;
  int Hq, Hkv, T;
  float scale_log2;
  float* out;
  float* lse;
  float* partial;                    // [rows, wpr, step_partial_stride(G)]: G x (max, sum, d outputs)
  uint32_t* ctrl;                    // step_ctrl_words(rows) control words
  int rows;
  int wpr;                           // workgroups per row: ceil(T / step_chunk_slots())
  int nxcc;                          // the device's XCDs (1..8): row r runs on XCD r % nxcc
};
int step_ctrl_words(int rows);
int step_ctrl_row0();                 // first per-row control word
int step_ctrl_per_row();              // control words per row
int step_chunk_slots();
int step_meta_stride();              // int4 per part of meta
int step_partial_stride(int G);      // floats per part of partial
// The fused step takes bf16 / fp8 projected-key caches of 64 or 128 bytes
// per key, fp32 / bf16 K/V with head_dim 128 and 1, 2, 4 or 8 query heads
// per KV head, rows of at most 32 chunks, B a multiple of 32, and hints
// that vouch for B keys; selected positions must start on a 128-byte line.
bool decode_step_supported(int rows, int n, int B, int r, int k_dt, int kv_dt, int G, int d, int hint_count,
                           int hint_k);
hipError_t launch_decode_step(const StepArgs& a, int k_dt, hipStream_t s);

// ----- indexed attention -----------------------------------------------------
struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  int64_t s_seq, s_tok, s_head;
  const int32_t* idx;
  int rows, Hq, Hkv, d, B, T;
  int prefill;
  float scale_log2;                  // scale * log2(e)
  float* out;
  float* lse;
  float* partial;                    // [rows*Hkv, splits, G, d + 2] when splits > 1
  int splits, keys_per_split;
  int qblk;                          // prefill: row i reads index row i / qblk
  const int32_t* slot;               // paged: [n_seq, slot_ld] position -> pool row
  int64_t slot_ld;
  int n_rows_kv;                     // rows addressable per sequence (T, or the pool size)
  // decode on the matrix cores only: with ctrl set, a (sequence, KV head)'s
  // splits run on one XCD (tickets per XCD, nxcc XCDs) and the last split to
  // finish merges them in place of the merge kernel; partials then sit
  // decode_partial_stride(G) floats apart. ctrl: zero before the launch and
  // left zero ([0..7] tickets, [8] finished workgroups, [16 + rowg] arrivals)
  uint32_t* ctrl = nullptr;
  int nxcc = 0;
};
int decode_partial_stride(int G);   // floats per split partial when merged in the launch
// Decode on the matrix cores (bf16, d = 128, G = 4 or 8, at most 64
// splits): one workgroup per split of kDecodeSplit list entries, writing a
// split partial, merged by launch_attention_merge.
constexpr int kDecodeSplit = 256;
bool attention_decode_mfma_supported(int G, int d, int B, bool bf16);
hipError_t launch_attention_decode_mfma(const AttnArgs& a, hipStream_t s);
hipError_t launch_attention_merge(const AttnArgs& a, hipStream_t s);
void attention_plan(int rows, int Hkv, int G, int d, int B, bool mfma_decode, int* splits,
                    int* keys_per_split);
size_t attention_workspace(int rows, int Hkv, int G, int d, int B, bool mfma_decode);
hipError_t launch_attention(const AttnArgs& a, bool q_bf16, bool kv_bf16, hipStream_t s);
// Matrix-core path for prefill with 8 query heads per KV head, head_dim 128,
// bf16 (no split partials, no workspace).
bool attention_mfma_supported(const AttnArgs& a, bool bf16);
hipError_t launch_attention_mfma(const AttnArgs& a, hipStream_t s);
bool attention_supported(int G, int d);

// ----- setup -----------------------------------------------------------------
struct ProjectArgs {
  const void* k;
  int64_t ks_seq, ks_tok, ks_head;
  const float* w;
  int w_per_head;
  void* out;
  int64_t os_seq, os_head, os_tok;
  int N, Hkv, d, r, tok_begin, n_tok;
};
// Storage dtypes: 0 fp32, 1 bf16, 2 OCP E4M3 fp8.
hipError_t launch_project(const ProjectArgs& a, bool k_bf16, int out_dt, hipStream_t s);

struct CentroidArgs {
  const void* in;
  int64_t is_seq, is_head, is_tok;
  void* out;
  int64_t os_seq, os_head, os_blk;
  int N, Hkv, T, r, block;
};
hipError_t launch_centroids(const CentroidArgs& a, int dt, hipStream_t s);

// Streaming read of bytes (a multiple of 16, 16-byte aligned) by
// kStreamReadBlocks workgroups; sink[b] = the XOR of the 32-bit words
// workgroup b read.
constexpr unsigned kStreamReadBlocks = 8192;   // = LSA_STREAM_READ_SINK_WORDS
hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t s);

}  // namespace lsa
