// Indexer scoring kernels (gfx950). The decode scoring body lives in
// score_body.hpp (shared with the fused decode step).
//
// score_emit_kernel is the decode step's scoring launch: it also does the
// top-B selection's collect (JSSA, "Joint Subspace Sparse Attention for
// Efficient Long-Context Decoding", Fig. 9: candidate scoring feeding top-B
// selection), so the step needs no collect launch and writes no scores.
// A row's threshold comes from a sample of its keys scored at the start of
// every chunk; the chunks of a row, on any XCD, hand the sample over only
// through device-scope atomics, never wait for one another, and fall back
// to the select's path over recomputed scores when anything is missing.
#include <algorithm>
#include <cmath>

#include "common.hpp"
#include "kernels.hpp"
#include "score_body.hpp"

#ifndef LSA_SCORE_WG_TARGET
#define LSA_SCORE_WG_TARGET 1024   // workgroups per scoring launch: one resident round (4 per CU)
#endif

namespace lsa {
namespace {

using namespace scoring;

constexpr int kStageSlots = 4096;   // scores one workgroup gathers in LDS before writing them

template <int DT, int LPK, bool CAND>
__global__ __launch_bounds__(kScoreThreads) void score_decode_kernel(ScoreDecodeArgs a) {
  __shared__ ScoreShared sh;
  __shared__ __align__(16) float stage[kStageSlots];   // a.chunk <= kStageSlots
  __shared__ uint32_t hstage[kStageSlots / 64];         // 4 hint entries per step of >= 256 slots
  const int64_t c0 = (int64_t)blockIdx.x * a.chunk;
  const int64_t c1 = min((int64_t)a.n_out, c0 + a.chunk);
  score_chunk<DT, LPK, CAND>(a, (int)blockIdx.y, c0, c1, sh, true, nullptr, stage, hstage);
}

// ---- decode scoring with the candidate lists of the row select ----

// Slot of sample i (global 64-slot group index gi) of a row: one slot per
// group, at a fixed pseudo-random offset, clamped to the row's end.
__device__ __forceinline__ int64_t sample_slot(int64_t gi, int row, int64_t n) {
  const uint32_t h = ((uint32_t)gi * 0x9E3779B1u) ^ ((uint32_t)row * 0x85EBCA77u);
  return min(gi * 64 + (int64_t)((h * 0xC2B2AE3Du) >> 26), n - 1);
}

// The bin (of 256, scanned from the top) that holds the need-th largest
// counted value, and the count above it, written to res[0] / res[1]
// (unchanged when fewer than need are counted). 256 threads; barriers.
__device__ __forceinline__ void emit_top_bin(const uint32_t* hist, int need, int* wsum, int* res) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int c = (int)hist[255 - t];
  int x = c;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  int base = 0;
#pragma unroll
  for (int q = 0; q < kScoreThreads / 64; ++q) base += q < w ? wsum[q] : 0;
  const int excl = base + x - c;
  if (excl < need && need <= excl + c) {
    res[0] = 255 - t;
    res[1] = excl;
  }
  __syncthreads();
}

template <int DT, int LPK, bool CAND>
__global__ __launch_bounds__(kScoreThreads) void score_emit_kernel(ScoreDecodeArgs a, ScoreEmitArgs e) {
  constexpr int ESZ = DT == 2 ? 1 : DT == 1 ? 2 : 4;
  constexpr int E = 16 / ESZ;
  constexpr int NG = kScoreThreads / LPK;                       // lane groups, one key each
  constexpr int SJ = (kStageSlots / 64 + NG - 1) / NG;          // sample keys per lane group
  constexpr int kSB = 8;                                        // sample entries per thread and batch
  constexpr uint32_t kMark = 1u << 16;                          // an entry written in this call
  constexpr int kSampleRetries = 16;                            // re-reads of an incomplete sample
  __shared__ ScoreShared sh;
  __shared__ __align__(16) float stage[kStageSlots];
  __shared__ uint32_t hstage[kStageSlots / 64];
  __shared__ uint32_t hist[256];
  __shared__ int wsum[kScoreThreads / 64];
  __shared__ int res[4];
  const int row = blockIdx.y, seg = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int64_t c0 = (int64_t)seg * a.chunk;
  const int64_t c1 = min((int64_t)a.n_out, c0 + a.chunk);
  const int ns = (int)((c1 - c0 + 63) / 64);   // this chunk's sample keys
  const int S = (int)((a.n_out + 63) / 64);    // the row's
  const int l = lane % LPK, grp = tid / LPK;
  const int n = row / a.Hkv, g = row % a.Hkv;
  const char* kbase = (const char*)a.k_idx + ((int64_t)n * a.ks_seq + (int64_t)g * a.ks_head) * ESZ + l * 16;
  uint32_t* rc = e.ctrl + (int64_t)row * e.ctrl_stride;
  uint32_t* sent = e.samples + (int64_t)row * e.s_ld;   // the row's sample entries

  // Hand-off between the row's chunks, which run on any XCD and never wait
  // for one another: each chunk writes its sample entries, mark | the key's
  // 16-bit prefix, early, and reads all of the row's entries after its
  // stream, by device-scope atomics (no fences: a device-scope fence writes
  // back or invalidates a whole L2). An entry without the mark (not yet
  // written) makes the chunk list nothing. The row's last chunk out clears
  // the entries for the next call.
  // sample slots are slots of the row (through the candidate map, when
  // there is one, like every slot: a slot that covers no token scores -inf)
  const int32_t* crow = CAND ? a.cand + (int64_t)row * a.cand_ld : nullptr;
  int64_t spos[SJ];
#pragma unroll
  for (int j = 0; j < SJ; ++j) spos[j] = sample_slot(c0 / 64 + min(grp + j * NG, ns - 1), row, a.n_out);
  if constexpr (CAND) {
    int32_t cb[SJ];
#pragma unroll
    for (int j = 0; j < SJ; ++j) cb[j] = crow[spos[j] / a.cand_block];   // map entries first, then keys
#pragma unroll
    for (int j = 0; j < SJ; ++j) {
      const int64_t p = cb[j] < 0 ? -1 : (int64_t)cb[j] * a.cand_block + spos[j] % a.cand_block;
      spos[j] = p < a.T ? p : -1;
    }
  }
  uint4 sraw[SJ];
#pragma unroll
  for (int j = 0; j < SJ; ++j) sraw[j] = load_key16(kbase + (spos[j] > 0 ? spos[j] : (int64_t)0) * a.ks_tok * ESZ);
  auto contribute = [&](const float (&qv)[E]) {
#pragma unroll
    for (int j = 0; j < SJ; ++j) {
      float sc = sum_lanes<LPK>(dot16<DT>(sraw[j], qv));
      if (spos[j] < 0) sc = -INFINITY;
      const int i = grp + j * NG;
      if (l == 0 && i < ns)
        __hip_atomic_store(sent + c0 / 64 + i, kMark | (order_key(sc) >> 16), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
  };
  uint32_t ent[kSB];
  auto load_batch = [&](int i0) {
#pragma unroll
    for (int q = 0; q < kSB; ++q)
      ent[q] = __hip_atomic_load(sent + min(i0 + q * kScoreThreads + tid, S - 1), __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
  };
  // The row's threshold word (1 << 32 | t_lo once set): the first chunks out
  // compute t_lo and set it, the later ones (those that end the launch)
  // only read it; its load is issued while the staged scores go out.
  uint64_t* tword = reinterpret_cast<uint64_t*>(rc + 2);
  uint64_t tw = 0;
  score_chunk<DT, LPK, CAND>(a, row, c0, c1, sh, true, nullptr, stage, hstage, contribute, [&]() {
    if (tid == 0) tw = __hip_atomic_load(tword, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  });
  if (tid == 0) res[3] = (tw >> 32) ? (int)(uint32_t)tw : -1;
  __syncthreads();
  uint32_t t_lo = (uint32_t)res[3];
  bool complete = res[3] != -1;
  __syncthreads();   // res is reused below
  if (!complete) {
    // ---- t_lo: the 16-bit prefix of the k_rank-th largest sample key, by two
    // 8-bit radix levels over the row's entries ----
    load_batch(0);
    auto each_entry = [&](auto fn) {
#pragma unroll
      for (int q = 0; q < kSB; ++q)
        if (q * kScoreThreads + tid < S) fn(ent[q]);
      for (int i0 = kSB * kScoreThreads; i0 < S; i0 += kSB * kScoreThreads) {   // rows of more samples
        load_batch(i0);
#pragma unroll
        for (int q = 0; q < kSB; ++q)
          if (i0 + q * kScoreThreads + tid < S) fn(ent[q]);
      }
    };
    // With short chunks a chunk can get here before a later chunk of its
    // row has written its entries: the entries are read again, a bounded
    // number of times (each writer is already running and writes its
    // entries right after its query prep), before the chunk gives up.
    for (int attempt = 0;; ++attempt) {
      if (tid == 0) res[2] = 0;
      __syncthreads();
      int unmarked = 0;
      each_entry([&](uint32_t v) { unmarked += (v >> 16) != 1u; });
      if (unmarked) atomicAdd(&res[2], unmarked);
      __syncthreads();
      complete = res[2] == 0;
      if (complete || attempt == kSampleRetries) break;
      __builtin_amdgcn_s_sleep(32);
      load_batch(0);
    }
    if (S > kSB * kScoreThreads) load_batch(0);
    hist[tid] = 0u;
    if (tid == 0) res[0] = 0, res[1] = 0;
    __syncthreads();
    each_entry([&](uint32_t v) { atomicAdd(&hist[(v >> 8) & 255u], 1u); });
    __syncthreads();
    emit_top_bin(hist, e.k_rank, wsum, res);
    const uint32_t b1 = (uint32_t)res[0];
    const int need = e.k_rank - res[1];
    hist[tid] = 0u;
    __syncthreads();
    if (S > kSB * kScoreThreads) load_batch(0);
    each_entry([&](uint32_t v) {
      if ((v >> 16) == 1u && ((v >> 8) & 255u) == b1) atomicAdd(&hist[v & 255u], 1u);
    });
    __syncthreads();
    emit_top_bin(hist, need, wsum, res);
    t_lo = ((b1 << 8) | (uint32_t)res[0]) << 16;
    if (tid == 0 && complete)   // every chunk that computes it finds the same value
      __hip_atomic_store(tword, (1ull << 32) | t_lo, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // ---- list this chunk's keys >= t_lo, in slot order ----
  int4* meta = e.meta + (int64_t)row * e.wpr + seg;
  const int len = (int)(c1 - c0);
  if (!complete) {   // the sample is not all there: the select takes the scores instead
    if (tid == 0) *meta = make_int4(e.no_list, 0, 0, 0);
  } else {
    if (tid == 0) res[3] = 0;   // max listed key
    // thread t owns slots 4(t + 256j) .. +3, j < 4: in slot order by (j, t)
    constexpr int kJ = kStageSlots / (4 * kScoreThreads);
    float v[kJ][4];
    uint32_t pass = 0;   // bit 4j + k
    int cnt[kJ];
    uint32_t kmax = 0u;
#pragma unroll
    for (int j = 0; j < kJ; ++j) {
      const int s0 = 4 * (tid + kScoreThreads * j);
      const float4 x = *reinterpret_cast<const float4*>(stage + s0);
      v[j][0] = x.x; v[j][1] = x.y; v[j][2] = x.z; v[j][3] = x.w;
      cnt[j] = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t key = order_key(v[j][k]);
        if (s0 + k < len && key >= t_lo) {
          pass |= 1u << (4 * j + k);
          ++cnt[j];
          kmax = max(kmax, key);
        }
      }
    }
    static_assert(kJ == 4, "four 16-bit counts in two words");
    int tot01, tot23;
    const int p01 = block_exclusive_scan<kScoreThreads>(cnt[0] | (cnt[1] << 16), wsum, &tot01);
    const int p23 = block_exclusive_scan<kScoreThreads>(cnt[2] | (cnt[3] << 16), wsum, &tot23);
    const int base[kJ] = {p01 & 0xffff, (tot01 & 0xffff) + (p01 >> 16),
                          (tot01 & 0xffff) + (tot01 >> 16) + (p23 & 0xffff),
                          (tot01 & 0xffff) + (tot01 >> 16) + (tot23 & 0xffff) + (p23 >> 16)};
    int2* lrow = e.lists + ((int64_t)row * e.wpr + seg) * e.list_stride;
#pragma unroll
    for (int j = 0; j < kJ; ++j) {
      int o = base[j];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if ((pass >> (4 * j + k)) & 1u)
          lrow[o++] = make_int2(__float_as_int(v[j][k]), (int)(c0 + 4 * (tid + kScoreThreads * j) + k));
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o, 64));
    if (lane == 0 && kmax) atomicMax(reinterpret_cast<uint32_t*>(&res[3]), kmax);
    __syncthreads();
    if (tid == 0) {
      const int total = (tot01 & 0xffff) + (tot01 >> 16) + (tot23 & 0xffff) + (tot23 >> 16);
      *meta = make_int4(total, res[3], (int)t_lo, 0);
    }
  }
  // the row's last chunk out clears the row's count and sample entries
  if (tid == 0)
    res[2] = __hip_atomic_fetch_add(rc, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)(e.wpr - 1);
  __syncthreads();
  if (res[2]) {
    if (tid == 0) {
      __hip_atomic_store(rc, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(tword, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    for (int i = tid; i < S; i += kScoreThreads)
      __hip_atomic_store(sent + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Small-L causal score matrix (unfused prefill scoring, for checking the
// fused path and for short prompts). One thread per (row, key).
template <bool BF16>
__global__ __launch_bounds__(256) void score_prefill_kernel(ScorePrefillArgs a) {
  __shared__ float s_q[kMaxR];
  const int row = blockIdx.y;  // i * Hkv + g
  const int i = row / a.Hkv, g = row % a.Hkv;
  for (int c = threadIdx.x; c < a.r; c += blockDim.x) {
    int64_t off = (int64_t)row * a.r + c;
    s_q[c] = BF16 ? bf16_to_f32(((const uint16_t*)a.q_idx)[off]) : ((const float*)a.q_idx)[off];
  }
  __syncthreads();
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= a.L) return;
  float acc = -INFINITY;
  if (j <= i) {
    acc = 0.f;
    int64_t kb = (int64_t)g * a.ks_head + (int64_t)j * a.ks_tok;
    for (int c = 0; c < a.r; ++c) {
      float k = BF16 ? bf16_to_f32(((const uint16_t*)a.k_idx)[kb + c]) : ((const float*)a.k_idx)[kb + c];
      acc = fmaf(s_q[c], k, acc);
    }
  }
  a.scores[(int64_t)row * a.scores_ld + j] = acc;
}

template <int DT, int LPK>
hipError_t launch_decode_lpk(const ScoreDecodeArgs& a, int rows, hipStream_t s) {
  dim3 grid((unsigned)((a.n_out + a.chunk - 1) / a.chunk), (unsigned)rows);
  if (a.cand)
    hipLaunchKernelGGL((score_decode_kernel<DT, LPK, true>), grid, dim3(kScoreThreads), 0, s, a);
  else
    hipLaunchKernelGGL((score_decode_kernel<DT, LPK, false>), grid, dim3(kScoreThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

int score_hint_count(int n_out, int k_dt) {
  const int step = groups_in_flight(k_dt) * 4 * 64;
  return (n_out + step - 1) / step * 4;
}

int score_hint_k(int k_dt) { return hint_k(k_dt); }

int score_chunk_slots(int n_out, int rows, int k_dt) {
  // about LSA_SCORE_WG_TARGET workgroups for a bf16 cache, scaled by the row
  // bytes so every workgroup streams about as many bytes whatever the dtype;
  // a chunk is a whole number of the slots one workgroup covers per step
  const int esz = k_dt == 2 ? 1 : k_dt == 1 ? 2 : 4;
  const int64_t step = (int64_t)groups_in_flight(k_dt) * 4 * 64;
  const int64_t target = std::max<int64_t>(256, (int64_t)LSA_SCORE_WG_TARGET * esz / 2);
  const int64_t per_row = (target + rows - 1) / rows;
  int64_t chunk = (n_out + per_row - 1) / per_row;
  chunk = (chunk + step - 1) / step * step;
  // at most kStageSlots, the LDS staging of the chunk's scores
  chunk = std::min<int64_t>(chunk, kStageSlots / step * step);
  return (int)std::max<int64_t>(step, chunk);
}

int score_emit_samples(int n_out) { return (n_out + 63) / 64; }

int score_emit_rank(int n_out, int rows, int B, int r, int k_dt, int seg_cap, int max_segs, int max_listed) {
  const int esz = k_dt == 2 ? 1 : k_dt == 1 ? 2 : 4;
  const int lpk = r * esz / 16;
  if (lpk != 4 && lpk != 8 && lpk != 16) return 0;
  if (B < 1 || n_out < 1 || B >= n_out) return 0;
  const int chunk = score_chunk_slots(n_out, rows, k_dt);
  if (chunk > kStageSlots || chunk > seg_cap || (n_out + chunk - 1) / chunk > max_segs) return 0;
  // about S*B/n sample keys reach the B-th key of the row; the rank adds
  // 3.5 standard deviations and 6, so that fewer than B of the row's keys
  // reach t_lo only rarely (the select then takes the scores)
  const double S = score_emit_samples(n_out);
  const double mu = S * B / n_out;
  const int k = (int)std::ceil(mu + 3.5 * std::sqrt(mu) + 6.0);
  // expected listed keys: about 64 k; the list path takes at most max_lists
  if (k > S / 2 || 64.0 * k > 0.8 * max_listed) return 0;
  return k;
}

template <int DT, int LPK>
hipError_t launch_emit_lpk(const ScoreDecodeArgs& a, const ScoreEmitArgs& e, int rows, hipStream_t s) {
  dim3 grid((unsigned)((a.n_out + a.chunk - 1) / a.chunk), (unsigned)rows);
  if ((int)grid.x != e.wpr) return hipErrorInvalidValue;
  if (a.cand)
    hipLaunchKernelGGL((score_emit_kernel<DT, LPK, true>), grid, dim3(kScoreThreads), 0, s, a, e);
  else
    hipLaunchKernelGGL((score_emit_kernel<DT, LPK, false>), grid, dim3(kScoreThreads), 0, s, a, e);
  return hipGetLastError();
}

hipError_t launch_score_emit(const ScoreDecodeArgs& a, const ScoreEmitArgs& e, int rows, int k_dt,
                             hipStream_t s) {
  if ((a.cand != nullptr && a.cand_block < 1) || a.hint != nullptr || a.chunk > kStageSlots || a.chunk % 4 != 0 ||
      e.list_stride < a.chunk || e.s_ld < score_emit_samples(a.n_out) || e.k_rank < 1)
    return hipErrorInvalidValue;
  const int esz = k_dt == 2 ? 1 : k_dt == 1 ? 2 : 4;
  const int lpk = a.r * esz / 16;
  if (k_dt == 2) {
    switch (lpk) {
      case 4: return launch_emit_lpk<2, 4>(a, e, rows, s);
      case 8: return launch_emit_lpk<2, 8>(a, e, rows, s);
      case 16: return launch_emit_lpk<2, 16>(a, e, rows, s);
    }
  } else if (k_dt == 1) {
    switch (lpk) {
      case 4: return launch_emit_lpk<1, 4>(a, e, rows, s);
      case 8: return launch_emit_lpk<1, 8>(a, e, rows, s);
      case 16: return launch_emit_lpk<1, 16>(a, e, rows, s);
    }
  } else {
    switch (lpk) {
      case 4: return launch_emit_lpk<0, 4>(a, e, rows, s);
      case 8: return launch_emit_lpk<0, 8>(a, e, rows, s);
      case 16: return launch_emit_lpk<0, 16>(a, e, rows, s);
    }
  }
  return hipErrorInvalidValue;
}

hipError_t launch_score_decode(const ScoreDecodeArgs& a, int rows, int k_dt, hipStream_t s) {
  const int esz = k_dt == 2 ? 1 : k_dt == 1 ? 2 : 4;
  const int lpk = a.r * esz / 16;
  if (k_dt == 2) {
    switch (lpk) {
      case 1: return launch_decode_lpk<2, 1>(a, rows, s);
      case 2: return launch_decode_lpk<2, 2>(a, rows, s);
      case 4: return launch_decode_lpk<2, 4>(a, rows, s);
      case 8: return launch_decode_lpk<2, 8>(a, rows, s);
      case 16: return launch_decode_lpk<2, 16>(a, rows, s);
    }
  } else if (k_dt == 1) {
    switch (lpk) {
      case 1: return launch_decode_lpk<1, 1>(a, rows, s);
      case 2: return launch_decode_lpk<1, 2>(a, rows, s);
      case 4: return launch_decode_lpk<1, 4>(a, rows, s);
      case 8: return launch_decode_lpk<1, 8>(a, rows, s);
      case 16: return launch_decode_lpk<1, 16>(a, rows, s);
    }
  } else {
    switch (lpk) {
      case 1: return launch_decode_lpk<0, 1>(a, rows, s);
      case 2: return launch_decode_lpk<0, 2>(a, rows, s);
      case 4: return launch_decode_lpk<0, 4>(a, rows, s);
      case 8: return launch_decode_lpk<0, 8>(a, rows, s);
      case 16: return launch_decode_lpk<0, 16>(a, rows, s);
    }
  }
  return hipErrorInvalidValue;
}

hipError_t launch_score_prefill(const ScorePrefillArgs& a, bool bf16, hipStream_t s) {
  dim3 grid((unsigned)((a.L + 255) / 256), (unsigned)(a.L * a.Hkv));
  if (bf16)
    hipLaunchKernelGGL((score_prefill_kernel<true>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((score_prefill_kernel<false>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace lsa
