// Indexer scoring kernels (gfx950).
//
// Decode scoring streams the projected-key cache once: the mean of a KV
// head's query heads, projected to r dims, is dotted with every cached
// projected key (JSSA, "Joint Subspace Sparse Attention for Efficient
// Long-Context Decoding", Fig. 1; Fig. 9 "scoring preparation" and
// "candidate scoring"). It is HBM-bound (r=64 bf16: 128 bytes and 64 FMAs
// per key), so the design is about the memory stream:
//   * LPK = r*esize/16 lanes share one key row and each issues one 128-bit
//     load, so every wave-wide load instruction reads 1 KiB of consecutive
//     rows (fully coalesced);
//   * the partial dot products are summed across those LPK lanes with DPP
//     (no LDS), and after LPK loads each lane owns one of 64 consecutive
//     scores, so the fp32 score store is one coalesced 256-byte write;
//   * the query prep (mean of the G heads, times W) runs at the top of each
//     workgroup, so the step needs no separate launch for it, and its
//     latency is hidden behind the workgroup's first cache loads.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

#ifndef LSA_SCORE_WG_TARGET
#define LSA_SCORE_WG_TARGET 2048   // workgroups per scoring launch (about 8 per CU)
#endif

namespace lsa {
namespace {

constexpr int kScoreThreads = 256;
constexpr int kMaxD = 512;
constexpr int kMaxR = 128;

// Build-time tuning knobs (defaults are the tuned values for gfx950).
#ifndef LSA_SCORE_GROUPS
#define LSA_SCORE_GROUPS 2   // 64-slot groups per wave whose loads are issued together
#endif
#ifndef LSA_SCORE_NT
#define LSA_SCORE_NT 1       // stream the projected-key cache with nontemporal loads
#endif
// 64-slot groups per wave in flight (the same for every cache dtype: more
// groups for fp8 cost more occupancy than they gain)
constexpr int groups_in_flight(int dt) { return (void)dt, LSA_SCORE_GROUPS; }
// keys a hint vouches for: 1 in 32 of its group's slots
constexpr int hint_k(int dt) { return 2 * groups_in_flight(dt); }

__device__ __forceinline__ uint4 load_key16(const char* p) {
#if LSA_SCORE_NT
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_nontemporal_load((const u32x4*)p);
  return make_uint4(v.x, v.y, v.z, v.w);
#else
  return *(const uint4*)p;
#endif
}

// Storage dtypes of the projected-key cache: 0 fp32, 1 bf16, 2 OCP E4M3.
template <int DT>
__device__ __forceinline__ float dot16(const uint4& w, const float* q) {
  if constexpr (DT == 2) {
    // 16 fp8 values, two per hardware conversion (OCP E4M3 on gfx950)
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(ws[k], false);
      const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(ws[k], true);
      s = k == 0 ? q[0] * lo[0] : fmaf(q[4 * k], lo[0], s);
      s = fmaf(q[4 * k + 1], lo[1], s);
      s = fmaf(q[4 * k + 2], hi[0], s);
      s = fmaf(q[4 * k + 3], hi[1], s);
    }
    return s;
  } else if constexpr (DT == 1) {
    float s = q[0] * bf16_lo(w.x);
    s = fmaf(q[1], bf16_hi(w.x), s);
    s = fmaf(q[2], bf16_lo(w.y), s);
    s = fmaf(q[3], bf16_hi(w.y), s);
    s = fmaf(q[4], bf16_lo(w.z), s);
    s = fmaf(q[5], bf16_hi(w.z), s);
    s = fmaf(q[6], bf16_lo(w.w), s);
    s = fmaf(q[7], bf16_hi(w.w), s);
    return s;
  } else {
    float s = q[0] * __uint_as_float(w.x);
    s = fmaf(q[1], __uint_as_float(w.y), s);
    s = fmaf(q[2], __uint_as_float(w.z), s);
    s = fmaf(q[3], __uint_as_float(w.w), s);
    return s;
  }
}

// Slot -> token position, or -1 when the slot covers no token.
template <bool CAND>
__device__ __forceinline__ int64_t slot_position(const ScoreDecodeArgs& a, const int32_t* crow,
                                                 int64_t slot) {
  if constexpr (!CAND) {
    return slot;
  } else {
    int32_t c = crow[slot / a.cand_block];
    if (c < 0) return -1;
    int64_t p = (int64_t)c * a.cand_block + slot % a.cand_block;
    return p < a.T ? p : -1;
  }
}

template <int DT, int LPK, bool CAND>
__global__ __launch_bounds__(kScoreThreads) void score_decode_kernel(ScoreDecodeArgs a) {
  constexpr int ESZ = DT == 2 ? 1 : DT == 1 ? 2 : 4;
  constexpr int kGroupsInFlight = groups_in_flight(DT);
  constexpr int kHintK = hint_k(DT);
  constexpr int E = 16 / ESZ;        // channels per lane
  constexpr int KPI = kWave / LPK;   // keys per wave-wide load
  constexpr int64_t kStep = (int64_t)kGroupsInFlight * 4 * 64;   // slots per workgroup step
  __shared__ float s_qbar[kMaxD];
  __shared__ float s_part[kScoreThreads];
  __shared__ float s_q[kMaxR];

  const int row = blockIdx.y;
  const int n = row / a.Hkv, g = row % a.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int r = a.r;
  const int l = lane % LPK, kg = lane / LPK;

  // this workgroup's chunk of slots
  const int64_t c0 = (int64_t)blockIdx.x * a.chunk;
  const int64_t c1 = min((int64_t)a.n_out, c0 + a.chunk);
  const char* kbase =
      (const char*)a.k_idx + ((int64_t)n * a.ks_seq + (int64_t)g * a.ks_head) * ESZ + l * 16;
  const int64_t tok_bytes = a.ks_tok * ESZ;
  float* srow = a.scores + (int64_t)row * a.scores_ld;
  const int32_t* crow = CAND ? a.cand + (int64_t)row * a.cand_ld : nullptr;

  // one wave's loads of one step: kGroupsInFlight groups of 64 slots
  uint4 raw[kGroupsInFlight][LPK];
  bool ok[kGroupsInFlight][LPK];
  auto issue_group = [&](int64_t gb, int u) {
#pragma unroll
    for (int it = 0; it < LPK; ++it) {
      const int64_t slot = gb + (int64_t)u * 4 * 64 + it * KPI + kg;
      bool valid = slot < c1;
      int64_t pos = 0;
      if (valid) {
        pos = slot_position<CAND>(a, crow, slot);
        valid = pos >= 0;
      }
      ok[u][it] = valid;
      // unconditional load (row 0 stands in for a slot past the chunk or a
      // missing position; its score is replaced by -inf below)
      raw[u][it] = load_key16(kbase + (valid ? pos : 0) * tok_bytes);
    }
  };

  // ---- scoring preparation: q_idx = mean of the group's heads . W ----
  // Vector loads complete in issue order, so the order of issue decides
  // what the prep waits for: the prep's own loads (W: thread (j, p) owns
  // output channel j over input channels c = p + k*parts; the query values,
  // index clamped and value masked) go out first, then the first group of
  // cache loads, and the prep's math waits only for its own loads while the
  // cache loads are in flight. The empty asm statements keep the compiler
  // from reordering the two batches.
  const int64_t gfirst = c0 + (int64_t)wid * 64;
  const bool prep = a.q != nullptr;
  const int G = prep ? a.Hq / a.Hkv : 1;
  const int parts = kScoreThreads / r;
  const int j = tid % r, p = tid / r;
  constexpr int kPre = 32;
  float wv[kPre];
  constexpr int kQG = 8;
  uint32_t xbits[kQG];   // raw query bits, converted after the cache loads are issued
  const float* W = prep ? a.w + (a.w_per_head ? (int64_t)g * a.d * r : 0) : nullptr;
  if (prep) {
#pragma unroll
    for (int k = 0; k < kPre; ++k) wv[k] = W[(int64_t)min(p + k * parts, a.d - 1) * r + j];
    const int cq = min(tid, a.d - 1);
    const int64_t off0 = ((int64_t)n * a.Hq + (int64_t)g * G) * a.d + cq;
    if (a.q_bf16) {
#pragma unroll
      for (int i = 0; i < kQG; ++i) xbits[i] = ((const uint16_t*)a.q)[off0 + (int64_t)min(i, G - 1) * a.d];
    } else {
#pragma unroll
      for (int i = 0; i < kQG; ++i) xbits[i] = ((const uint32_t*)a.q)[off0 + (int64_t)min(i, G - 1) * a.d];
    }
  }
  asm volatile("" ::: "memory");
  issue_group(gfirst, 0);   // unconditional: a wave past its chunk reads row 0, masked below
  asm volatile("" ::: "memory");

  if (prep) {
    if (tid < a.d) {
      float sq = 0.f;
#pragma unroll
      for (int i = 0; i < kQG; ++i)
        if (i < G) sq += a.q_bf16 ? __uint_as_float(xbits[i] << 16) : __uint_as_float(xbits[i]);
      const int64_t off0 = ((int64_t)n * a.Hq + (int64_t)g * G) * a.d + tid;
      for (int i = kQG; i < G; ++i)
        sq += a.q_bf16 ? bf16_to_f32(((const uint16_t*)a.q)[off0 + (int64_t)i * a.d])
                       : ((const float*)a.q)[off0 + (int64_t)i * a.d];
      s_qbar[tid] = sq / (float)G;
    }
    for (int c = kScoreThreads + tid; c < a.d; c += kScoreThreads) {
      float sq = 0.f;
      for (int i = 0; i < G; ++i) {
        const int64_t off = ((int64_t)n * a.Hq + (int64_t)g * G + i) * a.d + c;
        sq += a.q_bf16 ? bf16_to_f32(((const uint16_t*)a.q)[off]) : ((const float*)a.q)[off];
      }
      s_qbar[c] = sq / (float)G;
    }
    __syncthreads();
    float acc = 0.f;
#pragma unroll
    for (int k = 0; k < kPre; ++k) {
      const int c = p + k * parts;
      if (c < a.d) acc = fmaf(s_qbar[c], wv[k], acc);
    }
    for (int c = p + kPre * parts; c < a.d; c += parts) acc = fmaf(s_qbar[c], W[(int64_t)c * r + j], acc);
    s_part[tid] = acc;
    __syncthreads();
    if (tid < r) {
      float t = 0.f;
      for (int k = 0; k < parts; ++k) t += s_part[k * r + tid];
      s_q[tid] = t;
      if (a.q_idx_out != nullptr && blockIdx.x == 0) a.q_idx_out[(int64_t)row * r + tid] = t;
    }
  } else if (tid < r) {
    s_q[tid] = a.q_idx_in[(int64_t)row * r + tid];
  }
  __syncthreads();

  float qv[E];
#pragma unroll
  for (int e = 0; e < E; ++e) qv[e] = s_q[l * E + e];

  // ---- stream this workgroup's chunk ----
  for (int64_t gb = gfirst; gb < c1; gb += kStep) {
#pragma unroll
    for (int u = 0; u < kGroupsInFlight; ++u)   // the first step's group 0 is in flight already
      if (gb != gfirst || u > 0) issue_group(gb, u);
    uint32_t hkey[kGroupsInFlight];
#pragma unroll
    for (int u = 0; u < kGroupsInFlight; ++u) {
      float mine = 0.f;
#pragma unroll
      for (int it = 0; it < LPK; ++it) {
        float s = sum_lanes<LPK>(dot16<DT>(raw[u][it], qv));
        if (!ok[u][it]) s = -INFINITY;
        if (l == it) mine = s;
      }
      const int64_t myslot = gb + (int64_t)u * 4 * 64 + (int64_t)l * KPI + kg;
      if (myslot < c1) srow[myslot] = mine;
      hkey[u] = myslot < c1 ? order_key(mine) : 0u;
    }
    if (a.hint != nullptr) {
      // selection hint of this wave's group of kGroupsInFlight*64 slots: the
      // largest 16-bit key prefix that at least kHintK of them reach, by
      // bisection with ballots (the same value on every lane)
      uint32_t hp = 0;
#pragma unroll
      for (int bit = 15; bit >= 0; --bit) {
        const uint32_t cand = (hp | (1u << bit)) << 16;
        int cnt = 0;
#pragma unroll
        for (int u = 0; u < kGroupsInFlight; ++u) cnt += __popcll(__ballot(hkey[u] >= cand));
        if (cnt >= kHintK) hp |= 1u << bit;
      }
      if (lane == 0) {
        const int64_t step = (gb - (int64_t)wid * 64) / kStep;
        a.hint[(int64_t)row * a.hint_ld + step * 4 + wid] = hp << 16;
      }
    }
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
  return (int)std::max<int64_t>(step, chunk);
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
