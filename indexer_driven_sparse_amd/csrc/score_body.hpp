// Decode scoring of one chunk of a row by one workgroup: the body of the
// scoring kernel (score.hip) and of the fused decode step (step.hip), kept
// in one place so both compute bit-identical scores and hints. Included by
// one translation unit each (device code is not linked across them).
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
//     chunk, and its latency is hidden behind the chunk's first cache loads.
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace lsa {
namespace scoring {

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

// LDS of one scoring workgroup.
struct ScoreShared {
  float qbar[kMaxD];
  float part[kScoreThreads];
  float q[kMaxR];
};

// A 32-bit store, device-coherent (visible to every XCD once complete) when
// COHERENT, else a plain store.
template <bool COHERENT>
__device__ __forceinline__ void store_u32(uint32_t* p, uint32_t v) {
  if constexpr (COHERENT) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else *p = v;
}
template <bool COHERENT>
__device__ __forceinline__ void store_u32x4(uint32_t* p, uint4 v) {
  if constexpr (COHERENT) {
    store_u32<true>(p, v.x);
    store_u32<true>(p + 1, v.y);
    store_u32<true>(p + 2, v.z);
    store_u32<true>(p + 3, v.w);
  } else {
    *reinterpret_cast<uint4*>(p) = v;
  }
}

// Scores (and selection hints) of slots [c0, c1) of one row, by one
// 256-thread workgroup; c0 is a multiple of the workgroup step. Every
// thread of the workgroup must call it. With a.q set, the row's q_idx is
// computed here (overlapped with the first cache loads) when PREP and
// do_prep; otherwise the caller has left it in sh.q.
// STEPS > 0: the chunk is at most STEPS workgroup steps long, the loop is
// unrolled, and each thread keeps its scores in the LDS array keep, at
// keep[(s * G + u) * 256 + thread] (step s, group u; slots past c1 hold
// NaN), instead of storing them to a.scores; every hint entry of a step that
// starts inside the row is written (0 for a wave left with no slot). COHERENT: scores and hints are stored device-coherently, for
// readers on other XCDs inside the same launch. stage (STEPS == 0 only):
// an LDS array of at least c1 - c0 floats, hstage one of the chunk's hint
// entries (4 per step); scores and hints are gathered there and written out
// in one burst (16-byte stores for the scores) after the chunk's last load,
// every hint entry of the chunk's steps included (0 for a wave that had no
// slot left in the last step).
// Scattered score stores in the middle of the cache stream cost the stream
// far more than their share of the bytes on MI355X; one burst per chunk
// costs little.
// after_prep(qv), if given, runs on every thread once the row's q_idx is
// ready (qv: this lane's E channels of it) and before the chunk's stream
// goes on; before_burst(), if given, runs on every thread after the
// chunk's last cache load has been used and before the staged scores are
// written (STEPS == 0 with stage). Either may contain barriers.
struct NoHook {
  template <class... T>
  __device__ __forceinline__ void operator()(const T&...) const {}
};
template <int DT, int LPK, bool CAND, bool PREP = true, int STEPS = 0, bool COHERENT = false,
          class Hook = NoHook, class Hook2 = NoHook>
__device__ __forceinline__ void score_chunk(const ScoreDecodeArgs& a, int row, int64_t c0, int64_t c1,
                                            ScoreShared& sh, bool do_prep = true, float* keep = nullptr,
                                            float* stage = nullptr, uint32_t* hstage = nullptr,
                                            Hook after_prep = Hook{}, Hook2 before_burst = Hook2{}) {
  constexpr int ESZ = DT == 2 ? 1 : DT == 1 ? 2 : 4;
  constexpr int kGroupsInFlight = groups_in_flight(DT);
  constexpr int kHintK = hint_k(DT);
  constexpr int E = 16 / ESZ;        // channels per lane
  constexpr int KPI = kWave / LPK;   // keys per wave-wide load
  constexpr int64_t kStep = (int64_t)kGroupsInFlight * 4 * 64;   // slots per workgroup step
  float* const s_qbar = sh.qbar;
  float* const s_part = sh.part;
  float* const s_q = sh.q;

  const int n = row / a.Hkv, g = row % a.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int r = a.r;
  const int l = lane % LPK, kg = lane / LPK;
  const char* kbase =
      (const char*)a.k_idx + ((int64_t)n * a.ks_seq + (int64_t)g * a.ks_head) * ESZ + l * 16;
  const int64_t tok_bytes = a.ks_tok * ESZ;
  float* srow = a.scores != nullptr ? a.scores + (int64_t)row * a.scores_ld : nullptr;
  const int32_t* crow = CAND ? a.cand + (int64_t)row * a.cand_ld : nullptr;

  // one wave's loads of one step: kGroupsInFlight groups of 64 slots
  uint4 raw[kGroupsInFlight][LPK];
  bool ok[kGroupsInFlight][LPK];
  auto issue_group = [&](int64_t gb, int u) {
    // with a candidate map, every map entry of the group is loaded before
    // any key: vector loads complete in order, so a key load issued between
    // two map loads would make the second map entry wait for it
    int32_t cpos[LPK];
    if constexpr (CAND) {
#pragma unroll
      for (int it = 0; it < LPK; ++it) {
        const int64_t slot = gb + (int64_t)u * 4 * 64 + it * KPI + kg;
        cpos[it] = slot < c1 ? crow[slot / a.cand_block] : -1;
      }
    }
#pragma unroll
    for (int it = 0; it < LPK; ++it) {
      const int64_t slot = gb + (int64_t)u * 4 * 64 + it * KPI + kg;
      bool valid = slot < c1;
      int64_t pos = 0;
      if (valid) {
        if constexpr (CAND) {
          pos = cpos[it] < 0 ? -1 : (int64_t)cpos[it] * a.cand_block + slot % a.cand_block;
          if (pos >= a.T) pos = -1;
        } else {
          pos = slot;
        }
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
  const int n_hst = (int)((c1 - c0 + kStep - 1) / kStep) * 4;   // hint entries of the chunk's steps
  if (STEPS == 0 && stage != nullptr)
    for (int k = tid; k < n_hst; k += kScoreThreads) hstage[k] = 0u;   // ordered by the prep's barrier
  const bool prep = PREP && a.q != nullptr && do_prep;
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
      if (a.q_idx_out != nullptr && c0 == 0) a.q_idx_out[(int64_t)row * r + tid] = t;
    }
  } else if (a.q == nullptr && tid < r) {
    s_q[tid] = a.q_idx_in[(int64_t)row * r + tid];
  }
  __syncthreads();

  float qv[E];
#pragma unroll
  for (int e = 0; e < E; ++e) qv[e] = s_q[l * E + e];
  after_prep(qv);

  // ---- stream this workgroup's chunk ----
  auto one_step = [&](int64_t gb, int si) {
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
      if constexpr (STEPS == 0) {
        if (myslot < c1) {
          if (stage != nullptr) stage[myslot - c0] = mine;
          else store_u32<COHERENT>(reinterpret_cast<uint32_t*>(srow + myslot), __float_as_uint(mine));
        }
      }
      if constexpr (STEPS > 0)
        keep[(si * kGroupsInFlight + u) * kScoreThreads + tid] = myslot < c1 ? mine : __builtin_nanf("");
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
        if (STEPS == 0 && stage != nullptr) hstage[(step - c0 / kStep) * 4 + wid] = hp << 16;
        else store_u32<COHERENT>(a.hint + (int64_t)row * a.hint_ld + step * 4 + wid, hp << 16);
      }
    }
  };
  if constexpr (STEPS == 0) {
    for (int64_t gb = gfirst; gb < c1; gb += kStep) one_step(gb, 0);
    if (stage != nullptr) {
      before_burst();
      // srow + c0 is 16-byte aligned (16-byte aligned rows, c0 a multiple of the step)
      __syncthreads();
      const int n = a.scores != nullptr ? (int)(c1 - c0) : 0, nq = n / 4;   // no scores: none written
      float* dst = srow + c0;
      for (int k = tid; k < nq; k += kScoreThreads)
        store_u32x4<COHERENT>(reinterpret_cast<uint32_t*>(dst + 4 * k), *reinterpret_cast<const uint4*>(stage + 4 * k));
      for (int k = 4 * nq + tid; k < n; k += kScoreThreads)
        store_u32<COHERENT>(reinterpret_cast<uint32_t*>(dst + k), __float_as_uint(stage[k]));
      if (a.hint != nullptr) {
        uint32_t* hdst = a.hint + (int64_t)row * a.hint_ld + c0 / kStep * 4;
        for (int k = tid; k < n_hst; k += kScoreThreads) store_u32<COHERENT>(hdst + k, hstage[k]);
      }
    }
  } else {
#pragma unroll
    for (int si = 0; si < STEPS; ++si) {
      const int64_t gb = gfirst + (int64_t)si * kStep;
      if (gb < c1) {
        one_step(gb, si);
      } else {
#pragma unroll
        for (int u = 0; u < kGroupsInFlight; ++u)
          keep[(si * kGroupsInFlight + u) * kScoreThreads + tid] = __builtin_nanf("");
        // a step that starts inside the row but leaves this wave no slot:
        // its hint entry vouches for nothing
        const int64_t step0 = c0 + (int64_t)si * kStep;
        if (a.hint != nullptr && lane == 0 && step0 < a.n_out)
          store_u32<COHERENT>(a.hint + (int64_t)row * a.hint_ld + step0 / kStep * 4 + wid, 0u);
      }
    }
  }
}

}  // namespace scoring
}  // namespace lsa
