// Fused decode step: one launch computes the whole step of every
// (sequence, KV head) row -- scoring preparation, projected-key scores,
// exact top-B and indexed attention (JSSA, "Joint Subspace Sparse Attention
// for Efficient Long-Context Decoding", Fig. 1, and the four stages of
// Fig. 9).
//
// Why one launch: scoring is a long HBM stream, while the selection and the
// attention are chains of short, latency-bound steps over a few MB; in one
// launch the scores never leave LDS and no kernel boundary separates the
// phases. (Measured on MI355X a boundary costs only about 1 us on one
// stream, and with every workgroup resident the rows finish scoring
// together, so the phases do not overlap the stream: this launch is slower
// than the separate kernels and is opt-in.)
//
// Layout: the device's XCDs each take rows x, x + nxcc, ... (nxcc XCDs):
// a workgroup reads its XCD from the hardware, draws a ticket from that
// XCD's queue and becomes one (row, chunk) of kChunk slots, so all of a
// row's workgroups share one L2. Each scores its chunk (the stream of
// score_body.hpp, unchanged) and keeps the scores in LDS. After that the
// row's workgroups work together, with no further pass over the scores:
//   1. threshold  the last workgroup of the row to finish scoring derives a
//                 lower bound t_lo of the row's B-th key from the row's
//                 selection hints (the r-th largest of hints that each
//                 vouch for hint_k keys) and publishes it;
//   2. collect    every workgroup lists its slots whose key reaches t_lo,
//                 in slot order, as (score bits, slot), straight from its
//                 LDS; the last one to finish runs the exact selection over
//                 the row's lists (an LDS histogram, then bisection, the
//                 positions written in ascending order by one prefix scan;
//                 lists too long for the registers are selected by radix
//                 passes over the lists in memory);
//   3. attend     every workgroup attends over its share of the row's B
//                 selected positions (each K and V row read in place, one
//                 256-byte row per wave-wide load, softmax in fp32 in the
//                 log2 domain) and writes a partial (max, sum, output);
//                 the last one merges the row's partials by log-sum-exp.
// The hand-offs stay inside the row's XCD (the rules are stated beside
// add_l below). The waits in 1-3 only ever wait for workgroups of the same
// row, which hold consecutive tickets of one XCD's queue; every wait is
// bounded, and a timeout only sets an error bit, so every wave exits. The
// last workgroup out leaves the control words zero for the next launch.
//
// The indices equal those of the separate scoring and select calls bit for
// bit (both are the exact top-B of the same scores); the attention's
// arithmetic differs from the separate call's kernels only in summation
// order.
#include "common.hpp"
#include "kernels.hpp"
#include "score_body.hpp"
#include "select_row.hpp"

#ifndef LSA_STEP_WG_PER_CU
#define LSA_STEP_WG_PER_CU 4   // resident workgroups per CU the register budget allows
#endif

namespace lsa {
namespace {

using namespace scoring;
using namespace sel;

constexpr int kWgThreads = 256;
static_assert(kWgThreads == kScoreThreads, "the scoring body is written for 256 threads");
constexpr int kGroups = 2;                       // groups_in_flight(): 64-slot groups per wave step
constexpr int kWgStep = kGroups * 4 * 64;        // slots one workgroup covers per step
constexpr int kSteps = 8;                        // steps per chunk
constexpr int kChunk = kSteps * kWgStep;         // 4096 slots per workgroup
constexpr int kKeep = kSteps * kGroups;          // scores each lane keeps
constexpr int kFinPer = 32;                      // list entries per thread in the exact selection
constexpr int kFinCap = kWgThreads * kFinPer;      // longest list refined in registers
constexpr int kCompCap = 1024;                     // keys of one histogram bin bisected from LDS
static_assert(kCompCap <= kKeep * kWgThreads && kCompCap % kWgThreads == 0, "the compaction reuses the keep array");
constexpr int kMaxG = 8;                         // query heads per KV head (attention)
constexpr int kD = 128;                          // head dim (attention: two channels per lane)
constexpr int kBatch = 8;                        // list entries per wave per attention batch
constexpr int kMaxParts = 32;                    // workgroups per row (merge weights in LDS)
constexpr int kSpinLimit = 1 << 21;              // polls before a wait gives up
// floats per part's partial (G heads of max, sum and kD outputs), rounded
// up to whole 128-byte lines
__host__ __device__ constexpr int partial_stride(int G) { return (G * (kD + 2) + 31) / 32 * 32; }

// control words: [0..7] per-XCD tickets, [8] finished workgroups, [9] error
// bits (device-coherent), then one block per row, each in its own 4 KiB,
// used only by the row's XCD
enum { kCtlQueue = 0, kCtlDone = 8, kCtlErr = 9, kCtlRow0 = 1024, kCtlPerRow = 1024 };
enum { kRowScored = 0, kRowThr = 2, kRowCollected = 3, kRowSelected = 4, kRowAttended = 5 };
constexpr int kMetaStride = 8;   // int4 per part's meta: one 128-byte line each

__device__ __forceinline__ void st_c(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t add_c(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Hand-off inside one XCD. A row's workgroups all run on one XCD and so
// share one L2; the L1 of each CU writes through to it. The row's counters
// and flags are read and written only by atomics, which are performed in
// that L2 (a polled plain load would be served by a stale L1 line). The
// shared data (hints, lists, meta, selected positions, partials) is stored
// plainly and loaded plainly, under two rules that keep every L1 line a
// reader hits current: every 128-byte line of it has one writing workgroup
// (a chunk's 32 hint words fill one line of a 128-byte-aligned hint row),
// and nothing loads it before the counter that publishes it has been seen
// (the L1s start each launch empty). A writer waits for its stores before
// it bumps the counter.
__device__ __forceinline__ uint32_t add_l(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
// An atomic read: an OR with zero, the zero hidden from the compiler (which
// would otherwise turn the idempotent atomic into a load).
__device__ __forceinline__ uint32_t ld_l(uint32_t* p) {
  uint32_t zero;
  asm volatile("v_mov_b32 %0, 0" : "=v"(zero));
  return __hip_atomic_fetch_or(p, zero, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ unsigned xcd_id() {
  return __builtin_amdgcn_s_getreg((15 << 11) | 20) & 15u;   // HW_REG_XCC_ID
}

// Every memory operation of the workgroup has completed before thread 0
// publishes it.
__device__ __forceinline__ void all_done() {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
}

// Thread 0 polls the XCD-local word *p until it reaches target (bounded);
// a timeout sets error bit 0. Returns the value seen last, to every thread
// (through *slot in LDS).
__device__ __forceinline__ uint32_t wait_until(uint32_t* p, uint32_t target, uint32_t* err, int* slot) {
  if (threadIdx.x == 0) {
    int spins = 0;
    uint32_t v;
    while ((v = ld_l(p)) < target && spins < kSpinLimit) {
      __builtin_amdgcn_s_sleep(4);
      ++spins;
    }
    if (spins >= kSpinLimit) __hip_atomic_fetch_or(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *slot = (int)v;
  }
  __syncthreads();
  const uint32_t v = (uint32_t)*slot;
  __syncthreads();   // the slot is reused
  return v;
}

struct FinShared {
  uint32_t hist[256];
  int scan[kWgThreads / 64 + 1];
  int seg_off[kMaxParts + 1];
  int cnt[2][kWgThreads / 64];   // per-wave counts of a bisection step (two steps in flight)
  int ncomp;                     // keys compacted for the bisection
  uint32_t kmax;
  int bin, above;
};

struct CollectShared {
  int cnt[kSteps * kGroups * 4];
  int off[kSteps * kGroups * 4];
  uint32_t wmax[4];
  int total;
};

struct AttnShared {
  int32_t idx[kWgThreads];
  float m[4][kMaxG];
  float l[4][kMaxG];
  float o[4][kMaxG][kD];
  float w[kMaxParts][kMaxG];   // merge: per-partial weights
  float mstar[kMaxG];
};

struct StepShared {
  ScoreShared score;
  float keep[kKeep * kWgThreads];   // this workgroup's scores, kept for the collect
  union {
    SegShared seg;       // threshold
    CollectShared col;
    FinShared fin;
    AttnShared att;
  } u;
  int flag;   // a role decision (ticket, last arrival), read by every wave
  int wval;   // a value waited for or published to the workgroup
};

// ---------------------------------------------------------------------------
// 1. the row's threshold from its hints (the r-th largest of folded hint
// entries, on 16-bit prefixes, by two 8-bit radix levels; 0 = take all)
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t row_threshold(const uint32_t* hrow, int hint_count, int hint_k, int B, SegShared& sh) {
  const int tid = threadIdx.x;
  const int m = (hint_count + 4 * kWgThreads - 1) / (4 * kWgThreads);
  const int ne = (hint_count + m - 1) / m;
  const int r = (B + m * hint_k - 1) / (m * hint_k);
  uint32_t p[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = tid + q * kWgThreads;
    uint32_t val = 0xffffffffu;
    for (int mm = 0; mm < m; ++mm) {
      const int h = e * m + mm;
      val = min(val, h < hint_count ? hrow[h] : 0u);
    }
    p[q] = (e < ne ? val : 0u) >> 16;
  }
  sh.h1[tid] = 0u;
  sh.h2[tid] = 0u;
  if (tid == 0) sh.bin = -1;
  __syncthreads();
#pragma unroll
  for (int q = 0; q < 4; ++q)
    if (tid + q * kWgThreads < ne) atomicAdd(&sh.h1[p[q] >> 8], 1u);
  __syncthreads();
  uint32_t t_lo = 0u;
  if (r <= ne) {
    seg_level(sh, sh.h1, r);
    const int b1 = sh.bin, r2 = r - sh.above;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (tid + q * kWgThreads < ne && (int)(p[q] >> 8) == b1) atomicAdd(&sh.h2[p[q] & 255u], 1u);
    __syncthreads();
    seg_level(sh, sh.h2, r2);
    t_lo = ((uint32_t)b1 << 24) | ((uint32_t)sh.bin << 16);
  }
  return t_lo;
}

// ---------------------------------------------------------------------------
// 2b. exact top-B of a row from its lists (every key >= t_lo, in slot order;
// the hints guarantee at least B of them)
// ---------------------------------------------------------------------------

// Rows whose lists hold more than kFinCap entries: 8-bit radix levels over
// the lists in memory, then the positions in list (= slot) order, the lowest
// slots first among keys equal to the B-th. Each level is one pass over the
// lists; the case needs a flat or heavily tied row.
__device__ __forceinline__ void select_lists_general(const StepArgs& a, FinShared& sh, int row, int total) {
  const int tid = threadIdx.x;
  const int B = a.B, nseg = a.wpr;
  const uint64_t* lrow = (const uint64_t*)(a.lists + (int64_t)row * nseg * kChunk);
  int32_t* orow = a.out_idx + (int64_t)row * B;
  float* osc = a.out_score ? a.out_score + (int64_t)row * B : nullptr;
  uint32_t pre = 0u;
  int fixed = 0, nd = B;
  while (fixed < 32) {
    const int shift = 24 - fixed;
    const uint32_t pmask = fixed == 0 ? 0u : (~0u << (32 - fixed));
    sh.hist[tid] = 0u;
    __syncthreads();
    for (int p = 0; p < nseg; ++p) {
      const int n = sh.seg_off[p + 1] - sh.seg_off[p];
      for (int i = tid; i < n; i += kWgThreads) {
        const uint32_t key = order_key(__uint_as_float((uint32_t)lrow[(int64_t)p * kChunk + i]));
        if ((key & pmask) == pre) atomicAdd(&sh.hist[(key >> shift) & 255u], 1u);
      }
    }
    __syncthreads();
    const int c = (int)sh.hist[255 - tid];
    int tot;
    const int excl = block_exclusive_scan<kWgThreads>(c, sh.scan, &tot);
    if (excl < nd && nd <= excl + c) {
      sh.bin = 255 - tid;
      sh.above = excl;
    }
    __syncthreads();
    const int bin = sh.bin;
    nd -= sh.above;
    const int cnt = (int)sh.hist[bin];
    pre |= (uint32_t)bin << shift;
    fixed += 8;
    __syncthreads();
    if (cnt == nd) break;
  }
  const uint32_t bmask = fixed >= 32 ? ~0u : (~0u << (32 - fixed));
  const uint32_t top = pre | ~bmask;
  // list order, 4 entries per thread per tile of each part: a taken entry's
  // position counts the keys above the bin before it plus its rank among
  // the in-bin keys before it (only the first nd of those are taken)
  int a_before = 0, i_before = 0;
  for (int p = 0; p < nseg; ++p) {
    const int n = sh.seg_off[p + 1] - sh.seg_off[p];
    for (int t0 = 0; t0 < n; t0 += 4 * kWgThreads) {
      uint64_t e[4];
      uint32_t key[4];
      bool ok[4];
      int na = 0, ni = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int i = t0 + 4 * tid + k;
        ok[k] = i < n;
        e[k] = ok[k] ? lrow[(int64_t)p * kChunk + i] : 0ull;
        key[k] = order_key(__uint_as_float((uint32_t)e[k]));
        na += ok[k] && key[k] > top;
        ni += ok[k] && (key[k] & bmask) == pre;
      }
      int tot;
      const int pref = block_exclusive_scan<kWgThreads>(na | (ni << 16), sh.scan, &tot);
      int pa = a_before + (pref & 0xffff), pi = i_before + (pref >> 16);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if (!ok[k]) continue;
        int pos = -1;
        if (key[k] > top) {
          pos = pa + min(pi, nd);
          ++pa;
        } else if ((key[k] & bmask) == pre) {
          if (pi < nd) pos = pa + pi;
          ++pi;
        }
        if (pos >= 0) {
          orow[pos] = (int32_t)(e[k] >> 32);
          if (osc) osc[pos] = __uint_as_float((uint32_t)e[k]);
        }
      }
      a_before += tot & 0xffff;
      i_before += tot >> 16;
    }
  }
}

// The row's lists are loaded once, kFinPer entries per thread in list
// order (every address worked out from the LDS segment offsets first, so
// all loads are in flight together). The B-th key tau is found by bisection
// on the bits below the common prefix of t_lo and the row's largest key:
// each step counts the keys at or above a candidate with one ballot per
// register slot and one barrier. One prefix scan then writes the positions
// in ascending order, the lowest slots first among keys equal to tau.
__device__ __forceinline__ void select_row_exact(const StepArgs& a, FinShared& sh, int row, uint32_t* err,
                                                 float* keep_lds) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int B = a.B, nseg = a.wpr;
  const int4* meta = a.meta + (int64_t)row * nseg * kMetaStride;
  int cnt = 0;
  uint32_t km = 0u;
  if (tid < nseg) {
    const uint64_t lo = *(const uint64_t*)(meta + tid * kMetaStride);
    cnt = (int)(uint32_t)lo;
    km = (uint32_t)(lo >> 32);
  }
  const uint32_t t_lo = ((const uint32_t*)meta)[2];
  if (tid == 0) sh.kmax = 0u;
  int total;
  const int off = block_exclusive_scan<kWgThreads>(cnt, sh.scan, &total);
  if (tid < nseg) sh.seg_off[tid] = off;
  if (tid == 0) sh.seg_off[nseg] = total;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) km = max(km, (uint32_t)__shfl_xor((int)km, o, 64));
  if (lane == 0) atomicMax(&sh.kmax, km);
  __syncthreads();
  if (total < B) {   // cannot happen: the hints vouch for B keys >= t_lo
    if (tid == 0) __hip_atomic_fetch_or(err, 2u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  if (total > kFinCap) {
    select_lists_general(a, sh, row, total);
    return;
  }
  const int i0 = tid * kFinPer;
  const int nv = max(0, min(kFinPer, total - i0));   // this thread's valid entries
  const uint64_t* lrow = (const uint64_t*)(a.lists + (int64_t)row * nseg * kChunk);
  uint32_t key[kFinPer];
  {
    int addr[kFinPer];
    int sg = 0;
    if (nv > 0) {
      int lo = 0, hi = nseg - 1;   // last segment starting at or before i0
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (sh.seg_off[mid] <= i0) lo = mid; else hi = mid - 1;
      }
      sg = lo;
    }
    int next = sh.seg_off[sg + 1];
#pragma unroll
    for (int j = 0; j < kFinPer; ++j) {
      const int i = i0 + j;
      addr[j] = -1;
      if (j < nv) {
        while (next <= i) next = sh.seg_off[++sg + 1];
        addr[j] = sg * kChunk + (i - sh.seg_off[sg]);
      }
    }
#pragma unroll
    for (int j = 0; j < kFinPer; ++j) {
      const uint64_t e = addr[j] >= 0 ? lrow[addr[j]] : 0ull;
      key[j] = order_key(__uint_as_float((uint32_t)e));
    }
  }
  // tau = the largest t with at least B keys >= t. The keys share the
  // common prefix of t_lo and the row's largest key; one 256-bin LDS
  // histogram fixes the next 8 bits, the keys of the chosen bin (usually a
  // few hundred) are compacted into LDS, and bisection over their
  // remaining bits finishes it, each step one compare per entry, a ballot
  // and a barrier. A bin too big for the compaction is bisected in the
  // registers instead.
  const uint32_t kmax = sh.kmax;
  const int fixed = t_lo == kmax ? 32 : __clz(t_lo ^ kmax);
  uint32_t tau = fixed == 0 ? 0u : (t_lo & (~0u << (32 - fixed)));
  if (fixed < 32) {
    const int wA = min(8, 32 - fixed), shA = 32 - fixed - wA;
    const int nb = 1 << wA;
    sh.hist[tid] = 0u;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kFinPer; ++j)
      if (j < nv) atomicAdd(&sh.hist[(key[j] >> shA) & (uint32_t)(nb - 1)], 1u);
    __syncthreads();
    const int c = tid < nb ? (int)sh.hist[nb - 1 - tid] : 0;
    int tot;
    const int excl = block_exclusive_scan<kWgThreads>(c, sh.scan, &tot);
    if (tid < nb && excl < B && B <= excl + c) {
      sh.bin = nb - 1 - tid;
      sh.above = excl;
    }
    if (tid == 0) sh.ncomp = 0;
    __syncthreads();
    const uint32_t b1 = (uint32_t)sh.bin;
    const int need = B - sh.above;        // keys of the bin at or above tau
    const int c1 = (int)sh.hist[b1];
    tau |= b1 << shA;
    if (shA > 0) {
      const uint32_t top = tau >> shA;
      if (c1 <= kCompCap) {
        uint32_t* comp = (uint32_t*)keep_lds;
#pragma unroll
        for (int j = 0; j < kFinPer; ++j) {
          const bool in = j < nv && (key[j] >> shA) == top;
          const uint64_t bm = ballot64(in);
          if (bm == 0ull) continue;
          int base = 0;
          if (lane == 0) base = atomicAdd(&sh.ncomp, __popcll(bm));
          base = __shfl(base, 0, 64);
          if (in) comp[base + rank_below(bm)] = key[j];
        }
        __syncthreads();
        uint32_t ck[kCompCap / kWgThreads];
#pragma unroll
        for (int q = 0; q < kCompCap / kWgThreads; ++q) {
          const int i = tid + q * kWgThreads;
          ck[q] = i < c1 ? comp[i] : 0u;
        }
        for (int bit = shA - 1; bit >= 0; --bit) {
          const uint32_t cand = tau | (1u << bit);
          int cc = 0;
#pragma unroll
          for (int q = 0; q < kCompCap / kWgThreads; ++q)
            cc += __popcll(ballot64(tid + q * kWgThreads < c1 && ck[q] >= cand));
          if (lane == 0) sh.cnt[bit & 1][wid] = cc;
          __syncthreads();
          int tc = 0;
#pragma unroll
          for (int w = 0; w < kWgThreads / 64; ++w) tc += sh.cnt[bit & 1][w];
          if (tc >= need) tau = cand;
        }
      } else {
        for (int bit = shA - 1; bit >= 0; --bit) {
          const uint32_t cand = tau | (1u << bit);
          int cc = 0;
#pragma unroll
          for (int j = 0; j < kFinPer; ++j) cc += __popcll(ballot64(j < nv && key[j] >= cand));
          if (lane == 0) sh.cnt[bit & 1][wid] = cc;
          __syncthreads();
          int tc = 0;
#pragma unroll
          for (int w = 0; w < kWgThreads / 64; ++w) tc += sh.cnt[bit & 1][w];
          if (tc >= B) tau = cand;
        }
      }
    }
  }
  int na = 0, ni = 0;
#pragma unroll
  for (int j = 0; j < kFinPer; ++j) {
    na += j < nv && key[j] > tau;
    ni += j < nv && key[j] == tau;
  }
  int tot2;
  const int pref = block_exclusive_scan<kWgThreads>(na | (ni << 16), sh.scan, &tot2);
  const int nd = B - (tot2 & 0xffff);   // keys equal to tau that are taken
  int pa = pref & 0xffff, pi = pref >> 16;
  // each taken entry's position and list address, packed in one word (the
  // keys die as they go), then the taken entries are read again from the
  // lists kOutBatch at a time, all in flight together
  static_assert(kFinCap <= (1 << 14) && kChunk * kMaxParts <= (1 << 17), "position and address pack in 31 bits");
  int packed[kFinPer];
  {
    int sg = 0;
    if (nv > 0)
      while (sh.seg_off[sg + 1] <= i0) ++sg;
    int next = sh.seg_off[sg + 1];
#pragma unroll
    for (int j = 0; j < kFinPer; ++j) {
      const int i = i0 + j;
      packed[j] = -1;
      if (j >= nv) continue;
      while (next <= i) next = sh.seg_off[++sg + 1];
      int pos = -1;
      if (key[j] > tau) {
        pos = pa + min(pi, nd);
        ++pa;
      } else if (key[j] == tau) {
        if (pi < nd) pos = pa + pi;
        ++pi;
      }
      if (pos >= 0) packed[j] = (pos << 17) | (sg * kChunk + (i - sh.seg_off[sg]));
    }
  }
  int32_t* orow = a.out_idx + (int64_t)row * B;
  float* osc = a.out_score ? a.out_score + (int64_t)row * B : nullptr;
  constexpr int kOutBatch = 16;
#pragma unroll
  for (int j0 = 0; j0 < kFinPer; j0 += kOutBatch) {
    uint64_t e[kOutBatch];
#pragma unroll
    for (int jj = 0; jj < kOutBatch; ++jj)
      e[jj] = packed[j0 + jj] >= 0 ? lrow[packed[j0 + jj] & 0x1ffff] : 0ull;
#pragma unroll
    for (int jj = 0; jj < kOutBatch; ++jj) {
      const int pk = packed[j0 + jj];
      if (pk < 0) continue;
      orow[pk >> 17] = (int32_t)(e[jj] >> 32);
      if (osc) osc[pk >> 17] = __uint_as_float((uint32_t)e[jj]);   // the score's own bits
    }
  }
}

// ---------------------------------------------------------------------------
// 3. attention over this workgroup's share of the row's list: a partial
// (max m, sum l, output o; log2 domain) per query head
// ---------------------------------------------------------------------------
template <bool BF16>
__device__ __forceinline__ void load_ch2(const void* base, int64_t off, bool ok, float& x0, float& x1) {
  // channels 2 * lane and 2 * lane + 1 of one row; a skipped entry reads
  // row 0 and is masked
  if constexpr (BF16) {
    const uint32_t w = *((const uint32_t*)((const uint16_t*)base + (ok ? off : 0)) + threadIdx.x % 64);
    x0 = bf16_lo(w);
    x1 = bf16_hi(w);
  } else {
    const float2 v = *((const float2*)((const float*)base + (ok ? off : 0)) + threadIdx.x % 64);
    x0 = v.x;
    x1 = v.y;
  }
}

template <bool BF16, int G>
__device__ __forceinline__ void attend_part(const StepArgs& a, AttnShared& sh, int row, int part) {
  // list entries per wave per batch: with four or fewer heads a wave holds
  // 16 K and V rows at once (a part of 64 entries is one round trip)
  constexpr int KB = G <= 4 ? 2 * kBatch : kBatch;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int n = row / a.Hkv, g = row % a.Hkv;
  const int B = a.B;
  const int per = (B + a.wpr - 1) / a.wpr;
  const int e0 = part * per, e1 = min(B, e0 + per);
  const int ne = max(0, e1 - e0);
  const int32_t* irow = a.out_idx + (int64_t)row * B;
  // the part's list entries (written by another workgroup of the row)
  for (int i = tid; i < ne; i += kWgThreads) sh.idx[i] = irow[e0 + i];
  // this lane's two channels of each of the group's query heads
  float q0[G], q1[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const int64_t qo = ((int64_t)n * a.Hq + (int64_t)g * G + h) * kD;
    load_ch2<BF16>(a.q, qo, true, q0[h], q1[h]);
  }
  __syncthreads();
  const int64_t kv0 = (int64_t)n * a.kv_s_seq + (int64_t)g * a.kv_s_head;
  float m[G], l[G], o0[G], o1[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
    o0[h] = 0.f;
    o1[h] = 0.f;
  }
  // wave wid takes batches wid, wid + 4, ... of KB entries
  for (int b0 = wid * KB; b0 < ne; b0 += 4 * KB) {
    float k0[KB], k1[KB], v0[KB], v1[KB];
    bool ok[KB];
#pragma unroll
    for (int i = 0; i < KB; ++i) {
      const int t = b0 + i < ne ? sh.idx[b0 + i] : -1;
      ok[i] = t >= 0 && t < a.T;
      const int64_t off = kv0 + (int64_t)t * a.kv_s_tok;
      load_ch2<BF16>(a.k, off, ok[i], k0[i], k1[i]);
      load_ch2<BF16>(a.v, off, ok[i], v0[i], v1[i]);
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float z[KB];
      float mb = -INFINITY;
#pragma unroll
      for (int i = 0; i < KB; ++i) {
        float s = sum_lanes<16>(fmaf(q0[h], k0[i], q1[h] * k1[i]));
        s += __shfl_xor(s, 16, 64);
        s += __shfl_xor(s, 32, 64);
        z[i] = ok[i] ? s * a.scale_log2 : -INFINITY;
        mb = fmaxf(mb, z[i]);
      }
      const float mn = fmaxf(m[h], mb);
      if (mn == -INFINITY) continue;   // nothing valid yet for this head
      const float f = exp2f(m[h] - mn);   // 0 when m was -inf
      l[h] *= f;
      o0[h] *= f;
      o1[h] *= f;
#pragma unroll
      for (int i = 0; i < KB; ++i) {
        const float pz = exp2f(z[i] - mn);
        l[h] += pz;
        o0[h] = fmaf(pz, v0[i], o0[h]);
        o1[h] = fmaf(pz, v1[i], o1[h]);
      }
      m[h] = mn;
    }
  }
  // combine the four waves into the workgroup's partial
#pragma unroll
  for (int h = 0; h < G; ++h) {
    if (lane == 0) {
      sh.m[wid][h] = m[h];
      sh.l[wid][h] = l[h];
    }
    sh.o[wid][h][2 * lane] = o0[h];
    sh.o[wid][h][2 * lane + 1] = o1[h];
  }
  __syncthreads();
  float* pbase = a.partial + ((int64_t)row * a.wpr + part) * partial_stride(G);
  for (int e = tid; e < G * kD; e += kWgThreads) {
    const int h = e / kD, c = e % kD;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, sh.m[w][h]);
    float L = 0.f, O = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float f = exp2f(sh.m[w][h] - M);
        L = fmaf(sh.l[w][h], f, L);
        O = fmaf(sh.o[w][h][c], f, O);
      }
    }
    float* ph = pbase + h * (kD + 2);
    ph[2 + c] = O;
    if (c == 0) {
      ph[0] = M;
      ph[1] = L;
    }
  }
}

// Merge of the row's partials by log-sum-exp into out and lse.
template <int G>
__device__ __forceinline__ void merge_row(const StepArgs& a, AttnShared& sh, int row) {
  const int tid = threadIdx.x;
  const int n = row / a.Hkv, g = row % a.Hkv;
  const int P = a.wpr;
  const float* base = a.partial + (int64_t)row * P * partial_stride(G);
  for (int e = tid; e < P * G; e += kWgThreads) {
    const int p = e / G, h = e % G;
    sh.w[p][h] = base[(int64_t)p * partial_stride(G) + h * (kD + 2)];
  }
  __syncthreads();
  if (tid < G) {
    float M = -INFINITY;
    for (int p = 0; p < P; ++p) M = fmaxf(M, sh.w[p][tid]);
    sh.mstar[tid] = M;
  }
  __syncthreads();
  for (int e = tid; e < P * G; e += kWgThreads) {
    const int p = e / G, h = e % G;
    const float M = sh.mstar[h];
    sh.w[p][h] = M == -INFINITY ? 0.f : exp2f(sh.w[p][h] - M);
  }
  __syncthreads();
  // thread (h, c): c < kD the head's output channel, c == kD its sum; the
  // parts' values are loaded all at once
  for (int e = tid; e < G * (kD + 1); e += kWgThreads) {
    const int h = e / (kD + 1), c = e % (kD + 1);
    const float* col = base + h * (kD + 2) + (c == kD ? 1 : 2 + c);
    float x[kMaxParts];
#pragma unroll
    for (int q = 0; q < kMaxParts; ++q) x[q] = q < P ? col[(int64_t)q * partial_stride(G)] : 0.f;
    float acc = 0.f;
#pragma unroll
    for (int q = 0; q < kMaxParts; ++q)
      if (q < P) acc = fmaf(sh.w[q][h], x[q], acc);
    if (c == kD) sh.l[0][h] = acc;
    else sh.o[0][h][c] = acc;
  }
  __syncthreads();
  const float kLn2 = 0.69314718055994531f;
  for (int e = tid; e < G * kD; e += kWgThreads) {
    const int h = e / kD, c = e % kD;
    const float L = sh.l[0][h];
    const int64_t oh = (int64_t)n * a.Hq + (int64_t)g * G + h;
    a.out[oh * kD + c] = L > 0.f ? sh.o[0][h][c] / L : 0.f;
    if (c == 0 && a.lse) a.lse[oh] = L > 0.f ? (sh.mstar[h] + log2f(L)) * kLn2 : -INFINITY;
  }
}

// The last workgroup out clears the launch-wide words (tickets, count)
// for the next launch; the error word stays set for the caller to read.
__device__ __forceinline__ void finish_launch(const StepArgs& a) {
  if (threadIdx.x == 0) {
    uint32_t* const ctl = a.ctrl;
    if (add_c(ctl + kCtlDone, 1u) == gridDim.x - 1u) {
      for (int i = 0; i < 8; ++i) st_c(ctl + kCtlQueue + i, 0u);
      st_c(ctl + kCtlDone, 0u);
    }
  }
}

// ---------------------------------------------------------------------------
template <int DT, int LPK, bool BF16, int G>
__global__ __launch_bounds__(kWgThreads, LSA_STEP_WG_PER_CU) void decode_step_kernel(StepArgs a) {
  __shared__ StepShared sh;
  constexpr int KPI = kWave / LPK;
  constexpr uint64_t kColumn = LPK == 8 ? 0x0101010101010101ull : 0x1111111111111111ull;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  uint32_t* const ctl = a.ctrl;
  uint32_t* const err = ctl + kCtlErr;
  // this workgroup's (row, part), from its XCD's queue: of nxcc XCDs, XCD x
  // serves rows x, x + nxcc, ..., so all of a row's workgroups share one L2
  const int nx = a.nxcc;
  const int x = (int)(xcd_id() % (unsigned)nx);
  if (tid == 0) sh.flag = (int)add_c(ctl + kCtlQueue + x, 1u);
  __syncthreads();
  const int ticket = __builtin_amdgcn_readfirstlane(sh.flag);
  const int nr = x < a.rows ? (a.rows - x + nx - 1) / nx : 0;
  __syncthreads();
  if (ticket >= nr * a.wpr) {   // more workgroups landed on this XCD than it has work
    finish_launch(a);
    return;
  }
  const int row = x + nx * (ticket / a.wpr), part = ticket % a.wpr;
  uint32_t* const rc = ctl + kCtlRow0 + row * kCtlPerRow;
  const int64_t c0 = (int64_t)part * kChunk;
  const int64_t c1 = min((int64_t)a.sc.n_out, c0 + kChunk);

  // ---- scoring (the unchanged stream), keeping the scores in LDS ----
  score_chunk<DT, LPK, false, true, kSteps, false>(a.sc, row, c0, c1, sh.score, true, sh.keep);
  all_done();

  // ---- 1. threshold: the row's last scorer derives it from the hints ----
  if (tid == 0) sh.flag = add_l(rc + kRowScored, 1u) == (uint32_t)a.wpr - 1u;
  __syncthreads();
  if (__builtin_amdgcn_readfirstlane(sh.flag)) {
    const uint32_t t = row_threshold(a.sc.hint + (int64_t)row * a.sc.hint_ld, a.hint_count, a.hint_k, a.B,
                                     sh.u.seg);
    // the threshold's low 16 bits are zero: bit 0 marks the word as set
    if (tid == 0) add_l(rc + kRowThr, t | 1u);
    if (tid == 0) sh.wval = (int)t;
    __syncthreads();
  } else {
    wait_until(rc + kRowThr, 1u, err, &sh.wval);
  }
  const uint32_t t_lo = __builtin_amdgcn_readfirstlane((uint32_t)sh.wval) & ~0xffffu;

  // ---- 2. collect from LDS: keys >= t_lo, in slot order ----
  {
    const int l = lane % LPK;
    // lanes of column b (lane % LPK == b) hold slots b * KPI + lane / LPK of
    // a 64-slot group, so a lane's rank in slot order counts the taken lanes
    // of the lower columns and the lower taken lanes of its own column
    const uint64_t colmask = kColumn << l;
    // the ballot of group (s, u): which lanes take their slot (computed again
    // when the entries are written, rather than held in registers)
    auto taken = [&](int s, int u, uint32_t* key_out) {
      const int64_t slot = c0 + (int64_t)s * kWgStep + u * 256 + wid * 64 + l * KPI + lane / LPK;
      const uint32_t key = order_key(sh.keep[(s * kGroups + u) * kWgThreads + tid]);
      *key_out = key;
      return slot < c1 && (t_lo == 0u || key >= t_lo);
    };
    uint32_t kmax = 0u;
#pragma unroll
    for (int s = 0; s < kSteps; ++s)
#pragma unroll
      for (int u = 0; u < kGroups; ++u) {
        uint32_t key;
        const bool take = taken(s, u, &key);
        const uint64_t bm = ballot64(take);
        if (take) kmax = max(kmax, key);
        if (lane == 0) sh.u.col.cnt[s * 8 + u * 4 + wid] = __popcll(bm);
      }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o, 64));
    if (lane == 0) sh.u.col.wmax[wid] = kmax;
    __syncthreads();
    if (wid == 0) {   // groups in slot order: (step, u, wave)
      const int c = sh.u.col.cnt[lane];
      int v = c;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(v, o, 64);
        if (lane >= o) v += y;
      }
      sh.u.col.off[lane] = v - c;
      if (lane == 63) sh.u.col.total = v;
    }
    __syncthreads();
    uint64_t* lout = (uint64_t*)(a.lists + ((int64_t)row * a.wpr + part) * kChunk);
#pragma unroll
    for (int s = 0; s < kSteps; ++s)
#pragma unroll
      for (int u = 0; u < kGroups; ++u) {
        uint32_t key;
        const uint64_t bm = ballot64(taken(s, u, &key));
        if (!((bm >> lane) & 1ull)) continue;
        int rank = rank_below(bm & colmask);
#pragma unroll
        for (int b = 0; b < LPK; ++b)
          if (b < l) rank += __popcll(bm & (kColumn << b));
        const int64_t slot = c0 + (int64_t)s * kWgStep + u * 256 + wid * 64 + l * KPI + lane / LPK;
        const int pos = sh.u.col.off[s * 8 + u * 4 + wid] + rank;
        lout[pos] = (((uint64_t)(uint32_t)slot << 32) |
                     __float_as_uint(sh.keep[(s * kGroups + u) * kWgThreads + tid]));
      }
    if (tid == 0) {
      uint32_t km = sh.u.col.wmax[0];
#pragma unroll
      for (int w = 1; w < 4; ++w) km = max(km, sh.u.col.wmax[w]);
      uint64_t* mt = (uint64_t*)(a.meta + ((int64_t)row * a.wpr + part) * kMetaStride);
      mt[0] = ((uint64_t)km << 32) | (uint32_t)sh.u.col.total;
      mt[1] = (uint64_t)t_lo;
    }
  }
  all_done();
  if (tid == 0) sh.flag = add_l(rc + kRowCollected, 1u) == (uint32_t)a.wpr - 1u;
  __syncthreads();
  if (__builtin_amdgcn_readfirstlane(sh.flag)) {
    select_row_exact(a, sh.u.fin, row, err, sh.keep);   // the scores kept in LDS are spent
    all_done();
    if (tid == 0) add_l(rc + kRowSelected, 1u);
  } else {
    wait_until(rc + kRowSelected, 1u, err, &sh.wval);
  }

  // ---- 3. attention over this workgroup's share of the row's positions ----
  attend_part<BF16, G>(a, sh.u.att, row, part);
  all_done();
  if (tid == 0) sh.flag = add_l(rc + kRowAttended, 1u) == (uint32_t)a.wpr - 1u;
  __syncthreads();
  if (__builtin_amdgcn_readfirstlane(sh.flag)) {
    merge_row<G>(a, sh.u.att, row);
    // every workgroup of the row is past its last use of the row's words:
    // clear them here, in the L2 that holds them, for the next launch
    if (tid < 6) rc[tid] = 0u;
  }
  finish_launch(a);
}

template <int DT, int LPK, bool BF16>
hipError_t launch_g(const StepArgs& a, hipStream_t s) {
  // workgroups are dealt to the XCDs in turn: nxcc equal shares
  const dim3 grid((unsigned)(a.nxcc * ((a.rows + a.nxcc - 1) / a.nxcc) * a.wpr));
  switch (a.Hq / a.Hkv) {
    case 1: hipLaunchKernelGGL((decode_step_kernel<DT, LPK, BF16, 1>), grid, dim3(kWgThreads), 0, s, a); break;
    case 2: hipLaunchKernelGGL((decode_step_kernel<DT, LPK, BF16, 2>), grid, dim3(kWgThreads), 0, s, a); break;
    case 4: hipLaunchKernelGGL((decode_step_kernel<DT, LPK, BF16, 4>), grid, dim3(kWgThreads), 0, s, a); break;
    case 8: hipLaunchKernelGGL((decode_step_kernel<DT, LPK, BF16, 8>), grid, dim3(kWgThreads), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

int step_ctrl_words(int rows) { return kCtlRow0 + kCtlPerRow * rows; }
int step_ctrl_row0() { return kCtlRow0; }
int step_ctrl_per_row() { return kCtlPerRow; }
int step_chunk_slots() { return kChunk; }

bool decode_step_supported(int rows, int n, int B, int r, int k_dt, int kv_dt, int G, int d, int hint_count,
                           int hint_k_) {
  const int esz = k_dt == 2 ? 1 : k_dt == 1 ? 2 : 4;
  const int lpk = r * esz / 16;
  if ((k_dt != 1 && k_dt != 2) || (lpk != 4 && lpk != 8)) return false;
  if (kv_dt != 0 && kv_dt != 1) return false;
  if (d != kD || (G != 1 && G != 2 && G != 4 && G != 8)) return false;
  const int64_t wpr = ((int64_t)n + kChunk - 1) / kChunk;
  if (wpr > kMaxParts || rows < 1 || (int64_t)rows * wpr > (1 << 20)) return false;
  if ((int64_t)B > (int64_t)wpr * kWgThreads) return false;      // a part's entries fit the LDS list
  if ((int64_t)hint_count * hint_k_ < B) return false;        // the hints vouch for B keys
  // whole 128-byte lines of selected positions per row (one writer each)
  if (B % 32 != 0) return false;
  return B <= kFinCap && B <= n;
}

int step_meta_stride() { return kMetaStride; }
int step_partial_stride(int G) { return partial_stride(G); }

hipError_t launch_decode_step(const StepArgs& a, int k_dt, hipStream_t s) {
  if (a.nxcc < 1 || a.nxcc > 8) return hipErrorInvalidValue;
  const int esz = k_dt == 2 ? 1 : 2;
  const int lpk = a.sc.r * esz / 16;
  if (k_dt == 1 && lpk == 8) return a.kv_bf16 ? launch_g<1, 8, true>(a, s) : launch_g<1, 8, false>(a, s);
  if (k_dt == 1 && lpk == 4) return a.kv_bf16 ? launch_g<1, 4, true>(a, s) : launch_g<1, 4, false>(a, s);
  if (k_dt == 2 && lpk == 4) return a.kv_bf16 ? launch_g<2, 4, true>(a, s) : launch_g<2, 4, false>(a, s);
  if (k_dt == 2 && lpk == 8) return a.kv_bf16 ? launch_g<2, 8, true>(a, s) : launch_g<2, 8, false>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace lsa
