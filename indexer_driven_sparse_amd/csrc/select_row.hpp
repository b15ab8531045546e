// Exact top-B selection of one row by one workgroup: the device code shared
// by the select kernels and the causal prefill fallback. Included by one
// translation unit each (device code is not linked across them).
#pragma once

#include "common.hpp"
#include "kernels.hpp"
#include "score_body.hpp"

namespace lsa {
namespace sel {


constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kBins = 2048;
constexpr int kCap = 8192;          // LDS candidate list
constexpr int kSampleBlocks = 64;   // fast-path sample: blocks ...
constexpr int kSampleBlock = 128;   // ... of contiguous slots
constexpr int kUnroll = 8;          // 128-bit loads in flight per thread (general path)
constexpr int kCollectUnroll = 8;   // ... in the fast path's collect pass

struct SelShared {
  uint32_t hist[kBins];
  uint32_t ckey[kCap];
  int32_t cslot[kCap];
  int scan[kWaves + 1];
  int ncand;
  int nsample;
  uint32_t kmax;
  int wval[kWaves];   // per-wave values (sample counts, thresholds)
  int bin;      // result of find_bin
  int above;    // keys in higher bins
};

template <bool CAND>
__device__ __forceinline__ bool slot_ok(const SelectArgs& a, const int32_t* crow, int64_t slot,
                                        int64_t nv) {
  if (slot >= nv) return false;
  if constexpr (!CAND) {
    return true;
  } else {
    int32_t c = crow[slot / a.cand_block];
    if (c < 0) return false;
    int64_t p = (int64_t)c * a.cand_block + slot % a.cand_block;
    return p < a.n_positions;
  }
}

template <bool CAND>
__device__ __forceinline__ int32_t slot_pos(const SelectArgs& a, const int32_t* crow, int64_t slot) {
  if constexpr (!CAND) {
    return (int32_t)slot;
  } else {
    return crow[slot / a.cand_block] * a.cand_block + (int32_t)(slot % a.cand_block);
  }
}

// Four consecutive slots [s0, s0+4): order keys and validity bits. FULL:
// the caller knows s0 + 3 < nv, so the 128-bit load is unconditional and
// several of them issue back to back; otherwise each slot is guarded.
template <bool CAND, bool FULL = false>
__device__ __forceinline__ void load4(const SelectArgs& a, const float* srow, const int32_t* crow,
                                      int64_t s0, int64_t nv, uint32_t key[4], bool ok[4]) {
  float v[4];
  if (FULL || s0 + 3 < nv) {
    const float4 x = *(const float4*)(srow + s0);
    v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = srow[min(s0 + k, nv - 1)];
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    ok[k] = slot_ok<CAND>(a, crow, s0 + k, nv);
    key[k] = order_key(v[k]);
  }
}

// The 32-bit bitmap word of 32 consecutive slots held 4 per lane by 8
// consecutive lanes: every lane contributes a nibble, OR-combined with DPP.
// All 8 lanes of the group must be active.
__device__ __forceinline__ uint32_t word_from_nibbles(uint32_t nib, int lane) {
  uint32_t w = nib << (4 * (lane & 7));
  w |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)w, kDppXor1, 0xf, 0xf, false);
  w |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)w, kDppXor2, 0xf, 0xf, false);
  w |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)w, kDppHalfMirror, 0xf, 0xf, false);
  return w;
}

// Find the bin holding the need-th largest key: the highest bin b with
// (count above b) < need <= (count above b) + hist[b], for nb <= 2048 bins.
// Writes sh.bin / sh.above (left unchanged when the total is below need)
// and returns the total through *total. Contains barriers.
__device__ __forceinline__ void find_bin(SelShared& sh, const uint32_t* hist, int nb, int need,
                                         int* total) {
  const int t = threadIdx.x;
  const int per = (nb + kThreads - 1) / kThreads;
  const int hi = nb - 1 - t * per;
  int c = 0;
  for (int k = 0; k < per; ++k)
    if (hi - k >= 0) c += (int)hist[hi - k];
  int tot;
  const int above = block_exclusive_scan<kThreads>(c, sh.scan, &tot);
  int acc = above;
  for (int k = 0; k < per; ++k) {
    if (hi - k < 0) break;
    const int h = (int)hist[hi - k];
    if (acc < need && need <= acc + h) {
      sh.bin = hi - k;
      sh.above = acc;
    }
    acc += h;
  }
  *total = tot;
  __syncthreads();
}

__device__ __forceinline__ void zero_hist(SelShared& sh) {
  for (int i = threadIdx.x; i < kBins; i += kThreads) sh.hist[i] = 0u;
}

// Append this lane's flagged slots (their order keys and slot numbers) to
// the LDS list with one LDS atomic per wave; the lane then walks only its
// set flag bits. Item i = 4*j + k of a lane holds slot first + j*kThreads*4
// + k. Entries past kCap are dropped while the count still grows, so the
// caller sees the overflow. All 64 lanes of the wave must call it.
template <int M>
__device__ __forceinline__ void wave_append(SelShared& sh, const float* val, int64_t first,
                                            uint32_t flags, int lane) {
  const int mine = __popc(flags);
  int incl = mine;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  const int total = __shfl(incl, 63, 64);
  if (total == 0) return;
  int base = 0;
  if (lane == 63) base = atomicAdd(&sh.ncand, total);
  base = __shfl(base, 63, 64) + incl - mine;
  while (flags) {
    const int i = __ffs(flags) - 1;
    flags &= flags - 1;
    if (base < kCap) {
      float v = val[0];
#pragma unroll
      for (int q = 1; q < M; ++q) v = q == i ? val[q] : v;   // register select, no local memory
      sh.ckey[base] = order_key(v);
      sh.cslot[base] = (int32_t)(first + (int64_t)(i / 4) * kThreads * 4 + (i % 4));
    }
    ++base;
  }
}

// Exact refine of an LDS list whose keys all lie in [lo, hi]: radix levels
// of up to 11 bits below the common prefix of lo and hi, each a block-wide
// histogram of the listed keys that match the prefix so far. On return tau
// is the need-th largest listed key, *need the number of keys equal to tau
// to take and *ties the number of listed keys equal to tau. Contains
// barriers.
__device__ __forceinline__ uint32_t refine_list(SelShared& sh, int ncand, uint32_t lo, uint32_t hi,
                                                int* need, int* ties) {
  int fixed = lo == hi ? 32 : __clz(lo ^ hi);
  uint32_t tau = fixed == 0 ? 0u : (lo & (~0u << (32 - fixed)));
  int nd = *need;
  int eq = ncand;   // with no level, every listed key equals tau
  while (fixed < 32) {
    const int width = min(11, 32 - fixed);
    const int shift = 32 - fixed - width;
    const uint32_t pmask = fixed == 0 ? 0u : (~0u << (32 - fixed));
    const int nb = 1 << width;
    zero_hist(sh);
    __syncthreads();
    for (int i = threadIdx.x; i < ncand; i += kThreads) {
      const uint32_t key = sh.ckey[i];
      if ((key & pmask) == tau) atomicAdd(&sh.hist[(key >> shift) & (nb - 1)], 1u);
    }
    __syncthreads();
    int tl;
    find_bin(sh, sh.hist, nb, nd, &tl);
    const int bin = sh.bin;
    nd -= sh.above;
    eq = (int)sh.hist[bin];
    tau |= (uint32_t)bin << shift;
    fixed += width;
    __syncthreads();   // hist and bin are rewritten by the next level
  }
  *need = nd;
  *ties = eq;
  return tau;
}

constexpr int kSegThreads = 256;
constexpr int kSegWaves = kSegThreads / 64;
constexpr int kSegUnroll = 8;
constexpr int kSeg = kSegThreads * 4 * kSegUnroll;   // 8192 slots
constexpr int kSegUnits = kSegUnroll * kSegWaves;    // (loop step, wave) units, in slot order

// The scores of slots [0, nv) of a row recomputed into srow with the
// scoring kernels' arithmetic: each 16-byte piece of the key dotted with
// its q_idx channels (scoring::dot16), the P pieces summed pairwise in the
// tree the scoring kernels' lane sums form (((p0+p1)+(p2+p3))+...), so
// every score is bit-identical to the scoring launch's. The whole
// workgroup calls it; the scores are complete and visible to the
// workgroup on return.
template <int DT, int P>
__device__ __forceinline__ void rescore_row_t(const SelectArgs& a, int row, float* srow, int64_t nv,
                                              const float* sq) {
  constexpr int ESZ = DT == 2 ? 1 : DT == 1 ? 2 : 4;
  constexpr int E = 16 / ESZ;
  static_assert(P % 4 == 0 && P <= 16, "4, 8 or 16 pieces");
  const int n = row / a.rs_Hkv, g = row % a.rs_Hkv;
  const char* base = (const char*)a.rs_k_idx + ((int64_t)n * a.rs_ks_seq + (int64_t)g * a.rs_ks_head) * ESZ;
  const int32_t* crow = a.cand ? a.cand + (int64_t)row * a.cand_ld : nullptr;
#pragma unroll 1
  for (int64_t t = threadIdx.x; t < nv; t += kThreads) {
    // q_idx is read from LDS for every key: held in registers across the
    // loop, its up to 128 values would crowd the whole kernel into spills
    asm volatile("" ::: "memory");
    int64_t pos = t;   // slot t's position (through the candidate map), or -1
    if (crow) {
      const int32_t c = crow[t / a.cand_block];
      pos = c < 0 ? -1 : (int64_t)c * a.cand_block + t % a.cand_block;
      if (pos >= a.n_positions) pos = -1;
    }
    if (pos < 0) {   // a slot that covers no token scores -inf, as in the scoring kernels
      srow[t] = -INFINITY;
      continue;
    }
    const char* kr = base + pos * a.rs_ks_tok * ESZ;
    // pieces four at a time: ((p0+p1)+(p2+p3)) per group, then the groups
    // pairwise -- the same tree as pairwise over all P pieces
    float grp[P / 4];
#pragma unroll
    for (int q = 0; q < P / 4; ++q) {
      float d[4];
#pragma unroll
      for (int l = 0; l < 4; ++l)
        d[l] = scoring::dot16<DT>(*(const uint4*)(kr + 16 * (4 * q + l)), sq + (4 * q + l) * E);
      grp[q] = (d[0] + d[1]) + (d[2] + d[3]);
    }
    float v = grp[0];
    if constexpr (P == 8) v = grp[0] + grp[1];
    if constexpr (P == 16) v = (grp[0] + grp[1]) + (grp[2] + grp[3]);
    srow[t] = v;
  }
}

__device__ __forceinline__ void rescore_row(const SelectArgs& a, int row, float* srow, int64_t nv) {
  __shared__ float sq[scoring::kMaxR];
  for (int c = threadIdx.x; c < a.rs_r; c += kThreads) sq[c] = a.rs_q_idx[(int64_t)row * a.rs_r + c];
  __syncthreads();
  const int esz = a.rs_dt == 2 ? 1 : a.rs_dt == 1 ? 2 : 4;
  const int P = a.rs_r * esz / 16;
  if (a.rs_dt == 2) {
    if (P == 4) rescore_row_t<2, 4>(a, row, srow, nv, sq);
    else if (P == 8) rescore_row_t<2, 8>(a, row, srow, nv, sq);
    else if (P == 16) rescore_row_t<2, 16>(a, row, srow, nv, sq);
  } else if (a.rs_dt == 1) {
    if (P == 4) rescore_row_t<1, 4>(a, row, srow, nv, sq);
    else if (P == 8) rescore_row_t<1, 8>(a, row, srow, nv, sq);
    else if (P == 16) rescore_row_t<1, 16>(a, row, srow, nv, sq);
  } else {
    if (P == 4) rescore_row_t<0, 4>(a, row, srow, nv, sq);
    else if (P == 8) rescore_row_t<0, 8>(a, row, srow, nv, sq);
    else if (P == 16) rescore_row_t<0, 16>(a, row, srow, nv, sq);
  }
  // every store is complete before any thread of the workgroup reads the
  // row (the lines were never read in this launch, so no L1 copy is stale)
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
}

// One row of the selection, run by a whole kThreads-thread workgroup.
// `row` indexes the outputs (out_idx, out_score, out_count), the workspace
// bitmaps (GBM), the candidate map and the segment lists (PRE); srow holds
// the row's scores and nv its valid length. smem_raw: sizeof(SelShared),
// plus two bitmaps of n bits when !GBM.
// Exact top-B of `total` (>= B) entries held in registers: thread t holds
// entries i0 .. i0 + kPer - 1 (i0 = t * kPer) of a list in slot order, every
// key of the list is >= t_lo and the largest is kmax. Radix levels of up to
// 11 bits run below the common prefix of [t_lo, kmax] and stop as soon as
// the B-th key's bin is taken whole; then the taken entries -- keys above
// the bin and the first `nd` keys inside it, in slot order -- are written
// in slot order with one packed prefix scan. Writes out_idx, out_score and
// out_count (B). Every thread of the block must call it.
// Most listed keys the value-bin refine ranks directly.
constexpr int kRankCap = 1024;

// The exact top-B of entries held in registers (as select_in_registers
// below), in one pass when the keys spread out: the entries are binned by
// value, bin(v) = floor((v - vlo) * 2048 / (vhi - vlo)) over [vlo, vhi] =
// the values of [t_lo, kmax]. That map never decreases with v, and equal
// values (+0 and -0 too) share a bin, so every key of a higher bin is
// larger than every key of a lower one; 2048 bins over the values' range
// hold a few keys each where the top 11 key bits (sign and exponent) would
// put most keys in a handful of bins. The B-th key's bin is found from the
// histogram; its entries are ranked exactly (key descending, then slot
// ascending) by comparing each with every other, and the rest of the
// selection is every key of a higher bin. Returns false, with the
// histograms zeroed again and nothing written, where it does not apply:
// a NaN or infinite bound, a bin of more than kRankCap entries, or fewer
// than B entries in the bins. Every thread of the block must call it.
template <bool CAND, int kPer>
__device__ __forceinline__ bool select_by_value_bins(const SelectArgs& a, SelShared& sh, int row,
                                                     const int32_t* crow, const uint32_t (&key)[kPer],
                                                     const float (&val)[kPer], const int32_t (&slot)[kPer],
                                                     int i0, int total, uint32_t t_lo, uint32_t kmax) {
  const int tid = threadIdx.x;
  const int B = a.B;
  // Measured on gfx950: one pass over value bins beats the radix levels
  // when B is a small share of the entries (8 rows of 16384 at top-128:
  // 11.5 against 14.6 us), and loses where it is not (3700 listed keys to
  // 2048: 14.0 against 11.8 us; 8192 to 2048: 21.1 against 19.2 us).
  if ((int64_t)B * 16 > total) return false;
  if (t_lo == 0u || kmax <= t_lo) return false;   // a NaN bound, or every key equal
  const float vlo = key_to_float(t_lo), vhi = key_to_float(kmax);
  const float scale = (float)kBins / (vhi - vlo);
  if (!__builtin_isfinite(vlo) || !__builtin_isfinite(vhi) || !(scale > 0.f) || !__builtin_isfinite(scale))
    return false;
  int bin[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    bin[j] = -1;   // past the list, or a NaN (below every bin)
    if (i0 + j < total && key[j] != 0u) {
      bin[j] = min(kBins - 1, (int)((val[j] - vlo) * scale));
      atomicAdd(&sh.hist[bin[j]], 1u);
    }
  }
  if (tid == 0) {
    sh.ncand = 0;
    sh.bin = 0;   // left as is when the bins hold fewer than B entries
    sh.above = 0;
  }
  __syncthreads();
  int tot;
  find_bin(sh, sh.hist, kBins, B, &tot);
  const int b = sh.bin;
  const int nd = B - sh.above;
  const int cnt_b = (int)sh.hist[b];
  const bool ok = tot >= B && cnt_b <= kRankCap;
  __syncthreads();   // hist and bin are read above
  if (!ok) {
    for (int i = tid; i < kBins; i += kThreads) sh.hist[i] = 0u;
    __syncthreads();
    return false;
  }
  // the B-th key's bin: its entries to LDS, then each ranked against all
  uint32_t take = 0;   // bit j: entry j is selected
  if (cnt_b == nd) {
#pragma unroll
    for (int j = 0; j < kPer; ++j) take |= (uint32_t)(bin[j] >= b) << j;
  } else {
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      if (bin[j] == b) {
        const int k = atomicAdd(&sh.ncand, 1);
        sh.ckey[k] = key[j];
        sh.cslot[k] = slot[j];
      }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      if (bin[j] > b) {
        take |= 1u << j;
      } else if (bin[j] == b) {
        int rank = 0;
        for (int k = 0; k < cnt_b; ++k) {
          const uint32_t kk = sh.ckey[k];
          rank += kk > key[j] || (kk == key[j] && sh.cslot[k] < slot[j]);
        }
        take |= (uint32_t)(rank < nd) << j;
      }
    }
  }
  // ascending positions: the taken entries in list (slot) order
  int tot2;
  const int pos0 = block_exclusive_scan<kThreads>(__popc(take), sh.scan, &tot2);
  int32_t* orow = a.out_idx + (int64_t)row * B;
  float* osc = a.out_score ? a.out_score + (int64_t)row * B : nullptr;
  int pos = pos0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    if ((take >> j) & 1u) {
      orow[pos] = slot_pos<CAND>(a, crow, slot[j]);
      if (osc) osc[pos] = val[j];
      ++pos;
    }
  }
  if (tid == 0 && a.out_count) a.out_count[row] = B;
  return true;
}

template <bool CAND, int kPer>
__device__ __forceinline__ void select_in_registers(const SelectArgs& a, SelShared& sh, int row,
                                                    const int32_t* crow, const uint32_t (&key)[kPer],
                                                    const float (&val)[kPer], const int32_t (&slot)[kPer],
                                                    int i0, int total, uint32_t t_lo, uint32_t kmax) {
  if (select_by_value_bins<CAND, kPer>(a, sh, row, crow, key, val, slot, i0, total, t_lo, kmax)) return;
  const int tid = threadIdx.x;
  const int B = a.B;
  int fixed = t_lo == kmax ? 32 : __clz(t_lo ^ kmax);
  uint32_t pre = fixed == 0 ? 0u : (t_lo & (~0u << (32 - fixed)));
  int nd = B;
  int lev = 0;
  while (fixed < 32) {
    const int width = min(11, 32 - fixed);
    const int shift = 32 - fixed - width;
    const uint32_t pmask = fixed == 0 ? 0u : (~0u << (32 - fixed));
    const int nb = 1 << width;
    uint32_t* h = lev == 0 ? sh.hist : reinterpret_cast<uint32_t*>(sh.cslot) + (lev - 1) * kBins;
#pragma unroll
    for (int j = 0; j < kPer; ++j)
      if (i0 + j < total && (key[j] & pmask) == pre) atomicAdd(&h[(key[j] >> shift) & (nb - 1)], 1u);
    __syncthreads();
    int tl;
    find_bin(sh, h, nb, nd, &tl);
    const int bin = sh.bin;
    nd -= sh.above;
    const int cnt_bin = (int)h[bin];
    pre |= (uint32_t)bin << shift;
    fixed += width;
    ++lev;
    if (cnt_bin == nd) break;   // the whole bin is taken
  }
  const uint32_t bmask = fixed >= 32 ? ~0u : (fixed == 0 ? 0u : (~0u << (32 - fixed)));
  const uint32_t top = pre | ~bmask;
  int na = 0, ni = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    if (i0 + j < total) {
      na += key[j] > top;
      ni += (key[j] & bmask) == pre;
    }
  }
  int tot2;
  const int pref = block_exclusive_scan<kThreads>(na | (ni << 16), sh.scan, &tot2);
  int pa = pref & 0xffff, pi = pref >> 16;
  int32_t* orow = a.out_idx + (int64_t)row * B;
  float* osc = a.out_score ? a.out_score + (int64_t)row * B : nullptr;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    if (i0 + j >= total) continue;
    int pos = -1;
    if (key[j] > top) {
      pos = pa + min(pi, nd);
      ++pa;
    } else if ((key[j] & bmask) == pre) {
      if (pi < nd) pos = pa + pi;
      ++pi;
    }
    if (pos >= 0) {
      orow[pos] = slot_pos<CAND>(a, crow, slot[j]);
      if (osc) osc[pos] = val[j];
    }
  }
  if (tid == 0 && a.out_count) a.out_count[row] = B;
}

// Short rows (n <= kThreads * 8): every slot in registers, thread t holding
// slots 8t .. 8t+7; invalid slots are dropped by a compaction in slot order
// (one prefix scan), then the exact selection runs in registers. Returns
// false (nothing written) when the row is longer.
template <bool CAND>
__device__ __forceinline__ bool select_short_row(const SelectArgs& a, SelShared& sh, int row,
                                                 const float* srow, int64_t nv, const int32_t* crow) {
  constexpr int kPer = 8;
  if (nv > (int64_t)kThreads * kPer) return false;
  const int tid = threadIdx.x, lane = tid & 63;
  const int B = a.B;
  const int s0 = tid * kPer;
  float v[kPer];
  if (s0 + kPer <= nv && (((uintptr_t)(srow + s0)) & 15u) == 0) {
    const float4 x = *(const float4*)(srow + s0);
    const float4 y = *(const float4*)(srow + s0 + 4);
    v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w; v[4] = y.x; v[5] = y.y; v[6] = y.z; v[7] = y.w;
  } else {
#pragma unroll
    for (int j = 0; j < kPer; ++j) v[j] = s0 + j < nv ? srow[s0 + j] : 0.f;
  }
  uint32_t ok = 0;
  int mine = 0;
  uint32_t lo = 0xffffffffu, hi = 0u;
  uint32_t k8[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    k8[j] = order_key(v[j]);
    if (slot_ok<CAND>(a, crow, s0 + j, nv)) {
      ok |= 1u << j;
      ++mine;
      lo = min(lo, k8[j]);
      hi = max(hi, k8[j]);
    }
  }
  // compact the valid slots, keeping slot order: thread t's entries start
  // at the count of valid slots before it
  if (tid == 0) {
    sh.kmax = 0u;
    sh.nsample = -1;           // reused below as the minimum key (0xffffffff as unsigned)
  }
  int total;
  const int first = block_exclusive_scan<kThreads>(mine, sh.scan, &total);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    lo = min(lo, (uint32_t)__shfl_xor((int)lo, o, 64));
    hi = max(hi, (uint32_t)__shfl_xor((int)hi, o, 64));
  }
  if (lane == 0) {
    atomicMax(&sh.kmax, hi);
    atomicMin(reinterpret_cast<uint32_t*>(&sh.nsample), lo);
  }
  int32_t* orow = a.out_idx + (int64_t)row * B;
  float* osc = a.out_score ? a.out_score + (int64_t)row * B : nullptr;
  if (total <= B) {   // every valid slot is taken, in slot order; pad
    int pos = first;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      if (!((ok >> j) & 1u)) continue;
      orow[pos] = slot_pos<CAND>(a, crow, s0 + j);
      if (osc) osc[pos] = v[j];
      ++pos;
    }
    for (int p = total + tid; p < B; p += kThreads) {
      orow[p] = -1;
      if (osc) osc[p] = -INFINITY;
    }
    if (tid == 0 && a.out_count) a.out_count[row] = total;
    return true;
  }
  // the valid entries, compacted into the list layout select_in_registers
  // expects (thread t: entries t*kPer ..), through the LDS key/slot lists
  {
    int pos = first;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      if (!((ok >> j) & 1u)) continue;
      sh.ckey[pos] = __float_as_uint(v[j]);
      sh.cslot[pos] = s0 + j;
      ++pos;
    }
  }
  __syncthreads();
  uint32_t key[kPer];
  float val[kPer];
  int32_t slot[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int e = s0 + j;
    val[j] = e < total ? __uint_as_float(sh.ckey[e]) : 0.f;
    slot[j] = e < total ? sh.cslot[e] : 0;
    key[j] = order_key(val[j]);
  }
  const uint32_t t_lo = (uint32_t)sh.nsample, kmax = sh.kmax;
  __syncthreads();   // the refine histograms reuse cslot
  for (int i = tid; i < 2 * kBins; i += kThreads) sh.cslot[i] = 0;
  zero_hist(sh);
  __syncthreads();
  select_in_registers<CAND, kPer>(a, sh, row, crow, key, val, slot, s0, total, t_lo, kmax);
  return true;
}

// Rows of kThreads * 8 < n <= kThreads * 16 slots, all of them valid: every
// slot in registers (thread t holding slots 16t .. 16t+15, already in list
// order), then the exact selection in registers. Returns false (nothing
// written) for other rows or when a slot is invalid.
template <bool CAND>
__device__ __forceinline__ bool select_short_row16(const SelectArgs& a, SelShared& sh, int row,
                                                   const float* srow, int64_t nv, const int32_t* crow) {
  constexpr int kPer = 16;
  if (nv <= (int64_t)kThreads * 8 || nv > (int64_t)kThreads * kPer) return false;
  const int tid = threadIdx.x, lane = tid & 63;
  const int B = a.B;
  const int s0 = tid * kPer;
  float val[kPer];
  if (s0 + kPer <= nv && (((uintptr_t)(srow + s0)) & 15u) == 0) {
#pragma unroll
    for (int q = 0; q < kPer / 4; ++q) {
      const float4 x = *(const float4*)(srow + s0 + 4 * q);
      val[4 * q] = x.x; val[4 * q + 1] = x.y; val[4 * q + 2] = x.z; val[4 * q + 3] = x.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < kPer; ++j) val[j] = s0 + j < nv ? srow[s0 + j] : 0.f;
  }
  uint32_t key[kPer];
  int32_t slot[kPer];
  int bad = 0;
  uint32_t lo = 0xffffffffu, hi = 0u;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    key[j] = order_key(val[j]);
    slot[j] = s0 + j;
    if (s0 + j < nv) {
      if (slot_ok<CAND>(a, crow, s0 + j, nv)) {
        lo = min(lo, key[j]);
        hi = max(hi, key[j]);
      } else {
        ++bad;
      }
    }
  }
  if (tid == 0) {
    sh.kmax = 0u;
    sh.nsample = -1;           // the minimum key (0xffffffff as unsigned)
    sh.ncand = 0;
  }
  __syncthreads();
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    lo = min(lo, (uint32_t)__shfl_xor((int)lo, o, 64));
    hi = max(hi, (uint32_t)__shfl_xor((int)hi, o, 64));
    bad += __shfl_xor(bad, o, 64);
  }
  if (lane == 0) {
    atomicMax(&sh.kmax, hi);
    atomicMin(reinterpret_cast<uint32_t*>(&sh.nsample), lo);
    if (bad) atomicAdd(&sh.ncand, bad);
  }
  __syncthreads();
  const bool any_bad = sh.ncand != 0;
  const uint32_t t_lo = (uint32_t)sh.nsample, kmax = sh.kmax;
  __syncthreads();   // the general path resets these words
  if (any_bad) return false;
  const int total = (int)nv;
  if (total <= B) {   // every slot is taken, in slot order; pad
    int32_t* orow = a.out_idx + (int64_t)row * B;
    float* osc = a.out_score ? a.out_score + (int64_t)row * B : nullptr;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      if (s0 + j >= total) continue;
      orow[s0 + j] = slot_pos<CAND>(a, crow, s0 + j);
      if (osc) osc[s0 + j] = val[j];
    }
    for (int p = total + tid; p < B; p += kThreads) {
      orow[p] = -1;
      if (osc) osc[p] = -INFINITY;
    }
    if (tid == 0 && a.out_count) a.out_count[row] = total;
    return true;
  }
  for (int i = tid; i < 2 * kBins; i += kThreads) sh.cslot[i] = 0;   // the refine histograms
  zero_hist(sh);
  __syncthreads();
  select_in_registers<CAND, kPer>(a, sh, row, crow, key, val, slot, s0, total, t_lo, kmax);
  return true;
}

template <bool CAND, bool GBM, bool PRE>
__device__ __forceinline__ void select_row(const SelectArgs& a, int row, const float* srow,
                                           int64_t nv, unsigned char* smem_raw) {
  SelShared& sh = *reinterpret_cast<SelShared*>(smem_raw);
  const int tid = threadIdx.x, lane = tid & 63;
  const int64_t n = a.n;
  const int nw = (int)((n + 31) >> 5);
  uint32_t* bm_sel;
  uint32_t* bm_tie;
  if constexpr (GBM) {
    bm_sel = a.gbitmap + (int64_t)row * 2 * nw;
    bm_tie = bm_sel + nw;
  } else {
    bm_sel = reinterpret_cast<uint32_t*>(smem_raw + sizeof(SelShared));
    bm_tie = bm_sel + nw;
  }

  const int32_t* crow = CAND ? a.cand + (int64_t)row * a.cand_ld : nullptr;
  const int B = a.B;
  // passes over the row walk block-uniform tiles of kThreads * 4 * kUnroll slots
  const int64_t tile = (int64_t)kThreads * 4 * kUnroll;

  if constexpr (!PRE) {
    if (select_short_row<CAND>(a, sh, row, srow, nv, crow)) return;
    if (select_short_row16<CAND>(a, sh, row, srow, nv, crow)) return;
  }
  zero_hist(sh);
  if constexpr (PRE) {
    // two more refine histograms, in the (still unused) slot list
    for (int i = tid; i < 2 * kBins; i += kThreads) sh.cslot[i] = 0;
  } else {
    for (int i = tid; i < nw; i += kThreads) {
      bm_sel[i] = 0u;
      bm_tie[i] = 0u;
    }
  }
  if (tid == 0) {
    sh.ncand = 0;
    sh.nsample = 0;
    sh.kmax = 0u;
  }
  __syncthreads();

  // Outcome of the search: tau is the exact B-th key and `need` the number
  // of keys equal to tau to take (lowest slots first). With in_lds every key
  // >= tau is in the LDS list (ncand entries). `all`: take every valid slot.
  uint32_t tau = 0;
  int need = 0;
  int ncand = 0;
  bool in_lds = false;
  bool all = false;
  bool found = false;
  bool list_has_all = false;   // the LDS list holds every selected slot
  int ties_known = -1;         // keys equal to tau, when the list refine counted them

  // ---------------- pre-collected lists (segmented collect) ----------------
  if constexpr (PRE) {
    // segment offsets of the concatenated list, in the (unused) key list
    int32_t* seg_off = reinterpret_cast<int32_t*>(sh.ckey);
    const int4* meta = a.seg_meta + (int64_t)row * a.nseg;
    int cnt = 0;
    uint32_t km = 0u;
    const uint32_t t_lo = (uint32_t)meta[0].z;
    bool other_t = false;   // a segment listed against another threshold
    if (tid < a.nseg) {
      const int4 mm = meta[tid];
      cnt = mm.x;
      km = (uint32_t)mm.y;
      other_t = (uint32_t)mm.z != t_lo;
    }
    const bool same_t = !__syncthreads_or(other_t);
    int total;
    const int off = block_exclusive_scan<kThreads>(cnt, sh.scan, &total);
    if (tid < a.nseg) seg_off[tid] = off;
    if (tid == 0) seg_off[a.nseg] = total;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) km = max(km, (uint32_t)__shfl_xor((int)km, o, 64));
    if (lane == 0) atomicMax(&sh.kmax, km);
    __syncthreads();
    if (same_t && total >= B && total <= kCap) {
      // Every key >= t_lo of the row is listed and at least B are, so the
      // B-th key is among them. Thread t holds entries 8t .. 8t+7 (list
      // order is slot order) in registers.
      constexpr int kPer = kCap / kThreads;
      const int i0 = tid * kPer;
      int sg = 0;
      if (i0 < total) {
        int lo = 0, hi = a.nseg - 1;   // last segment starting at or before i0
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (seg_off[mid] <= i0) lo = mid; else hi = mid - 1;
        }
        sg = lo;
      }
      const int2* lrow = a.seg_list + (int64_t)row * a.nseg * kSeg;
      int64_t addr[kPer];
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const int i = i0 + j;
        if (i < total) {
          while (seg_off[sg + 1] <= i) ++sg;
          addr[j] = (int64_t)sg * kSeg + (i - seg_off[sg]);
        } else {
          addr[j] = -1;
        }
      }
      uint32_t key[kPer];
      float val[kPer];
      int32_t slot[kPer];
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const int2 e = addr[j] >= 0 ? lrow[addr[j]] : make_int2(0, 0);
        val[j] = __int_as_float(e.x);
        key[j] = order_key(val[j]);
        slot[j] = e.y;
      }
      select_in_registers<CAND, kPer>(a, sh, row, crow, key, val, slot, i0, total, t_lo, sh.kmax);
      return;
    }
    // the lists do not settle it: general path over the row (its scores
    // recomputed first when the listing launch wrote none)
    if (a.rs_k_idx != nullptr) rescore_row(a, row, const_cast<float*>(srow), nv);
    for (int i = tid; i < nw; i += kThreads) {
      bm_sel[i] = 0u;
      bm_tie[i] = 0u;
    }
    __syncthreads();
  }

  // ---------------- fast path: threshold, then collect keys >= t_lo ----------------
  if (!PRE && B <= kCap / 2 && nv > B) {
    uint32_t t_lo = 0u;
    // the hints can vouch for at most hint_count*hint_k keys
    const bool use_hint = a.hint != nullptr && a.hint_k > 0 && a.hint_count > 0 &&
                          (int64_t)a.hint_count * a.hint_k >= B;
    if (use_hint) {
      // Hints: entry h vouches that at least hint_k valid keys of its group
      // reach it. Wave 0 folds them into at most 1024 entries (the min of m
      // hints vouches for m*hint_k keys) and finds the r-th largest entry,
      // r = ceil(B / (m*hint_k)), by bisection on the 16-bit prefixes: at
      // least r entries reach it, so at least B keys of the row do.
      if (tid < 64) {
        const uint32_t* hrow = a.hint + (int64_t)row * a.hint_ld;
        const int m = (a.hint_count + 1023) / 1024;
        const int ne = (a.hint_count + m - 1) / m;
        const int r = (B + m * a.hint_k - 1) / (m * a.hint_k);
        uint32_t e[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int idx = lane + 64 * j;
          uint32_t v = idx < ne ? 0xffffffffu : 0u;
          for (int q = 0; q < m; ++q) {
            const int h = idx * m + q;
            if (idx < ne) v = min(v, h < a.hint_count ? hrow[h] : 0u);
          }
          e[j] = v;
        }
        uint32_t p = 0;
        if (r <= ne) {
          for (int bit = 15; bit >= 0; --bit) {
            const uint32_t cand = (p | (1u << bit)) << 16;
            int cnt = 0;
#pragma unroll
            for (int j = 0; j < 16; ++j) cnt += __popcll(ballot64(e[j] >= cand));
            if (cnt >= r) p |= 1u << bit;
          }
        }
        if (lane == 0) sh.wval[0] = (int)(p << 16);
      }
      __syncthreads();
      t_lo = (uint32_t)sh.wval[0];
    } else {
      // No hint: 64 evenly spaced blocks of 128 slots are radix-histogrammed
      // (top 11 key bits, then the next 11 inside the chosen bin); t_lo sits
      // where the sample's suffix count passes twice B's share plus 64.
      const int64_t nblk = (nv + kSampleBlock - 1) / kSampleBlock;
      const int64_t stride = max<int64_t>(1, nblk / kSampleBlocks);
      constexpr int kPer = kSampleBlocks * kSampleBlock / kThreads;
      float sval[kPer];
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        const int i = tid + k * kThreads;
        const int64_t s = (int64_t)(i / kSampleBlock) * stride * kSampleBlock + (i % kSampleBlock);
        sval[k] = srow[min(s, nv - 1)];   // clamped: every load issues unconditionally
      }
      uint32_t skey[kPer];
      uint32_t sok = 0;
      int mine = 0;
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        const int i = tid + k * kThreads;
        const int64_t s = (int64_t)(i / kSampleBlock) * stride * kSampleBlock + (i % kSampleBlock);
        const bool ok = slot_ok<CAND>(a, crow, s, nv);
        skey[k] = ok ? order_key(sval[k]) : 0u;
        sok |= (uint32_t)ok << k;
        if (ok) {
          atomicAdd(&sh.hist[skey[k] >> 21], 1u);
          ++mine;
        }
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) mine += __shfl_xor(mine, o, 64);
      if (lane == 0) atomicAdd(&sh.nsample, mine);
      __syncthreads();
      const double share = (double)sh.nsample / (double)nv;
      const int target = (int)min<double>((double)sh.nsample, ceil(2.0 * B * share) + 64.0);
      if (target >= 1) {
        int tot_s;
        find_bin(sh, sh.hist, kBins, target, &tot_s);
        if (tot_s >= target) {
          const uint32_t sb = (uint32_t)sh.bin;
          const int need_s = target - sh.above;
          zero_hist(sh);
          __syncthreads();
#pragma unroll
          for (int k = 0; k < kPer; ++k)
            if ((sok & (1u << k)) && (skey[k] >> 21) == sb) atomicAdd(&sh.hist[(skey[k] >> 10) & 2047u], 1u);
          __syncthreads();
          int tot2;
          find_bin(sh, sh.hist, kBins, need_s, &tot2);
          t_lo = (sb << 21) | ((uint32_t)sh.bin << 10);
        }
      }
    }

    // collect every valid key >= t_lo: one float compare per slot (the key
    // order is the float order with -0 == +0; NaN only when t_lo is 0)
    const bool take_all = t_lo == 0u;
    const float t_f = key_to_float(t_lo);
    constexpr int kCU = kCollectUnroll;
    const int64_t ctile = (int64_t)kThreads * 4 * kCU;
    int64_t t0 = 0;
    for (; t0 + ctile <= nv; t0 += ctile) {   // full tiles: straight-line 128-bit loads
      float4 raw[kCU];
#pragma unroll
      for (int j = 0; j < kCU; ++j)
        raw[j] = *(const float4*)(srow + t0 + (int64_t)j * kThreads * 4 + (int64_t)tid * 4);
      float v[4 * kCU];
      uint32_t flags = 0;
#pragma unroll
      for (int j = 0; j < kCU; ++j) {
        v[4 * j] = raw[j].x; v[4 * j + 1] = raw[j].y; v[4 * j + 2] = raw[j].z; v[4 * j + 3] = raw[j].w;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          bool take = take_all || v[4 * j + k] >= t_f;
          if constexpr (CAND) take = take && slot_ok<CAND>(a, crow, t0 + (int64_t)j * kThreads * 4 + (int64_t)tid * 4 + k, nv);
          flags |= (uint32_t)take << (4 * j + k);
        }
      }
      wave_append<4 * kCU>(sh, v, t0 + (int64_t)tid * 4, flags, lane);
    }
    if (t0 < nv) {   // the partial last tile, clamped scalar loads
      float v[4 * kCU];
#pragma unroll
      for (int j = 0; j < kCU; ++j)
#pragma unroll
        for (int k = 0; k < 4; ++k)
          v[4 * j + k] = srow[min(t0 + (int64_t)j * kThreads * 4 + (int64_t)tid * 4 + k, nv - 1)];
      uint32_t flags = 0;
#pragma unroll
      for (int j = 0; j < kCU; ++j)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const bool take = take_all || v[4 * j + k] >= t_f;
          flags |= (uint32_t)(take && slot_ok<CAND>(a, crow, t0 + (int64_t)j * kThreads * 4 + (int64_t)tid * 4 + k, nv)) << (4 * j + k);
        }
      wave_append<4 * kCU>(sh, v, t0 + (int64_t)tid * 4, flags, lane);
    }
    __syncthreads();
    ncand = sh.ncand;
    if (ncand >= B && ncand <= kCap) {
      in_lds = true;
      found = true;
      list_has_all = true;
      uint32_t kmax = 0;
      for (int i = tid; i < ncand; i += kThreads) kmax = max(kmax, sh.ckey[i]);
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o, 64));
      if (lane == 0) atomicMax(&sh.kmax, kmax);
      __syncthreads();
      need = B;
      tau = refine_list(sh, ncand, t_lo, sh.kmax, &need, &ties_known);
    } else {
      zero_hist(sh);   // the guess failed: start the general path clean
      __syncthreads();
      if (tid == 0) sh.ncand = 0;
      __syncthreads();
    }
  }

  // ---------------- general path ----------------
  if (!found) {
    // pass A: histogram of every valid key; bm_tie temporarily holds "valid"
    for (int64_t t0 = 0; t0 < nv; t0 += tile) {
#pragma unroll
      for (int j = 0; j < kUnroll; ++j) {
        const int64_t s0 = t0 + (int64_t)j * kThreads * 4 + (int64_t)tid * 4;
        uint32_t key[4];
        bool ok[4];
        load4<CAND>(a, srow, crow, s0, nv, key, ok);
        uint32_t nib = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          if (ok[k]) {
            atomicAdd(&sh.hist[key[k] >> 21], 1u);
            nib |= 1u << k;
          }
        }
        const uint32_t w = word_from_nibbles(nib, lane);
        if ((lane & 7) == 0 && s0 < nv) bm_tie[s0 >> 5] = w;
      }
    }
    __syncthreads();
    int total;
    find_bin(sh, sh.hist, kBins, B, &total);
    if (total <= B) {
      all = true;
    } else {
      const uint32_t b0 = (uint32_t)sh.bin;
      need = B - sh.above;
      const int cnt_b0 = (int)sh.hist[b0];
      in_lds = cnt_b0 <= kCap;
      for (int i = tid; i < nw; i += kThreads) bm_tie[i] = 0u;
      __syncthreads();
      // pass B: above b0 -> selected outright; inside b0 -> LDS list
      for (int64_t t0 = 0; t0 < nv; t0 += tile) {
#pragma unroll
        for (int j = 0; j < kUnroll; ++j) {
          const int64_t s0 = t0 + (int64_t)j * kThreads * 4 + (int64_t)tid * 4;
          uint32_t key[4];
          bool ok[4];
          load4<CAND>(a, srow, crow, s0, nv, key, ok);
          uint32_t nib = 0, flags = 0;
          float val[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            nib |= (uint32_t)(ok[k] && (key[k] >> 21) > b0) << k;
            flags |= (uint32_t)(ok[k] && (key[k] >> 21) == b0) << k;
            val[k] = key_to_float(key[k]);
          }
          const uint32_t w = word_from_nibbles(nib, lane);
          if ((lane & 7) == 0 && s0 < nv) bm_sel[s0 >> 5] = w;
          if (in_lds) wave_append<4>(sh, val, s0, flags, lane);
        }
      }
      __syncthreads();
      tau = b0 << 21;
      if (in_lds) {
        ncand = cnt_b0;
        tau = refine_list(sh, ncand, b0 << 21, (b0 << 21) | 0x1fffffu, &need, &ties_known);
      } else {
        for (int level = 1; level <= 2; ++level) {
          const int shift = level == 1 ? 10 : 0;
          const int nb = level == 1 ? 2048 : 1024;
          const uint32_t pmask = level == 1 ? 0xffe00000u : 0xfffffc00u;
          zero_hist(sh);
          __syncthreads();
          for (int64_t t0 = 0; t0 < nv; t0 += tile) {
#pragma unroll
            for (int j = 0; j < kUnroll; ++j) {
              const int64_t s0 = t0 + (int64_t)j * kThreads * 4 + (int64_t)tid * 4;
              uint32_t key[4];
              bool ok[4];
              load4<CAND>(a, srow, crow, s0, nv, key, ok);
#pragma unroll
              for (int k = 0; k < 4; ++k)
                if (ok[k] && (key[k] & pmask) == tau) atomicAdd(&sh.hist[(key[k] >> shift) & (nb - 1)], 1u);
            }
          }
          __syncthreads();
          int tl;
          find_bin(sh, sh.hist, nb, need, &tl);
          tau |= (uint32_t)sh.bin << shift;
          need -= sh.above;
        }
      }
    }
  }

  // ---------------- mark keys above tau, and the ties ----------------
  const int wpt = (nw + kThreads - 1) / kThreads;
  const int w0 = tid * wpt, w1 = min(nw, w0 + wpt);
  if (!all) {
    // keys equal to tau: from the list refine, or the last global level's bin
    const int ties = ties_known >= 0 ? ties_known : (int)sh.hist[tau & 1023u];
    __syncthreads();
    if (in_lds) {
      for (int i = tid; i < ncand; i += kThreads) {
        const uint32_t key = sh.ckey[i];
        const int32_t s = sh.cslot[i];
        if (key > tau) atomicOr(&bm_sel[s >> 5], 1u << (s & 31));
        else if (key == tau) atomicOr(&bm_tie[s >> 5], 1u << (s & 31));
      }
    } else {
      const uint32_t b0 = tau >> 21;
      for (int64_t t0 = 0; t0 < nv; t0 += tile) {
#pragma unroll
        for (int j = 0; j < kUnroll; ++j) {
          const int64_t s0 = t0 + (int64_t)j * kThreads * 4 + (int64_t)tid * 4;
          uint32_t key[4];
          bool ok[4];
          load4<CAND>(a, srow, crow, s0, nv, key, ok);
          uint32_t ns = 0, nt = 0;
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const bool inb = ok[k] && (key[k] >> 21) == b0;
            ns |= (uint32_t)(inb && key[k] > tau) << k;
            nt |= (uint32_t)(inb && key[k] == tau) << k;
          }
          const uint32_t ws = word_from_nibbles(ns, lane);
          const uint32_t wt = word_from_nibbles(nt, lane);
          if ((lane & 7) == 0 && s0 < nv) {
            bm_sel[s0 >> 5] |= ws;
            bm_tie[s0 >> 5] = wt;
          }
        }
      }
    }
    __syncthreads();
    // take the `need` lowest tie slots
    if (need == ties) {
      for (int w = w0; w < w1; ++w) bm_sel[w] |= bm_tie[w];
    } else {
      int c = 0;
      for (int w = w0; w < w1; ++w) c += __popc(bm_tie[w]);
      int tot_t;
      const int before = block_exclusive_scan<kThreads>(c, sh.scan, &tot_t);
      int rem = need - before;
      for (int w = w0; w < w1 && rem > 0; ++w) {
        uint32_t t = bm_tie[w];
        const int pc = __popc(t);
        if (pc <= rem) {
          bm_sel[w] |= t;
          rem -= pc;
        } else {
          uint32_t keep = 0;
          while (rem > 0) {
            const uint32_t low = t & (0u - t);
            keep |= low;
            t ^= low;
            --rem;
          }
          bm_sel[w] |= keep;
        }
      }
    }
  } else {
    for (int w = w0; w < w1; ++w) bm_sel[w] = bm_tie[w];
  }
  __syncthreads();

  // ---------------- output: ascending positions ----------------
  int c = 0;
  for (int w = w0; w < w1; ++w) c += __popc(bm_sel[w]);
  int count;
  int off = block_exclusive_scan<kThreads>(c, sh.scan, &count);
  int32_t* orow = a.out_idx + (int64_t)row * B;
  float* osc = a.out_score ? a.out_score + (int64_t)row * B : nullptr;
  if (list_has_all) {
    // bm_tie becomes the per-word prefix count of bm_sel; each listed slot
    // that is selected finds its output position from it in parallel
    for (int w = w0; w < w1; ++w) {
      const uint32_t b = bm_sel[w];
      bm_tie[w] = (uint32_t)off;
      off += __popc(b);
    }
    __syncthreads();
    for (int i = tid; i < ncand; i += kThreads) {
      const int32_t s = sh.cslot[i];
      const uint32_t word = bm_sel[s >> 5];
      if ((word >> (s & 31)) & 1u) {
        const int pos = (int)bm_tie[s >> 5] + __popc(word & ((1u << (s & 31)) - 1u));
        if (pos < B) {
          orow[pos] = slot_pos<CAND>(a, crow, s);
          if (osc) osc[pos] = srow[s];
        }
      }
    }
  } else {
    for (int w = w0; w < w1; ++w) {
      uint32_t bits = bm_sel[w];
      while (bits) {
        const int b = __ffs(bits) - 1;
        bits &= bits - 1;
        const int64_t s = ((int64_t)w << 5) + b;
        if (off < B) {
          orow[off] = slot_pos<CAND>(a, crow, s);
          if (osc) osc[off] = srow[s];
        }
        ++off;
      }
    }
  }
  for (int j = count + tid; j < B; j += kThreads) {
    orow[j] = -1;
    if (osc) osc[j] = -INFINITY;
  }
  if (tid == 0 && a.out_count) a.out_count[row] = min(count, B);
}

// ---------------------------------------------------------------------------
// Segmented collect (long rows with a selection hint). A row is cut into
// segments of kSeg slots, one 256-thread workgroup each, so a few rows
// still spread over every CU. Each workgroup issues its segment's loads,
// derives the row's threshold t_lo from the hint while they are in flight
// (every workgroup of the row gets the same value), and writes the
// segment's slots whose keys reach t_lo, in slot order, as (score bits,
// slot) pairs, with {count, max key, t_lo}. The row kernel then refines the
// concatenated lists (see select_kernel, PRE).
// ---------------------------------------------------------------------------

struct SegShared {
  uint32_t h1[256];
  uint32_t h2[256];
  int wsum[kSegWaves];
  int bin, above;
  int ucnt[kSegUnits];
  int uoff[kSegUnits];
  uint32_t wmax[kSegWaves];
};

// One 8-bit radix level over a 256-bin histogram: the bin holding the
// need-th largest value (bins scanned from the top), published in sh.bin /
// sh.above. sh.bin is left unchanged when the histogram holds fewer than
// need values. Contains barriers.
__device__ __forceinline__ void seg_level(SegShared& sh, const uint32_t* h, int need) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int c = (int)h[255 - t];
  int x = c;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) sh.wsum[w] = x;
  __syncthreads();
  int base = 0;
#pragma unroll
  for (int q = 0; q < kSegWaves; ++q) base += q < w ? sh.wsum[q] : 0;
  const int excl = base + x - c;
  if (excl < need && need <= excl + c) {
    sh.bin = 255 - t;
    sh.above = excl;
  }
  __syncthreads();
}

// Collect segment `seg` of row `row` (one 256-thread workgroup; every
// thread must call it).
template <bool CAND>
__device__ __forceinline__ void collect_segment(const SelectArgs& a, SegShared& sh, int row, int seg) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  int64_t nv = a.n;
  if (a.n_valid) nv = min<int64_t>(nv, (int64_t)max(0, a.n_valid[row]));
  if (a.causal_group > 0) nv = min<int64_t>(nv, ((int64_t)row / a.causal_group + 1) * a.causal_block);
  const int64_t s0 = (int64_t)seg * kSeg;
  int4* meta = a.seg_meta + (int64_t)row * a.nseg + seg;
  if (s0 >= nv) {   // nothing valid here (block-uniform)
    if (tid == 0) *meta = make_int4(0, 0, 0, 0);
    return;
  }
  const float* srow = a.scores + (int64_t)row * a.scores_ld;
  const int32_t* crow = CAND ? a.cand + (int64_t)row * a.cand_ld : nullptr;

  // 1. the hint loads go out first (vector loads return in order, so the
  // threshold search below then overlaps the segment's loads)
  const uint32_t* hrow = a.hint + (int64_t)row * a.hint_ld;
  const int m = (a.hint_count + 4 * kSegThreads - 1) / (4 * kSegThreads);
  const int ne = (a.hint_count + m - 1) / m;
  const int r = (a.B + m * a.hint_k - 1) / (m * a.hint_k);
  uint32_t p[4];
  if (m == 1) {   // plain loads, first used after the segment's loads are issued
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = tid + q * kSegThreads;
      p[q] = e < a.hint_count ? hrow[e] : 0u;
    }
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = tid + q * kSegThreads;
      uint32_t val = 0xffffffffu;
      for (int mm = 0; mm < m; ++mm) {
        const int h = e * m + mm;
        val = min(val, h < a.hint_count ? hrow[h] : 0u);
      }
      p[q] = val;
    }
  }
  float v[4 * kSegUnroll];
  const bool full = s0 + kSeg <= nv;
  if (full) {
#pragma unroll
    for (int j = 0; j < kSegUnroll; ++j) {
      const float4 x = *(const float4*)(srow + s0 + j * kSegThreads * 4 + tid * 4);
      v[4 * j] = x.x; v[4 * j + 1] = x.y; v[4 * j + 2] = x.z; v[4 * j + 3] = x.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < kSegUnroll; ++j)
#pragma unroll
      for (int k = 0; k < 4; ++k)
        v[4 * j + k] = srow[min(s0 + j * kSegThreads * 4 + tid * 4 + k, nv - 1)];
    // keeps these clamped loads in this branch: merged with the branch
    // above, every 128-bit load would become four 32-bit ones
    asm volatile("" ::: "memory");
  }

  // 2. t_lo from the hint (loaded above). Entry h vouches that hint_k valid
  // keys of its (disjoint) slot group reach it; folding m entries into
  // their minimum vouches for m*hint_k keys. The r-th largest folded entry,
  // with r = ceil(B / (m*hint_k)), is then reached by at least B keys. It
  // is found on the 16-bit prefixes by two 8-bit radix levels.
#pragma unroll
  for (int q = 0; q < 4; ++q) p[q] >>= 16;
  sh.h1[tid] = 0u;
  sh.h2[tid] = 0u;
  if (tid == 0) sh.bin = -1;
  __syncthreads();
#pragma unroll
  for (int q = 0; q < 4; ++q)
    if (tid + q * kSegThreads < ne) atomicAdd(&sh.h1[p[q] >> 8], 1u);
  __syncthreads();
  uint32_t t_lo = 0u;
  if (r <= ne) {
    seg_level(sh, sh.h1, r);
    const int b1 = sh.bin, r2 = r - sh.above;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (tid + q * kSegThreads < ne && (int)(p[q] >> 8) == b1) atomicAdd(&sh.h2[p[q] & 255u], 1u);
    __syncthreads();
    seg_level(sh, sh.h2, r2);
    t_lo = ((uint32_t)b1 << 24) | ((uint32_t)sh.bin << 16);
  }

  // 3. compare (float order is key order, -0 == +0; a threshold at or below
  // the key of -inf takes every non-NaN score, t_lo == 0 takes everything)
  const bool take_all = t_lo == 0u;
  const float t_f = t_lo <= 0x007fffffu ? -INFINITY : key_to_float(t_lo);
  uint32_t flags = 0;
  float vmax = v[0];
#pragma unroll
  for (int j = 0; j < kSegUnroll; ++j)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int64_t s = s0 + j * kSegThreads * 4 + tid * 4 + k;
      bool take = take_all || v[4 * j + k] >= t_f;
      if (!full) take = take && s < nv;
      if constexpr (CAND) take = take && slot_ok<CAND>(a, crow, s, nv);
      flags |= (uint32_t)take << (4 * j + k);
      vmax = fmaxf(vmax, v[4 * j + k]);   // an upper bound of the listed keys
    }

  // 4. ranks in slot order: unit (j, wave) holds 256 consecutive slots,
  // lane-major; a lane's entries follow those of the lanes below it
  int lb[kSegUnroll];
#pragma unroll
  for (int j = 0; j < kSegUnroll; ++j) {
    int cnt = 0, below = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint64_t mk = ballot64((flags >> (4 * j + k)) & 1u);
      cnt += __popcll(mk);
      below += rank_below(mk);
    }
    lb[j] = below;
    if (lane == 0) sh.ucnt[j * kSegWaves + wid] = cnt;
  }
  uint32_t kmax = order_key(vmax);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o, 64));
  if (lane == 0) sh.wmax[wid] = kmax;
  __syncthreads();
  if (tid < 64) {
    const int c = lane < kSegUnits ? sh.ucnt[lane] : 0;
    int x = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    if (lane < kSegUnits) sh.uoff[lane] = x - c;
    if (lane == 63) {
      uint32_t km = sh.wmax[0];
#pragma unroll
      for (int q = 1; q < kSegWaves; ++q) km = max(km, sh.wmax[q]);
      *meta = make_int4(x, (int)km, (int)t_lo, 0);
    }
  }
  __syncthreads();

  // 5. write the listed (score bits, slot) pairs
  int2* out = a.seg_list + ((int64_t)row * a.nseg + seg) * kSeg;
#pragma unroll
  for (int j = 0; j < kSegUnroll; ++j) {
    uint32_t f = (flags >> (4 * j)) & 15u;
    int pos = sh.uoff[j * kSegWaves + wid] + lb[j];
    while (f) {
      const int k = __ffs(f) - 1;
      f &= f - 1;
      const float x = k == 0 ? v[4 * j] : k == 1 ? v[4 * j + 1] : k == 2 ? v[4 * j + 2] : v[4 * j + 3];
      out[pos++] = make_int2(__float_as_int(x), (int)(s0 + j * kSegThreads * 4 + tid * 4 + k));
    }
  }
}

}  // namespace sel
}  // namespace lsa
