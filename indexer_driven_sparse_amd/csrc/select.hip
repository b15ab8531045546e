// Exact top-B selection per row (JSSA, "Joint Subspace Sparse Attention for
// Efficient Long-Context Decoding", Fig. 1: the top-B token positions of
// each KV head; Fig. 9 "top-B selection"), lowest position on equal scores.
//
// The selection is integer work on 32-bit order-preserving keys of the fp32
// scores, so it is exact and independent of the launch shape. One
// 1024-thread workgroup owns a row:
//   pass A  reads the row once: 2048-bin LDS histogram of the top 11 key
//           bits; the bin holding the B-th key (b0) follows by a suffix scan;
//   pass B  reads the row again: keys above b0 are selected outright (their
//           bits go straight into a selection bitmap from wave ballots);
//           keys inside b0 are appended to an LDS candidate list;
//   refine  two more radix levels (11 + 10 bits) run on that small list and
//           give the exact B-th key tau and how many keys equal to tau are
//           taken; keys above tau join the selection bitmap, keys equal to
//           tau a tie bitmap, of which the lowest slots are taken;
//   output  a prefix count over the bitmap writes the selected positions in
//           ascending order, then -1 padding.
// When the boundary bin does not fit the LDS list (e.g. all scores equal)
// the refine levels re-read the row from memory instead. Rows longer than
// kSelectLdsMaxSlots keep their bitmaps in workspace.
#include "common.hpp"
#include "kernels.hpp"

namespace lsa {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kBins = 2048;
constexpr int kCap = 8192;

struct SelShared {
  uint32_t hist[kBins];
  uint32_t ckey[kCap];
  int32_t cslot[kCap];
  int scan[kWaves + 1];
  int ncand;
  int bin;      // result of find_bin
  int above;    // keys in higher bins
};

// Validity of one slot of this row, and its token position.
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

// Four consecutive slots [s0, s0+4) of the row, with their validity bits.
template <bool CAND>
__device__ __forceinline__ void load4(const SelectArgs& a, const float* srow, const int32_t* crow,
                                      int64_t s0, int64_t nv, float v[4], bool ok[4]) {
  if (s0 + 3 < nv) {
    float4 x = *(const float4*)(srow + s0);
    v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = (s0 + k < nv) ? srow[s0 + k] : 0.f;
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) ok[k] = slot_ok<CAND>(a, crow, s0 + k, nv);
}

// The 32-bit bitmap word of 32 consecutive slots held 4 per lane by 8
// consecutive lanes: every lane contributes a nibble, OR-combined with DPP.
// Returns the word on every lane of the 8-lane group.
__device__ __forceinline__ uint32_t word_from_nibbles(uint32_t nib, int lane) {
  uint32_t w = nib << (4 * (lane & 7));
  w |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)w, kDppXor1, 0xf, 0xf, false);
  w |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)w, kDppXor2, 0xf, 0xf, false);
  w |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)w, kDppHalfMirror, 0xf, 0xf, false);
  return w;
}

// Find the bin holding the need-th largest key: the highest bin b with
// (count above b) < need <= (count above b) + hist[b]. nb in {1024, 2048}.
// Writes sh.bin and sh.above; returns the total count via *total.
__device__ __forceinline__ void find_bin(SelShared& sh, int nb, int need, int* total) {
  const int t = threadIdx.x;
  const int per = nb / kThreads;  // 1 or 2 bins per thread, walked from the top
  const int hi = nb - 1 - t * per;
  int c = 0;
  for (int k = 0; k < per; ++k) c += (int)sh.hist[hi - k];
  int tot;
  int above = block_exclusive_scan<kThreads>(c, sh.scan, &tot);
  int acc = above;
  for (int k = 0; k < per; ++k) {
    int h = (int)sh.hist[hi - k];
    if (acc < need && need <= acc + h) {
      sh.bin = hi - k;
      sh.above = acc;
    }
    acc += h;
  }
  *total = tot;
  __syncthreads();
}

template <bool GBM>
__device__ __forceinline__ void zero_words(uint32_t* w, int nw) {
  for (int i = threadIdx.x; i < nw; i += kThreads) w[i] = 0u;
}

template <bool CAND, bool GBM>
__global__ __launch_bounds__(kThreads) void select_kernel(SelectArgs a) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  SelShared& sh = *reinterpret_cast<SelShared*>(smem_raw);
  const int row = blockIdx.x;
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

  int64_t nv = n;
  if (a.n_valid) nv = min<int64_t>(n, (int64_t)max(0, a.n_valid[row]));
  if (a.causal_group > 0) nv = min<int64_t>(n, (int64_t)row / a.causal_group + 1);
  const float* srow = a.scores + (int64_t)row * a.scores_ld;
  const int32_t* crow = CAND ? a.cand + (int64_t)row * a.cand_ld : nullptr;
  const int B = a.B;

  for (int i = tid; i < kBins; i += kThreads) sh.hist[i] = 0u;
  zero_words<GBM>(bm_sel, nw);
  zero_words<GBM>(bm_tie, nw);
  if (tid == 0) sh.ncand = 0;
  __syncthreads();

  // Every pass walks the row in wave-uniform steps (w0 is the wave's first
  // slot), so all 64 lanes stay active for the DPP and ballot work even in the
  // ragged tail; slots at or beyond nv are simply invalid.

  // ---- pass A: level-0 histogram; bm_tie temporarily holds "valid" ----
  for (int64_t w0 = (int64_t)(tid & ~63) * 4; w0 < nv; w0 += (int64_t)kThreads * 4) {
    const int64_t s0 = w0 + lane * 4;
    float v[4];
    bool ok[4];
    load4<CAND>(a, srow, crow, s0, nv, v, ok);
    uint32_t nib = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (ok[k]) {
        atomicAdd(&sh.hist[order_key(v[k]) >> 21], 1u);
        nib |= 1u << k;
      }
    }
    uint32_t w = word_from_nibbles(nib, lane);
    if ((lane & 7) == 0 && s0 < nv) bm_tie[s0 >> 5] = w;
  }
  __syncthreads();
  int total;
  find_bin(sh, kBins, B, &total);

  if (total > B) {
    const uint32_t b0 = (uint32_t)sh.bin;
    int need = B - sh.above;
    const int cnt_b0 = (int)sh.hist[b0];
    const bool in_lds = cnt_b0 <= kCap;
    zero_words<GBM>(bm_tie, nw);
    __syncthreads();

    // ---- pass B: above b0 -> selected; inside b0 -> candidate list ----
    for (int64_t w0 = (int64_t)(tid & ~63) * 4; w0 < nv; w0 += (int64_t)kThreads * 4) {
      const int64_t s0 = w0 + lane * 4;
      float v[4];
      bool ok[4];
      load4<CAND>(a, srow, crow, s0, nv, v, ok);
      uint32_t nib = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t key = order_key(v[k]);
        const bool sel = ok[k] && (key >> 21) > b0;
        nib |= (uint32_t)sel << k;
        if (in_lds) {
          const bool eq = ok[k] && (key >> 21) == b0;
          const uint64_t m = ballot64(eq);
          if (m) {
            int base = 0;
            if (lane == 0) base = atomicAdd(&sh.ncand, __popcll(m));
            base = __shfl(base, 0, 64);
            if (eq) {
              const int at = base + rank_below(m);
              sh.ckey[at] = key;
              sh.cslot[at] = (int32_t)(s0 + k);
            }
          }
        }
      }
      uint32_t w = word_from_nibbles(nib, lane);
      if ((lane & 7) == 0 && s0 < nv) bm_sel[s0 >> 5] = w;
    }
    __syncthreads();

    // ---- refine: bits 20..10, then 9..0, inside the boundary bin ----
    uint32_t prefix = b0 << 21;
    for (int level = 1; level <= 2; ++level) {
      const int shift = level == 1 ? 10 : 0;
      const int nb = level == 1 ? 2048 : 1024;
      const uint32_t pmask = level == 1 ? 0xffe00000u : 0xfffffc00u;
      for (int i = tid; i < kBins; i += kThreads) sh.hist[i] = 0u;
      __syncthreads();
      if (in_lds) {
        for (int i = tid; i < cnt_b0; i += kThreads) {
          const uint32_t key = sh.ckey[i];
          if ((key & pmask) == prefix) atomicAdd(&sh.hist[(key >> shift) & (nb - 1)], 1u);
        }
      } else {
        for (int64_t w0 = (int64_t)(tid & ~63) * 4; w0 < nv; w0 += (int64_t)kThreads * 4) {
      const int64_t s0 = w0 + lane * 4;
          float v[4];
          bool ok[4];
          load4<CAND>(a, srow, crow, s0, nv, v, ok);
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const uint32_t key = order_key(v[k]);
            if (ok[k] && (key & pmask) == prefix) atomicAdd(&sh.hist[(key >> shift) & (nb - 1)], 1u);
          }
        }
      }
      __syncthreads();
      int tot_level;
      find_bin(sh, nb, need, &tot_level);
      prefix |= (uint32_t)sh.bin << shift;
      need -= sh.above;
    }
    const uint32_t tau = prefix;
    const int ties = (int)sh.hist[tau & 1023u];
    __syncthreads();

    // keys above tau inside b0 join the selection; keys equal to tau are ties
    if (in_lds) {
      for (int i = tid; i < cnt_b0; i += kThreads) {
        const uint32_t key = sh.ckey[i];
        const int32_t s = sh.cslot[i];
        if (key > tau) atomicOr(&bm_sel[s >> 5], 1u << (s & 31));
        else if (key == tau) atomicOr(&bm_tie[s >> 5], 1u << (s & 31));
      }
    } else {
      for (int64_t w0 = (int64_t)(tid & ~63) * 4; w0 < nv; w0 += (int64_t)kThreads * 4) {
      const int64_t s0 = w0 + lane * 4;
        float v[4];
        bool ok[4];
        load4<CAND>(a, srow, crow, s0, nv, v, ok);
        uint32_t ns = 0, nt = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t key = order_key(v[k]);
          const bool inb = ok[k] && (key >> 21) == b0;
          ns |= (uint32_t)(inb && key > tau) << k;
          nt |= (uint32_t)(inb && key == tau) << k;
        }
        const uint32_t ws = word_from_nibbles(ns, lane);
        const uint32_t wt = word_from_nibbles(nt, lane);
        if ((lane & 7) == 0 && s0 < nv) {
          bm_sel[s0 >> 5] |= ws;
          bm_tie[s0 >> 5] = wt;
        }
      }
    }
    __syncthreads();

    // take the `need` lowest tie slots
    const int wpt = (nw + kThreads - 1) / kThreads;
    const int w0 = tid * wpt, w1 = min(nw, w0 + wpt);
    if (need == ties) {
      for (int w = w0; w < w1; ++w) bm_sel[w] |= bm_tie[w];
    } else {
      int c = 0;
      for (int w = w0; w < w1; ++w) c += __popc(bm_tie[w]);
      int tot_t;
      int before = block_exclusive_scan<kThreads>(c, sh.scan, &tot_t);
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
    // every valid slot is selected
    const int wpt = (nw + kThreads - 1) / kThreads;
    const int w0 = tid * wpt, w1 = min(nw, w0 + wpt);
    for (int w = w0; w < w1; ++w) bm_sel[w] = bm_tie[w];
  }
  __syncthreads();

  // ---- output: ascending positions from the selection bitmap ----
  const int wpt = (nw + kThreads - 1) / kThreads;
  const int w0 = tid * wpt, w1 = min(nw, w0 + wpt);
  int c = 0;
  for (int w = w0; w < w1; ++w) c += __popc(bm_sel[w]);
  int count;
  int off = block_exclusive_scan<kThreads>(c, sh.scan, &count);
  int32_t* orow = a.out_idx + (int64_t)row * B;
  float* osc = a.out_score ? a.out_score + (int64_t)row * B : nullptr;
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
  for (int j = count + tid; j < B; j += kThreads) {
    orow[j] = -1;
    if (osc) osc[j] = -INFINITY;
  }
  if (tid == 0 && a.out_count) a.out_count[row] = min(count, B);
}

template <bool CAND>
hipError_t launch_select_t(const SelectArgs& a, int rows, hipStream_t s) {
  const int nw = (a.n + 31) / 32;
  if (a.gbitmap) {
    hipLaunchKernelGGL((select_kernel<CAND, true>), dim3(rows), dim3(kThreads), sizeof(SelShared), s, a);
  } else {
    const size_t lds = sizeof(SelShared) + (size_t)2 * nw * sizeof(uint32_t);
    hipLaunchKernelGGL((select_kernel<CAND, false>), dim3(rows), dim3(kThreads), lds, s, a);
  }
  return hipGetLastError();
}

}  // namespace

size_t select_workspace(int rows, int n) {
  if (n <= kSelectLdsMaxSlots) return 0;
  const size_t nw = ((size_t)n + 31) / 32;
  return (size_t)rows * 2 * nw * sizeof(uint32_t);
}

hipError_t launch_select(const SelectArgs& a, int rows, hipStream_t s) {
  // allow the largest LDS footprint (SelShared + two bitmaps of the longest
  // LDS-resident row); a function-local static runs this once, thread-safely
  static const hipError_t attr = [] {
    const int lds = (int)(sizeof(SelShared) + (size_t)2 * (kSelectLdsMaxSlots / 32) * sizeof(uint32_t));
    hipError_t e1 = hipFuncSetAttribute((const void*)select_kernel<false, false>,
                                        hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    hipError_t e2 = hipFuncSetAttribute((const void*)select_kernel<true, false>,
                                        hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    return e1 != hipSuccess ? e1 : e2;
  }();
  if (attr != hipSuccess) return attr;
  return a.cand ? launch_select_t<true>(a, rows, s) : launch_select_t<false>(a, rows, s);
}

}  // namespace lsa
