// Exact top-B selection per row (JSSA, "Joint Subspace Sparse Attention for
// Efficient Long-Context Decoding", Fig. 1: the top-B token positions of
// each KV head; Fig. 9 "top-B selection"), lowest position on equal scores.
//
// The selection is integer work on 32-bit order-preserving keys of the fp32
// scores, so it is exact and independent of the launch shape. One
// 1024-thread workgroup owns a row.
//
// Fast path (B small against the row, the decode case):
//   sample   64 evenly spaced blocks of 128 slots are radix-histogrammed
//            (top 11 key bits, then the next 11 inside the chosen bin); where
//            the sample's suffix count passes twice B's share plus a margin
//            gives a threshold t_lo that keeps at least B keys of the row with
//            high probability;
//   collect  one pass over the row, 8 x 128-bit loads in flight per thread,
//            appends every key >= t_lo (a few B) to an LDS list;
//   verify   fewer than B kept, or more than fit, means the guess was wrong
//            and the general path runs instead: the sample decides speed,
//            never the result.
// General path: a 2048-bin histogram pass finds the bin b0 of the B-th key;
// a second pass selects keys above b0 outright and lists the keys inside b0
// (re-reading the row per refine level if they do not fit in LDS).
// Both paths then refine to the exact B-th key tau with radix levels of 11,
// 11 and 10 bits, select keys above tau plus the lowest slots among keys
// equal to tau through two bitmaps, and write the selected positions in
// ascending order from a prefix count over the bitmap, then -1 padding.
// Rows longer than kSelectLdsMaxSlots keep their bitmaps in workspace.
#include "select_row.hpp"

namespace lsa {
namespace {

using namespace sel;

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

template <bool CAND>
__global__ __launch_bounds__(kSegThreads) void select_collect_kernel(SelectArgs a) {
  __shared__ SegShared sh;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int row = blockIdx.x / a.nseg, seg = blockIdx.x - row * a.nseg;
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

template <bool CAND, bool GBM, bool PRE>
__global__ __launch_bounds__(kThreads) void select_kernel(SelectArgs a) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  const int row = blockIdx.x;
  int64_t nv = a.n;
  if (a.n_valid) nv = min<int64_t>(nv, (int64_t)max(0, a.n_valid[row]));
  if (a.causal_group > 0) nv = min<int64_t>(nv, ((int64_t)row / a.causal_group + 1) * a.causal_block);
  select_row<CAND, GBM, PRE>(a, row, a.scores + (int64_t)row * a.scores_ld, nv, smem_raw);
}

template <bool CAND>
hipError_t launch_select_t(const SelectArgs& a, int rows, hipStream_t s) {
  const int nw = (a.n + 31) / 32;
  const size_t lds = a.gbitmap ? sizeof(SelShared) : sizeof(SelShared) + (size_t)2 * nw * sizeof(uint32_t);
  if (a.nseg > 0) {
    hipLaunchKernelGGL((select_collect_kernel<CAND>), dim3(rows * a.nseg), dim3(kSegThreads), 0, s, a);
    if (a.gbitmap)
      hipLaunchKernelGGL((select_kernel<CAND, true, true>), dim3(rows), dim3(kThreads), lds, s, a);
    else
      hipLaunchKernelGGL((select_kernel<CAND, false, true>), dim3(rows), dim3(kThreads), lds, s, a);
  } else {
    if (a.gbitmap)
      hipLaunchKernelGGL((select_kernel<CAND, true, false>), dim3(rows), dim3(kThreads), lds, s, a);
    else
      hipLaunchKernelGGL((select_kernel<CAND, false, false>), dim3(rows), dim3(kThreads), lds, s, a);
  }
  return hipGetLastError();
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t bitmap_bytes(int rows, int n) {
  if (n <= kSelectLdsMaxSlots) return 0;
  return (size_t)rows * 2 * (((size_t)n + 31) / 32) * sizeof(uint32_t);
}

}  // namespace

int select_segments(int n, int B, bool hint_usable) {
  if (!hint_usable || B > kCap / 2 || n < 2 * kSeg) return 0;
  const int nseg = (n + kSeg - 1) / kSeg;
  return nseg <= kThreads ? nseg : 0;   // the row kernel scans one count per thread
}

size_t select_workspace(int rows, int n, int B, bool hint_usable) {
  size_t bytes = bitmap_bytes(rows, n);
  const int nseg = select_segments(n, B, hint_usable);
  if (nseg > 0)
    bytes = align256(bytes) + align256((size_t)rows * nseg * sizeof(int4)) +
            (size_t)rows * nseg * kSeg * sizeof(int2);
  return bytes;
}

void select_bind_workspace(SelectArgs& a, int rows, void* ws) {
  const bool hint_usable = a.hint != nullptr && a.hint_count > 0 && a.hint_k > 0 &&
                           (int64_t)a.hint_count * a.hint_k >= a.B;
  unsigned char* p = static_cast<unsigned char*>(ws);
  const size_t gb = bitmap_bytes(rows, a.n);
  a.gbitmap = gb ? reinterpret_cast<uint32_t*>(p) : nullptr;
  a.nseg = select_segments(a.n, a.B, hint_usable);
  if (a.nseg > 0) {
    a.seg_meta = reinterpret_cast<int4*>(p + align256(gb));
    a.seg_list = reinterpret_cast<int2*>(p + align256(gb) + align256((size_t)rows * a.nseg * sizeof(int4)));
  } else {
    a.seg_meta = nullptr;
    a.seg_list = nullptr;
  }
}

hipError_t launch_select(const SelectArgs& a, int rows, hipStream_t s) {
  // allow the largest LDS footprint (SelShared + two bitmaps of the longest
  // LDS-resident row); a function-local static runs this once, thread-safely
  static const hipError_t attr = [] {
    const int lds = (int)(sizeof(SelShared) + (size_t)2 * (kSelectLdsMaxSlots / 32) * sizeof(uint32_t));
    const void* fns[] = {(const void*)select_kernel<false, false, false>,
                         (const void*)select_kernel<true, false, false>,
                         (const void*)select_kernel<false, false, true>,
                         (const void*)select_kernel<true, false, true>};
    for (const void* f : fns) {
      const hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }();
  if (attr != hipSuccess) return attr;
  return a.cand ? launch_select_t<true>(a, rows, s) : launch_select_t<false>(a, rows, s);
}

}  // namespace lsa
