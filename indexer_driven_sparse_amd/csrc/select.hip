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

#ifndef LSA_SELECT_SEGMENTED
#define LSA_SELECT_SEGMENTED 1   // long hinted rows: segmented collect, then the row select
#endif
#ifndef LSA_SELECT_SEG_MIN
// shortest row that takes the segmented collect: rows up to 16384 slots are
// held in registers by one workgroup (13.6 us against 18.0 segmented for
// 8 rows of 16384 at top-128)
#define LSA_SELECT_SEG_MIN (kThreads * 16 + 1)
#endif

namespace lsa {
namespace {

using namespace sel;

template <bool CAND>
__global__ __launch_bounds__(kSegThreads) void select_collect_kernel(SelectArgs a) {
  __shared__ SegShared sh;
  const int row = blockIdx.x / a.nseg, seg = blockIdx.x - row * a.nseg;
  collect_segment<CAND>(a, sh, row, seg);
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
  if (!LSA_SELECT_SEGMENTED || !hint_usable || B > kCap / 2 || n < 2 * kSeg || n < LSA_SELECT_SEG_MIN) return 0;
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

namespace {
// allow the largest LDS footprint (SelShared + two bitmaps of the longest
// LDS-resident row); a function-local static runs this once, thread-safely
hipError_t select_attributes() {
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
  return attr;
}
}  // namespace

hipError_t launch_select(const SelectArgs& a, int rows, hipStream_t s) {
  const hipError_t attr = select_attributes();
  if (attr != hipSuccess) return attr;
  return a.cand ? launch_select_t<true>(a, rows, s) : launch_select_t<false>(a, rows, s);
}

hipError_t launch_select_lists(const SelectArgs& a, int rows, hipStream_t s) {
  if (a.nseg < 1 || a.nseg > kThreads || !a.seg_list || !a.seg_meta) return hipErrorInvalidValue;
  const hipError_t attr = select_attributes();
  if (attr != hipSuccess) return attr;
  const int nw = (a.n + 31) / 32;
  const size_t lds = a.gbitmap ? sizeof(SelShared) : sizeof(SelShared) + (size_t)2 * nw * sizeof(uint32_t);
  if (a.cand) {
    if (a.gbitmap)
      hipLaunchKernelGGL((select_kernel<true, true, true>), dim3(rows), dim3(kThreads), lds, s, a);
    else
      hipLaunchKernelGGL((select_kernel<true, false, true>), dim3(rows), dim3(kThreads), lds, s, a);
  } else {
    if (a.gbitmap)
      hipLaunchKernelGGL((select_kernel<false, true, true>), dim3(rows), dim3(kThreads), lds, s, a);
    else
      hipLaunchKernelGGL((select_kernel<false, false, true>), dim3(rows), dim3(kThreads), lds, s, a);
  }
  return hipGetLastError();
}

int select_list_stride() { return kSeg; }
int select_list_max() { return kCap; }
int select_list_max_segments() { return kThreads; }

}  // namespace lsa
