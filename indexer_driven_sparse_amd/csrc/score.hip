// Indexer scoring kernels (gfx950). The decode scoring body lives in
// score_body.hpp (shared with the fused decode step).
#include <algorithm>

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
