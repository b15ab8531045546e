// Setup kernels, outside the decode step:
//   * the projected-key cache k_idx = K . W (JSSA, "Joint Subspace Sparse
//     Attention for Efficient Long-Context Decoding", Fig. 1; Fig. 9 calls
//     the key projection negligible), built for a range of tokens so a
//     decode loop can append the newest token;
//   * block centroids, the mean projected key of each block, scored by the
//     coarse pass of hierarchical indexing (LongCat Sparse Attention
//     abstract, item 3).
// Each output is a sum of exact products taken in fp64 and rounded once to
// the storage dtype (nearest-even), so it matches a double-precision
// reference bit for bit whatever the summation order.
#include "common.hpp"
#include "kernels.hpp"

namespace lsa {
namespace {

constexpr int kProjThreads = 256;
constexpr int kProjTokens = 32;

// Storage dtypes: 0 fp32, 1 bf16, 2 OCP E4M3 fp8.
template <int DT>
__device__ __forceinline__ void store_rounded(void* out, int64_t i, double x) {
  if constexpr (DT == 1) ((uint16_t*)out)[i] = f64_to_bf16_rne(x);
  else if constexpr (DT == 2) ((uint8_t*)out)[i] = f64_to_fp8_e4m3_rne(x);
  else ((float*)out)[i] = (float)x;
}

template <int DT>
__device__ __forceinline__ double load_stored(const void* p, int64_t i) {
  if constexpr (DT == 1) return (double)bf16_to_f32(((const uint16_t*)p)[i]);
  else if constexpr (DT == 2) return (double)__builtin_amdgcn_cvt_f32_fp8(((const uint8_t*)p)[i], 0);
  else return (double)((const float*)p)[i];
}

template <bool K_BF16, int OUT_DT>
__global__ __launch_bounds__(kProjThreads) void project_kernel(ProjectArgs a) {
  extern __shared__ float s_k[];  // [kProjTokens][d]
  const int g = blockIdx.y, n = blockIdx.z;
  const int t0 = a.tok_begin + blockIdx.x * kProjTokens;
  const int nt = min(kProjTokens, a.tok_begin + a.n_tok - t0);
  for (int e = threadIdx.x; e < nt * a.d; e += kProjThreads) {
    const int t = e / a.d, c = e % a.d;
    const int64_t off = (int64_t)n * a.ks_seq + (int64_t)(t0 + t) * a.ks_tok + (int64_t)g * a.ks_head + c;
    s_k[e] = K_BF16 ? bf16_to_f32(((const uint16_t*)a.k)[off]) : ((const float*)a.k)[off];
  }
  __syncthreads();
  const float* W = a.w + (a.w_per_head ? (int64_t)g * a.d * a.r : 0);
  const int tpar = kProjThreads / a.r;  // token lanes (r divides 256)
  const int j = threadIdx.x % a.r, tl = threadIdx.x / a.r;
  for (int t = tl; t < nt; t += tpar) {
    double acc = 0.0;
    const float* kt = s_k + t * a.d;
    for (int c = 0; c < a.d; ++c) acc = fma((double)kt[c], (double)W[(int64_t)c * a.r + j], acc);
    const int64_t o = (int64_t)n * a.os_seq + (int64_t)g * a.os_head + (int64_t)(t0 + t) * a.os_tok + j;
    store_rounded<OUT_DT>(a.out, o, acc);
  }
}

template <int DT>
__global__ __launch_bounds__(256) void centroid_kernel(CentroidArgs a) {
  const int b = blockIdx.x, g = blockIdx.y, n = blockIdx.z;
  const int t0 = b * a.block, t1 = min(a.T, t0 + a.block);
  for (int j = threadIdx.x; j < a.r; j += 256) {
    double s = 0.0;
    for (int t = t0; t < t1; ++t) {
      const int64_t off = (int64_t)n * a.is_seq + (int64_t)g * a.is_head + (int64_t)t * a.is_tok + j;
      s += load_stored<DT>(a.in, off);
    }
    const int64_t o = (int64_t)n * a.os_seq + (int64_t)g * a.os_head + (int64_t)b * a.os_blk + j;
    store_rounded<DT>(a.out, o, s / (double)(t1 - t0));
  }
}

template <bool K_BF16>
void launch_project_k(const ProjectArgs& a, int out_dt, dim3 grid, size_t lds, hipStream_t s) {
  if (out_dt == 1) hipLaunchKernelGGL((project_kernel<K_BF16, 1>), grid, dim3(kProjThreads), lds, s, a);
  else if (out_dt == 2) hipLaunchKernelGGL((project_kernel<K_BF16, 2>), grid, dim3(kProjThreads), lds, s, a);
  else hipLaunchKernelGGL((project_kernel<K_BF16, 0>), grid, dim3(kProjThreads), lds, s, a);
}

}  // namespace

hipError_t launch_project(const ProjectArgs& a, bool k_bf16, int out_dt, hipStream_t s) {
  if (a.n_tok <= 0) return hipSuccess;
  dim3 grid((unsigned)((a.n_tok + kProjTokens - 1) / kProjTokens), (unsigned)a.Hkv, (unsigned)a.N);
  const size_t lds = (size_t)kProjTokens * a.d * sizeof(float);
  if (k_bf16) launch_project_k<true>(a, out_dt, grid, lds, s);
  else launch_project_k<false>(a, out_dt, grid, lds, s);
  return hipGetLastError();
}

hipError_t launch_centroids(const CentroidArgs& a, int dt, hipStream_t s) {
  const int nb = (a.T + a.block - 1) / a.block;
  if (nb <= 0) return hipSuccess;
  dim3 grid((unsigned)nb, (unsigned)a.Hkv, (unsigned)a.N);
  if (dt == 1) hipLaunchKernelGGL((centroid_kernel<1>), grid, dim3(256), 0, s, a);
  else if (dt == 2) hipLaunchKernelGGL((centroid_kernel<2>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((centroid_kernel<0>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace lsa
