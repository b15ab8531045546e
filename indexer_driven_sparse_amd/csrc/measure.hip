// Measurement helper: a plain streaming read of a device buffer, the
// achievable-bandwidth reference against which the HBM-bound kernels of
// the hot path are judged (its rate, not the published peak alone, is what
// a memory-bound kernel can reach on this part).
//
// Workgroup b streams one contiguous share of the buffer (its 16-byte
// words [b * n16 / nb, (b + 1) * n16 / nb)), every lane issuing eight
// 16-byte nontemporal loads per loop step, each wave-wide load 1 KB of
// consecutive bytes. Contiguous shares read about a seventh faster on
// MI355X than a grid-stride sweep of the same buffer. The words are
// XOR-folded so the loads cannot be dropped, and workgroup b stores its
// fold to sink[b] (plain stores: no atomics contend on one address).
#include "common.hpp"
#include "kernels.hpp"

namespace lsa {
namespace {

constexpr int kReadThreads = 256;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(const u32x4* p, size_t n16,
                                                                   uint32_t* sink) {
  __shared__ uint32_t s_fold[kReadThreads / 64];
  constexpr int kU = 8;
  const size_t b0 = n16 * blockIdx.x / gridDim.x, b1 = n16 * (blockIdx.x + 1) / gridDim.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  size_t i = b0 + threadIdx.x;
  for (; i + (kU - 1) * kReadThreads < b1; i += kU * kReadThreads) {
    u32x4 v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) v[u] = __builtin_nontemporal_load(p + i + u * kReadThreads);
#pragma unroll
    for (int u = 0; u < kU; ++u) acc ^= v[u];
  }
  for (; i < b1; i += kReadThreads) acc ^= __builtin_nontemporal_load(p + i);
  uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x ^= (uint32_t)__shfl_xor((int)x, o, 64);
  if ((threadIdx.x & 63) == 0) s_fold[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t f = 0u;
#pragma unroll
    for (int w = 0; w < kReadThreads / 64; ++w) f ^= s_fold[w];
    sink[blockIdx.x] = f;
  }
}

}  // namespace

hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t s) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(kStreamReadBlocks), dim3(kReadThreads), 0, s,
                     (const u32x4*)buf, bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace lsa
