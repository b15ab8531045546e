// Measurement helper: a plain streaming read of a device buffer, the
// achievable-bandwidth reference against which the HBM-bound kernels of
// the hot path are judged (its rate, not the published peak alone, is what
// a memory-bound kernel can reach on this part).
//
// Every lane streams 16-byte nontemporal loads, four in flight per loop
// step, over a grid-stride range; the words are XOR-folded so the loads
// cannot be dropped, and workgroup b stores its fold to sink[b] (plain
// stores: no atomics contend on one address).
#include "common.hpp"
#include "kernels.hpp"

namespace lsa {
namespace {

constexpr int kReadThreads = 256;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(const u32x4* p, size_t n16,
                                                                   uint32_t* sink) {
  __shared__ uint32_t s_fold[kReadThreads / 64];
  const size_t stride = (size_t)gridDim.x * kReadThreads;
  size_t i = (size_t)blockIdx.x * kReadThreads + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = __builtin_nontemporal_load(p + i);
    const u32x4 b = __builtin_nontemporal_load(p + i + stride);
    const u32x4 c = __builtin_nontemporal_load(p + i + 2 * stride);
    const u32x4 d = __builtin_nontemporal_load(p + i + 3 * stride);
    acc ^= a ^ b ^ c ^ d;
  }
  for (; i < n16; i += stride) acc ^= __builtin_nontemporal_load(p + i);
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
