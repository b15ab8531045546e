// Device helpers shared by the liblsa kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lsa {

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// bf16 <-> fp32. bf16 is the top half of an IEEE binary32, so decoding is a
// shift; packed pairs come out of one 32-bit word.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Round a double to bf16, nearest-even, in one step (no intermediate float):
// drop the low 45 of the 52 fraction bits with the usual add-and-carry
// trick; below 2^-126 count units of 2^-133 with rint (exact scaling).
__device__ __forceinline__ uint16_t f64_to_bf16_rne(double x) {
  uint64_t u = (uint64_t)__double_as_longlong(x);
  uint16_t sign = (uint16_t)((u >> 48) & 0x8000u);
  uint64_t a = u & 0x7fffffffffffffffull;
  if (a > 0x7ff0000000000000ull) return sign | 0x7fc0u;   // NaN
  if (a == 0x7ff0000000000000ull) return sign | 0x7f80u;  // inf
  int e = (int)(a >> 52) - 1023;
  if (e >= -126) {
    uint64_t m = a & 0x000fffffffffffffull;
    uint64_t r = m + ((1ull << 44) - 1) + ((m >> 45) & 1);
    int e2 = e + (int)(r >> 52);
    if (e2 > 127) return sign | 0x7f80u;
    uint32_t f7 = (uint32_t)((r >> 45) & 0x7f);
    return sign | (uint16_t)(((uint32_t)(e2 + 127) << 7) | f7);
  }
  double q = rint(fabs(x) * 0x1p133);  // 0..128; 128 is the smallest normal
  return sign | (uint16_t)(uint32_t)q;
}

// OCP 8-bit float E4M3 ("FN": no infinities, largest finite 448, NaN 0x7f
// and 0xff): round a double to the nearest value, ties to even, straight
// from the double; beyond 448 the result saturates (the format has no
// infinity). Normal values keep 3 fraction bits: drop the low 49 of the 52
// with add-and-carry; below 2^-6 count units of 2^-9 with rint (exact
// scaling), which also rounds up into the smallest normal (0x08) correctly.
__device__ __forceinline__ uint8_t f64_to_fp8_e4m3_rne(double x) {
  const uint64_t u = (uint64_t)__double_as_longlong(x);
  const uint8_t sign = (uint8_t)((u >> 56) & 0x80u);
  const uint64_t a = u & 0x7fffffffffffffffull;
  if (a > 0x7ff0000000000000ull) return 0x7f;               // NaN
  const int e = (int)(a >> 52) - 1023;
  if (e < -6) return sign | (uint8_t)(int)rint(fabs(x) * 0x1p9);   // 0..8 units of 2^-9
  if (e > 8) return sign | 0x7e;                             // saturate (also inf)
  const uint64_t m = a & 0x000fffffffffffffull;
  const uint64_t r = m + ((1ull << 48) - 1) + ((m >> 49) & 1);
  const int e2 = e + (int)(r >> 52);
  const uint32_t f3 = (uint32_t)((r >> 49) & 7);
  if (e2 > 8 || (e2 == 8 && f3 == 7)) return sign | 0x7e;
  return sign | (uint8_t)(((uint32_t)(e2 + 7) << 3) | f3);
}

// Order-preserving key of an fp32 score: a larger score gives a larger key;
// -0 maps to +0; every NaN maps to 0, below -inf (0x007fffff).
__device__ __forceinline__ uint32_t order_key(float s) {
  uint32_t u = __float_as_uint(s);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0u;
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inverse of order_key (a NaN key gives a NaN; -0 comes back as +0).
__device__ __forceinline__ float key_to_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k ^ 0x80000000u) : ~k);
}

// ---------------------------------------------------------------------------
// Cross-lane sums with DPP (no LDS traffic). After sum_lanes<N>, every lane
// of each aligned group of N lanes (N in 1..16) holds the group's sum. The
// pairing (xor 1, xor 2, then mirror within 8 and 16) is fixed, so results
// are deterministic.
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
constexpr int kDppXor1 = 0xb1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4e;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7-i within 8
constexpr int kDppMirror = 0x140;     // lane i <-> 15-i within 16

template <int N>
__device__ __forceinline__ float sum_lanes(float v) {
  static_assert(N == 1 || N == 2 || N == 4 || N == 8 || N == 16, "group size");
  if constexpr (N >= 2) v += dpp<kDppXor1>(v);
  if constexpr (N >= 4) v += dpp<kDppXor2>(v);
  if constexpr (N >= 8) v += dpp<kDppHalfMirror>(v);
  if constexpr (N >= 16) v += dpp<kDppMirror>(v);
  return v;
}

template <int N>
__device__ __forceinline__ float max_lanes(float v) {
  if constexpr (N >= 2) v = fmaxf(v, dpp<kDppXor1>(v));
  if constexpr (N >= 4) v = fmaxf(v, dpp<kDppXor2>(v));
  if constexpr (N >= 8) v = fmaxf(v, dpp<kDppHalfMirror>(v));
  if constexpr (N >= 16) v = fmaxf(v, dpp<kDppMirror>(v));
  return v;
}

// 64-bit ballot and lane rank among the set lanes below this one.
__device__ __forceinline__ uint64_t ballot64(bool p) { return __ballot(p); }
__device__ __forceinline__ int rank_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
}

// Exclusive prefix sum over a block of NT threads (NT a multiple of 64, at
// most 1024). `scratch` holds NT/64 ints of LDS. Returns the exclusive
// prefix of `v`; *total receives the block sum. Every thread reads all wave
// totals (broadcast LDS reads), so only two barriers are paid. Every thread
// of the block must call it.
template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int v, int* scratch, int* total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) scratch[wid] = x;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const int t = scratch[w];
    base += w < wid ? t : 0;
    tot += t;
  }
  *total = tot;
  __syncthreads();   // scratch may be reused right after
  return base + x - v;
}

}  // namespace lsa
