// Indexed attention over per-KV-head index sets (JSSA, "Joint Subspace
// Sparse Attention for Efficient Long-Context Decoding": Fig. 1 -- the query
// heads of a group share their KV head's top-B set; Key contributions -- a
// gather-free kernel for distinct per-KV-head selections under the standard
// GQA KV-cache layout; Fig. 6 -- gather-free versus gather-then-attend).
//
// Nothing is gathered into a copy: each selected K and V row is read once,
// in place, by 16 lanes (D/16 channels each), straight into registers.
// A workgroup of 4 waves = 16 lane groups owns one (row, KV head, split of
// the index list); the split's indices are staged in LDS, every lane group
// walks its share of keys 4 at a time (all 8 row loads issued before any
// math), keeps an online softmax in the log2 domain for all G heads and
// accumulates in fp32. Lane groups merge through DPP/LDS; splits merge in a
// second small kernel by log-sum-exp. Decode with G=4 is far too narrow for
// MFMA, so the math is fp32 FMA; the kernel is bound by the latency of the
// random 256-byte row reads, hence many splits and loads in flight.
#include "common.hpp"
#include "kernels.hpp"

namespace lsa {
namespace {

constexpr int kThreads = 256;
constexpr int kGroups = kThreads / 16;   // lane groups per workgroup
constexpr float kLn2 = 0.69314718055994530942f;

// keys a lane group loads per step: all of their K and V rows are requested
// before any math; fewer for wide groups to bound registers
template <int G>
constexpr int keys_per_step() { return G <= 4 ? 8 : 4; }

template <bool BF16, int CH>
struct RowLoad {
  static constexpr int kWords = CH * (BF16 ? 2 : 4) / 4;
  uint32_t w[kWords];
};

template <bool BF16, int CH>
__device__ __forceinline__ void load_row(RowLoad<BF16, CH>& r, const char* p) {
  constexpr int NW = RowLoad<BF16, CH>::kWords;
  if constexpr (NW == 2) {
    uint2 x = *(const uint2*)p;
    r.w[0] = x.x; r.w[1] = x.y;
  } else {
#pragma unroll
    for (int i = 0; i < NW / 4; ++i) {
      uint4 x = *(const uint4*)(p + 16 * i);
      r.w[4 * i] = x.x; r.w[4 * i + 1] = x.y; r.w[4 * i + 2] = x.z; r.w[4 * i + 3] = x.w;
    }
  }
}

template <bool BF16, int CH>
__device__ __forceinline__ float chan(const RowLoad<BF16, CH>& r, int c) {
  if constexpr (BF16) return (c & 1) ? bf16_hi(r.w[c >> 1]) : bf16_lo(r.w[c >> 1]);
  else return __uint_as_float(r.w[c]);
}

template <bool BF16, int G, int D>
__global__ __launch_bounds__(kThreads) void attn_kernel(AttnArgs a) {
  constexpr int kKC = keys_per_step<G>();
  constexpr int CH = D / 16;             // channels per lane
  constexpr int ESZ = BF16 ? 2 : 4;
  extern __shared__ __align__(16) unsigned char smem[];
  int32_t* s_idx = reinterpret_cast<int32_t*>(smem);                 // keys_per_split
  float* s_red = reinterpret_cast<float*>(smem) + a.keys_per_split;  // 4 waves x G x (D + 2)

  // flat grid: consecutive workgroups are the splits of one (row, KV head)
  const int64_t blk = blockIdx.x;
  const int split = (int)(blk % a.splits);
  const int g = (int)((blk / a.splits) % a.Hkv);
  const int row = (int)(blk / ((int64_t)a.splits * a.Hkv));
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int sub = lane & 15, grp = tid >> 4;   // lane within group, group within WG
  const int64_t seq = a.prefill ? 0 : row;

  // stage this split's indices
  const int k0 = split * a.keys_per_split;
  const int nk = max(0, min(a.B - k0, a.keys_per_split));
  // prefill: a selection may be shared by qblk consecutive query tokens,
  // and each token reads only positions up to its own (causal)
  const int64_t isel = a.prefill ? row / a.qblk : row;
  const int32_t* irow = a.idx + (isel * a.Hkv + g) * a.B + k0;
  const int tlim = a.prefill ? min(a.T, row + 1) : a.T;   // readable positions [0, tlim)
  if (a.slot) {
    // paged pool: translate position -> pool row once, here, so the row loads
    // below are the unpaged ones
    const int32_t* tab = a.slot + seq * a.slot_ld;
    for (int i = tid; i < nk; i += kThreads) {
      const int32_t t = irow[i];
      s_idx[i] = (t >= 0 && t < tlim) ? tab[t] : -1;
    }
  } else {
    for (int i = tid; i < nk; i += kThreads) {
      const int32_t t = irow[i];
      s_idx[i] = t < tlim ? t : -1;
    }
  }

  // this lane's query channels for the G heads, pre-scaled into log2 units
  float q[G][CH];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const int64_t qoff = ((int64_t)row * a.Hq + (int64_t)g * G + h) * D + sub * CH;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      float x = BF16 ? bf16_to_f32(((const uint16_t*)a.q)[qoff + c]) : ((const float*)a.q)[qoff + c];
      q[h][c] = x * a.scale_log2;
    }
  }
  float m[G], l[G], acc[G][CH];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int c = 0; c < CH; ++c) acc[h][c] = 0.f;
  }
  __syncthreads();

  const char* kbase = (const char*)a.k + (seq * a.s_seq + (int64_t)g * a.s_head) * ESZ + sub * CH * ESZ;
  const char* vbase = (const char*)a.v + (seq * a.s_seq + (int64_t)g * a.s_head) * ESZ + sub * CH * ESZ;
  const int64_t tok_bytes = a.s_tok * ESZ;

  for (int base = grp * kKC; base < nk; base += kGroups * kKC) {
    RowLoad<BF16, CH> kr[kKC], vr[kKC];
    bool ok[kKC];
#pragma unroll
    for (int j = 0; j < kKC; ++j) {
      const int i = base + j;
      const int32_t t = i < nk ? s_idx[i] : -1;
      ok[j] = t >= 0 && t < a.n_rows_kv;
      // unconditional loads (a skipped entry reads row 0, then is zeroed), so
      // all 2*kKC row requests of the step issue back to back
      const int64_t tc = ok[j] ? t : 0;
      load_row<BF16, CH>(kr[j], kbase + tc * tok_bytes);
      load_row<BF16, CH>(vr[j], vbase + tc * tok_bytes);
    }
#pragma unroll
    for (int j = 0; j < kKC; ++j) {
      if (!ok[j]) {
#pragma unroll
        for (int w = 0; w < RowLoad<BF16, CH>::kWords; ++w) kr[j].w[w] = vr[j].w[w] = 0u;
      }
    }
    float z[kKC][G];
#pragma unroll
    for (int j = 0; j < kKC; ++j) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float s = 0.f;
#pragma unroll
        for (int c = 0; c < CH; ++c) s = fmaf(q[h][c], chan<BF16, CH>(kr[j], c), s);
        s = sum_lanes<16>(s);
        z[j][h] = ok[j] ? s : -INFINITY;
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mc = z[0][h];
#pragma unroll
      for (int j = 1; j < kKC; ++j) mc = fmaxf(mc, z[j][h]);
      const float mn = fmaxf(m[h], mc);
      if (mn == -INFINITY) continue;         // nothing valid yet for this head
      const float rs = exp2f(m[h] - mn);     // 0 when m was -inf
      l[h] *= rs;
#pragma unroll
      for (int c = 0; c < CH; ++c) acc[h][c] *= rs;
#pragma unroll
      for (int j = 0; j < kKC; ++j) {
        const float p = exp2f(z[j][h] - mn);  // 0 for skipped keys
        l[h] += p;
#pragma unroll
        for (int c = 0; c < CH; ++c) acc[h][c] = fmaf(p, chan<BF16, CH>(vr[j], c), acc[h][c]);
      }
      m[h] = mn;
    }
  }

  // merge the 4 lane groups of this wave (lanes sub, sub+16, sub+32, sub+48)
#pragma unroll
  for (int off = 16; off <= 32; off <<= 1) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mo = __shfl_xor(m[h], off, 64);
      const float lo = __shfl_xor(l[h], off, 64);
      const float mn = fmaxf(m[h], mo);
      const float ra = mn == -INFINITY ? 0.f : exp2f(m[h] - mn);
      const float rb = mn == -INFINITY ? 0.f : exp2f(mo - mn);
      l[h] = l[h] * ra + lo * rb;
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        const float ao = __shfl_xor(acc[h][c], off, 64);
        acc[h][c] = acc[h][c] * ra + ao * rb;
      }
      m[h] = mn;
    }
  }
  // waves -> LDS: wave w stores m, l, acc for its G heads
  float* red = s_red + wid * G * (D + 2);
  if (lane < 16) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      if (sub == 0) {
        red[h * (D + 2)] = m[h];
        red[h * (D + 2) + 1] = l[h];
      }
#pragma unroll
      for (int c = 0; c < CH; ++c) red[h * (D + 2) + 2 + sub * CH + c] = acc[h][c];
    }
  }
  __syncthreads();

  const int64_t rowg = (int64_t)row * a.Hkv + g;
  for (int e = tid; e < G * D; e += kThreads) {
    const int h = e / D, c = e % D;
    float M = -INFINITY;
    for (int w = 0; w < 4; ++w) M = fmaxf(M, s_red[(w * G + h) * (D + 2)]);
    float L = 0.f, O = 0.f;
    if (M != -INFINITY) {
      for (int w = 0; w < 4; ++w) {
        const float* rw = s_red + (w * G + h) * (D + 2);
        const float f = exp2f(rw[0] - M);
        L += rw[1] * f;
        O += rw[2 + c] * f;
      }
    }
    if (a.splits == 1) {
      const int64_t oh = (int64_t)row * a.Hq + (int64_t)g * G + h;
      a.out[oh * D + c] = M == -INFINITY ? 0.f : O / L;
      if (c == 0 && a.lse) a.lse[oh] = M == -INFINITY ? -INFINITY : (M + log2f(L)) * kLn2;
    } else {
      float* pr = a.partial + ((rowg * a.splits + split) * G + h) * (D + 2);
      pr[2 + c] = O;
      if (c == 0) {
        pr[0] = M;
        pr[1] = L;
      }
    }
  }
}

// Merge the split partials of one (row, KV head) by log-sum-exp: one
// workgroup of G*D threads; thread (h, c) owns output channel c of head h.
// Every load is issued before any dependent math: (m, l) of all splits into
// LDS, and this thread's o of every split into registers.
constexpr int kMaxSplits = 64;

template <int G, int D>
__global__ __launch_bounds__(G * D) void attn_merge_kernel(AttnArgs a) {
  __shared__ float s_m[kMaxSplits * G], s_l[kMaxSplits * G];
  const int64_t rowg = blockIdx.x;
  const int row = (int)(rowg / a.Hkv), g = (int)(rowg % a.Hkv);
  const int t = threadIdx.x, h = t / D, c = t % D;
  const int S = a.splits;
  const int64_t sstride = (int64_t)G * (D + 2);
  const float* base = a.partial + rowg * S * sstride;
  if (t < S * G) {
    const int s = t / G, hh = t % G;
    s_m[t] = base[s * sstride + hh * (D + 2)];
    s_l[t] = base[s * sstride + hh * (D + 2) + 1];
  }
  float o[kMaxSplits];
#pragma unroll
  for (int s = 0; s < kMaxSplits; ++s)
    if (s < S) o[s] = base[s * sstride + h * (D + 2) + 2 + c];
  __syncthreads();
  float M = -INFINITY;
  for (int s = 0; s < S; ++s) M = fmaxf(M, s_m[s * G + h]);
  float L = 0.f, O = 0.f;
  if (M != -INFINITY) {
#pragma unroll
    for (int s = 0; s < kMaxSplits; ++s) {
      if (s < S) {
        const float f = exp2f(s_m[s * G + h] - M);
        L += s_l[s * G + h] * f;
        O += o[s] * f;
      }
    }
  }
  const int64_t oh = (int64_t)row * a.Hq + (int64_t)g * G + h;
  a.out[oh * D + c] = M == -INFINITY ? 0.f : O / L;
  if (c == 0 && a.lse) a.lse[oh] = M == -INFINITY ? -INFINITY : (M + log2f(L)) * kLn2;
}

template <bool BF16, int G, int D>
hipError_t launch_t(const AttnArgs& a, hipStream_t s) {
  const size_t lds = (size_t)a.keys_per_split * sizeof(int32_t) + (size_t)4 * G * (D + 2) * sizeof(float);
  dim3 grid((unsigned)((int64_t)a.splits * a.Hkv * a.rows));
  hipLaunchKernelGGL((attn_kernel<BF16, G, D>), grid, dim3(kThreads), lds, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.splits == 1) return e;
  hipLaunchKernelGGL((attn_merge_kernel<G, D>), dim3((unsigned)(a.rows * a.Hkv)), dim3(G * D), 0, s, a);
  return hipGetLastError();
}

template <bool BF16, int D>
hipError_t launch_g(const AttnArgs& a, int G, hipStream_t s) {
  switch (G) {
    case 1: return launch_t<BF16, 1, D>(a, s);
    case 2: return launch_t<BF16, 2, D>(a, s);
    case 4: return launch_t<BF16, 4, D>(a, s);
    case 8: return launch_t<BF16, 8, D>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_attention_merge(const AttnArgs& a, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  if (a.splits < 1 || a.splits > kMaxSplits) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(a.rows * a.Hkv));
#define LSA_MERGE(GG, DD)                                                            \
  if (G == GG && a.d == DD) {                                                        \
    hipLaunchKernelGGL((attn_merge_kernel<GG, DD>), grid, dim3(GG * DD), 0, s, a);   \
    return hipGetLastError();                                                        \
  }
  LSA_MERGE(4, 128)
  LSA_MERGE(8, 128)
#undef LSA_MERGE
  return hipErrorInvalidValue;
}

bool attention_supported(int G, int d) {
  return (d == 64 || d == 128) && (G == 1 || G == 2 || G == 4 || G == 8);
}

void attention_plan(int rows, int Hkv, int G, int d, int B, bool mfma_decode, int* splits,
                    int* keys_per_split) {
  (void)d;
  if (mfma_decode) {   // one workgroup per kDecodeSplit list entries
    *keys_per_split = kDecodeSplit;
    *splits = (B + kDecodeSplit - 1) / kDecodeSplit;
    return;
  }
  const int64_t units = (int64_t)rows * Hkv;
  const int unit_keys = kGroups * (G <= 4 ? 8 : 4);   // keys one workgroup covers per step
  int max_splits = min(kMaxSplits, (B + unit_keys - 1) / unit_keys);
  int sp = (int)((512 + units - 1) / units);  // about 2 workgroups per CU, all resident at once
  sp = max(1, min(sp, max_splits));
  int kps = (B + sp - 1) / sp;
  kps = (kps + unit_keys - 1) / unit_keys * unit_keys;
  sp = (B + kps - 1) / kps;
  *splits = sp;
  *keys_per_split = kps;
}

size_t attention_workspace(int rows, int Hkv, int G, int d, int B, bool mfma_decode) {
  int sp, kps;
  attention_plan(rows, Hkv, G, d, B, mfma_decode, &sp, &kps);
  if (sp == 1) return 0;
  return (size_t)rows * Hkv * sp * G * (d + 2) * sizeof(float);
}

hipError_t launch_attention(const AttnArgs& a, bool q_bf16, bool kv_bf16, hipStream_t s) {
  if (q_bf16 != kv_bf16) return hipErrorInvalidValue;
  const int G = a.Hq / a.Hkv;
  if (kv_bf16) return a.d == 128 ? launch_g<true, 128>(a, G, s) : launch_g<true, 64>(a, G, s);
  return a.d == 128 ? launch_g<false, 128>(a, G, s) : launch_g<false, 64>(a, G, s);
}

}  // namespace lsa
