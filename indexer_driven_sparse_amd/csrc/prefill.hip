// Causal prefill indexer (LongCat Sparse Attention, abstract: the indexer's
// O(L^2) causal scoring) with the per-row exact top-B of JSSA ("Joint
// Subspace Sparse Attention for Efficient Long-Context Decoding", Fig. 1:
// top-B positions, lowest position on equal scores) fused in: no L x L score
// matrix is written.
//
// Scores S[i,j] = q_idx[i] . k_idx[j] (j <= i) come from MFMA tiles
// (v_mfma_f32_32x32x16_bf16, r = 64 as four 16-deep chunks). Every prefill
// path -- the fused one, its fallback and the unfused score kernel -- runs
// the same MFMA sequence per tile, so equal inputs give bit-equal scores and
// the fused selection equals select-over-unfused-scores exactly.
//
// Fused selection, four kernels:
//   sample  per block of 32 query rows, MFMA scores against a jittered
//           stratified sample of at most 4096 keys of the causal prefix; per
//           row, two 8-bit radix levels give a threshold tau that the sample
//           says about B plus a 3.5-sigma margin of the row's keys reach;
//   cand    per block of 128 query rows (4 waves x 32) and one of two
//           interleaved halves of its causal key tiles (two workgroups per
//           block, so the longest blocks spread over two CUs); each score
//           >= tau of its row is appended, as (score bits, j), to the row's
//           sub-list for that half;
//   final   per row: if the list did not overflow and holds at least
//           min(B, i+1) entries, every key ranking above the B-th one is
//           among them, so a radix select over them is exact; the positions
//           go out ascending through an LDS bitmap. Otherwise the row is put
//           on a redo list (the sample decides speed, never the result);
//   redo    recomputes each listed row's scores (same MFMA sequence) into a
//           scratch row, then the general single-row select runs on it.
#include "select_row.hpp"

namespace lsa {
namespace {

using namespace sel;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kT = 32;           // keys per MFMA tile = query rows per block
constexpr int kCh = 4;           // rank 64 = four 16-deep chunks
constexpr int kRank = 16 * kCh;

constexpr int kSampleMax = 4096; // sampled keys per block of 32 query rows
constexpr int kHistLd = 257;     // padded histogram row: rows fall on different LDS banks
constexpr int kRowsA = 128;      // query rows per candidate workgroup
constexpr int kCandCap = 8192;   // candidate list entries per row
constexpr int kSplit = 2;        // workgroups per block of rows, each with its own sub-list
constexpr int kSubCap = kCandCap / kSplit;
constexpr int kFinThreads = 256;
constexpr int kFinPerMax = kCandCap / kFinThreads;  // candidates per thread, largest build (32)
constexpr int kRedoBlocks = 256;

// 8 bf16 of row p for chunk c and lane half h: elements 16c + 8h .. +8.
__device__ __forceinline__ bf16x8 frag(const uint16_t* p, int c, int h) {
  return __builtin_bit_cast(bf16x8, *(const u32x4*)(p + 16 * c + 8 * h));
}

// One tile: D[m][n] = sum_k K[m][k] * Q[n][k] for 32 keys m (operand A) and
// 32 queries n (operand B). Lane l holds query n = l % 32 and the keys
// tile_key(v, l / 32), v = 0..15.
__device__ __forceinline__ f32x16 tile_scores(const bf16x8 (&ka)[kCh], const bf16x8 (&qb)[kCh]) {
  f32x16 acc = {};
#pragma unroll
  for (int c = 0; c < kCh; ++c) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[c], qb[c], acc, 0, 0, 0);
  return acc;
}
__device__ __forceinline__ int tile_key(int v, int h) { return 8 * (v >> 2) + 4 * h + (v & 3); }

__device__ __forceinline__ const uint16_t* krow(const PrefillTopkArgs& a, int g, int j) {
  return a.k_idx + (int64_t)g * a.ks_head + (int64_t)j * a.ks_tok;
}
__device__ __forceinline__ const uint16_t* qrow(const PrefillTopkArgs& a, int g, int i) {
  return a.q_idx + ((int64_t)i * a.Hkv + g) * kRank;
}

// A tile of 32 rank-64 bf16 rows (keys or queries, 128 bytes each) staged
// through LDS. Loading operands straight from the rows puts a different row
// in each adjacent lane, so every lane's 16 bytes cost an L1 access of
// their own; the staged load reads each row with 8 lanes (lane l, step i:
// row 8i + l/8, 16-byte piece l%8), one access per 64 bytes. Piece p of
// row m sits at slot p ^ ((m/2) % 8), so the stores (two rows per 16
// lanes) and the operand reads (16 rows, one piece each per 16 lanes) both
// touch every bank once.
typedef uint32_t lds_x4 __attribute__((ext_vector_type(4), __may_alias__));
constexpr int kRowB = 2 * kRank;   // bytes per row
__device__ __forceinline__ int rtile_byte(int row, int piece) {
  return row * kRowB + 16 * (piece ^ ((row >> 1) & 7));
}
// step i of the staged load: 16 bytes of row 8i + l/8 (p = that row)
__device__ __forceinline__ u32x4 rtile_piece(const uint16_t* p, int lane) {
  return *(const u32x4*)(p + 8 * (lane & 7));
}
__device__ __forceinline__ void rtile_put(uint8_t* t, int i, int lane, u32x4 x) {
  *(lds_x4*)(t + rtile_byte(8 * i + (lane >> 3), lane & 7)) = x;
}
// the MFMA fragment frag() would load for row n, chunk c, lane half h
__device__ __forceinline__ bf16x8 rtile_frag(const uint8_t* t, int n, int c, int h) {
  return __builtin_bit_cast(bf16x8, *(const lds_x4*)(t + rtile_byte(n, 2 * c + h)));
}

// ---------------------------------------------------------------------------
// Unfused scores (topk == 0): full causal rows, -inf past each row's keys.
// Row i sees keys j < (i+1)*qblk (qblk = 1: j <= i; qblk > 1: the keys of a
// block of qblk query tokens). One wave per 32 x 32 tile; the tile is
// transposed through LDS so each row's 32 scores leave as 128 contiguous
// bytes.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void prefill_scores_mfma_kernel(PrefillTopkArgs a, float* scores,
                                                                 int64_t ld) {
  // the key and query tiles, then (once the operands are in registers) the
  // score tile over the same bytes: one wave, so its LDS reads of the
  // operands complete before its stores of the scores
  __shared__ __align__(16) uint8_t smem[2 * kT * kRowB];
  static_assert(sizeof(float) * kT * (kT + 1) <= sizeof(smem), "score tile fits");
  uint8_t* sk = smem;
  uint8_t* sq = smem + kT * kRowB;
  float (*tile)[kT + 1] = reinterpret_cast<float (*)[kT + 1]>(smem);
  const int lane = threadIdx.x, h = lane >> 5, n = lane & 31;
  const int kt = blockIdx.x, qt = blockIdx.y, g = blockIdx.z;
  const int j0 = kt * kT, i0 = qt * kT;
  if ((int64_t)j0 < (int64_t)(i0 + kT) * a.qblk) {   // some key of the tile is visible to some row
    u32x4 xk[4], xq[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = 8 * i + (lane >> 3);
      xk[i] = rtile_piece(krow(a, g, min(j0 + m, a.L - 1)), lane);
      xq[i] = rtile_piece(qrow(a, g, min(i0 + m, a.Lq - 1)), lane);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      rtile_put(sk, i, lane, xk[i]);
      rtile_put(sq, i, lane, xq[i]);
    }
    // one wave: its LDS stores complete before its reads
    bf16x8 ka[kCh], qb[kCh];
#pragma unroll
    for (int c = 0; c < kCh; ++c) {
      ka[c] = rtile_frag(sk, n, c, h);
      qb[c] = rtile_frag(sq, n, c, h);
    }
    const f32x16 acc = tile_scores(ka, qb);
#pragma unroll
    for (int v = 0; v < 16; ++v) tile[n][tile_key(v, h)] = acc[v];
  }
  __syncthreads();
  if (j0 + kT <= a.L && (ld & 3) == 0 && ((uintptr_t)scores & 15) == 0) {
    // 8 lanes per row, 16 bytes each: rows 8s + l/8, columns 4(l%8)..+3
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      const int r = 8 * s4 + (lane >> 3), q0 = 4 * (lane & 7);
      const int i = i0 + r;
      if (i >= a.Lq) continue;
      const int64_t jend = (int64_t)(i + 1) * a.qblk;   // this row's keys: j < jend
      float4 v;
      v.x = j0 + q0 < jend ? tile[r][q0] : -INFINITY;
      v.y = j0 + q0 + 1 < jend ? tile[r][q0 + 1] : -INFINITY;
      v.z = j0 + q0 + 2 < jend ? tile[r][q0 + 2] : -INFINITY;
      v.w = j0 + q0 + 3 < jend ? tile[r][q0 + 3] : -INFINITY;
      *reinterpret_cast<float4*>(scores + ((int64_t)i * a.Hkv + g) * ld + j0 + q0) = v;
    }
    return;
  }
  // the last tile of a row (the API keeps rows 16-byte aligned; the check
  // above also guards direct callers): lane pair (2r, 2r+1) writes row r's
  // scores, 16 each
  const int r = lane >> 1, half = lane & 1;
  const int i = i0 + r;
  if (i < a.Lq) {
    const int64_t jend = (int64_t)(i + 1) * a.qblk;   // this row's keys: j < jend
    float* out = scores + ((int64_t)i * a.Hkv + g) * ld + j0 + 16 * half;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int j = j0 + 16 * half + q;
      if (j < a.L) out[q] = (j < jend) ? tile[r][16 * half + q] : -INFINITY;
    }
  }
}

// Block queries: one workgroup of 64 lanes per (block, KV head); lane c
// adds channel c of the block's tokens in fp64, in token order, divides by
// the token count and rounds that mean once to bf16 (nearest-even). For
// inputs of ordinary range the fp64 sum is exact.
__global__ __launch_bounds__(kRank) void block_query_kernel(const uint16_t* q_idx, int L, int Hkv,
                                                           int qblk, uint16_t* out) {
  const int b = blockIdx.x, g = blockIdx.y, c = threadIdx.x;
  const int i0 = b * qblk, i1 = min(L, i0 + qblk);
  double s = 0.0;
  for (int i = i0; i < i1; ++i) s += (double)bf16_to_f32(q_idx[((int64_t)i * Hkv + g) * kRank + c]);
  out[((int64_t)b * Hkv + g) * kRank + c] = f64_to_bf16_rne(s / (double)(i1 - i0));
}

// ---------------------------------------------------------------------------
// sample: per-row threshold tau
// ---------------------------------------------------------------------------
// The histograms of two rows share words (row 2p in the low half of row
// p's words, row 2p + 1 in the high half): a count never exceeds
// kSampleMax < 2^16, and the halved size lets four workgroups share a CU.
struct SampleShared {
  uint32_t hist[kT / 2][kHistLd];
  int pos[kSampleMax];   // the block's sample positions, increasing
  int nvalid[kT];
  int target[kT];   // sample keys that should reach tau (0: no threshold)
  int bin1[kT];
  int bin2[kT];
  int need2[kT];    // of those, the ones inside bin1
};

// Sample position k of m over the prefix [0, nb): one key per stratum
// [k nb / m, (k+1) nb / m), at a fixed pseudo-random offset inside it (no
// aliasing with periodic structure in the keys). Increasing in k.
__device__ __forceinline__ int sample_pos(int k, int m, int nb) {
  if (nb <= m) return k;
  const int lo = (int)((int64_t)k * nb / m), hi = (int)((int64_t)(k + 1) * nb / m);
  return lo + (int)(((uint32_t)k * 2654435761u >> 8) % (uint32_t)(hi - lo));
}

// 8 threads per row: the bin where the count from the top of hist[row]
// reaches tgt; writes *bin_out and need2[row] = tgt - (count above).
__device__ __forceinline__ void sample_find(SampleShared& sh, const int* tgts, int* bin_out) {
  const int tid = threadIdx.x, row = tid >> 3, part = tid & 7;
  const int tgt = tgts[row];
  const uint32_t* hr = sh.hist[row >> 1];
  const int sh16 = 16 * (row & 1);
  int c = 0;
  for (int q = 0; q < 32; ++q) c += (int)((hr[255 - 32 * part - q] >> sh16) & 0xffffu);
  int incl = c;
#pragma unroll
  for (int o = 1; o < 8; o <<= 1) {
    const int y = __shfl_up(incl, o, 8);
    if (part >= o) incl += y;
  }
  int acc = incl - c;
  if (tgt > 0 && acc < tgt && tgt <= incl) {
    for (int q = 0; q < 32; ++q) {
      const int b = 255 - 32 * part - q;
      const int hb = (int)((hr[b] >> sh16) & 0xffffu);
      if (acc + hb >= tgt) {
        bin_out[row] = b;
        sh.need2[row] = tgt - acc;
        break;
      }
      acc += hb;
    }
  }
}

// at most 128 VGPRs: with the shared histogram words (33 KiB of LDS) four
// workgroups fit per CU, so more of the sample's gathers are in flight
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4, 8))) void prefill_sample_kernel(PrefillTopkArgs a, float* tau,
                                                             int* redo) {
  __shared__ SampleShared sh;
  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, n = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, uniform
  const int qt = blockIdx.x, g = blockIdx.y;
  const int i0 = qt * kT;
  if (qt == 0 && g == 0 && tid == 0) redo[0] = 0;   // the redo list starts empty
  if (i0 + kT <= a.B) {   // every row of the block keeps all its keys
    if (tid < kT && i0 + tid < a.L) tau[(int64_t)(i0 + tid) * a.Hkv + g] = -INFINITY;
    return;
  }
  const int nb = min(a.L, i0 + kT);          // keys any row of the block can see
  const int m = min(nb, kSampleMax);
  const int ntiles = (m + kT - 1) / kT;
  const int i = i0 + n;                      // this lane's query row
  bf16x8 qb[kCh];
  {
    const uint16_t* qp = qrow(a, g, min(i, a.L - 1));
#pragma unroll
    for (int c = 0; c < kCh; ++c) qb[c] = frag(qp, c, h);
  }
  for (int q = tid; q < kT / 2 * kHistLd; q += 256) (&sh.hist[0][0])[q] = 0u;
  for (int q = tid; q < m; q += 256) sh.pos[q] = sample_pos(q, m, nb);
  if (tid < kT) {
    sh.nvalid[tid] = 0;
    sh.bin1[tid] = -1;
    sh.bin2[tid] = -1;
    sh.need2[tid] = 0;
  }
  __syncthreads();
  // Tiles wholly inside every row's prefix (the common case) skip the
  // per-score checks; the order key here ignores the NaN and -0 cases,
  // which can only move tau (speed), never a result.
  const bool rows_in = i0 + kT <= a.L;
  uint32_t* hrow = &sh.hist[n >> 1][0];
  const uint32_t one = 1u << (16 * (n & 1));   // this row's half of the shared words
  for (int pass = 0; pass < 2; ++pass) {
    int nval = 0;
    const uint32_t b1 = pass ? (uint32_t)sh.bin1[n] : 0u;
    bf16x8 ka[kCh];
    if (w < ntiles) {
      const uint16_t* kp = krow(a, g, sh.pos[min(w * kT + n, m - 1)]);
#pragma unroll
      for (int c = 0; c < kCh; ++c) ka[c] = frag(kp, c, h);
    }
    for (int t = w; t < ntiles; t += 4) {
      // the products first, then the next tile's gathers into the same
      // registers: they fly during this tile's histogram work
      const f32x16 acc = tile_scores(ka, qb);
      if (t + 4 < ntiles) {
        const uint16_t* kp = krow(a, g, sh.pos[min((t + 4) * kT + n, m - 1)]);
#pragma unroll
        for (int c = 0; c < kCh; ++c) ka[c] = frag(kp, c, h);
      }
      const bool full = rows_in && (t + 1) * kT <= m && sh.pos[t * kT + kT - 1] <= i0;
      if (full) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const uint32_t u = __float_as_uint(acc[v]);
          const uint32_t key = u ^ ((uint32_t)((int)u >> 31) | 0x80000000u);
          if (pass == 0) atomicAdd(&hrow[key >> 24], one);
          else if ((key >> 24) == b1) atomicAdd(&hrow[(key >> 16) & 255u], one);
        }
        nval += 16;
      } else {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int k = t * kT + tile_key(v, h);
          if (k < m && i < a.L && sh.pos[k] <= i) {
            const uint32_t u = __float_as_uint(acc[v]);
            const uint32_t key = u ^ ((uint32_t)((int)u >> 31) | 0x80000000u);
            if (pass == 0) {
              atomicAdd(&hrow[key >> 24], one);
              ++nval;
            } else if ((key >> 24) == b1) {
              atomicAdd(&hrow[(key >> 16) & 255u], one);
            }
          }
        }
      }
    }
    if (pass == 0) atomicAdd(&sh.nvalid[n], nval);
    __syncthreads();
    if (pass == 0 && tid < kT) {
      // sample keys expected to rank among the row's top B, plus a
      // 3.5-sigma (binomial) margin and 6; 0 (no threshold) when that is the
      // whole sample. A miss costs a recomputed row, never the result.
      const int row = i0 + tid;
      const int mv = sh.nvalid[tid];
      int tgt = 0;
      if (row < a.L && mv > 0) {
        const double e = (double)a.B * mv / (double)(row + 1);
        const double k = ceil(e + 3.5 * sqrt(e) + 6.0);
        tgt = k < (double)mv ? (int)k : 0;
      }
      sh.target[tid] = tgt;
    }
    __syncthreads();
    if (pass == 0) sample_find(sh, sh.target, sh.bin1);
    else sample_find(sh, sh.need2, sh.bin2);
    __syncthreads();
    if (pass == 0) {
      for (int q = tid; q < kT / 2 * kHistLd; q += 256) (&sh.hist[0][0])[q] = 0u;
      __syncthreads();
    }
  }
  if (tid < kT && i0 + tid < a.L) {
    float t = -INFINITY;
    if (sh.target[tid] > 0 && sh.bin1[tid] >= 0 && sh.bin2[tid] >= 0) {
      const uint32_t key = ((uint32_t)sh.bin1[tid] << 24) | ((uint32_t)sh.bin2[tid] << 16);
      // every score whose key is >= this one; at or below -inf's key, all
      // scores but NaN
      t = key <= 0x007fffffu ? -INFINITY : key_to_float(key);
    }
    tau[(int64_t)(i0 + tid) * a.Hkv + g] = t;
  }
}

// ---------------------------------------------------------------------------
// cand: MFMA scores of 128 query rows x all their causal keys; every score
// >= its row's tau goes to the row's sub-list (wave w, lane half h).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void prefill_cand_kernel(PrefillTopkArgs a, const float* tau,
                                                           int2* cand, int* cnt) {
  __shared__ __align__(16) float stash[4][64][20];   // per wave, per lane: 16 scores (+pad)
  __shared__ int rcnt[kRowsA];                       // candidates appended per row
  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, n = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, uniform
  // kSplit workgroups share a block of rows: split s takes the groups of 4
  // tiles whose index is s modulo kSplit and fills sub-list s of each row
  const int job = gridDim.x - 1 - blockIdx.x;  // longest prefixes first
  const int blk = job / kSplit, split = job % kSplit;
  const int g = blockIdx.y;
  const int r0 = blk * kRowsA;
  const int kend = min(a.L, r0 + kRowsA);      // keys [0, kend) reach some row here
  if (tid < kRowsA) rcnt[tid] = 0;
  bf16x8 qb[4][kCh];
  float tq[4];
  int2* list[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int i = r0 + kT * b + n;
    const uint16_t* qp = qrow(a, g, min(i, a.L - 1));
#pragma unroll
    for (int ch = 0; ch < kCh; ++ch) qb[b][ch] = frag(qp, ch, h);
    tq[b] = i < a.L ? tau[(int64_t)i * a.Hkv + g] : INFINITY;
    list[b] = cand + ((int64_t)min(i, a.L - 1) * a.Hkv + g) * kCandCap + split * kSubCap;
  }
  __syncthreads();
  // Per tile: two row blocks' MFMAs, their epilogues, then the other two
  // blocks' MFMAs (after which the next tile's key loads go out) and their
  // epilogues. Each row has
  // one list; a lane reserves room for its candidates of the tile with one
  // LDS atomic and writes them as a contiguous run, so every row's list
  // grows at a single tail and the stores combine into full lines in L2.
  constexpr int kStep = 4 * kSplit;            // tiles between a wave's consecutive tiles
  const int t_first = 4 * split + w;
  bf16x8 ka[kCh];
  {
    const uint16_t* kp = krow(a, g, min(t_first * kT + n, a.L - 1));
#pragma unroll
    for (int ch = 0; ch < kCh; ++ch) ka[ch] = frag(kp, ch, h);
  }
  for (int t = t_first; t * kT < kend; t += kStep) {
    const int j0 = t * kT;
    // the tile's four row blocks in two halves of two: two accumulators
    // live instead of four (a third wave per SIMD fits in the registers);
    // the next tile's loads go out after the last products
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      f32x16 acc[2];
#pragma unroll
      for (int bb = 0; bb < 2; ++bb) acc[bb] = tile_scores(ka, qb[2 * hb + bb]);
      if (hb == 1 && (t + kStep) * kT < kend) {
        const uint16_t* kp = krow(a, g, min(j0 + kStep * kT + n, a.L - 1));
#pragma unroll
        for (int ch = 0; ch < kCh; ++ch) ka[ch] = frag(kp, ch, h);
      }
#pragma unroll
      for (int bb = 0; bb < 2; ++bb) {
        const int b = 2 * hb + bb;
        const int qlo = r0 + kT * b;
        if (j0 > qlo + kT - 1) continue;            // above every row's diagonal
        const int i = qlo + n;
        uint32_t flags = 0;
        if (j0 + kT - 1 <= qlo) {                   // the whole tile is causal for every row
#pragma unroll
          for (int v = 0; v < 16; ++v) flags |= (uint32_t)(acc[bb][v] >= tq[b]) << v;
        } else {
#pragma unroll
          for (int v = 0; v < 16; ++v)
            flags |= (uint32_t)(acc[bb][v] >= tq[b] && j0 + tile_key(v, h) <= i) << v;
        }
        if (__ballot(flags != 0)) {
          int pos = 0;
          if (flags) pos = atomicAdd(&rcnt[kT * b + n], __popc(flags));
          float4* st = reinterpret_cast<float4*>(&stash[w][lane][0]);
          st[0] = make_float4(acc[bb][0], acc[bb][1], acc[bb][2], acc[bb][3]);
          st[1] = make_float4(acc[bb][4], acc[bb][5], acc[bb][6], acc[bb][7]);
          st[2] = make_float4(acc[bb][8], acc[bb][9], acc[bb][10], acc[bb][11]);
          st[3] = make_float4(acc[bb][12], acc[bb][13], acc[bb][14], acc[bb][15]);
          while (flags) {
            const int v = __ffs(flags) - 1;
            flags &= flags - 1;
            if (pos < kSubCap)
              list[b][pos] = make_int2(__float_as_int(stash[w][lane][v]), j0 + tile_key(v, h));
            ++pos;
          }
        }
      }
    }
  }
  __syncthreads();
  if (tid < kRowsA && r0 + tid < a.L) cnt[((int64_t)(r0 + tid) * a.Hkv + g) * kSplit + split] = rcnt[tid];
}

// ---------------------------------------------------------------------------
// final: exact top-B of each row from its candidates
// ---------------------------------------------------------------------------
struct FinShared {
  uint32_t hist[kBins];
  int scan[kFinThreads / 64];
  uint32_t kmin, kmax;
  int bin, above;
};

// The bin holding the need-th largest of nb bins (scanned from the top):
// sh.bin, sh.above. Contains barriers.
__device__ __forceinline__ void fin_find_bin(FinShared& sh, int nb, int need) {
  const int t = threadIdx.x;
  const int per = (nb + kFinThreads - 1) / kFinThreads;
  const int hi = nb - 1 - t * per;
  int c = 0;
  if (per == 8) {   // 2048 bins: two 16-byte reads per thread, no bank conflicts
    const uint4 x = *(const uint4*)&sh.hist[hi - 7];
    const uint4 y = *(const uint4*)&sh.hist[hi - 3];
    c = (int)(x.x + x.y + x.z + x.w + y.x + y.y + y.z + y.w);
  } else {
    for (int k = 0; k < per; ++k)
      if (hi - k >= 0) c += (int)sh.hist[hi - k];
  }
  int tot;
  int acc = block_exclusive_scan<kFinThreads>(c, sh.scan, &tot);
  for (int k = 0; k < per; ++k) {
    if (hi - k < 0) break;
    const int hb = (int)sh.hist[hi - k];
    if (acc < need && need <= acc + hb) {
      sh.bin = hi - k;
      sh.above = acc;
    }
    acc += hb;
  }
  __syncthreads();
}

// Exclusive prefix of popcounts over words[0, nw) into pre[0, nw) (pre may
// not alias words). Contains barriers.
__device__ __forceinline__ void word_prefix(FinShared& sh, const uint32_t* words, uint32_t* pre,
                                            int nw) {
  const int per = (nw + kFinThreads - 1) / kFinThreads;
  const int w0 = threadIdx.x * per, w1 = min(nw, w0 + per);
  if (per == 8) {   // 32-byte runs: vector LDS access, no bank conflicts (the choice is block-uniform)
    uint32_t wv[8];
    if (w1 == w0 + 8) {
      const uint4 x = *(const uint4*)&words[w0];
      const uint4 y = *(const uint4*)&words[w0 + 4];
      wv[0] = x.x; wv[1] = x.y; wv[2] = x.z; wv[3] = x.w;
      wv[4] = y.x; wv[5] = y.y; wv[6] = y.z; wv[7] = y.w;
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) wv[q] = w0 + q < w1 ? words[w0 + q] : 0u;
    }
    uint32_t p[8], c = 0;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      p[q] = c;
      c += __popc(wv[q]);
    }
    int tot;
    const uint32_t off = (uint32_t)block_exclusive_scan<kFinThreads>((int)c, sh.scan, &tot);
    if (w1 == w0 + 8) {
      *(uint4*)&pre[w0] = make_uint4(off + p[0], off + p[1], off + p[2], off + p[3]);
      *(uint4*)&pre[w0 + 4] = make_uint4(off + p[4], off + p[5], off + p[6], off + p[7]);
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (w0 + q < w1) pre[w0 + q] = off + p[q];
    }
    __syncthreads();
    return;
  }
  int c = 0;
  for (int q = w0; q < w1; ++q) c += __popc(words[q]);
  int tot;
  int off = block_exclusive_scan<kFinThreads>(c, sh.scan, &tot);
  for (int q = w0; q < w1; ++q) {
    pre[q] = (uint32_t)off;
    off += __popc(words[q]);
  }
  __syncthreads();
}

template <int PER>   // candidates per thread: 16 (B <= 2048) or 32
__global__ __launch_bounds__(kFinThreads) void prefill_final_kernel(PrefillTopkArgs a,
                                                                   const int2* cand,
                                                                   const int* cnt, int* redo) {
  extern __shared__ __align__(16) unsigned char smem[];
  FinShared& sh = *reinterpret_cast<FinShared*>(smem);
  const int nw_max = (a.L + 31) >> 5;
  uint32_t* bm = reinterpret_cast<uint32_t*>(smem + sizeof(FinShared));   // selected
  // ties, then prefixes: used only after the radix levels, so it shares the
  // histogram's space when it fits (less LDS, more rows in flight per CU)
  uint32_t* aux = nw_max <= kBins ? sh.hist : bm + nw_max;
  const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
  const int i = row / a.Hkv;
  const int nv = i + 1;
  const int Bq = min(a.B, nv);
  const int nw = (nv + 31) >> 5;
  // slot k reads sub-list k / kPer, entry tid + 256 (k mod kPer); the
  // first 3/4 of each sub-list's slots are read together with the counts
  // (one memory latency; a typical list fills about that much), the rest
  // only when the sub-list is longer
  constexpr int kPer = PER / kSplit;
  constexpr int kSpec = (kPer * 3 + 3) / 4;
  const int2* crow = cand + (int64_t)row * kCandCap;
  int2 raw[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k)
    if (k % kPer < kSpec) raw[k] = crow[(k / kPer) * kSubCap + tid + kFinThreads * (k % kPer)];
  int tc[kSplit];
  int total = 0, longest = 0;
#pragma unroll
  for (int q = 0; q < kSplit; ++q) {
    tc[q] = cnt[(int64_t)row * kSplit + q];
    total += tc[q];
    longest = max(longest, tc[q]);
  }
  if (longest > kFinThreads * kPer || total < Bq) {   // the threshold missed: recompute this row
    if (tid == 0) redo[1 + atomicAdd(&redo[0], 1)] = row;
    return;
  }
#pragma unroll
  for (int k = 0; k < PER; ++k)
    if (k % kPer >= kSpec && kFinThreads * (k % kPer) < tc[k / kPer])
      raw[k] = crow[(k / kPer) * kSubCap + tid + kFinThreads * (k % kPer)];
  for (int q = tid; q < nw; q += kFinThreads) bm[q] = 0u;
  if (tid == 0) {
    sh.kmin = 0xffffffffu;
    sh.kmax = 0u;
  }
  // candidates e = tid + 256 k of the row's list
  uint32_t key[PER];
  int32_t jj[PER];
  uint32_t lo = 0xffffffffu, hi = 0u;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int e = tid + kFinThreads * (k % kPer);
    key[k] = 0u;
    jj[k] = -1;
    if (e < tc[k / kPer]) {
      const int2 x = raw[k];
      if (x.y >= 0 && x.y <= i) {   // always, for lists the candidate kernel wrote
        key[k] = order_key(__int_as_float(x.x));
        jj[k] = x.y;
        lo = min(lo, key[k]);
        hi = max(hi, key[k]);
      }
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    lo = min(lo, (uint32_t)__shfl_xor((int)lo, o, 64));
    hi = max(hi, (uint32_t)__shfl_xor((int)hi, o, 64));
  }
  __syncthreads();
  if (lane == 0) {
    atomicMin(&sh.kmin, lo);
    atomicMax(&sh.kmax, hi);
  }
  __syncthreads();

  // radix levels below the common prefix of [kmin, kmax], up to 11 bits
  // each; stop once the need-th key's bin is taken whole
  uint32_t pfx = 0u, bmask = 0u;
  int need = Bq, cnt_bin = total;
  bool all = total <= Bq;
  if (!all) {
    const uint32_t kmin = sh.kmin, kmax = sh.kmax;
    int fixed = kmin == kmax ? 32 : __clz(kmin ^ kmax);
    pfx = fixed == 0 ? 0u : (kmin & (~0u << (32 - fixed)));
    while (fixed < 32) {
      const int width = min(11, 32 - fixed);
      const int shift = 32 - fixed - width;
      const uint32_t pmask = fixed == 0 ? 0u : (~0u << (32 - fixed));
      const int nb = 1 << width;
      for (int q = tid; q < nb; q += kFinThreads) sh.hist[q] = 0u;
      __syncthreads();
#pragma unroll
      for (int k = 0; k < PER; ++k)
        if (jj[k] >= 0 && (key[k] & pmask) == pfx) atomicAdd(&sh.hist[(key[k] >> shift) & (nb - 1)], 1u);
      __syncthreads();
      fin_find_bin(sh, nb, need);
      const int bin = sh.bin;
      need -= sh.above;
      cnt_bin = (int)sh.hist[bin];
      pfx |= (uint32_t)bin << shift;
      fixed += width;
      __syncthreads();   // hist and bin are rewritten by the next level
      if (cnt_bin == need) break;
    }
    bmask = fixed >= 32 ? ~0u : (~0u << (32 - fixed));
  }
  const uint32_t top = pfx | ~bmask;

  // exact ties at the B-th key: the lowest positions win
  uint32_t tie_take = 0u;   // bit k: candidate k is a tie that is taken
  if (!all && cnt_bin > need) {
    for (int q = tid; q < nw; q += kFinThreads) aux[q] = 0u;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < PER; ++k)
      if (jj[k] >= 0 && key[k] == pfx) atomicOr(&aux[jj[k] >> 5], 1u << (jj[k] & 31));
    __syncthreads();
    word_prefix(sh, aux, bm, nw);   // bm holds the tie prefixes for now
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      if (jj[k] >= 0 && key[k] == pfx) {
        const int j = jj[k];
        const int rank = (int)bm[j >> 5] + __popc(aux[j >> 5] & ((1u << (j & 31)) - 1u));
        tie_take |= (uint32_t)(rank < need) << k;
      }
    }
    __syncthreads();
    for (int q = tid; q < nw; q += kFinThreads) bm[q] = 0u;
    __syncthreads();
  }

  // mark the selected positions, then write them in ascending order
  uint32_t sel = 0u;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    if (jj[k] < 0) continue;
    bool take;
    if (all) take = true;
    else if (key[k] > top) take = true;
    else if ((key[k] & bmask) != pfx) take = false;
    else take = cnt_bin == need || ((tie_take >> k) & 1u);
    if (take) {
      sel |= 1u << k;
      atomicOr(&bm[jj[k] >> 5], 1u << (jj[k] & 31));
    }
  }
  __syncthreads();
  word_prefix(sh, bm, aux, nw);
  int32_t* orow = a.out_idx + (int64_t)row * a.B;
  float* osc = a.out_score ? a.out_score + (int64_t)row * a.B : nullptr;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    if (!((sel >> k) & 1u)) continue;
    const int j = jj[k];
    const int pos = (int)aux[j >> 5] + __popc(bm[j >> 5] & ((1u << (j & 31)) - 1u));
    if (pos < a.B) {
      orow[pos] = j;
      if (osc) osc[pos] = key_to_float(key[k]);
    }
  }
  for (int p = Bq + tid; p < a.B; p += kFinThreads) {
    orow[p] = -1;
    if (osc) osc[p] = -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// redo: rows whose candidates did not settle the selection. The first
// kRedoBlocks listed rows: redo_scores writes row f's causal scores (same
// MFMA sequence, the query in every column) to scratch row f, then
// redo_select runs the general single-row select on it. Any further rows
// (a pathological input) go through redo_loop, which does both per row in
// one workgroup, kRedoBlocks rows at a time.
// ---------------------------------------------------------------------------
// Causal scores of one row into srow; this workgroup takes the tiles
// t = first + w, first + w + stride, ... (w its wave index).
__device__ __forceinline__ void redo_row_scores(const PrefillTopkArgs& a, int row, float* srow,
                                                int first, int stride) {
  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, n = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, uniform
  const int i = row / a.Hkv, g = row % a.Hkv;
  bf16x8 qb[kCh];
  {
    const uint16_t* qp = qrow(a, g, i);
#pragma unroll
    for (int c = 0; c < kCh; ++c) qb[c] = frag(qp, c, h);
  }
  for (int t = first + w; t * kT <= i; t += stride) {
    const int j0 = t * kT;
    bf16x8 ka[kCh];
    const uint16_t* kp = krow(a, g, min(j0 + n, a.L - 1));
#pragma unroll
    for (int c = 0; c < kCh; ++c) ka[c] = frag(kp, c, h);
    const f32x16 acc = tile_scores(ka, qb);
    // every column holds the same 32 scores: lane (n < 16, h) stores value n
    float x = acc[0];
#pragma unroll
    for (int v = 1; v < 16; ++v) x = (n & 15) == v ? acc[v] : x;
    const int j = j0 + tile_key(n & 15, h);
    if (n < 16 && j <= i) srow[j] = x;
  }
}

constexpr int kRedoSlices = 16;      // workgroups per redo row when all kRedoBlocks rows are listed
constexpr int kRedoSlicesMax = 128;  // ... and at most, when few are (16 waves each)

// The kRedoBlocks x kRedoSlices workgroups are shared by the listed rows:
// S = kRedoBlocks * kRedoSlices / n per row (at most kRedoSlicesMax), so a
// single listed row is scored by 2048 waves instead of 256.
__global__ __launch_bounds__(1024) void prefill_redo_scores_kernel(PrefillTopkArgs a, const int* redo,
                                                                   float* scratch) {
  const int n = min(redo[0], kRedoBlocks);
  if (n == 0) return;
  const int S = min(kRedoSlicesMax, kRedoBlocks * kRedoSlices / n);
  const int f = blockIdx.x / S, slice = blockIdx.x % S;
  if (f >= n) return;
  redo_row_scores(a, redo[1 + f], scratch + (int64_t)f * a.L, 16 * slice, 16 * S);
}

__device__ __forceinline__ void redo_row_select(const PrefillTopkArgs& a, int row, const float* srow,
                                                unsigned char* smem_raw) {
  const int i = row / a.Hkv;
  SelectArgs s{};
  s.scores = srow;
  s.scores_ld = a.L;
  s.n = i + 1;
  s.B = a.B;
  s.cand_block = 1;
  s.n_positions = i + 1;
  s.out_idx = a.out_idx;
  s.out_score = a.out_score;
  select_row<false, false, false>(s, row, srow, (int64_t)i + 1, smem_raw);
}

__global__ __launch_bounds__(kThreads) void prefill_redo_select_kernel(PrefillTopkArgs a,
                                                                       const int* redo,
                                                                       const float* scratch) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  const int f = blockIdx.x;
  if (f >= redo[0]) return;
  redo_row_select(a, redo[1 + f], scratch + (int64_t)f * a.L, smem_raw);
}

__global__ __launch_bounds__(kThreads) void prefill_redo_loop_kernel(PrefillTopkArgs a, const int* redo,
                                                                     float* scratch) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  float* srow = scratch + (int64_t)blockIdx.x * a.L;
  const int count = redo[0];
  for (int f = kRedoBlocks + blockIdx.x; f < count; f += gridDim.x) {
    const int row = redo[1 + f];
    redo_row_scores(a, row, srow, 0, kWaves);
    // the scratch row is complete and visible to the whole workgroup (the
    // acquire also drops lines the previous row left in the vector L1)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __syncthreads();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    redo_row_select(a, row, srow, smem_raw);
    __syncthreads();   // done with the scratch row before the next one
  }
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct PrefillWs {
  float* tau;
  int* cnt;
  int* redo;
  int2* cand;
  float* scratch;
};

size_t prefill_layout(int L, int Hkv, void* base, PrefillWs* ws) {
  const size_t rows = (size_t)L * Hkv;
  size_t off = 0;
  unsigned char* p = static_cast<unsigned char*>(base);
  const size_t o_tau = off;
  off = align256(off + rows * sizeof(float));
  const size_t o_cnt = off;
  off = align256(off + rows * kSplit * sizeof(int));
  const size_t o_redo = off;
  off = align256(off + (rows + 1) * sizeof(int));
  const size_t o_scr = off;
  off = align256(off + (size_t)kRedoBlocks * L * sizeof(float));
  const size_t o_cand = off;
  off += rows * kCandCap * sizeof(int2);
  if (ws) {
    ws->tau = reinterpret_cast<float*>(p + o_tau);
    ws->cnt = reinterpret_cast<int*>(p + o_cnt);
    ws->redo = reinterpret_cast<int*>(p + o_redo);
    ws->scratch = reinterpret_cast<float*>(p + o_scr);
    ws->cand = reinterpret_cast<int2*>(p + o_cand);
  }
  return off;
}

size_t fin_lds(int L) {
  const size_t nw = (L + 31) / 32;
  return sizeof(FinShared) + (nw <= (size_t)kBins ? 1 : 2) * nw * sizeof(uint32_t);
}
size_t redo_lds(int L) { return sizeof(SelShared) + (size_t)2 * ((L + 31) / 32) * sizeof(uint32_t); }

}  // namespace

bool prefill_topk_supported(int L, int r, int B) {
  return r == kRank && B >= 1 && B <= 4096 && L >= 1 && L <= kSelectLdsMaxSlots;
}

bool prefill_mfma_scores_supported(int r) { return r == kRank; }

size_t prefill_topk_workspace(int L, int Hkv, int B) {
  (void)B;
  return prefill_layout(L, Hkv, nullptr, nullptr);
}

hipError_t launch_prefill_topk(const PrefillTopkArgs& a, hipStream_t s) {
  static const hipError_t attr = [] {
    hipError_t e = hipFuncSetAttribute((const void*)prefill_final_kernel<16>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)fin_lds(kSelectLdsMaxSlots));
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute((const void*)prefill_final_kernel<kFinPerMax>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)fin_lds(kSelectLdsMaxSlots));
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute((const void*)prefill_redo_select_kernel,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)redo_lds(kSelectLdsMaxSlots));
    if (e != hipSuccess) return e;
    return hipFuncSetAttribute((const void*)prefill_redo_loop_kernel,
                               hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)redo_lds(kSelectLdsMaxSlots));
  }();
  if (attr != hipSuccess) return attr;
  PrefillWs ws;
  prefill_layout(a.L, a.Hkv, a.ws, &ws);
  const int rows = a.L * a.Hkv;
  hipLaunchKernelGGL(prefill_sample_kernel, dim3((a.L + kT - 1) / kT, a.Hkv), dim3(256), 0, s, a,
                     ws.tau, ws.redo);
  hipLaunchKernelGGL(prefill_cand_kernel, dim3((a.L + kRowsA - 1) / kRowsA * kSplit, a.Hkv),
                     dim3(256), 0, s, a, ws.tau, ws.cand, ws.cnt);
  // 16 register slots per thread hold 4096 candidates, twice a budget of
  // 2048 (the sample aims at about 1.4 B); larger budgets take 32
  if (a.B <= 2048)
    hipLaunchKernelGGL(prefill_final_kernel<16>, dim3(rows), dim3(kFinThreads), fin_lds(a.L), s, a,
                       ws.cand, ws.cnt, ws.redo);
  else
    hipLaunchKernelGGL(prefill_final_kernel<kFinPerMax>, dim3(rows), dim3(kFinThreads), fin_lds(a.L),
                       s, a, ws.cand, ws.cnt, ws.redo);
  hipLaunchKernelGGL(prefill_redo_scores_kernel, dim3(kRedoBlocks * kRedoSlices), dim3(1024), 0, s, a,
                     ws.redo, ws.scratch);
  hipLaunchKernelGGL(prefill_redo_select_kernel, dim3(kRedoBlocks), dim3(kThreads), redo_lds(a.L), s,
                     a, ws.redo, ws.scratch);
  hipLaunchKernelGGL(prefill_redo_loop_kernel, dim3(kRedoBlocks), dim3(kThreads), redo_lds(a.L), s, a,
                     ws.redo, ws.scratch);
  return hipGetLastError();
}

hipError_t launch_prefill_scores_mfma(const PrefillTopkArgs& a, float* scores, int64_t ld,
                                      hipStream_t s) {
  const dim3 grid((a.L + kT - 1) / kT, (a.Lq + kT - 1) / kT, a.Hkv);
  hipLaunchKernelGGL(prefill_scores_mfma_kernel, grid, dim3(64), 0, s, a, scores, ld);
  return hipGetLastError();
}

hipError_t launch_block_queries(const uint16_t* q_idx, int L, int Hkv, int qblk, uint16_t* out,
                                hipStream_t s) {
  const int nb = (L + qblk - 1) / qblk;
  hipLaunchKernelGGL(block_query_kernel, dim3(nb, Hkv), dim3(kRank), 0, s, q_idx, L, Hkv, qblk, out);
  return hipGetLastError();
}

}  // namespace lsa
