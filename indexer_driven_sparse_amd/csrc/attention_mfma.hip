// Prefill indexed attention on the matrix cores (JSSA, "Joint Subspace
// Sparse Attention for Efficient Long-Context Decoding": Fig. 1 -- a KV
// head's query heads attend to its selected positions; Key contributions
// -- the selected rows are read in place from the standard GQA cache).
//
// Shapes served: bf16, head_dim 128; prefill with G = 8 query heads per KV
// head, decode with G = 4 or 8. Three kernels:
//   attn_mfma16_kernel  per-token selections: one wave per (token, KV head)
//                       on 16x16x32 tiles, rows = the 8 heads (+8 idle);
//   attn_mfma_kernel    selections shared by a block of tokens: a workgroup
//                       of 4 waves serves 16 tokens of the block, each wave
//                       32 rows (4 tokens x 8 heads) on 32x32x16 tiles;
//   attn_decode_mfma_kernel  decode: a workgroup of 8 waves per (sequence,
//                       KV head, split of 256 entries), one 32-key chunk per
//                       wave, combined in LDS into a split partial.
// Keys go by in chunks of 32 selected positions:
//   gather   each quad of lanes reads 64 contiguous bytes of one selected
//            K or V row (a wave covers whole 256-byte rows), and the rows
//            land in K and V tiles in LDS, one row per key with its 16-byte
//            pieces XOR-permuted per key so the stores and the operand reads
//            touch every bank once; QK reads its B operand from the K tile
//            with 128-bit LDS loads, PV reads V through gfx950's transposing
//            LDS read (ds_read_b64_tr_b16); the next chunk's list entries
//            and rows are in flight during the current chunk's products;
//   QK       S = Q K^T over the chunk's keys;
//   softmax  causal and list masks, scale, log2 domain; O and the row sums
//            stay relative to a reference max raised only when a score
//            passes it by 8, so p <= 256 and most chunks touch O only
//            through the MFMA; the row sum stays a per-lane partial;
//   PV       O += P V.
// Accumulation is fp32 throughout. p enters the PV product as two bf16
// terms, hi = bf16(p) and lo = bf16(p - hi), so its operand error is about
// 2^-17 relative instead of bf16's 2^-9 (one more MFMA per PV step). A
// skipped key's V row is zeroed before the product.
#include "common.hpp"
#include "kernels.hpp"

namespace lsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
// 128-bit LDS accesses of tiles that are also read or written at other
// widths (16-bit stores, transposing reads, float partials): the type
// aliases anything, so the compiler keeps them in program order
typedef uint32_t lds_x4 __attribute__((ext_vector_type(4), __may_alias__));

constexpr int kD = 128;          // head_dim
constexpr int kG = 8;            // query heads per KV head
constexpr int kKC = 32;          // keys per chunk
constexpr int kPLd = 40;         // LDS P row: 32 bf16 + 8 pad
constexpr float kLn2f = 0.69314718055994530942f;

// K and V of a 32-key chunk in LDS: one 256-byte row per key, its 16-byte
// pieces permuted by XOR with a per-key pattern. The gather fills them with
// each quad of lanes reading 64 contiguous bytes of one row (one L1 access
// per quad); the matrix-core operands are read back from them:
//   K: f(k) = 4 (k % 4) + (k / 4) % 4. The gather's stores (4 keys x 64
//      bytes per 16 lanes) and the QK B-operand reads (16 keys, one piece
//      each) touch every bank once.
//   V: f(k) = 4 (k % 4) + 2 ((k / 8) % 2). The stores as for K, and the P.V
//      B operand comes from gfx950's transposing LDS read: it gives lane j
//      of each 16-lane block element j%4 of the 8 bytes that lane 4e + j/4
//      of the block loaded, as its element e. For the 16x16x32 operand
//      (lane l: keys 8(l/16) + e, e = 0..7, of channel 16t + l%16), lane i
//      of block b loads channels 16t + 4(i%4)..+3 of key 8b + 4h + i/4, for
//      h = 0 and h = 1; the 8 keys a half wave reads sit in 8 bank groups.
constexpr int kRowBytes = 2 * kD;   // one key's K or V row
__device__ __forceinline__ int ktile_byte(int key, int byte) {
  const int f = 4 * (key & 3) + ((key >> 2) & 3);
  return key * kRowBytes + (((byte >> 4) ^ f) << 4) + (byte & 15);
}
__device__ __forceinline__ int vtile_byte(int key, int byte) {
  const int f = 4 * (key & 3) + 2 * ((key >> 3) & 1);
  return key * kRowBytes + (((byte >> 4) ^ f) << 4) + (byte & 15);
}
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4* lds_i16x4_ptr;
// the B operand of O += P V for channels 16t..16t+15 over keys 0..31
__device__ __forceinline__ bf16x8 vtile_operand16(const uint8_t* sV, int t, int lane) {
  const int i = lane & 15, key = 8 * (lane >> 4) + (i >> 2), byte = 32 * t + 8 * (i & 3);
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr)(sV + vtile_byte(key, byte)));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr)(sV + vtile_byte(key + 4, byte)));
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  const i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// two p values as hi + lo bf16 terms, hi = bf16(p) and lo = bf16(p - hi),
// both round-to-nearest-even by gfx950's packed conversion; element 0 in
// the low halves
__device__ __forceinline__ void split2_bf16(float p0, float p1, uint32_t& hi, uint32_t& lo) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  hi = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){p0, p1}, bf16x2));
  const float h0 = __uint_as_float(hi << 16), h1 = __uint_as_float(hi & 0xffff0000u);
  lo = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){p0 - h0, p1 - h1}, bf16x2));
}

// Block-shared selections: kTPW tokens per wave, kNW waves per workgroup; a
// workgroup serves the tokens [tok0, tok0 + kTPW * kNW) of one block, which
// share index row `isel`. The workgroup gathers each 32-key chunk once, into
// K and V tiles in LDS (double-buffered: the next chunk's rows are in flight
// while every wave computes on this one), one barrier per chunk.
constexpr int kTPW = 4, kNW = 4;
constexpr int kTileBytes = kKC * kRowBytes;                    // one K or V tile
constexpr int kBlkWaveBytes = 2 * kKC * kPLd * 2;              // per wave: P hi, P lo
constexpr int kBlkLds = 2 * (2 * kTileBytes + kKC * 4) + kNW * kBlkWaveBytes;

// the B operand of O += P V on 32x32x16 tiles for channels 32t..32t+31 and
// keys 16kc..16kc+15 (lane l: keys 16kc + 8(l/32) + e of channel 32t +
// l%32): lane i of 16-lane block b loads channels 32t + 16(b%2) + 4(i%4)..+3
// of key 16kc + 8(b/2) + 4h + i/4, for h = 0 and h = 1
__device__ __forceinline__ bf16x8 vtile_operand32(const uint8_t* sV, int t, int kc, int lane) {
  const int b = lane >> 4, i = lane & 15;
  const int key = 16 * kc + 8 * (b >> 1) + (i >> 2), byte = 64 * t + 32 * (b & 1) + 8 * (i & 3);
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr)(sV + vtile_byte(key, byte)));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr)(sV + vtile_byte(key + 4, byte)));
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  const i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

__global__ __launch_bounds__(64 * kNW) void attn_mfma_kernel(AttnArgs a) {
  constexpr int TPW = kTPW, NW = kNW;
  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5, n = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // two buffers of (K tile, V tile, key positions), then each wave's P
  uint8_t* sBuf = smem;
  uint16_t* sP = reinterpret_cast<uint16_t*>(smem + 2 * (2 * kTileBytes + kKC * 4) + w * kBlkWaveBytes);
  uint16_t* sPl = sP + kKC * kPLd;

  // ceil(qblk / (TPW NW)) workgroups per (block, KV head)
  const int g = blockIdx.y;
  const int per_blk = (a.qblk + TPW * NW - 1) / (TPW * NW);
  const int blk = blockIdx.x / per_blk, part = blockIdx.x % per_blk;
  const int isel = blk;
  const int tok0 = blk * a.qblk + part * TPW * NW;
  const int ntok = min(min(TPW * NW, a.qblk - part * TPW * NW), a.rows - tok0);
  const int32_t* ilist = a.idx + ((int64_t)isel * a.Hkv + g) * a.B;

  // this wave's 32 rows: row r -> token w*TPW + r/8, head r%8
  bf16x8 qa[kD / 16];
  {
    const int r = n;
    const int tt = w * TPW + r / kG;
    const bool live = tt < ntok;
    const int64_t qoff = ((int64_t)(tok0 + (live ? tt : 0)) * a.Hq + (int64_t)g * kG + (r % kG)) * kD;
    const uint16_t* qp = (const uint16_t*)a.q + qoff + 8 * hh;
#pragma unroll
    for (int c = 0; c < kD / 16; ++c) {
      u32x4 x = live ? *(const u32x4*)(qp + 16 * c) : u32x4{0u, 0u, 0u, 0u};
      qa[c] = __builtin_bit_cast(bf16x8, x);
    }
  }
  // rows this lane holds in S and O (v = 0..15): 8(v/4) + 4hh + v%4; the
  // token of row v is v/4
  constexpr int kV = 16;                   // row slots per lane
  int ipos[kV];                            // each live row's token position (-1: none)
#pragma unroll
  for (int v = 0; v < kV; ++v) {
    const int tt = w * TPW + v / 4;
    ipos[v] = tt < ntok ? tok0 + tt : -1;
  }

  float m[kV], l[kV];
  f32x16 o[kD / 32];
#pragma unroll
  for (int v = 0; v < kV; ++v) {
    m[v] = -INFINITY;
    l[v] = 0.f;
  }
#pragma unroll
  for (int t = 0; t < kD / 32; ++t) o[t] = f32x16{};

  const int nch = (a.B + kKC - 1) / kKC;
  const int64_t tok_bytes = a.s_tok * 2;
  const int tlim = a.T;
  // The gather: thread t reads pieces t%8 and 8 + t%8 (16 bytes each) of
  // the K and V rows of one key of a chunk -- a quad per 64 contiguous
  // bytes. Threads 8j..8j+7 serve key gk(j), a bijection on 0..31 that gives
  // each 16 threads two keys whose tile pieces land in opposite bank halves.
  const int gk = ((tid >> 5) << 2) | (((tid >> 3) & 1) << 1) | ((tid >> 4) & 1), gp = tid & 7;
  const char* kb0 = (const char*)a.k + ((int64_t)g * a.s_head) * 2 + 16 * gp;
  const char* vb0 = (const char*)a.v + ((int64_t)g * a.s_head) * 2 + 16 * gp;
  u32x4 kreg[2], vreg[2];
  int32_t gpos = -1;   // key gk of the chunk in flight: its position (-1: skipped)
  auto fetch = [&](int c) {
    const int e = c * kKC + gk;
    int32_t t = e < a.B ? ilist[e] : -1;
    if (t < 0 || t >= tlim) t = -1;
    int64_t row = t < 0 ? 0 : t;
    if (a.slot && t >= 0) {
      const int32_t pr = a.slot[t];
      if (pr < 0 || pr >= a.n_rows_kv) t = -1;
      row = t < 0 ? 0 : pr;
    }
    gpos = t;
    const char* kr = kb0 + row * tok_bytes;
    const char* vr = vb0 + row * tok_bytes;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      kreg[u] = *(const u32x4*)(kr + 128 * u);
      vreg[u] = *(const u32x4*)(vr + 128 * u);
    }
  };

  if (nch > 0) fetch(0);
  for (int c = 0; c < nch; ++c) {
    uint8_t* sK = sBuf + (c & 1) * (2 * kTileBytes + kKC * 4);
    uint8_t* sV = sK + kTileBytes;
    int32_t* sPos = reinterpret_cast<int32_t*>(sV + kTileBytes);
    // this chunk's rows to the tiles; a skipped key's V row is zeroed, so
    // its p = 0 never meets a NaN or Inf (the buffer was last read two
    // chunks ago, before the previous barrier)
    {
      const uint32_t vkeep = gpos >= 0 ? ~0u : 0u;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        *(lds_x4*)(sK + ktile_byte(gk, 16 * gp + 128 * u)) = kreg[u];
        *(lds_x4*)(sV + vtile_byte(gk, 16 * gp + 128 * u)) = vreg[u] & vkeep;
      }
      if (gp == 0) sPos[gk] = gpos;
    }
    __syncthreads();
    if (c + 1 < nch) fetch(c + 1);   // the next chunk's rows fly during this chunk's products
    const int32_t pos = sPos[n];     // key n of chunk c: its position in the sequence (-1: none)
    // S = Q K^T over the chunk's 32 keys: B = K (key n, channels 16q + 8hh ..)
    f32x16 s = f32x16{};
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const u32x4 kb = *(const lds_x4*)(sK + ktile_byte(n, 32 * q + 16 * hh));
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[q], __builtin_bit_cast(bf16x8, kb), s, 0, 0, 0);
    }
    // masks and scale; O and l stay relative to a reference max m per row,
    // raised (with a rescale of O and l) only when a score passes m + 8 in
    // the log2 domain -- a few times per row -- so p = exp2(x - m) <= 256
    // and the common chunk touches O only through the MFMA. y = the scaled
    // score minus m (-inf where masked; +inf while m is -inf).
    const bool kvalid = pos >= 0;
    const float sc = a.scale_log2;
    bool ok[4];   // rows v hold token v/4
#pragma unroll
    for (int tq = 0; tq < 4; ++tq) ok[tq] = kvalid && pos <= ipos[4 * tq];
    float y[kV];
    bool raise = false;
#pragma unroll
    for (int v = 0; v < kV; ++v) {
      y[v] = ok[v >> 2] ? fmaf(s[v], sc, -m[v]) : -INFINITY;
      raise |= y[v] > 8.f;
    }
    if (__builtin_amdgcn_ballot_w64(raise)) {
#pragma unroll
      for (int v = 0; v < kV; ++v) {
        float mm = ok[v >> 2] ? s[v] * sc : -INFINITY;
#pragma unroll
        for (int off = 1; off < 32; off <<= 1) mm = fmaxf(mm, __shfl_xor(mm, off, 64));
        const float mn = fmaxf(m[v], mm);
        const float alpha = mn == -INFINITY || m[v] == -INFINITY ? 0.f : exp2f(m[v] - mn);
        l[v] *= alpha;
#pragma unroll
        for (int t = 0; t < kD / 32; ++t) o[t][v] *= alpha;
        m[v] = mn;
        y[v] = ok[v >> 2] ? fmaf(s[v], sc, -mn) : -INFINITY;
      }
    }
#pragma unroll
    for (int v = 0; v < kV; v += 2) {
      // y <= 8 or -inf here: the raw exp2 (no denormal rescaling) suffices
      const float p0 = __builtin_amdgcn_exp2f(y[v]);
      const float p1 = __builtin_amdgcn_exp2f(y[v + 1]);
      l[v] += p0;
      l[v + 1] += p1;
      uint32_t hi, lo;
      split2_bf16(p0, p1, hi, lo);
      const int r0 = 8 * (v >> 2) + 4 * hh + (v & 3);
      sP[r0 * kPLd + n] = (uint16_t)hi;
      sP[(r0 + 1) * kPLd + n] = (uint16_t)(hi >> 16);
      sPl[r0 * kPLd + n] = (uint16_t)lo;
      sPl[(r0 + 1) * kPLd + n] = (uint16_t)(lo >> 16);
    }
    // O += P V (two 16-key halves of the chunk)
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      const bf16x8 pa = __builtin_bit_cast(bf16x8, *(const lds_x4*)(sP + n * kPLd + 16 * kc + 8 * hh));
      const bf16x8 pl = __builtin_bit_cast(bf16x8, *(const lds_x4*)(sPl + n * kPLd + 16 * kc + 8 * hh));
#pragma unroll
      for (int t = 0; t < kD / 32; ++t) {
        const bf16x8 vb = vtile_operand32(sV, t, kc, lane);
        o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa, vb, o[t], 0, 0, 0);
        o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pl, vb, o[t], 0, 0, 0);
      }
    }
  }

  // row sums over the 32 key lanes, then out = O / L, lse = m + log2 L
#pragma unroll
  for (int v = 0; v < kV; ++v) {
    float L = l[v];
#pragma unroll
    for (int off = 1; off < 32; off <<= 1) L += __shfl_xor(L, off, 64);
    const int r = 8 * (v >> 2) + 4 * hh + (v & 3);
    const int tt = w * TPW + v / 4;
    if (ipos[v] < 0 || tt >= ntok) continue;
    const int head = r % kG;
    const int64_t oh = (int64_t)(tok0 + tt) * a.Hq + (int64_t)g * kG + head;
    const bool empty = m[v] == -INFINITY;
#pragma unroll
    for (int t = 0; t < kD / 32; ++t) a.out[oh * kD + 32 * t + n] = empty ? 0.f : o[t][v] / L;
    if (n == 0 && a.lse) a.lse[oh] = empty ? -INFINITY : (m[v] + log2f(L)) * kLn2f;
  }
}

// Per-token selections: one wave per (token, KV head) on 16x16x32 tiles:
// rows = the 8 heads (+ 8 idle), columns = 16 keys. Lane l: A row / B
// column / D column l % 16, operand k-elements 8 (l / 16) + e, D rows
// 4 (l / 16) + v -- heads live in lanes 0..31. A 32-key chunk is two
// 16-key column tiles for QK and one 32-deep step for PV.
constexpr int kP16Ld = 40;   // LDS P row: 32 bf16 + 8 pad
__global__ __launch_bounds__(64) void attn_mfma16_kernel(AttnArgs a) {
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  __shared__ __align__(16) uint8_t sK[kKC * kRowBytes];   // K of the chunk
  __shared__ __align__(16) uint8_t sV[kKC * kRowBytes];   // V of the chunk
  __shared__ __align__(16) uint16_t sP[16 * kP16Ld];    // P hi (rows 8..15 stay zero)
  __shared__ __align__(16) uint16_t sPl[16 * kP16Ld];   // P lo
  const int lane = threadIdx.x, q4 = lane >> 4, c16 = lane & 15;
  const int g = blockIdx.y;
  const int tok = blockIdx.x;
  const int32_t* ilist = a.idx + ((int64_t)tok * a.Hkv + g) * a.B;

  // Q: row c16 = head c16 (< 8; idle rows are zero), channels 32c + 8 q4 ..
  bf16x8 qa[kD / 32];
  {
    const bool live = c16 < kG;
    const uint16_t* qp = (const uint16_t*)a.q + ((int64_t)tok * a.Hq + (int64_t)g * kG + (live ? c16 : 0)) * kD + 8 * q4;
#pragma unroll
    for (int c = 0; c < kD / 32; ++c) {
      u32x4 x = live ? *(const u32x4*)(qp + 32 * c) : u32x4{0u, 0u, 0u, 0u};
      qa[c] = __builtin_bit_cast(bf16x8, x);
    }
  }
  for (int e = lane; e < 8 * kP16Ld; e += 64) sP[8 * kP16Ld + e] = sPl[8 * kP16Ld + e] = 0;

  float m[4], l[4];   // rows 4 q4 + v (heads in lanes 0..31)
  f32x4 o[kD / 16];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    m[v] = -INFINITY;
    l[v] = 0.f;
  }
#pragma unroll
  for (int t = 0; t < kD / 16; ++t) o[t] = f32x4{};

  const int nch = (a.B + kKC - 1) / kKC;
  const int64_t tok_bytes = a.s_tok * 2;
  // The gather: lane l reads bytes 64j + 16(l%4) (j < 4) of the K and V
  // rows of keys l/4 and 16 + l/4 of a chunk -- a quad per 64 contiguous
  // bytes -- and stores them to the LDS tiles.
  const int kq = lane >> 2, r4 = lane & 3;
  const char* kb0 = (const char*)a.k + ((int64_t)g * a.s_head) * 2 + 16 * r4;
  const char* vb0 = (const char*)a.v + ((int64_t)g * a.s_head) * 2 + 16 * r4;
  const int tlim = a.T;
  // A chunk's list entries are loaded a chunk ahead of its rows (clamped
  // into the list, unconditionally, and checked only when used), so the
  // gather never waits for its own index load.
  u32x4 kreg[2][4], vreg[2][4];
  auto load_entries = [&](int c, int32_t (&ent)[2]) {
#pragma unroll
    for (int tn = 0; tn < 2; ++tn) ent[tn] = ilist[min(c * kKC + 16 * tn + kq, a.B - 1)];
  };
  // pos: this lane's gather keys (-1 = skipped); posc: the keys of its
  // score columns c16 and 16 + c16
  auto fetch = [&](int c, const int32_t (&ent)[2], int32_t (&pos)[2], int32_t (&posc)[2]) {
#pragma unroll
    for (int tn = 0; tn < 2; ++tn) {
      int32_t t = c * kKC + 16 * tn + kq < a.B ? ent[tn] : -1;
      if (t < 0 || t >= tlim) t = -1;
      int64_t row = t < 0 ? 0 : t;
      if (a.slot && t >= 0) {
        const int32_t pr = a.slot[t];
        if (pr < 0 || pr >= a.n_rows_kv) t = -1;
        row = t < 0 ? 0 : pr;
      }
      pos[tn] = t;
      const char* kr = kb0 + row * tok_bytes;
      const char* vr = vb0 + row * tok_bytes;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        kreg[tn][j] = *(const u32x4*)(kr + 64 * j);
        vreg[tn][j] = *(const u32x4*)(vr + 64 * j);
      }
    }
#pragma unroll
    for (int tn = 0; tn < 2; ++tn) posc[tn] = __shfl(pos[tn], 4 * c16, 64);
  };
  int32_t posg[2] = {-1, -1}, posn[2] = {-1, -1}, ent[2] = {-1, -1};
  if (nch > 0) {
    load_entries(0, ent);
    fetch(0, ent, posg, posn);
    load_entries(1, ent);
  }
  for (int c = 0; c < nch; ++c) {
    const int32_t pos0 = posn[0], pos1 = posn[1];
    // this chunk's rows to LDS (the previous chunk's reads are done: same
    // wave); a skipped key's V row is zeroed, so its p = 0 never meets a
    // NaN or Inf
    if (__builtin_amdgcn_ballot_w64(posg[0] < 0 || posg[1] < 0)) {
#pragma unroll
      for (int tn = 0; tn < 2; ++tn) {
        const uint32_t vkeep = posg[tn] >= 0 ? ~0u : 0u;
#pragma unroll
        for (int j = 0; j < 4; ++j) vreg[tn][j] &= vkeep;
      }
    }
#pragma unroll
    for (int tn = 0; tn < 2; ++tn) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        *(lds_x4*)(sK + ktile_byte(16 * tn + kq, 64 * j + 16 * r4)) = kreg[tn][j];
        *(lds_x4*)(sV + vtile_byte(16 * tn + kq, 64 * j + 16 * r4)) = vreg[tn][j];
      }
    }
    if (c + 1 < nch) {   // the next chunk's rows fly during this chunk's products
      const int32_t cur[2] = {ent[0], ent[1]};
      fetch(c + 1, cur, posg, posn);
      load_entries(c + 2, ent);
    }
    // S = Q K^T: B = K (key 16 tn + c16, channels 32q + 8 q4 ..)
    f32x4 s[2];
#pragma unroll
    for (int tn = 0; tn < 2; ++tn) {
      s[tn] = f32x4{};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const u32x4 kb = *(const lds_x4*)(sK + ktile_byte(16 * tn + c16, 64 * q + 16 * q4));
        s[tn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[q], __builtin_bit_cast(bf16x8, kb), s[tn], 0, 0, 0);
      }
    }
    // masks and scale; O and l relative to a reference max m raised only
    // when a score passes it by 8 (log2 domain), so p <= 256. y = the
    // scaled score minus m (-inf where masked; +inf while m is -inf).
    const int i = tok;   // causal: positions up to the token's own
    const bool ok0 = pos0 >= 0 && pos0 <= i, ok1 = pos1 >= 0 && pos1 <= i;
    const float sc = a.scale_log2;
    float y0[4], y1[4];
    bool raise = false;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      y0[v] = ok0 ? fmaf(s[0][v], sc, -m[v]) : -INFINITY;
      y1[v] = ok1 ? fmaf(s[1][v], sc, -m[v]) : -INFINITY;
      raise |= fmaxf(y0[v], y1[v]) > 8.f;
    }
    if (__builtin_amdgcn_ballot_w64(raise && lane < 32)) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float mm = fmaxf(ok0 ? s[0][v] * sc : -INFINITY, ok1 ? s[1][v] * sc : -INFINITY);
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) mm = fmaxf(mm, __shfl_xor(mm, off, 64));
        const float mn = fmaxf(m[v], mm);
        const float alpha = mn == -INFINITY || m[v] == -INFINITY ? 0.f : exp2f(m[v] - mn);
        l[v] *= alpha;
#pragma unroll
        for (int t = 0; t < kD / 16; ++t) o[t][v] *= alpha;
        m[v] = mn;
        y0[v] = ok0 ? fmaf(s[0][v], sc, -mn) : -INFINITY;
        y1[v] = ok1 ? fmaf(s[1][v], sc, -mn) : -INFINITY;
      }
    }
    if (lane < 32) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        // y <= 8 or -inf here: the raw exp2 (no denormal rescaling) suffices
        const float p0 = __builtin_amdgcn_exp2f(y0[v]);
        const float p1 = __builtin_amdgcn_exp2f(y1[v]);
        l[v] += p0 + p1;
        uint32_t hi, lo;
        split2_bf16(p0, p1, hi, lo);
        const int o16 = (4 * q4 + v) * kP16Ld + c16;
        sP[o16] = (uint16_t)hi;
        sP[o16 + 16] = (uint16_t)(hi >> 16);
        sPl[o16] = (uint16_t)lo;
        sPl[o16 + 16] = (uint16_t)(lo >> 16);
      }
    }
    // O += P V: A = P (row c16, keys 8 q4 ..), B = V (keys 8 q4 .., channel 16t + c16)
    const bf16x8 pa = __builtin_bit_cast(bf16x8, *(const lds_x4*)(sP + c16 * kP16Ld + 8 * q4));
    const bf16x8 pl = __builtin_bit_cast(bf16x8, *(const lds_x4*)(sPl + c16 * kP16Ld + 8 * q4));
#pragma unroll
    for (int t = 0; t < kD / 16; ++t) {
      const bf16x8 vb = vtile_operand16(sV, t, lane);
      o[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, vb, o[t], 0, 0, 0);
      o[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl, vb, o[t], 0, 0, 0);
    }
  }

  // heads 4 q4 + v (lanes 0..31): row sums over the 16 key lanes, out, lse
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    float L = l[v];
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) L += __shfl_xor(L, off, 64);
    if (lane >= 32) continue;
    const int head = 4 * q4 + v;
    const int64_t oh = (int64_t)tok * a.Hq + (int64_t)g * kG + head;
    const bool empty = m[v] == -INFINITY;
#pragma unroll
    for (int t = 0; t < kD / 16; ++t) a.out[oh * kD + 16 * t + c16] = empty ? 0.f : o[t][v] / L;
    if (c16 == 0 && a.lse) a.lse[oh] = empty ? -INFINITY : (m[v] + log2f(L)) * kLn2f;
  }
}

// Decode on the matrix cores: a workgroup of 8 waves per (sequence, KV
// head, split of 256 list entries), one wave per 32 of them, on the
// 16x16x32 tiles and lane layouts of the per-token kernel above (rows = the
// GL heads of the group, the rest idle; columns = 16 keys). Each wave
// gathers its 32 keys' K and V rows (one round trip), computes S = Q K^T,
// its chunk's softmax relative to the chunk's max, and O = P V with p as
// hi + lo bf16 terms; the 8 waves' (max, sum, O) are combined through LDS
// into the split partial that the merge kernel combines by log-sum-exp.
// (8 waves rather than 4 halve the partials the merge reads: 4.4 us against
// 5.0 for the merge at the 4 x 8-head, top-2048 decode shape.)
constexpr int kDecWaves = 8;
// floats per split partial when the splits are merged in the launch: G heads
// of (max, sum, kD outputs), rounded up to whole 128-byte lines
__host__ __device__ constexpr int dec_partial_stride(int G) { return (G * (kD + 2) + 31) / 32 * 32; }

// The last workgroup out clears the launch-wide control words.
__device__ __forceinline__ void decode_launch_done(const AttnArgs& a) {
  if (threadIdx.x == 0 &&
      __hip_atomic_fetch_add(a.ctrl + 8, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == gridDim.x - 1u) {
    for (int i = 0; i < 9; ++i) __hip_atomic_store(a.ctrl + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Log-sum-exp merge of a (sequence, KV head)'s split partials into out and
// lse, with the merge kernel's arithmetic in the same order (so the results
// are the same bits). lds: at least 2 * splits * GL floats.
template <int GL>
__device__ __forceinline__ void decode_merge_row(const AttnArgs& a, int64_t rowg, float* lds) {
  const int t = threadIdx.x, S = a.splits;
  const int row = (int)(rowg / a.Hkv), g = (int)(rowg % a.Hkv);
  const int ps = dec_partial_stride(GL);
  const float* base = a.partial + rowg * S * ps;
  float* s_m = lds;
  float* s_l = lds + S * GL;
  for (int e = t; e < S * GL; e += 64 * kDecWaves) {
    const int sp = e / GL, hh = e % GL;
    s_m[e] = base[sp * ps + hh * (kD + 2)];
    s_l[e] = base[sp * ps + hh * (kD + 2) + 1];
  }
  __syncthreads();
  for (int e = t; e < GL * kD; e += 64 * kDecWaves) {
    const int h = e / kD, c = e % kD;
    float M = -INFINITY;
    for (int sp = 0; sp < S; ++sp) M = fmaxf(M, s_m[sp * GL + h]);
    float L = 0.f, O = 0.f;
    for (int s0 = 0; s0 < S; s0 += 8) {   // eight splits' values in flight at once
      float o[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) o[u] = s0 + u < S ? base[(s0 + u) * ps + h * (kD + 2) + 2 + c] : 0.f;
      if (M != -INFINITY) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          if (s0 + u < S) {
            const float f = exp2f(s_m[(s0 + u) * GL + h] - M);
            L += s_l[(s0 + u) * GL + h] * f;
            O += o[u] * f;
          }
        }
      }
    }
    const int64_t oh = (int64_t)row * a.Hq + (int64_t)g * GL + h;
    a.out[oh * kD + c] = M == -INFINITY ? 0.f : O / L;
    if (c == 0 && a.lse) a.lse[oh] = M == -INFINITY ? -INFINITY : (M + log2f(L)) * kLn2f;
  }
}

template <int GL>
__global__ __launch_bounds__(64 * kDecWaves) void attn_decode_mfma_kernel(AttnArgs a) {
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  __shared__ __align__(16) uint8_t sKall[kDecWaves][kKC * kRowBytes];   // K of the chunk
  __shared__ __align__(16) uint8_t sVall[kDecWaves][kKC * kRowBytes];   // V of the chunk, then the wave's partial
  __shared__ __align__(16) uint16_t sPall[kDecWaves][16 * kP16Ld];      // P hi (rows >= 8 stay zero)
  __shared__ __align__(16) uint16_t sPlall[kDecWaves][16 * kP16Ld];     // P lo
  const int tid = threadIdx.x, lane = tid & 63, q4 = lane >> 4, c16 = lane & 15;
  const int kq = lane >> 2, r4 = lane & 3;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  uint8_t* sK = sKall[w];
  uint8_t* sV = sVall[w];
  uint16_t* sP = sPall[w];
  uint16_t* sPl = sPlall[w];
  __shared__ int s_flag;
  int split;
  int64_t rowg;
  if (a.ctrl != nullptr) {   // (row, split) from this XCD's queue: a row's splits share its L2
    const int nx = a.nxcc;
    const int x = (int)((__builtin_amdgcn_s_getreg((15 << 11) | 20) & 15u) % (unsigned)nx);   // HW_REG_XCC_ID
    if (tid == 0) s_flag = (int)__hip_atomic_fetch_add(a.ctrl + x, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const int ticket = __builtin_amdgcn_readfirstlane(s_flag);
    const int64_t nrg = (int64_t)a.rows * a.Hkv;
    const int nr = x < nrg ? (int)((nrg - x + nx - 1) / nx) : 0;
    __syncthreads();
    if (ticket >= nr * a.splits) {   // more workgroups landed on this XCD than it has splits
      decode_launch_done(a);
      return;
    }
    rowg = x + (int64_t)nx * (ticket / a.splits);
    split = ticket % a.splits;
  } else {
    split = (int)(blockIdx.x % a.splits);
    rowg = blockIdx.x / a.splits;
  }
  const int g = (int)(rowg % a.Hkv), row = (int)(rowg / a.Hkv);
  const int e0 = split * (kDecWaves * kKC) + w * kKC;   // this wave's first list entry
  const int32_t* ilist = a.idx + rowg * a.B;

  // list entries and rows first, so the gather starts at once: lane l reads
  // bytes 64j + 16(l%4) of the K and V rows of keys l/4 and 16 + l/4 (a
  // quad per 64 contiguous bytes)
  int32_t pos[2];
  u32x4 kreg[2][4], vreg[2][4];
  const int64_t tok_bytes = a.s_tok * 2;
  const int64_t base = ((int64_t)row * a.s_seq + (int64_t)g * a.s_head) * 2 + 16 * r4;
  const int32_t* tab = a.slot ? a.slot + (int64_t)row * a.slot_ld : nullptr;
#pragma unroll
  for (int tn = 0; tn < 2; ++tn) {
    const int e = e0 + 16 * tn + kq;
    int32_t t = e < a.B ? ilist[e] : -1;
    if (t < 0 || t >= a.T) t = -1;
    int64_t r = t < 0 ? 0 : t;
    if (tab && t >= 0) {
      const int32_t pr = tab[t];
      if (pr < 0 || pr >= a.n_rows_kv) t = -1;
      r = t < 0 ? 0 : pr;
    }
    pos[tn] = t;
    const char* kr = (const char*)a.k + base + r * tok_bytes;
    const char* vr = (const char*)a.v + base + r * tok_bytes;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      kreg[tn][j] = *(const u32x4*)(kr + 64 * j);
      vreg[tn][j] = *(const u32x4*)(vr + 64 * j);
    }
  }
  // Q: row c16 = head c16 (< GL; idle rows are zero), channels 32c + 8 q4 ..
  bf16x8 qa[kD / 32];
  {
    const bool live = c16 < GL;
    const uint16_t* qp = (const uint16_t*)a.q + ((int64_t)row * a.Hq + (int64_t)g * GL + (live ? c16 : 0)) * kD + 8 * q4;
#pragma unroll
    for (int c = 0; c < kD / 32; ++c) {
      u32x4 x = live ? *(const u32x4*)(qp + 32 * c) : u32x4{0u, 0u, 0u, 0u};
      qa[c] = __builtin_bit_cast(bf16x8, x);
    }
  }
  for (int e = lane; e < 8 * kP16Ld; e += 64) sP[8 * kP16Ld + e] = sPl[8 * kP16Ld + e] = 0;

  // the rows to the LDS tiles; a skipped key's V row is zeroed, so its
  // p = 0 never meets a NaN or Inf
#pragma unroll
  for (int tn = 0; tn < 2; ++tn) {
    const uint32_t vkeep = pos[tn] >= 0 ? ~0u : 0u;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      *(lds_x4*)(sK + ktile_byte(16 * tn + kq, 64 * j + 16 * r4)) = kreg[tn][j];
      *(lds_x4*)(sV + vtile_byte(16 * tn + kq, 64 * j + 16 * r4)) = vreg[tn][j] & vkeep;
    }
  }
  // the keys of this lane's score columns c16 and 16 + c16
  int32_t posc[2];
#pragma unroll
  for (int tn = 0; tn < 2; ++tn) posc[tn] = __shfl(pos[tn], 4 * c16, 64);
  // S = Q K^T: B = K (key 16 tn + c16, channels 32q + 8 q4 ..)
  f32x4 s[2];
#pragma unroll
  for (int tn = 0; tn < 2; ++tn) {
    s[tn] = f32x4{};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const u32x4 kb = *(const lds_x4*)(sK + ktile_byte(16 * tn + c16, 64 * q + 16 * q4));
      s[tn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[q], __builtin_bit_cast(bf16x8, kb), s[tn], 0, 0, 0);
    }
  }
  // softmax over the chunk, heads 4 q4 + v in lanes 0..31 (log2 domain)
  float m[4], l[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const float x0 = posc[0] >= 0 ? s[0][v] * a.scale_log2 : -INFINITY;
    const float x1 = posc[1] >= 0 ? s[1][v] * a.scale_log2 : -INFINITY;
    float mm = fmaxf(x0, x1);
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) mm = fmaxf(mm, __shfl_xor(mm, off, 64));
    m[v] = mm;
    // x - mm <= 0 or -inf: the raw exp2 (no denormal rescaling) suffices
    const float p0 = mm == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(x0 - mm);
    const float p1 = mm == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(x1 - mm);
    l[v] = p0 + p1;
    if (lane < 32) {
      uint32_t hi, lo;
      split2_bf16(p0, p1, hi, lo);
      const int o16 = (4 * q4 + v) * kP16Ld + c16;
      sP[o16] = (uint16_t)hi;
      sP[o16 + 16] = (uint16_t)(hi >> 16);
      sPl[o16] = (uint16_t)lo;
      sPl[o16 + 16] = (uint16_t)(lo >> 16);
    }
  }
  // O = P V: A = P (row c16, keys 8 q4 ..), B = V (keys 8 q4 .., channel 16t + c16)
  const bf16x8 pa = __builtin_bit_cast(bf16x8, *(const lds_x4*)(sP + c16 * kP16Ld + 8 * q4));
  const bf16x8 pl = __builtin_bit_cast(bf16x8, *(const lds_x4*)(sPl + c16 * kP16Ld + 8 * q4));
  f32x4 o[kD / 16];
#pragma unroll
  for (int t = 0; t < kD / 16; ++t) {
    const bf16x8 vb = vtile_operand16(sV, t, lane);
    o[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, vb, f32x4{}, 0, 0, 0);
    o[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl, vb, o[t], 0, 0, 0);
  }
  // this wave's (max, sum, O) of heads 4 q4 + v < GL into its own V tile
  // (its reads of the tile are done: a wave's LDS accesses execute in order)
  float* wp = reinterpret_cast<float*>(sV);   // [GL][kD + 2]
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    float L = l[v];
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) L += __shfl_xor(L, off, 64);
    const int head = 4 * q4 + v;
    if (lane >= 32 || head >= GL) continue;
    float* hp = wp + head * (kD + 2);
    if (c16 == 0) {
      hp[0] = m[v];
      hp[1] = L;
    }
#pragma unroll
    for (int t = 0; t < kD / 16; ++t) hp[2 + 16 * t + c16] = o[t][v];
  }
  __syncthreads();
  // combine the waves: thread (head, channel) pairs, written as the split's partial
  for (int e = tid; e < GL * kD; e += 64 * kDecWaves) {
    const int h = e / kD, c = e % kD;
    float M = -INFINITY;
#pragma unroll
    for (int q = 0; q < kDecWaves; ++q) M = fmaxf(M, reinterpret_cast<const float*>(sVall[q])[h * (kD + 2)]);
    float L = 0.f, O = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int q = 0; q < kDecWaves; ++q) {
        const float* hp = reinterpret_cast<const float*>(sVall[q]) + h * (kD + 2);
        const float f = exp2f(hp[0] - M);
        L += hp[1] * f;
        O += hp[2 + c] * f;
      }
    }
    if (a.splits == 1) {   // the whole list: the output itself
      const int64_t oh = (int64_t)row * a.Hq + (int64_t)g * GL + h;
      a.out[oh * kD + c] = M == -INFINITY ? 0.f : O / L;
      if (c == 0 && a.lse) a.lse[oh] = M == -INFINITY ? -INFINITY : (M + log2f(L)) * kLn2f;
      continue;
    }
    float* pr = a.ctrl ? a.partial + (rowg * a.splits + split) * dec_partial_stride(GL) + h * (kD + 2)
                       : a.partial + ((rowg * a.splits + split) * GL + h) * (kD + 2);
    pr[2 + c] = O;
    if (c == 0) {
      pr[0] = M;
      pr[1] = L;
    }
  }
  if (a.ctrl != nullptr && a.splits > 1) {
    // the last split of the row merges: the partials are in this XCD's L2,
    // one writing workgroup per 128-byte line, read only after the arrival
    // count (an atomic, performed in that L2) shows every split done
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0)
      s_flag = __hip_atomic_fetch_add(a.ctrl + 16 + rowg, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) ==
               (uint32_t)a.splits - 1u;
    __syncthreads();
    if (__builtin_amdgcn_readfirstlane(s_flag)) {
      if (tid == 0) __hip_atomic_store(a.ctrl + 16 + rowg, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      decode_merge_row<GL>(a, rowg, reinterpret_cast<float*>(&sVall[0][0]));
    }
  }
  if (a.ctrl != nullptr) decode_launch_done(a);
}

hipError_t launch_mfma_blocks(const AttnArgs& a, hipStream_t s) {
  const size_t lds = (size_t)kBlkLds;
  const int nsel = (a.rows + a.qblk - 1) / a.qblk;
  const unsigned nx = (unsigned)(nsel * ((a.qblk + kTPW * kNW - 1) / (kTPW * kNW)));
  hipLaunchKernelGGL(attn_mfma_kernel, dim3(nx, (unsigned)a.Hkv), dim3(64 * kNW), lds, s, a);
  return hipGetLastError();
}

}  // namespace

bool attention_mfma_supported(const AttnArgs& a, bool bf16) {
  return bf16 && a.prefill && a.d == kD && a.Hq == kG * a.Hkv && a.B >= 1 && a.Hkv <= 65535 &&
         a.rows <= 0x7fffffff;
}

bool attention_decode_mfma_supported(int G, int d, int B, bool bf16) {
  return bf16 && d == kD && (G == 4 || G == 8) && B >= 1 && (B + kDecodeSplit - 1) / kDecodeSplit <= 64;
}

int decode_partial_stride(int G) { return dec_partial_stride(G); }

hipError_t launch_attention_decode_mfma(const AttnArgs& a, hipStream_t s) {
  static_assert(kDecodeSplit == kDecWaves * kKC, "a split is one 32-key MFMA step per wave");
  const int G = a.Hq / a.Hkv;
  const int64_t nrg = (int64_t)a.rows * a.Hkv;
  if (a.ctrl != nullptr && (a.nxcc < 1 || a.nxcc > 8 || nrg > 1000)) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(a.ctrl ? a.nxcc * ((nrg + a.nxcc - 1) / a.nxcc) * a.splits : nrg * a.splits));
  if (G == 4)
    hipLaunchKernelGGL(attn_decode_mfma_kernel<4>, grid, dim3(64 * kDecWaves), 0, s, a);
  else if (G == 8)
    hipLaunchKernelGGL(attn_decode_mfma_kernel<8>, grid, dim3(64 * kDecWaves), 0, s, a);
  else
    return hipErrorInvalidValue;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.splits == 1 || a.ctrl != nullptr) return e;
  return launch_attention_merge(a, s);
}

hipError_t launch_attention_mfma(const AttnArgs& a, hipStream_t s) {
  if (a.qblk > 1) return launch_mfma_blocks(a, s);
  hipLaunchKernelGGL(attn_mfma16_kernel, dim3((unsigned)a.rows, (unsigned)a.Hkv), dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace lsa
