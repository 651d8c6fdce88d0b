// CSA ratio-4 selection producer (the indexer) on gfx950.
//
// The compressed-sparse-attention pages (onnx-runtime-ep-cpu,
// src/kernels/compressed_sparse_attention.rs: `select_ratio4_topk`,
// `finalize_index_query`, `apply_compressed_rope`, `hadamard_bf16`,
// `fp4_roundtrip`; onnx-runtime-ep-cuda, same file,
// `csa_ratio4_index_select`) score every causally complete record of a
// (batch, query) by sum over index heads of relu(q_h . k) w_h / (sqrt(D)
// sqrt(H)) with FP4 E2M1 block-32 index keys, and keep the top k in
// (-score, +record) order with -1 padding. Three launches:
//
//  1. finalize: one wave per (batch, query, index head): bf16 rounding,
//     compressed RoPE on the last 64 dims (pow, sin and cos taken in double
//     and rounded once, so they are reproducible), Walsh-Hadamard butterflies across
//     lanes, times 1/sqrt(128) rounded to bf16, FP4 round trip. The result is
//     FP4 values times a power of two, exact in bf16.
//  2. score: a workgroup per (batch, query, 1024 records). The keys are staged
//     in LDS, decoded to bf16 with v_cvt_scalef32_pk_bf16_fp4 (exact), and
//     S^T = K . Q^T runs on v_mfma_f32_16x16x32_bf16; every product is exact
//     and the dot products of FP4 operands are exact in fp32 for the value
//     ranges met here, so the order of accumulation does not change them.
//     The head sum is then taken one record per thread, in ascending head
//     order with the pages' fp32 operations (relu, times w, times the scale,
//     add), so a score is the pages' fp32 score.
//  3. select: a workgroup per (batch, query): the k-th largest total-order
//     key of the scores by a binary search over key values, the winners (ties
//     in ascending record order) ranked by (-score, +record), written to
//     every index-head row of the output.
#include "sa_mfma_dev.h"

// the pages' fp32 arithmetic here is separate multiplies and adds (no fused
// multiply-add); keep every one of them separately rounded
#pragma clang fp contract(off)

namespace sa {

namespace cx {
constexpr int D = 128;            // index head dim
constexpr int ROPE = 64;          // RoPE tail of the index query
constexpr int KB = 68;            // key bytes: 4 x (1 scale + 16 code bytes)
constexpr int HMAX = 64;          // index heads
constexpr int RC = 1024;          // records per score workgroup
constexpr int RB = 128;           // records per score pass (one per thread of waves 0, 1)
constexpr int DSTR = 68;          // LDS row stride (floats) of the dot table (16-byte rows)
constexpr int KMAX = 2048;        // selected width
constexpr int NMAX = 32768;       // records per (batch, query) (index keys per batch entry)
}  // namespace cx

// ---------------------------------------------------------------- finalize

// nearest E2M1 magnitude (0, .5, 1, 1.5, 2, 3, 4, 6) of v >= 0, ties to the even code
__device__ __forceinline__ float e2m1_round(float v) {
  if (v <= 0.25f) return 0.0f;
  if (v < 0.75f) return 0.5f;
  if (v <= 1.25f) return 1.0f;
  if (v < 1.75f) return 1.5f;
  if (v <= 2.5f) return 2.0f;
  if (v < 3.5f) return 3.0f;
  if (v <= 5.0f) return 4.0f;
  return 6.0f;
}

__device__ __forceinline__ float bf16_round(float x) { return bf16_to_f32(f32_to_bf16_rne(x)); }

// lane l of the wave holds elements 2l, 2l+1 of one head's 128 values
__global__ void __launch_bounds__(256)
csa_index_finalize_kernel(const float* __restrict__ iq, uint16_t* __restrict__ qf, uint8_t* __restrict__ qe,
                          int64_t rows, int H, int S, const int64_t* __restrict__ total_ptr) {
  using namespace cx;
  const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // (b, s, h) row
  if (wid >= rows) return;
  const int lane = threadIdx.x & 63;
  const int s = (int)((wid / H) % S);
  const int64_t pos = *total_ptr - S + s;
  const float* src = iq + wid * D;
  float v0 = bf16_round(src[2 * lane]), v1 = bf16_round(src[2 * lane + 1]);
  // compressed RoPE on dims 64..127 (lanes 32..63 hold pair p = lane - 32)
  if (lane >= 32) {
    const int p = lane - 32;
    float ramp = ((float)p - 15.0f) / (25.0f - 15.0f);
    ramp = fminf(fmaxf(ramp, 0.0f), 1.0f);
    // pow, sin and cos as exactly rounded fp32 values (double, rounded once)
    const float bf = (float)pow(160000.0, (double)(-((float)(2 * p)) / (float)ROPE));
    const float a = bf * (1.0f - ramp);
    const float c = bf / 16.0f * ramp;
    const float freq = a + c;
    const float ang = (float)pos * freq;
    const float sn = (float)sin((double)ang), cs = (float)cos((double)ang);
    const float r0 = v0 * cs, r1 = v1 * sn, i0 = v0 * sn, i1 = v1 * cs;
    v0 = bf16_round(r0 - r1);
    v1 = bf16_round(i0 + i1);
  }
  // Walsh-Hadamard butterflies: span 1 inside the lane, spans 2..64 across lanes
  {
    const float a = v0, b = v1;
    v0 = a + b;
    v1 = a - b;
  }
#pragma unroll
  for (int sl = 1; sl < 64; sl <<= 1) {  // element span 2 sl = lane distance sl
    const float p0 = __shfl_xor(v0, sl), p1 = __shfl_xor(v1, sl);
    if (lane & sl) {
      v0 = p0 - v0;
      v1 = p1 - v1;
    } else {
      v0 = v0 + p0;
      v1 = v1 + p1;
    }
  }
  const float hs = 1.0f / sqrtf((float)D);
  v0 = bf16_round(v0 * hs);
  v1 = bf16_round(v1 * hs);
  // FP4 round trip, block of 32 = 16 lanes
  float amax = fmaxf(fabsf(v0), fabsf(v1));
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m));
  int e = 127;
  if (amax > 0.0f) {
    int ex;
    frexpf(amax, &ex);  // floor(log2 amax) = ex - 1
    e = min(max(ex - 1 - 2 + 127, 0), 254);
  }
  const float inv = ldexpf(1.0f, 127 - e), sc = ldexpf(1.0f, e - 127);
  const float q0 = copysignf(e2m1_round(fabsf(v0) * inv), v0) * sc;
  const float q1 = copysignf(e2m1_round(fabsf(v1) * inv), v1) * sc;
  const uint32_t packed = (uint32_t)f32_to_bf16_rne(q0) | ((uint32_t)f32_to_bf16_rne(q1) << 16);
  ((uint32_t*)(qf + wid * D))[lane] = packed;
  if ((lane & 15) == 0) qe[wid * 4 + (lane >> 4)] = (uint8_t)e;  // the block's scale exponent (E8M0 byte)
}

// ---------------------------------------------------------------- score

// Exactness of a head dot taken by the matrix cores. With biased scale
// exponents q_c (query block c, from the finalize) and k_c (key block c), the
// products of block c are multiples of 2^(q_c + k_c - 256 - 2) and at most 36
// times 2^(q_c + k_c - 254); every partial sum of the 128 products is then an
// exact fp32 number (so any order of summation gives the same value) when
// each factor is normal (2 <= q_c, k_c <= 252), no product or sum leaves the
// normal range (q_c + k_c - 254 in [-124, 115]) and the block exponents span
// at most 9 (4608 * 2^9 * 4 < 2^24). qr packs the query's lowest and highest
// block exponent; the key's come in klo, khi; the per-block test runs only
// when the ranges alone do not settle it.
__device__ __forceinline__ bool range_is_exact(int qr, int klo, int khi) {
  const int qlo = qr & 255, qhi = qr >> 8;
  if (qlo < 2 || qhi > 252 || klo < 2 || khi > 252) return false;
  const int lo = qlo + klo - 254, hi = qhi + khi - 254;
  return lo >= -124 && hi <= 115 && hi - lo <= 9;
}

__device__ __forceinline__ bool dot_is_exact(int qr, int klo, int khi, uint32_t qx, const uint8_t* kk) {
  if (range_is_exact(qr, klo, khi)) return true;
  if ((qr & 255) < 2 || (qr >> 8) > 252 || klo < 2 || khi > 252) return false;
  int elo = 1 << 20, ehi = -(1 << 20);
#pragma unroll
  for (int c = 0; c < 4; c++) {
    const int e = (int)((qx >> (8 * c)) & 255u) + (int)kk[17 * c] - 254;
    elo = min(elo, e);
    ehi = max(ehi, e);
  }
  return elo >= -124 && ehi <= 115 && ehi - elo <= 9;
}

// The head dot in the pages' order: q (bf16, exact in fp32) times the
// decoded key value (E2M1 magnitude times the block's E8M0 scale, 255 = NaN),
// each product rounded, folded in ascending dimension order.
__device__ __forceinline__ float ordered_dot(const uint16_t* __restrict__ qh, const uint8_t* kk) {
  const float mag[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
  float acc = 0.0f;
#pragma unroll 1
  for (int c = 0; c < 4; c++) {
    const uint32_t e = kk[17 * c];
    const float sc = e == 255u ? __uint_as_float(0x7fc00000u) : (e ? __uint_as_float(e << 23) : 5.877471754e-39f);
#pragma unroll 1
    for (int i = 0; i < 32; i++) {
      const uint32_t code = ((uint32_t)kk[17 * c + 1 + (i >> 1)] >> (4 * (i & 1))) & 15u;
      const float m = mag[code & 7u];
      const float kv = ((code & 8u) ? -m : m) * sc;
      const float prod = bf16_to_f32(qh[32 * c + i]) * kv;
      acc = acc + prod;
    }
  }
  return acc;
}


// A workgroup scores RC records of one (batch, query) in passes of RB: the
// pass's keys (68 B each, contiguous) are copied to LDS from registers loaded
// during the previous pass; each wave computes S^T for two 16-record tiles and
// all heads, writes the fp32 dot products to an LDS table, and threads
// 0..RB-1 take the head sums (one record each).
template <int HT>
__global__ void __launch_bounds__(256)
csa_index_score_kernel(const uint16_t* __restrict__ qf, const uint8_t* __restrict__ qe,
                       const float* __restrict__ iw, const uint8_t* __restrict__ keys, float* __restrict__ scores,
                       int S, int64_t kcap, const int64_t* __restrict__ total_ptr, ErrorBlock* __restrict__ eb) {
  using namespace cx;
  constexpr int H = 16 * HT;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int i16 = lane & 15, g = lane >> 4;
  const int64_t row = blockIdx.y;  // (b, s)
  const int s = (int)(row % S);
  const int64_t b = row / S;
  const int64_t pos = *total_ptr - S + s;
  if (pos < s) return;  // total < S: the select launch flags it
  int64_t n = (pos + 1) / 4;
  if (n > kcap) n = kcap;
  const int64_t c0 = (int64_t)blockIdx.x * RC;
  if (c0 >= n) return;
  const int64_t c1 = min(c0 + RC, n);

  // the finalized query as B operands: lane (head i16 of tile ht, g) holds
  // dims 32 c + 8 g .. + 7
  u32x4_l qb[HT][4];
  const uint16_t* qrow = qf + row * H * D;
#pragma unroll
  for (int ht = 0; ht < HT; ht++)
#pragma unroll
    for (int c = 0; c < 4; c++) qb[ht][c] = *(const u32x4_l*)(qrow + (int64_t)(16 * ht + i16) * D + 32 * c + 8 * g);
  const float ws = (1.0f / sqrtf((float)D)) / sqrtf((float)H);
  float wv[H];  // the (batch, query)'s head weights, uniform
#pragma unroll
  for (int h = 0; h < H; h++) wv[h] = iw[row * H + h];

  uint8_t* kl = smem;                          // RB keys, 68 B each
  float* dt = (float*)(smem + RB * KB);        // [RB][DSTR] dot products
  // per head: the query blocks' scale exponents (4 bytes) and their range
  // (and, in qr[HMAX], the range over all heads)
  uint32_t* qx = (uint32_t*)(smem + RB * KB + RB * DSTR * 4);
  int* qr = (int*)(qx + HMAX);
  if (w == 0) {
    int lo = 255, hi = 0;
    if (tid < H) {
      const uint32_t x = *(const uint32_t*)(qe + (row * H + tid) * 4);
#pragma unroll
      for (int c = 0; c < 4; c++) {
        const int e = (int)((x >> (8 * c)) & 255u);
        lo = min(lo, e);
        hi = max(hi, e);
      }
      qx[tid] = x;
      qr[tid] = lo | (hi << 8);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      lo = min(lo, __shfl_xor(lo, o));
      hi = max(hi, __shfl_xor(hi, o));
    }
    if (tid == 0) qr[HMAX] = lo | (hi << 8);
  }  // read after the first pass's barriers
  // keys of the next two passes in flight (two register sets), each issue
  // the same loads with out-of-range offsets past the workgroup's records,
  // so the compiler's wait counts are exact
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(keys + (b * kcap) * KB), (short)0, (int)(kcap * KB), 0x00020000);
  constexpr int KW = RB * KB / 4;              // dwords of a pass's keys
  constexpr int KL = (KW + 255) / 256;         // loads per thread
  uint32_t kra[KL], krb[KL];
  auto load_keys = [&](uint32_t (&kr)[KL], int64_t r0) {
    const int64_t left = c1 - r0;
    const int64_t lim = (left < 0 ? 0 : (left > RB ? RB : left)) * (KB / 4);  // dwords of this pass's records
#pragma unroll
    for (int j = 0; j < KL; j++) {
      const int i = tid + 256 * j;
      const uint32_t off = (i < KW && i < lim) ? (uint32_t)((r0 * (KB / 4) + i) * 4) : 0x80000000u;
      kr[j] = __builtin_amdgcn_raw_buffer_load_b32(krs, off, 0, 0);
    }
  };
  bool bad = false;
  load_keys(kra, c0);
  load_keys(krb, c0 + RB);
  auto pass = [&](int64_t r0, uint32_t (&kr)[KL]) {
    __syncthreads();  // the previous pass's LDS reads are done
#pragma unroll
    for (int j = 0; j < KL; j++) {
      const int i = tid + 256 * j;
      if (i < KW) ((uint32_t*)kl)[i] = kr[j];
    }
    load_keys(kr, r0 + 2 * RB);
    __syncthreads();
    // S^T for the wave's two record tiles: all operand reads first, then the MFMAs
    bf16x8_l av[2][4];
#pragma unroll
    for (int rt = 0; rt < 2; rt++) {
      const uint8_t* kq = kl + (32 * w + 16 * rt + i16) * KB;
#pragma unroll
      for (int c = 0; c < 4; c++) {
        // 4 code bytes at 17 c + 1 + 4 g (unaligned) and the block's scale byte
        const int o = 17 * c + 1 + 4 * g;
        const uint32_t* wp = (const uint32_t*)(kq + (o & ~3));
        const uint32_t cw = __builtin_amdgcn_alignbyte(wp[1], wp[0], (uint32_t)(o & 3));
        const uint32_t e = kq[17 * c];
        const float sc = e == 255u ? __uint_as_float(0x7fc00000u) : (e ? __uint_as_float(e << 23) : 5.877471754e-39f);
        u32x4_l a;
        a[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, sc, 0));
        a[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, sc, 1));
        a[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, sc, 2));
        a[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, sc, 3));
        av[rt][c] = __builtin_bit_cast(bf16x8_l, a);
      }
    }
    f32x4_l acc[2][HT];
#pragma unroll
    for (int rt = 0; rt < 2; rt++)
#pragma unroll
      for (int ht = 0; ht < HT; ht++) acc[rt][ht] = (f32x4_l){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 4; c++)
#pragma unroll
      for (int rt = 0; rt < 2; rt++)
#pragma unroll
        for (int ht = 0; ht < HT; ht++)
          acc[rt][ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[rt][c], __builtin_bit_cast(bf16x8_l, qb[ht][c]),
                                                               acc[rt][ht], 0, 0, 0);
    // lane (head i16 of tile ht, g) holds records 4 g .. 4 g + 3 of tile rt
#pragma unroll
    for (int rt = 0; rt < 2; rt++)
#pragma unroll
      for (int ht = 0; ht < HT; ht++)
#pragma unroll
        for (int j = 0; j < 4; j++) dt[(32 * w + 16 * rt + 4 * g + j) * DSTR + 16 * ht + i16] = acc[rt][ht][j];
    __syncthreads();
    // one record per thread: the head sum in ascending head order
    const int64_t r = r0 + tid;
    if (tid < RB && r < c1) {
      float* drow = dt + tid * DSTR;
      const uint8_t* kk = kl + tid * KB;
      int klo = 255, khi = 0;
#pragma unroll
      for (int c = 0; c < 4; c++) {
        klo = min(klo, (int)kk[17 * c]);
        khi = max(khi, (int)kk[17 * c]);
      }
      // The matrix dot equals the pages' ascending fp32 fold when no partial
      // sum rounds: every factor a normal number and the block products within
      // 2^9 of each other. Where the exponent ranges over all heads do not
      // settle that, the heads that fail are redone in the pages' order (rare:
      // keys and queries of widely spread block scales).
      if (!range_is_exact(qr[HMAX], klo, khi)) {
#pragma unroll 1
        for (int h = 0; h < H; h++)
          if (!dot_is_exact(qr[h], klo, khi, qx[h], kk)) drow[h] = ordered_dot(qrow + (int64_t)h * D, kk);
      }
      const f32x4_l* d4 = (const f32x4_l*)drow;
      float score = 0.0f;
#pragma unroll
      for (int h4 = 0; h4 < H / 4; h4++) {
        const f32x4_l x4 = d4[h4];
#pragma unroll
        for (int j = 0; j < 4; j++) {
          const float x = x4[j];
          const float relu = x > 0.0f ? x : 0.0f;
          const float t0 = relu * wv[4 * h4 + j];
          const float t1 = t0 * ws;
          score = score + t1;
        }
      }
      bad |= !isfinite(score);
      scores[row * kcap + r] = score;
    }
  };
  for (int64_t r0 = c0; r0 < c1; r0 += 2 * RB) {
    pass(r0, kra);
    if (r0 + RB < c1) pass(r0 + RB, krb);
  }
  if (__builtin_amdgcn_ballot_w64(bad) != 0 && lane == 0) atomicOr(&eb->word, SA_ERR_INDEX_NONFINITE);
}

// ---------------------------------------------------------------- select

// strictly monotone map of a float's total order (Rust f32::total_cmp) to u32
__device__ __forceinline__ uint32_t total_key(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// One workgroup per (batch, query). Thread t holds the total-order keys of
// records t, t + 1024, ... in registers (key 0 for padding, below every
// score's key); the k-th largest key is found by a binary search over key
// values (each probe counted by wave ballots and summed over the waves
// through LDS), the winners take slots by one LDS atomic per wave and key
// register, and are sorted by rank (each winner counts the larger ones).
// Exact score ties, which the CSA CPU page rejects (`select_ratio4_topk`),
// are found by workgroups of their own beside the row's select workgroup: the
// row's scores are split by a hash of their value into P parts and each part
// inserted into an LDS hash table (linear probing, 2^15 slots, key 0 = empty);
// meeting its own key again is a tie. Scores compare as floats: -0 counts as
// +0, a NaN equals nothing. Equal scores share a part, so the parts together
// see every equal pair.
constexpr int TIE_SLOTS = 1 << 15;
__device__ __forceinline__ void tie_part(const float* __restrict__ src, int n, uint32_t p, uint32_t P,
                                         uint32_t* __restrict__ tab, ErrorBlock* __restrict__ eb) {
  const int tid = threadIdx.x;
  for (int i = tid; i < TIE_SLOTS / 4; i += 1024) ((uint4*)tab)[i] = make_uint4(0u, 0u, 0u, 0u);
  __syncthreads();
  bool tie = false;
  for (int i = tid; i < n; i += 1024) {
    float x = src[i];
    if (x != x) continue;     // NaN
    if (x == 0.0f) x = 0.0f;  // -0 -> +0
    const uint32_t key = total_key(x);  // never 0 for a number
    if ((uint32_t)(((uint64_t)(key * 0x85EBCA6Bu) * P) >> 32) != p) continue;
    uint32_t h = (key * 0x9E3779B1u) >> 17;
    for (int probe = 0; probe < TIE_SLOTS; probe++) {
      const uint32_t prev = atomicCAS(&tab[h], 0u, key);
      if (prev == 0u) break;
      if (prev == key) {
        tie = true;
        break;
      }
      h = (h + 1u) & (TIE_SLOTS - 1);
    }
  }
  if (__syncthreads_or(tie) && tid == 0) atomicOr(&eb->word, SA_ERR_INDEX_TIE);
}

template <int NJ>
__device__ __forceinline__ void select_row(const float* __restrict__ src, int32_t* __restrict__ outb, int n,
                                           int K, int S, int out_heads, uint8_t* smem) {
  using namespace cx;
  constexpr int NT = 1024, NW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  // [2 NW] probe partials (two buffers), [NW] partials of keys at the cut,
  // [48] winner slot counter
  uint32_t* tot = (uint32_t*)smem;
  unsigned long long* win = (unsigned long long*)(tot + 64);  // [KMAX] winners (key, ~record)
  uint32_t kv[NJ];
#pragma unroll
  for (int j = 0; j < NJ; j++) {
    const int i = tid + NT * j;
    const uint32_t x = total_key(src[i < n ? i : 0]);
    kv[j] = i < n ? x : 0u;
  }
  // the sum of this wave's partials over the NW waves (four 16-byte reads)
  auto sum_parts = [&](int base) {
    uint32_t c = 0;
#pragma unroll
    for (int q = 0; q < NW / 4; q++) {
      const uint4 v = *(const uint4*)(tot + base + 4 * q);
      c += (v.x + v.y) + (v.z + v.w);
    }
    return c;
  };
  // keys of this wave that satisfy pred, counted by ballots (uniform)
  auto wave_count = [&](auto pred) {
    uint32_t c = 0;
#pragma unroll
    for (int j = 0; j < NJ; j++) c += (uint32_t)__builtin_popcountll(__builtin_amdgcn_ballot_w64(pred(kv[j], j)));
    return c;
  };
  const int k = min(K, n);
  uint32_t T = 0;
  int need = k;
  if (tid == 0) tot[48] = 0u;
  if (k > 0 && k < n) {
    uint64_t lo = 1, hi = 1ull << 32;  // count(>= lo) >= k (every real key is >= 1), count(>= hi) < k
    uint32_t c_hi = 0;
    int par = 0;
    while (hi - lo > 1) {
      const uint64_t mid = lo + ((hi - lo) >> 1);
      const uint32_t t = (uint32_t)mid;
      const uint32_t cnt = wave_count([&](uint32_t x, int) { return x >= t; });
      if (lane == 0) tot[NW * par + w] = cnt;
      __syncthreads();
      // uniform: the loop's control stays on the scalar unit
      const uint32_t c = __builtin_amdgcn_readfirstlane(sum_parts(NW * par));
      par ^= 1;
      if (c >= (uint32_t)k) {
        lo = mid;
      } else {
        hi = mid;
        c_hi = c;
      }
    }
    T = (uint32_t)lo;
    need = k - (int)c_hi;  // keys > T number c_hi < k; the rest are keys == T
  }
  // winners: keys > T, and keys == T unless they straddle the cut
  uint32_t eq = 0;
  if (k < n) eq = wave_count([&](uint32_t x, int) { return x == T; });
  if (lane == 0) tot[2 * NW + w] = eq;
  __syncthreads();
  const uint32_t n_eq = __builtin_amdgcn_readfirstlane(sum_parts(2 * NW));
  const bool split_ties = k < n && n_eq > (uint32_t)need;
  // each wave takes slots for its winners of one register at a time (one
  // LDS atomic per wave); the order of the slots does not matter, the rank
  // sort below orders the winners
#pragma unroll
  for (int j = 0; j < NJ; j++) {
    const int i = tid + NT * j;
    const uint32_t x = kv[j];
    const bool won = i < n && (k >= n || x > T || (x == T && !split_ties));
    const uint64_t bal = __builtin_amdgcn_ballot_w64(won);
    if (bal == 0) continue;  // uniform
    uint32_t base = 0;
    if (lane == 0) base = atomicAdd(&tot[48], (uint32_t)__builtin_popcountll(bal));
    base = __builtin_amdgcn_readfirstlane(base);
    const uint32_t before = (uint32_t)__builtin_popcountll(bal & ((1ull << lane) - 1ull));
    if (won) win[base + before] = ((unsigned long long)x << 32) | (uint32_t)(~(uint32_t)i);
  }
  __syncthreads();
  const uint32_t n_win = tot[48];
  if (split_ties && w == 0) {
    // equal keys at the cut: the first `need` of them in ascending record order
    uint32_t taken = 0;
    for (int i0 = 0; i0 < n && taken < (uint32_t)need; i0 += 64) {
      const int i = i0 + lane;
      const bool isT = i < n && total_key(src[i]) == T;
      const uint64_t bal = __builtin_amdgcn_ballot_w64(isT);
      const uint32_t before = (uint32_t)__builtin_popcountll(bal & ((1ull << lane) - 1ull));
      if (isT && taken + before < (uint32_t)need)
        win[n_win + taken + before] = ((unsigned long long)T << 32) | (uint32_t)(~(uint32_t)i);
      taken += (uint32_t)__builtin_popcountll(bal);
    }
  }
  __syncthreads();
  // rank sort: the winners' composite keys are distinct; a winner's output
  // position is the number of larger ones. Two threads count for each winner,
  // over one half of the winners each (the halves in different waves, so the
  // waves of a half read the same winner at the same time: LDS broadcast), and
  // add their counts in LDS.
  int* rk = (int*)(win + KMAX);  // [KMAX] ranks
  for (int a = tid; a < k; a += NT) rk[a] = 0;
  __syncthreads();
  const int hk = (k + 1) >> 1;
  for (int it = tid; it < 2 * k; it += NT) {
    const int a = it < k ? it : it - k;
    const int q0 = it < k ? 0 : hk, q1 = it < k ? hk : k;
    const unsigned long long x = win[a];
    int r8[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    int q = q0;
    for (; q + 8 <= q1; q += 8) {
#pragma unroll
      for (int u = 0; u < 8; u++) r8[u] += win[q + u] > x ? 1 : 0;
    }
    for (; q < q1; q++) r8[0] += win[q] > x ? 1 : 0;
    atomicAdd(&rk[a], ((r8[0] + r8[1]) + (r8[2] + r8[3])) + ((r8[4] + r8[5]) + (r8[6] + r8[7])));
  }
  __syncthreads();
  int32_t* out0 = outb;
  for (int a = tid; a < k; a += NT) {
    const int32_t rec = (int32_t)(~(uint32_t)(win[a] & 0xffffffffull));
    const int rank = rk[a];
    for (int h = 0; h < out_heads; h++) out0[(int64_t)h * S * K + rank] = rec;
  }
  for (int j = k + tid; j < K; j += NT)
    for (int h = 0; h < out_heads; h++) out0[(int64_t)h * S * K + j] = -1;
}

__global__ void __launch_bounds__(1024)
csa_index_select_kernel(const float* __restrict__ scores, int32_t* __restrict__ sel, int S, int out_heads,
                        int64_t kcap, int K, const int64_t* __restrict__ total_ptr,
                        ErrorBlock* __restrict__ eb) {
  using namespace cx;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int64_t row = blockIdx.y;  // (b, s); x = 0 selects, x >= 1 looks for ties
  const int s = (int)(row % S);
  const int64_t b = row / S;
  const int64_t pos = *total_ptr - S + s;
  int32_t* outb = sel + (b * out_heads * S + s) * K;  // head 0 row; head h at + h S K
  if (pos < s) {  // total < S
    if (row == 0 && blockIdx.x == 0 && threadIdx.x == 0) atomicOr(&eb->word, SA_ERR_CSA_GEOMETRY);
    return;
  }
  int64_t n64 = (pos + 1) / 4;
  if (n64 > kcap) n64 = kcap;
  const int n = (int)n64;
  const float* src = scores + row * kcap;
  if (blockIdx.x > 0) {
    tie_part(src, n, blockIdx.x - 1, gridDim.x - 1, (uint32_t*)smem, eb);
    return;
  }
  // registers per thread sized to the records (uniform branch)
  if (n <= 1024 * 4)
    select_row<4>(src, outb, n, K, S, out_heads, smem);
  else if (n <= 1024 * 16)
    select_row<16>(src, outb, n, K, S, out_heads, smem);
  else
    select_row<NMAX / 1024>(src, outb, n, K, S, out_heads, smem);
}

size_t csa_index_workspace_bytes(int64_t rows, int64_t H, int64_t kcap) {
  // scores fp32 [rows][kcap], then the finalized queries bf16 [rows][H][128],
  // then their block scale exponents u8 [rows][H][4]
  const size_t sb = ((size_t)rows * (size_t)kcap * 4 + 255) & ~(size_t)255;
  return sb + (size_t)rows * (size_t)H * cx::D * 2 + (size_t)rows * (size_t)H * 4;
}

sa_status launch_csa_index_select(sparse_attn_ctx* c, const CsaIndexArgs& a) {
  using namespace cx;
  const int64_t rows = a.batch * a.q_seq;
  float* scores = (float*)a.workspace;
  const size_t sb = ((size_t)rows * (size_t)a.key_cap * 4 + 255) & ~(size_t)255;
  uint16_t* qf = (uint16_t*)((uint8_t*)a.workspace + sb);
  uint8_t* qe = (uint8_t*)(qf + (size_t)rows * (size_t)a.heads * D);
  const size_t score_lds = (size_t)RB * KB + (size_t)RB * DSTR * 4 + (size_t)HMAX * 8 + 16;
  const size_t select_lds = std::max((size_t)64 * 4 + (size_t)KMAX * 12, (size_t)TIE_SLOTS * 4);
  const void* score_fns[4] = {(const void*)csa_index_score_kernel<1>, (const void*)csa_index_score_kernel<2>,
                              (const void*)csa_index_score_kernel<3>, (const void*)csa_index_score_kernel<4>};
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipSuccess;
    for (int i = 0; i < 4 && e == hipSuccess; i++)
      e = hipFuncSetAttribute(score_fns[i], hipFuncAttributeMaxDynamicSharedMemorySize, (int)score_lds);
    if (e == hipSuccess)
      e = hipFuncSetAttribute((const void*)csa_index_select_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)select_lds);
    if (e != hipSuccess) return check_hip(c, e, "csa index LDS attribute");
    attr = true;
  }
  const int64_t hrows = rows * a.heads;
  hipLaunchKernelGGL(csa_index_finalize_kernel, dim3((unsigned)((hrows + 3) / 4)), dim3(256), 0, c->stream,
                     a.iq, qf, qe, hrows, (int)a.heads, (int)a.q_seq, a.total);
  sa_status st = check_hip(c, hipGetLastError(), "csa index finalize");
  if (st != SA_OK) return st;
  const ProfEvents pe = prof_next(c);
  const dim3 sgrid((unsigned)((a.key_cap + RC - 1) / RC), (unsigned)rows);
#define SA_IDX_SCORE(HTV)                                                                                       \
  SA_MAIN_LAUNCH(pe, csa_index_score_kernel<HTV>, sgrid, dim3(256), score_lds, c->stream, qf, qe, a.iw, a.keys, scores, \
                     (int)a.q_seq, a.key_cap, a.total, c->err)
  switch (a.heads / 16) {
    case 1: SA_IDX_SCORE(1); break;
    case 2: SA_IDX_SCORE(2); break;
    case 3: SA_IDX_SCORE(3); break;
    default: SA_IDX_SCORE(4); break;
  }
#undef SA_IDX_SCORE
  st = check_hip(c, hipGetLastError(), "csa index score");
  if (st != SA_OK) return st;
  // tie parts per row: enough to fill the chip beside the select workgroups
  const unsigned parts = (unsigned)std::max<int64_t>(1, std::min<int64_t>(3, 256 / rows - 1));
  hipLaunchKernelGGL(csa_index_select_kernel, dim3(1 + parts, (unsigned)rows), dim3(1024), select_lds, c->stream, scores,
                     a.selected, (int)a.q_seq, (int)a.out_heads, a.key_cap, (int)a.topk, a.total, c->err);
  return check_hip(c, hipGetLastError(), "csa index select");
}

}  // namespace sa
