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
//  3. select: a workgroup per (batch, query): the scores' total-order keys in
//     LDS, a radix select of the k-th largest key, the winners (ties in
//     ascending record order) sorted by (-score, +record) with a bitonic sort,
//     written to every index-head row of the output.
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
constexpr int RB = 256;           // records per score pass (one per thread)
constexpr int DSTR = 65;          // LDS row stride (floats) of the dot table
constexpr int KMAX = 2048;        // selected width
constexpr int NMAX = 32768;       // records per (batch, query) the select keeps in LDS
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
csa_index_finalize_kernel(const float* __restrict__ iq, uint16_t* __restrict__ qf, int64_t rows, int H,
                          int S, const int64_t* __restrict__ total_ptr) {
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
}

// ---------------------------------------------------------------- score

__global__ void __launch_bounds__(256, 1)
csa_index_score_kernel(const uint16_t* __restrict__ qf, const float* __restrict__ iw,
                       const uint8_t* __restrict__ keys, float* __restrict__ scores, int S, int H,
                       int64_t kcap, const int64_t* __restrict__ total_ptr, ErrorBlock* __restrict__ eb) {
  using namespace cx;
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
  const int HT = H / 16;

  // the finalized query as B operands: lane (head i16 of tile ht, g) holds
  // dims 32 c + 8 g .. + 7
  u32x4_l qb[HMAX / 16][4];
  const uint16_t* qrow = qf + row * H * D;
#pragma unroll
  for (int ht = 0; ht < HMAX / 16; ht++)
#pragma unroll
    for (int c = 0; c < 4; c++)
      qb[ht][c] = ht < HT ? *(const u32x4_l*)(qrow + (int64_t)(16 * ht + i16) * D + 32 * c + 8 * g)
                          : (u32x4_l){0u, 0u, 0u, 0u};
  const float ws = (1.0f / sqrtf((float)D)) / sqrtf((float)H);

  uint8_t* kl = smem;                                     // RB keys, 68 B each
  float* dt = (float*)(smem + RB * KB);                   // [RB][DSTR] dot products
  float* wl = dt + RB * DSTR;                             // [H] weights
  if (tid < H) wl[tid] = iw[row * H + tid];
  const uint8_t* kb = keys + (b * kcap) * KB;
  bool bad = false;

  for (int64_t r0 = c0; r0 < c0 + RC && r0 < n; r0 += RB) {
    __syncthreads();  // the previous pass's LDS reads are done
    // stage RB keys (coalesced dwords; records past the capacity read as zeros)
    const int64_t nk = min((int64_t)RB, kcap - r0);
    const uint32_t* src = (const uint32_t*)(kb + r0 * KB);
    for (int i = tid; i < RB * KB / 4; i += 256)
      ((uint32_t*)kl)[i] = i < nk * (KB / 4) ? src[i] : 0u;
    __syncthreads();
    // S^T for the wave's 64 records: record tiles rt, head tiles ht, blocks c
    f32x4_l acc[4][HMAX / 16];
#pragma unroll
    for (int rt = 0; rt < 4; rt++)
#pragma unroll
      for (int ht = 0; ht < HMAX / 16; ht++) acc[rt][ht] = (f32x4_l){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int rt = 0; rt < 4; rt++) {
      const int rec = 64 * w + 16 * rt + i16;
      const uint8_t* kr = kl + rec * KB;
#pragma unroll
      for (int c = 0; c < 4; c++) {
        // 4 code bytes at 17 c + 1 + 4 g (unaligned) and the block's scale byte
        const int o = 17 * c + 1 + 4 * g;
        const uint32_t* wp = (const uint32_t*)(kr + (o & ~3));
        const uint32_t cw = __builtin_amdgcn_alignbyte(wp[1], wp[0], (uint32_t)(o & 3));
        const uint32_t e = kr[17 * c];
        const float sc = e == 255u ? __uint_as_float(0x7fc00000u) : (e ? __uint_as_float(e << 23) : 5.877471754e-39f);
        u32x4_l a;
        a[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, sc, 0));
        a[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, sc, 1));
        a[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, sc, 2));
        a[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, sc, 3));
        const bf16x8_l av = __builtin_bit_cast(bf16x8_l, a);
#pragma unroll
        for (int ht = 0; ht < HMAX / 16; ht++)
          if (ht < HT)
            acc[rt][ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8_l, qb[ht][c]),
                                                                 acc[rt][ht], 0, 0, 0);
      }
    }
    // lane (head i16 of tile ht, g) holds records 4 g .. 4 g + 3 of tile rt
#pragma unroll
    for (int rt = 0; rt < 4; rt++)
#pragma unroll
      for (int ht = 0; ht < HMAX / 16; ht++)
        if (ht < HT)
#pragma unroll
          for (int j = 0; j < 4; j++) dt[(64 * w + 16 * rt + 4 * g + j) * DSTR + 16 * ht + i16] = acc[rt][ht][j];
    __syncthreads();
    // one record per thread: the head sum in ascending head order
    const int64_t r = r0 + tid;
    if (r < n) {
      const float* d = dt + tid * DSTR;
      float score = 0.0f;
      for (int h = 0; h < H; h++) {
        const float x = d[h];
        const float relu = x > 0.0f ? x : 0.0f;
        const float t0 = relu * wl[h];
        const float t1 = t0 * ws;
        score = score + t1;
      }
      bad |= !isfinite(score);
      scores[row * kcap + r] = score;
    }
  }
  if (__builtin_amdgcn_ballot_w64(bad) != 0 && lane == 0) atomicOr(&eb->word, SA_ERR_INDEX_NONFINITE);
}

// ---------------------------------------------------------------- select

// strictly monotone map of a float's total order (Rust f32::total_cmp) to u32
__device__ __forceinline__ uint32_t total_key(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__global__ void __launch_bounds__(256)
csa_index_select_kernel(const float* __restrict__ scores, int32_t* __restrict__ sel, int S, int out_heads,
                        int64_t kcap, int K, const int64_t* __restrict__ total_ptr,
                        ErrorBlock* __restrict__ eb) {
  using namespace cx;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;  // (b, s)
  const int s = (int)(row % S);
  const int64_t b = row / S;
  const int64_t total = *total_ptr;
  const int64_t pos = total - S + s;
  int32_t* outb = sel + (b * out_heads * S + s) * K;  // head 0 row; head h at + h S K
  if (pos < s) {  // total < S
    if (row == 0 && tid == 0) atomicOr(&eb->word, SA_ERR_CSA_GEOMETRY);
    return;
  }
  int64_t n64 = (pos + 1) / 4;
  if (n64 > kcap) n64 = kcap;
  const int n = (int)n64;
  uint32_t* key = (uint32_t*)smem;                       // [NMAX] total-order keys
  unsigned long long* win = (unsigned long long*)(smem + NMAX * 4);  // [KMAX] winners
  uint32_t* hist = (uint32_t*)(win + KMAX);              // [256]
  uint32_t* misc = hist + 256;                           // [8]
  const float* src = scores + row * kcap;
  for (int i = tid; i < n; i += 256) key[i] = total_key(src[i]);
  const int k = min(K, n);
  // threshold T: the k-th largest key (radix select, 8 bits at a time)
  uint32_t prefix = 0, pmask = 0;
  int need = k;  // how many of the keys matching the prefix are still to take
  if (k > 0 && k < n) {
    for (int shift = 24; shift >= 0; shift -= 8) {
      __syncthreads();
      hist[tid] = 0;
      __syncthreads();
      for (int i = tid; i < n; i += 256) {
        const uint32_t x = key[i];
        if ((x & pmask) == prefix) atomicAdd(&hist[(x >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (tid == 0) {
        int acc = 0, d = 255;
        for (; d > 0; d--) {
          if (acc + (int)hist[d] >= need) break;
          acc += (int)hist[d];
        }
        misc[0] = (uint32_t)d;
        misc[1] = (uint32_t)(need - acc);
      }
      __syncthreads();
      prefix |= misc[0] << shift;
      pmask |= 255u << shift;
      need = (int)misc[1];
    }
  }
  const uint32_t T = prefix;  // with k < n: keys > T all win, `need` of the keys == T win
  // gather the winners as (key, ~record) pairs: keys > T anywhere, ties by
  // ascending record (a scan over contiguous per-thread ranges)
  __syncthreads();
  if (tid == 0) misc[2] = 0;
  const int per = (n + 255) / 256;
  const int lo = min(n, tid * per), hi = min(n, lo + per);
  int eq = 0;
  if (k < n)
    for (int i = lo; i < hi; i++) eq += key[i] == T;
  // exclusive scan of eq over threads (in LDS)
  hist[tid] = (uint32_t)eq;
  __syncthreads();
  if (tid == 0) {
    uint32_t run = 0;
    for (int t = 0; t < 256; t++) {
      const uint32_t v = hist[t];
      hist[t] = run;
      run += v;
    }
  }
  __syncthreads();
  int eq_before = (int)hist[tid];
  for (int i = lo; i < hi; i++) {
    const uint32_t x = key[i];
    bool take;
    if (k >= n) {
      take = true;
    } else if (x > T) {
      take = true;
    } else if (x == T) {
      take = eq_before < need;
      eq_before++;
    } else {
      take = false;
    }
    if (take) {
      const uint32_t slot = atomicAdd(&misc[2], 1u);
      win[slot] = ((unsigned long long)x << 32) | (uint32_t)(~(uint32_t)i);
    }
  }
  __syncthreads();
  // bitonic sort, descending, over the next power of two >= k (padding 0)
  int m = 1;
  while (m < k) m <<= 1;
  for (int i = k + tid; i < m; i += 256) win[i] = 0ull;
  __syncthreads();
  for (int size = 2; size <= m; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < m / 2; i += 256) {
        const int lo_i = (i / stride) * 2 * stride + (i % stride);
        const int hi_i = lo_i + stride;
        const bool desc = ((lo_i & size) == 0);
        const unsigned long long a = win[lo_i], c = win[hi_i];
        if ((a < c) == desc) {
          win[lo_i] = c;
          win[hi_i] = a;
        }
      }
      __syncthreads();
    }
  }
  // write every index-head row
  for (int j = tid; j < K; j += 256) {
    const int32_t v = j < k ? (int32_t)(~(uint32_t)(win[j] & 0xffffffffull)) : -1;
    for (int h = 0; h < out_heads; h++) outb[(int64_t)h * S * K + j] = v;
  }
}

size_t csa_index_workspace_bytes(int64_t rows, int64_t H, int64_t kcap) {
  // scores fp32 [rows][kcap], then the finalized queries bf16 [rows][H][128]
  const size_t sb = ((size_t)rows * (size_t)kcap * 4 + 255) & ~(size_t)255;
  return sb + (size_t)rows * (size_t)H * cx::D * 2;
}

sa_status launch_csa_index_select(sparse_attn_ctx* c, const CsaIndexArgs& a) {
  using namespace cx;
  const int64_t rows = a.batch * a.q_seq;
  float* scores = (float*)a.workspace;
  const size_t sb = ((size_t)rows * (size_t)a.key_cap * 4 + 255) & ~(size_t)255;
  uint16_t* qf = (uint16_t*)((uint8_t*)a.workspace + sb);
  const size_t score_lds = (size_t)RB * KB + (size_t)RB * DSTR * 4 + HMAX * 4;
  const size_t select_lds = (size_t)NMAX * 4 + (size_t)KMAX * 8 + 264 * 4;
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute((const void*)csa_index_score_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)score_lds);
    if (e == hipSuccess)
      e = hipFuncSetAttribute((const void*)csa_index_select_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)select_lds);
    if (e != hipSuccess) return check_hip(c, e, "csa index LDS attribute");
    attr = true;
  }
  const int64_t hrows = rows * a.heads;
  hipLaunchKernelGGL(csa_index_finalize_kernel, dim3((unsigned)((hrows + 3) / 4)), dim3(256), 0, c->stream,
                     a.iq, qf, hrows, (int)a.heads, (int)a.q_seq, a.total);
  sa_status st = check_hip(c, hipGetLastError(), "csa index finalize");
  if (st != SA_OK) return st;
  prof_begin(c);
  hipLaunchKernelGGL(csa_index_score_kernel, dim3((unsigned)((a.key_cap + RC - 1) / RC), (unsigned)rows),
                     dim3(256), score_lds, c->stream, qf, a.iw, a.keys, scores, (int)a.q_seq, (int)a.heads,
                     a.key_cap, a.total, c->err);
  prof_end(c);
  st = check_hip(c, hipGetLastError(), "csa index score");
  if (st != SA_OK) return st;
  hipLaunchKernelGGL(csa_index_select_kernel, dim3((unsigned)rows), dim3(256), select_lds, c->stream, scores,
                     a.selected, (int)a.q_seq, (int)a.out_heads, a.key_cap, (int)a.topk, a.total, c->err);
  return check_hip(c, hipGetLastError(), "csa index select");
}

}  // namespace sa
