// Shared-latent selected-token attention on the matrix cores (gfx950).
//
// When every query head reads the same kv head through the same index row
// (one shared-latent cache row per token: key = the whole 576-dim row,
// value = its first 512 dims; the CSA pages' records are both key and value),
// the per-row work is two dense products over the gathered tile:
//   S^T[key, head] = K_sel[key, :] . Q[head, :]^T      (M=keys, N=heads, K=576)
//   O^T[dv, head] += V_sel^T[dv, key] . P^T[key, head]  (M=dv, N=heads, K=keys)
// both on v_mfma_f32_16x16x32_bf16 with fp32 accumulation. Semantics are the
// IndexShare `index_share_row` ones (scaled scores, fp32 softmax, probs . V);
// the schedule is FlashDecoding-style: an online softmax per head over 32-key
// tiles and, when there are too few rows to fill 256 CUs, a split of each
// row's selected keys across workgroups merged by a log-sum-exp combine (the
// standard Attention page's `attention_split` / `attention_combine`).
//
// Workgroup: 4 waves, wave w owns heads 16w..16w+15; Q^T for them stays in
// registers for the whole row (18 k-steps x 8 bf16 per lane). Per tile the
// workgroup gathers 32 selected rows (global -> registers, the next tile's
// loads in flight while the current tile computes), writes them to LDS twice:
// row-major K (A operand of S^T) and transposed V^T (A operand of O^T), with
// the key order inside V^T matching how S^T leaves the keys in each lane, so
// the probabilities feed the PV product straight from registers.
// fp8_e4m3_block64 records are decoded on the way in (E8M0 * E4M3FN -> bf16,
// exact for scale bytes 9..246; the BF16 tail is copied).
#include "sa_internal.h"

namespace sa {

namespace mla {
constexpr int DK = 576;
constexpr int DV = 512;
constexpr int NH = 64;
constexpr int KT = 32;                // keys per tile
constexpr int KSTEPS = DK / 32;       // 18
constexpr int DVT = DV / 16;          // 32 output tiles per wave
constexpr int KSTRIDE = DK + 8;       // bf16 elements per K row in LDS (1168 B)
constexpr int VSTRIDE = KT + 8;       // bf16 elements per V^T row in LDS (80 B)
constexpr int CHUNKS = DK / 8;        // 16-byte chunks per bf16 row (72)
constexpr int VCHUNKS = DV / 8;       // chunks that also feed V^T (64)
constexpr int UNITS = (KT / 4) * CHUNKS;   // (key quad, chunk) units per tile (576)
constexpr int UPT = (UNITS + 255) / 256;   // units per thread (3)
constexpr int IDX_STAGE = 2048;       // selected keys staged in LDS at a time
constexpr int REC = 648;              // fp8 record bytes: 8 * 65 + 64 * 2
constexpr int THREADS = 256;
constexpr size_t LDS_BYTES = (size_t)KT * KSTRIDE * 2 + (size_t)DV * VSTRIDE * 2 + IDX_STAGE * 4 + 16;
}  // namespace mla

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr float kLog2eM = 1.4426950408889634f;

// physical V^T slot of the first key of quad `quad` (keys 4*quad..4*quad+3):
// lane group g of an S^T tile pair holds keys {4g..4g+3, 16+4g..16+4g+3},
// which become slots 8g..8g+7 of the PV k-dimension.
__device__ __forceinline__ int vt_slot_of_quad(int quad) {
  return quad < 4 ? 8 * quad : 8 * (quad - 4) + 4;
}

// E4M3FN code + E8M0 scale byte -> bf16 bits (exact whenever representable).
__device__ __forceinline__ uint32_t fp8_to_bf16_bits(uint32_t code, int e) {
  const uint32_t s = (code & 0x80u) << 8;
  const uint32_t mag = code & 0x7fu;
  if (mag >= 8u && mag != 0x7fu && e >= 9 && e <= 246) {
    return s | ((mag << 4) + (uint32_t)((e - 7) << 7));
  }
  if (mag == 0u) return s;
  if (mag == 0x7fu || e == 255) return 0x7fc0u;
  // general case (subnormal codes, extreme scales): exact fp32 then RNE to bf16
  const uint32_t E = mag >> 3, M = mag & 7u;
  float v = E ? __uint_as_float(((E + 120u) << 23) | (M << 20)) : (float)M * 0.001953125f;
  v = ldexpf(v, e - 127);
  return (uint32_t)f32_to_bf16_rne(s ? -v : v);
}

// Bytes [off, off+8) of a record as two dwords, from 4-byte-aligned loads.
__device__ __forceinline__ uint2 load8_unaligned(const uint8_t* rec, int off) {
  const uint32_t* w = (const uint32_t*)(rec + (off & ~3));
  const uint32_t d0 = w[0], d1 = w[1], d2 = w[2];
  const uint32_t sh = (uint32_t)(off & 3);
  uint2 r;
  r.x = __builtin_amdgcn_alignbyte(d1, d0, sh);
  r.y = __builtin_amdgcn_alignbyte(d2, d1, sh);
  return r;
}

template <bool FP8>
struct TileRegs {
  // bf16: 4 keys x 16 bytes per unit; fp8: 4 keys x (8 code bytes + scale)
  uint4 d[mla::UPT][4];
  int sc[mla::UPT][4];
};

// Issue the global loads of one tile's rows into registers.
template <bool FP8>
__device__ __forceinline__ void tile_load(TileRegs<FP8>& r, const uint8_t* __restrict__ cache_b,
                                          const int* __restrict__ keys_s, int slot0, int kend) {
  using namespace mla;
#pragma unroll
  for (int j = 0; j < UPT; j++) {
    const int u = threadIdx.x + j * THREADS;
    const int quad = u & 7;
    const int chunk = u >> 3;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int slot = slot0 + 4 * quad + i;
      r.d[j][i] = make_uint4(0, 0, 0, 0);
      r.sc[j][i] = 0;
      if (u < UNITS && slot < kend) {
        const int64_t key = keys_s[slot];
        if constexpr (!FP8) {
          r.d[j][i] = *(const uint4*)(cache_b + (key * DK + chunk * 8) * 2);
        } else {
          const uint8_t* rec = cache_b + key * REC;
          if (chunk < VCHUNKS) {
            const int blk = chunk >> 3, sub = chunk & 7;
            const uint2 c8 = load8_unaligned(rec, 65 * blk + 1 + 8 * sub);
            r.d[j][i] = make_uint4(c8.x, c8.y, 0, 0);
            const uint32_t sw = *(const uint32_t*)(rec + ((65 * blk) & ~3));
            r.sc[j][i] = (int)((sw >> (8 * ((65 * blk) & 3))) & 0xffu);
          } else {
            const uint2* t2 = (const uint2*)(rec + 520 + 16 * (chunk - VCHUNKS));
            const uint2 lo = t2[0], hi = t2[1];
            r.d[j][i] = make_uint4(lo.x, lo.y, hi.x, hi.y);
          }
        }
      }
    }
  }
}

// Write one tile from registers to LDS: K row-major and the transposed V^T.
template <bool FP8>
__device__ __forceinline__ void tile_store(const TileRegs<FP8>& r, uint16_t* __restrict__ ks,
                                           uint16_t* __restrict__ vt) {
  using namespace mla;
#pragma unroll
  for (int j = 0; j < UPT; j++) {
    const int u = threadIdx.x + j * THREADS;
    if (u >= UNITS) continue;
    const int quad = u & 7;
    const int chunk = u >> 3;
    uint32_t w[4][4];  // [key][dword] bf16 pairs
#pragma unroll
    for (int i = 0; i < 4; i++) {
      if constexpr (!FP8) {
        w[i][0] = r.d[j][i].x;
        w[i][1] = r.d[j][i].y;
        w[i][2] = r.d[j][i].z;
        w[i][3] = r.d[j][i].w;
      } else {
        if (chunk < VCHUNKS) {
          const int e = r.sc[j][i];
          const uint32_t c0 = r.d[j][i].x, c1 = r.d[j][i].y;
#pragma unroll
          for (int p = 0; p < 4; p++) {
            const uint32_t src = p < 2 ? c0 : c1;
            const uint32_t lo = fp8_to_bf16_bits((src >> (16 * (p & 1))) & 0xffu, e);
            const uint32_t hi = fp8_to_bf16_bits((src >> (16 * (p & 1) + 8)) & 0xffu, e);
            w[i][p] = lo | (hi << 16);
          }
        } else {
          w[i][0] = r.d[j][i].x;
          w[i][1] = r.d[j][i].y;
          w[i][2] = r.d[j][i].z;
          w[i][3] = r.d[j][i].w;
        }
      }
      *(uint4*)(ks + (4 * quad + i) * KSTRIDE + chunk * 8) = make_uint4(w[i][0], w[i][1], w[i][2], w[i][3]);
    }
    if (chunk < VCHUNKS) {
      const int slot = vt_slot_of_quad(quad);
#pragma unroll
      for (int e = 0; e < 8; e++) {
        const int dw = e >> 1, sh = 16 * (e & 1);
        const uint32_t k0 = (w[0][dw] >> sh) & 0xffffu, k1 = (w[1][dw] >> sh) & 0xffffu;
        const uint32_t k2 = (w[2][dw] >> sh) & 0xffffu, k3 = (w[3][dw] >> sh) & 0xffffu;
        *(uint2*)(vt + (chunk * 8 + e) * VSTRIDE + slot) = make_uint2(k0 | (k1 << 16), k2 | (k3 << 16));
      }
    }
  }
}

template <bool FP8, bool I64>
__global__ void __launch_bounds__(mla::THREADS, 1)
mla_forward_kernel(const uint16_t* __restrict__ q, const uint8_t* __restrict__ cache,
                   const void* __restrict__ idx, const int32_t* __restrict__ valid_len,
                   uint16_t* __restrict__ y, float* __restrict__ part_o,
                   float* __restrict__ part_ml, int64_t q_seq, int64_t rows, int64_t cap,
                   int64_t width, int splits, float scale, float softcap) {
  using namespace mla;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  uint16_t* ks = (uint16_t*)lds;
  uint16_t* vt = ks + KT * KSTRIDE;
  int* keys_s = (int*)(vt + DV * VSTRIDE);
  int* n_s = keys_s + IDX_STAGE;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 4;
  const int c16 = lane & 15;

  const int split = (int)(blockIdx.x % (unsigned)splits);
  const int64_t row = rows - 1 - (int64_t)(blockIdx.x / (unsigned)splits);  // long rows first
  const int64_t b = row / q_seq;
  const int64_t qi = row - b * q_seq;
  int64_t bound = valid_len ? (int64_t)valid_len[b] : cap;
  bound = bound < 0 ? 0 : (bound > cap ? cap : bound);
  const int64_t ibase = row * width;
  const int64_t row_elems = FP8 ? REC : (int64_t)DK * 2;  // bytes per cache row
  const uint8_t* cache_b = cache + b * cap * row_elems;

  // n = entries before the first -1
  if (tid == 0) *n_s = (int)width;
  __syncthreads();
  for (int64_t c = tid; c < width; c += THREADS) {
    if (load_index<I64>(idx, ibase + c) == -1) atomicMin(n_s, (int)c);
  }
  __syncthreads();
  const int n = *n_s;
  const int tiles = (n + KT - 1) / KT;
  const int tps = (tiles + splits - 1) / splits;
  const int t_begin = split * tps;
  const int t_end = min(tiles, t_begin + tps);

  // Q^T for this wave's 16 heads: lane (c16, g) holds dims ks*32 + 8g .. +8
  const int head = wave * 16 + c16;
  bf16x8_t qreg[KSTEPS];
  {
    const uint16_t* qp = q + ((b * NH + head) * q_seq + qi) * DK + 8 * g;
#pragma unroll
    for (int s = 0; s < KSTEPS; s++) {
      const uint4 raw = *(const uint4*)(qp + s * 32);
      qreg[s] = __builtin_bit_cast(bf16x8_t, raw);
    }
  }
  f32x4_t o[DVT];
#pragma unroll
  for (int t = 0; t < DVT; t++) o[t] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.0f;
  const float sl2 = scale * kLog2eM;

  TileRegs<FP8> regs;
  for (int st0 = t_begin * KT; st0 < t_end * KT; st0 += IDX_STAGE) {
    const int st_end = min(min(st0 + IDX_STAGE, t_end * KT), n);
    __syncthreads();  // previous stage's LDS readers are done
    for (int s = tid; s < st_end - st0; s += THREADS) {
      int64_t key = load_index<I64>(idx, ibase + st0 + s);
      keys_s[s] = (int)((key >= 0 && key < bound) ? key : 0);  // clamp into range
    }
    __syncthreads();
    const int kcount = st_end - st0;
    const int ntile = (kcount + KT - 1) / KT;
    tile_load<FP8>(regs, cache_b, keys_s, 0, kcount);
    for (int t = 0; t < ntile; t++) {
      tile_store<FP8>(regs, ks, vt);
      __syncthreads();
      if (t + 1 < ntile) tile_load<FP8>(regs, cache_b, keys_s, (t + 1) * KT, kcount);

      // ---- S^T = K . Q^T for two 16-key halves
      f32x4_t sacc[2] = {(f32x4_t){0.f, 0.f, 0.f, 0.f}, (f32x4_t){0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int s = 0; s < KSTEPS; s++) {
#pragma unroll
        for (int h = 0; h < 2; h++) {
          const uint4 raw = *(const uint4*)(ks + (16 * h + c16) * KSTRIDE + s * 32 + 8 * g);
          sacc[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, raw),
                                                             qreg[s], sacc[h], 0, 0, 0);
        }
      }
      // ---- online softmax over the tile (lane holds keys 16h + 4g + r, head c16)
      const int slot_base = t * KT;
      float x[8];
      float tmax = -INFINITY;
#pragma unroll
      for (int h = 0; h < 2; h++) {
#pragma unroll
        for (int r4 = 0; r4 < 4; r4++) {
          const int slot = slot_base + 16 * h + 4 * g + r4;
          float s = sacc[h][r4];
          if (softcap != 0.0f) {
            s = softcap * tanhf(s * scale / softcap) * kLog2eM;
          } else {
            s = s * sl2;
          }
          s = slot < kcount ? s : -INFINITY;
          x[4 * h + r4] = s;
          tmax = fmaxf(tmax, s);
        }
      }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
      const float m_new = fmaxf(m_run, tmax);
      const float alpha = (m_new == -INFINITY) ? 1.0f : exp2f(m_run - m_new);
      float psum = 0.0f;
      float p[8];
#pragma unroll
      for (int i = 0; i < 8; i++) {
        p[i] = (m_new == -INFINITY) ? 0.0f : exp2f(x[i] - m_new);
        psum += p[i];
      }
      psum += __shfl_xor(psum, 16, 64);
      psum += __shfl_xor(psum, 32, 64);
      l_run = alpha * l_run + psum;
      m_run = m_new;
      bf16x8_t pb;
#pragma unroll
      for (int i = 0; i < 8; i++) pb[i] = (__bf16)p[i];
      // ---- O^T += V^T . P^T
#pragma unroll
      for (int dt = 0; dt < DVT; dt++) {
        const uint4 raw = *(const uint4*)(vt + (16 * dt + c16) * VSTRIDE + 8 * g);
        o[dt] *= alpha;
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, raw), pb,
                                                        o[dt], 0, 0, 0);
      }
      __syncthreads();  // LDS tile is rewritten next iteration
    }
  }

  // ---- epilogue: lane holds O^T[16 dt + 4g + r][head]
  if (splits == 1) {
    const float inv = l_run > 0.0f ? 1.0f / l_run : 0.0f;
    uint16_t* yp = y + ((b * NH + head) * q_seq + qi) * DV + 4 * g;
#pragma unroll
    for (int dt = 0; dt < DVT; dt++) {
      const uint32_t lo = (uint32_t)f32_to_bf16_rne(o[dt][0] * inv) |
                          ((uint32_t)f32_to_bf16_rne(o[dt][1] * inv) << 16);
      const uint32_t hi = (uint32_t)f32_to_bf16_rne(o[dt][2] * inv) |
                          ((uint32_t)f32_to_bf16_rne(o[dt][3] * inv) << 16);
      *(uint2*)(yp + 16 * dt) = make_uint2(lo, hi);
    }
  } else {
    const int64_t pr = (row * splits + split) * NH + head;
    float* op = part_o + pr * DV + 4 * g;
#pragma unroll
    for (int dt = 0; dt < DVT; dt++) *(float4*)(op + 16 * dt) = make_float4(o[dt][0], o[dt][1], o[dt][2], o[dt][3]);
    if (g == 0) {
      part_ml[pr * 2] = m_run;
      part_ml[pr * 2 + 1] = l_run;
    }
  }
}

// Log-sum-exp merge of the split partials (standard Attention page,
// `attention_combine`): M = max_j m_j, y = sum_j o_j 2^(m_j-M) / sum_j l_j 2^(m_j-M)
// (m in log2 units). One 128-thread workgroup per (row, head); thread owns 4
// channels. Block b serves row b % rows, so it runs on the XCD whose L2 took
// that row's partials. Every split's (m, l) and partial output in a round of
// CH splits is loaded before any is used, so the merge costs one memory round
// trip per CH splits, not one per split.
template <int CH>
__global__ void __launch_bounds__(128)
mla_combine_kernel(const float* __restrict__ part_o, const float* __restrict__ part_ml,
                   uint16_t* __restrict__ y, int64_t rows, int64_t q_seq, int splits) {
  using namespace mla;
  const int64_t row = (int64_t)(blockIdx.x % (unsigned)rows);
  const int head = (int)(blockIdx.x / (unsigned)rows);
  const int64_t b = row / q_seq, qi = row - b * q_seq;
  const int d = threadIdx.x * 4;
  float M = -INFINITY, L = 0.0f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j0 = 0; j0 < splits; j0 += CH) {
    float2 ml[CH];
    float4 v[CH];
#pragma unroll
    for (int j = 0; j < CH; j++) {
      const int64_t pr = (row * splits + j0 + j) * NH + head;
      if (j0 + j < splits) {
        ml[j] = *(const float2*)(part_ml + pr * 2);
        v[j] = *(const float4*)(part_o + pr * DV + d);
      } else {
        ml[j] = make_float2(-INFINITY, 0.0f);
        v[j] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
    float Mn = M;
#pragma unroll
    for (int j = 0; j < CH; j++) Mn = fmaxf(Mn, ml[j].x);
    if (Mn == -INFINITY) continue;  // no key in these splits yet
    const float r = M == -INFINITY ? 0.0f : exp2f(M - Mn);  // rescale what is merged so far
    L *= r;
    acc.x *= r;
    acc.y *= r;
    acc.z *= r;
    acc.w *= r;
#pragma unroll
    for (int j = 0; j < CH; j++) {
      const float w = ml[j].x == -INFINITY ? 0.0f : exp2f(ml[j].x - Mn);
      L += ml[j].y * w;
      acc.x += v[j].x * w;
      acc.y += v[j].y * w;
      acc.z += v[j].z * w;
      acc.w += v[j].w * w;
    }
    M = Mn;
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  uint16_t* yp = y + ((b * NH + head) * q_seq + qi) * DV + d;
  const uint32_t lo = (uint32_t)f32_to_bf16_rne(acc.x * inv) | ((uint32_t)f32_to_bf16_rne(acc.y * inv) << 16);
  const uint32_t hi = (uint32_t)f32_to_bf16_rne(acc.z * inv) | ((uint32_t)f32_to_bf16_rne(acc.w * inv) << 16);
  *(uint2*)yp = make_uint2(lo, hi);
}

sa_status launch_mla_combine(sparse_attn_ctx* c, int64_t rows, int64_t q_seq, int splits, uint16_t* y) {
  hipLaunchKernelGGL(mla_combine_kernel<8>, dim3((unsigned)(rows * mla::NH)), dim3(mla::DV / 4), 0,
                     c->stream, c->partial_o, c->partial_ml, y, rows, q_seq, splits);
  return check_hip(c, hipGetLastError(), "forward (combine)");
}

bool mla_supported(const sa_config& cfg, int64_t index_heads) {
  return cfg.kv_layout == SA_KV_SHARED_LATENT && cfg.dtype == SA_BF16 && cfg.num_heads == mla::NH &&
         cfg.kv_num_heads == 1 && cfg.head_dim_qk == mla::DK && cfg.head_dim_v == mla::DV &&
         index_heads == 1 &&
         (cfg.cache_format == SA_CACHE_DENSE ||
          (cfg.cache_format == SA_CACHE_FP8_E4M3_BLOCK64 && cfg.rope_dim == 64));
}

// Splits per row so that rows * splits covers the 256 CUs, keeping at least
// two 32-key tiles per split.
int mla_splits(int64_t rows, int64_t width) {
  if (rows >= kNumCUs) return 1;
  const int64_t want = (kNumCUs + rows - 1) / rows;
  const int64_t max_by_keys = std::max<int64_t>(1, (width + 2 * mla::KT - 1) / (2 * mla::KT));
  return (int)std::min<int64_t>(std::min<int64_t>(want, max_by_keys), 64);
}

static bool g_mla_attr_set[4] = {false, false, false, false};

sa_status launch_forward_mla(sparse_attn_ctx* c, const FwdArgs& a, int splits) {
  using namespace mla;
  const int64_t rows = a.batch * a.q_seq;
  if (rows <= 0) return SA_OK;
  if (splits > 1 && rows * splits > c->partial_rows)
    return set_error(c, SA_E_STATE, "forward: split-K partials exceed the context's buffers");
  const int64_t wgs = rows * splits;
  if (wgs > 0x7fffffffLL) return set_error(c, SA_E_SHAPE, "forward: too many rows for one launch");
  const bool fp8 = a.cache_format == SA_CACHE_FP8_E4M3_BLOCK64;
  const int variant = (fp8 ? 2 : 0) + (a.idx64 ? 1 : 0);
  const void* fn = nullptr;
  switch (variant) {
    case 0: fn = (const void*)mla_forward_kernel<false, false>; break;
    case 1: fn = (const void*)mla_forward_kernel<false, true>; break;
    case 2: fn = (const void*)mla_forward_kernel<true, false>; break;
    default: fn = (const void*)mla_forward_kernel<true, true>; break;
  }
  if (!g_mla_attr_set[variant]) {
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)LDS_BYTES);
    if (e != hipSuccess) return check_hip(c, e, "forward (mla) LDS attribute");
    g_mla_attr_set[variant] = true;
  }
  const dim3 grid((unsigned)wgs), block(THREADS);
  const ProfEvents pe = prof_next(c);
#define SA_MLA(F8, I)                                                                             \
  SA_MAIN_LAUNCH(pe, (mla_forward_kernel<F8, I>), grid, block, LDS_BYTES, c->stream,              \
                     (const uint16_t*)a.q, (const uint8_t*)a.k, a.idx, a.valid_len,               \
                     (uint16_t*)a.y, c->partial_o, c->partial_ml, a.q_seq, rows, a.cap, a.width, \
                     splits, a.scale, a.softcap)
  switch (variant) {
    case 0: SA_MLA(false, false); break;
    case 1: SA_MLA(false, true); break;
    case 2: SA_MLA(true, false); break;
    default: SA_MLA(true, true); break;
  }
#undef SA_MLA
  sa_status s = check_hip(c, hipGetLastError(), "forward (mla)");
  if (s != SA_OK || splits == 1) return s;
  return launch_mla_combine(c, rows, a.q_seq, splits, (uint16_t*)a.y);
}

}  // namespace sa
