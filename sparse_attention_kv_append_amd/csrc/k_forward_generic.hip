// Generic forward: selected-token attention on the vector ALUs, for every
// configuration the shared-latent MFMA kernel does not take (f32/f16/bf16,
// grouped-query heads, one index list per head or one per (batch, query),
// separate or shared-latent caches, fp8 records, softcap).
//
// Semantics are IndexShare's `index_share_row` (scaled dot products over the
// selected keys, fp32 softmax, probs . V). The schedule is not: one workgroup
// serves every head that shares one index row and one kv head (up to 8), so a
// gathered key row is read once for all of them; keys are processed 256 at a
// time with an online softmax (running max and sum per head, rescaling the
// accumulators), instead of a global score scratch and a serial lead thread.
#include "sa_internal.h"

namespace sa {

constexpr int kGenThreads = 256;
constexpr int kGenMaxHeads = 8;
constexpr int kGenPairs = 8;   // (head, 2 channels) output pairs per thread: 8*256*2 = 4096 >= 8*512
constexpr float kLog2e = 1.4426950408889634f;

// fp8_e4m3_block64 element d of a record (CSA CPU page `dequantize_cache`):
// E4M3FN code times 2^(scale-127) for the first `nope` dims, BF16 tail after.
__device__ __forceinline__ float fp8_record_elem(const uint8_t* __restrict__ rec, int d, int nope) {
  if (d < nope) {
    const int j = d >> 6;
    const uint32_t e = rec[65 * j];
    const uint32_t code = rec[65 * j + 1 + (d & 63)];
    const uint32_t E = (code >> 3) & 0xfu, M = code & 7u;
    float v;
    if (E == 0) {
      v = (float)M * 0.001953125f;  // M * 2^-9
    } else if (E == 15 && M == 7) {
      v = __uint_as_float(0x7fc00000u);
    } else {
      v = __uint_as_float(((E + 120u) << 23) | (M << 20));
    }
    if (code & 0x80u) v = -v;
    if (e == 255u) return __uint_as_float(0x7fc00000u);
    return ldexpf(v, (int)e - 127);
  }
  const int i = d - nope;
  const int t = 65 * (nope >> 6) + 2 * i;
  return bf16_to_f32((uint16_t)(rec[t] | (rec[t + 1] << 8)));
}

template <int DT, bool FP8>
__device__ __forceinline__ float cache_elem(const void* __restrict__ base, int64_t row,
                                            int64_t row_elems, int64_t rec_bytes, int d, int nope) {
  if constexpr (FP8) {
    return fp8_record_elem((const uint8_t*)base + row * rec_bytes, d, nope);
  } else {
    return load_elem<DT>(base, row * row_elems + d);
  }
}

template <int DT, bool FP8, bool I64>
__global__ void __launch_bounds__(kGenThreads)
generic_forward_kernel(const void* __restrict__ q, const void* __restrict__ kc,
                       const void* __restrict__ vc, const void* __restrict__ idx,
                       const int32_t* __restrict__ valid_len, void* __restrict__ y,
                       int64_t hq, int64_t hkv, int64_t q_seq, int dk, int dv, int rope,
                       int64_t cap, int64_t index_heads, int64_t width, int64_t head_chunks,
                       float scale, float softcap, const void* __restrict__ bias, int64_t bd0,
                       int64_t bd1, int64_t bd2, int64_t bd3) {
  extern __shared__ float smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t group = hq / hkv;

  // ---- which heads / index row this workgroup serves
  int64_t wg = blockIdx.x;
  int64_t b, qi, kvh, h0, ih;
  int nh;
  if (index_heads == 1) {
    const int64_t hc = wg % head_chunks;
    wg /= head_chunks;
    kvh = wg % hkv;
    wg /= hkv;
    qi = wg % q_seq;
    b = wg / q_seq;
    h0 = kvh * group + hc * kGenMaxHeads;
    nh = (int)min((int64_t)kGenMaxHeads, group - hc * kGenMaxHeads);
    ih = 0;
  } else {
    h0 = wg % hq;
    wg /= hq;
    qi = wg % q_seq;
    b = wg / q_seq;
    kvh = h0 / group;
    nh = 1;
    ih = h0;
  }
  int64_t bound = valid_len ? (int64_t)valid_len[b] : cap;
  bound = bound < 0 ? 0 : (bound > cap ? cap : bound);
  const int64_t ibase = ((b * index_heads + ih) * q_seq + qi) * width;
  const int nope = dk - rope;
  const int64_t rec_bytes = (int64_t)(nope / 64) * 65 + 2 * rope;
  const bool latent_v = (vc == nullptr);

  float* q_s = smem;                              // [nh][dk]
  float* s_s = q_s + kGenMaxHeads * dk;           // [kGenMaxHeads][256]
  int* key_s = (int*)(s_s + kGenMaxHeads * kGenThreads);  // [256]
  float* red = (float*)(key_s + kGenThreads);     // [4 waves][kGenMaxHeads]
  float* alpha_s = red + 4 * kGenMaxHeads;        // [kGenMaxHeads]
  int* n_s = (int*)(alpha_s + kGenMaxHeads);

  for (int i = tid; i < nh * dk; i += kGenThreads) {
    const int h = i / dk, d = i - h * dk;
    q_s[i] = load_elem<DT>(q, ((b * hq + h0 + h) * q_seq + qi) * dk + d);
  }
  // n = number of entries before the first -1
  if (tid == 0) *n_s = (int)width;
  __syncthreads();
  for (int64_t c = tid; c < width; c += kGenThreads) {
    if (load_index<I64>(idx, ibase + c) == -1) atomicMin(n_s, (int)c);
  }
  __syncthreads();
  const int n = *n_s;

  float m_run[kGenMaxHeads], l_run[kGenMaxHeads];
#pragma unroll
  for (int h = 0; h < kGenMaxHeads; h++) {
    m_run[h] = -INFINITY;
    l_run[h] = 0.0f;
  }
  const int half_dv = dv >> 1;
  float2 o[kGenPairs];
#pragma unroll
  for (int j = 0; j < kGenPairs; j++) o[j] = make_float2(0.0f, 0.0f);

  const int64_t kv_row0 = (b * hkv + kvh) * cap;
  const float sl2 = scale * kLog2e;

  for (int c0 = 0; c0 < n; c0 += kGenThreads) {
    const int cnt = min(kGenThreads, n - c0);
    // ---- scores: one key per thread, all heads of the group
    float sc[kGenMaxHeads];
    if (tid < cnt) {
      int64_t key = load_index<I64>(idx, ibase + c0 + tid);
      key = (key >= 0 && key < bound) ? key : 0;  // clamp: a bad row stays in bounds
      key_s[tid] = (int)key;
      float acc[kGenMaxHeads];
#pragma unroll
      for (int h = 0; h < kGenMaxHeads; h++) acc[h] = 0.0f;
      const int64_t krow = kv_row0 + key;
      if constexpr (!FP8 && DT == SA_BF16) {
        if ((dk & 7) == 0) {
          const uint4* kp = (const uint4*)((const uint16_t*)kc + krow * dk);
          for (int d8 = 0; d8 < dk / 8; d8++) {
            const uint4 raw = kp[d8];
            const uint32_t wv[4] = {raw.x, raw.y, raw.z, raw.w};
            float kf[8];
#pragma unroll
            for (int e = 0; e < 4; e++) {
              kf[2 * e] = __uint_as_float(wv[e] << 16);
              kf[2 * e + 1] = __uint_as_float(wv[e] & 0xffff0000u);
            }
#pragma unroll
            for (int h = 0; h < kGenMaxHeads; h++) {
              if (h < nh) {
                const float* qh = q_s + h * dk + d8 * 8;
#pragma unroll
                for (int e = 0; e < 8; e++) acc[h] = fmaf(qh[e], kf[e], acc[h]);
              }
            }
          }
        } else {
          for (int d = 0; d < dk; d++) {
            const float kd = load_elem<DT>(kc, krow * dk + d);
#pragma unroll
            for (int h = 0; h < kGenMaxHeads; h++)
              if (h < nh) acc[h] = fmaf(q_s[h * dk + d], kd, acc[h]);
          }
        }
      } else {
        for (int d = 0; d < dk; d++) {
          const float kd = cache_elem<DT, FP8>(kc, krow, dk, rec_bytes, d, nope);
#pragma unroll
          for (int h = 0; h < kGenMaxHeads; h++)
            if (h < nh) acc[h] = fmaf(q_s[h * dk + d], kd, acc[h]);
        }
      }
      // the optional bias of (b, head, query, key): an extent of 1 broadcasts
      // (IndexShare `bias_at`); added after the softcap
      int64_t boff = 0;
      if (bias) boff = (((bd0 == 1 ? 0 : b) * bd1) * bd2 + (bd2 == 1 ? 0 : qi)) * bd3 + (bd3 == 1 ? 0 : key);
#pragma unroll
      for (int h = 0; h < kGenMaxHeads; h++) {
        float s = acc[h] * scale;
        if (softcap != 0.0f) s = softcap * tanhf(s / softcap);
        if (bias && h < nh) s += load_elem<DT>(bias, boff + (bd1 == 1 ? 0 : (h0 + h) * bd2 * bd3));
        sc[h] = s * kLog2e;
      }
    } else {
#pragma unroll
      for (int h = 0; h < kGenMaxHeads; h++) sc[h] = -INFINITY;
    }
    (void)sl2;
    // ---- chunk max per head, then the online update
#pragma unroll
    for (int h = 0; h < kGenMaxHeads; h++) {
      if (h < nh) {
        const float mx = wave_max(sc[h]);
        if (lane == 0) red[wave * kGenMaxHeads + h] = mx;
      }
    }
    __syncthreads();
    float m_new[kGenMaxHeads];
#pragma unroll
    for (int h = 0; h < kGenMaxHeads; h++) {
      if (h < nh) {
        float cm = fmaxf(fmaxf(red[h], red[kGenMaxHeads + h]),
                         fmaxf(red[2 * kGenMaxHeads + h], red[3 * kGenMaxHeads + h]));
        m_new[h] = fmaxf(m_run[h], cm);
        const float p = (m_new[h] == -INFINITY) ? 0.0f : exp2f(sc[h] - m_new[h]);
        s_s[h * kGenThreads + tid] = p;
        sc[h] = p;
      }
    }
    __syncthreads();  // red reused below
#pragma unroll
    for (int h = 0; h < kGenMaxHeads; h++) {
      if (h < nh) {
        const float ps = wave_sum(sc[h]);
        if (lane == 0) red[wave * kGenMaxHeads + h] = ps;
      }
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < kGenMaxHeads; h++) {
      if (h < nh) {
        const float alpha = (m_new[h] == -INFINITY) ? 1.0f : exp2f(m_run[h] - m_new[h]);
        const float psum = (red[h] + red[kGenMaxHeads + h]) +
                           (red[2 * kGenMaxHeads + h] + red[3 * kGenMaxHeads + h]);
        l_run[h] = alpha * l_run[h] + psum;
        m_run[h] = m_new[h];
        if (tid == 0) alpha_s[h] = alpha;
      }
    }
    __syncthreads();
    // ---- PV: thread owns (head, channel pair) outputs
#pragma unroll
    for (int j = 0; j < kGenPairs; j++) {
      const int pi = tid + j * kGenThreads;
      if (pi < nh * half_dv) {
        const int h = pi / half_dv;
        const int d = 2 * (pi - h * half_dv);
        const float alpha = alpha_s[h];
        float ox = o[j].x * alpha, oy = o[j].y * alpha;
        const float* ph = s_s + h * kGenThreads;
        for (int t = 0; t < cnt; t++) {
          const int64_t vrow = kv_row0 + key_s[t];
          float vx, vy;
          if (latent_v) {
            if (!FP8 && DT == SA_BF16 && (dk & 1) == 0) {
              const uint32_t w2 = *(const uint32_t*)((const uint16_t*)kc + vrow * dk + d);
              vx = __uint_as_float(w2 << 16);
              vy = __uint_as_float(w2 & 0xffff0000u);
            } else {
              vx = cache_elem<DT, FP8>(kc, vrow, dk, rec_bytes, d, nope);
              vy = cache_elem<DT, FP8>(kc, vrow, dk, rec_bytes, d + 1, nope);
            }
          } else {
            vx = load_elem<DT>(vc, vrow * dv + d);
            vy = load_elem<DT>(vc, vrow * dv + d + 1);
          }
          const float p = ph[t];
          ox = fmaf(p, vx, ox);
          oy = fmaf(p, vy, oy);
        }
        o[j] = make_float2(ox, oy);
      }
    }
    __syncthreads();  // s_s / key_s / alpha_s are rewritten by the next chunk
  }

  // ---- normalise and store
  __shared__ float inv_s[kGenMaxHeads];
  if (tid < nh) {
    // every thread holds the same l_run; thread h publishes head h's reciprocal
    float l = 0.0f;
#pragma unroll
    for (int h = 0; h < kGenMaxHeads; h++)
      if (h == tid) l = l_run[h];
    inv_s[tid] = l > 0.0f ? 1.0f / l : 0.0f;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kGenPairs; j++) {
    const int pi = tid + j * kGenThreads;
    if (pi < nh * half_dv) {
      const int h = pi / half_dv;
      const int d = 2 * (pi - h * half_dv);
      const float inv = inv_s[h];
      const int64_t yo = ((b * hq + h0 + h) * q_seq + qi) * dv + d;
      store_elem<DT>(y, yo, o[j].x * inv);
      store_elem<DT>(y, yo + 1, o[j].y * inv);
    }
  }
}

sa_status launch_forward_generic(sparse_attn_ctx* c, const FwdArgs& a) {
  const int64_t group = a.hq / a.hkv;
  const int64_t head_chunks = (group + kGenMaxHeads - 1) / kGenMaxHeads;
  const int64_t wgs = (a.index_heads == 1) ? a.batch * a.q_seq * a.hkv * head_chunks
                                           : a.batch * a.q_seq * a.hq;
  if (wgs <= 0) return SA_OK;
  if (wgs > 0x7fffffffLL) return set_error(c, SA_E_SHAPE, "forward: too many rows for one launch");
  const size_t smem = sizeof(float) * (size_t)(kGenMaxHeads * a.dk + kGenMaxHeads * kGenThreads +
                                               kGenThreads + 4 * kGenMaxHeads + kGenMaxHeads + 1);
  const dim3 grid((unsigned)wgs), block(kGenThreads);
  const bool fp8 = a.cache_format == SA_CACHE_FP8_E4M3_BLOCK64;
  const ProfEvents pe = prof_next(c);
#define SA_GEN(DT, F8, I)                                                                        \
  SA_MAIN_LAUNCH(pe, (generic_forward_kernel<DT, F8, I>), grid, block, smem, c->stream, a.q, a.k, \
                     a.v, a.idx, a.valid_len, a.y, a.hq, a.hkv, a.q_seq, (int)a.dk, (int)a.dv,    \
                     (int)a.rope, a.cap, a.index_heads, a.width, head_chunks, a.scale, a.softcap,  \
                     a.bias, a.bd[0], a.bd[1], a.bd[2], a.bd[3])
#define SA_GEN_I(DT, F8) \
  if (a.idx64) { SA_GEN(DT, F8, true); } else { SA_GEN(DT, F8, false); }
  if (fp8) {
    SA_GEN_I(SA_BF16, true);
  } else if (a.dtype == SA_F32) {
    SA_GEN_I(SA_F32, false);
  } else if (a.dtype == SA_F16) {
    SA_GEN_I(SA_F16, false);
  } else {
    SA_GEN_I(SA_BF16, false);
  }
#undef SA_GEN_I
#undef SA_GEN
  return check_hip(c, hipGetLastError(), "forward (generic)");
}

}  // namespace sa
