// CSA ratio-4 selected sink attention on the gfx950 matrix cores.
//
// The compressed-sparse-attention pages (onnx-runtime-ep-cuda and -cpu,
// src/kernels/compressed_sparse_attention.rs: the `csa_ratio4_sink_attention`
// kernel, `ratio4_attention`, `AttentionBias`) attend each (batch, query,
// head) over a dense causal window of at most 128 current_kv rows plus the
// top-k selected 583-byte fp8 records, in fp32, with exp(head_sink - max)
// added to the softmax denominator after the candidates' maximum.
//
// Every head of a (batch, query) reads the same candidates, so per 32-key
// tile the scores S^T = K . Q^T and the update O^T += V^T . P^T are dense
// products. The operands are fp32, and the matrix cores take bf16: each fp32
// operand x is carried as three bf16 pieces x1 + x2 + x3 (each the nearest
// bf16 to what the previous ones leave), which hold x exactly, and a product
// sums the piece products whose weight is at least 2^-16 of the leading one.
// The records decode to bf16 exactly (an E4M3FN code times a power of two, or
// a BF16 tail value), so a record key or value takes one piece and its
// products with the query or probabilities are exact; a current_kv row takes
// three, and its product drops the terms below 2^-16 relative (x2*y3, x3*y2,
// x3*y3). Accumulation is fp32 on the matrix cores.
//
// Work split: one workgroup of four waves per (batch, query, 16-head group);
// wave w owns dims 128w .. 128w+127 of every key and of the output. Per tile
// each wave stages its own 128-dim slice of the 32 keys into LDS (bf16; a
// current_kv slice as three bf16 planes), computes the partial S^T over its
// dims, and the four partials are summed through LDS (one barrier per tile)
// in a fixed order, so every wave holds the same scores, maxima and sums.
// Global loads run two tiles ahead in registers.
//
// LDS rows of 256 bytes hold 16-byte chunk c of key row R at chunk
// c ^ 2 (R & 7) ^ ((R >> 3) & 1): the K reads (16 rows x one chunk) and the
// transposing V reads (8 rows x one 32-byte pair) both land on distinct banks.
#include "sa_mfma_dev.h"
#include "sa_quant_dev.h"

namespace sa {

namespace cs {
constexpr int D = 512;                  // logical dims of a key / value / query row
constexpr int REC = 583;                // record bytes: 7 x (1 + 64) + 64 x 2
constexpr int TAILB = 455;              // first BF16 tail byte of a record
constexpr int WIN = 128;                // dense window
constexpr int KT = 32;                  // keys per tile
constexpr int NH = 16;                  // heads per workgroup
constexpr int THREADS = 256;
constexpr int ROWB = 256;               // bytes of one key's 128-dim bf16 slice
constexpr int PLANE = KT * ROWB;        // 8192
constexpr int SLOT = 3 * PLANE;         // per wave: three planes
constexpr int HALF = 16 * ROWB;         // keys 16..31 of a plane
constexpr int KMAX = 2048;              // selected width limit (the index row lives in LDS)
constexpr int EXCH_OFF = 4 * SLOT;      // partial-score exchange, two buffers
constexpr int EXCH_WAVE = 64 * 32;
constexpr int EXCH_BUF = 4 * EXCH_WAVE;
constexpr int IDX_OFF = EXCH_OFF + 2 * EXCH_BUF;
constexpr size_t LDS_BYTES = (size_t)IDX_OFF + KMAX * 4;
constexpr int RAWN = 16;                // 16-byte loads per lane and tile (dense); records use 5 or 8 + 3 bytes
}  // namespace cs

__device__ __forceinline__ int csa_swz(int R, int ch) { return ch ^ (2 * (R & 7)) ^ ((R >> 3) & 1); }

// x = p1 + p2 + p3 exactly for eight fp32 values: three packed bf16x8 pieces,
// each the nearest bf16 to the remainder of the previous ones
__device__ __forceinline__ void split3x8(const float (&x)[8], u32x4_l& p1, u32x4_l& p2, u32x4_l& p3) {
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const float a = x[2 * i], b = x[2 * i + 1];
    const uint32_t h = pack_bf16x2(a, b);
    const float ra = a - __uint_as_float(h << 16), rb = b - __uint_as_float(h & 0xffff0000u);
    const uint32_t m = pack_bf16x2(ra, rb);
    const float sa = ra - __uint_as_float(m << 16), sb = rb - __uint_as_float(m & 0xffff0000u);
    p1[i] = h;
    p2[i] = m;
    p3[i] = pack_bf16x2(sa, sb);
  }
}

__device__ __forceinline__ f32x4_l mfma_bf16(u32x4_l a, u32x4_l b, f32x4_l c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_l, a), __builtin_bit_cast(bf16x8_l, b),
                                                 c, 0, 0, 0);
}

template <bool BIAS>
__global__ void __launch_bounds__(cs::THREADS, 1)
csa_attention_kernel(const float* __restrict__ q, const float* __restrict__ ckv,
                     const uint8_t* __restrict__ rec, const int32_t* __restrict__ sel,
                     const float* __restrict__ sink, const float* __restrict__ bias,
                     const int64_t* __restrict__ total_ptr, float* __restrict__ y, int B, int S, int H,
                     int Tcur, int64_t rcap, int idx_heads, int K, int bb, int bh, int bs, int bk,
                     float scale, ErrorBlock* __restrict__ eb) {
  using namespace cs;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int i16 = lane & 15, g = lane >> 4;
  const int HG = H / NH;
  const int G = B * S * HG;

  // workgroups of one (batch, query) share an XCD (blockIdx % 8) when the
  // grid divides evenly, so its candidates are fetched into one L2
  int L = (int)blockIdx.x;
  if (G % (8 * HG) == 0) L = (L & 7) * (G / 8) + (L >> 3);
  const int hg = L % HG;
  const int bsi = L / HG;
  const int s = bsi % S, b = bsi / S;

  // ---- cursors from total_sequence_length (read on the device)
  const int64_t total = *total_ptr;
  const int64_t start = total - S, base = total - Tcur;
  const int64_t earliest = start + 1 - WIN > 0 ? start + 1 - WIN : 0;
  const int64_t vr = total / 4;  // complete records
  const int64_t Dn = start == 0 ? (Tcur < WIN ? Tcur : WIN) : WIN;
  bool geom_bad = total < S || total < Tcur || base > earliest || vr > rcap;
  if (BIAS) geom_bad = geom_bad || (bk != 1 && (int64_t)bk != Dn + K);
  if (geom_bad) {
    if (blockIdx.x == 0 && tid == 0) atomicOr(&eb->word, SA_ERR_CSA_GEOMETRY);
    return;
  }
  const int64_t pos = start + s;
  const int64_t wstart = pos + 1 - WIN > base ? pos + 1 - WIN : base;
  const int nd = (int)min(Dn, pos - wstart + 1);  // valid dense keys (a prefix of the window)
  const int64_t r0 = wstart - base;                // current_kv row of dense key 0

  // ---- the index row (index head 0) into LDS, padded with -1
  __attribute__((address_space(3))) int32_t* idxl = (__attribute__((address_space(3))) int32_t*)(smem + IDX_OFF);
  __shared__ int s_last, s_bad;
  if (tid == 0) {
    s_last = 0;
    s_bad = 0;
  }
  __syncthreads();
  {
    const int32_t* srow = sel + ((int64_t)b * idx_heads * S + s) * K;
    int last = 0, bad = 0;
    for (int j = tid; j < KMAX; j += THREADS) {
      const int32_t v = j < K ? srow[j] : -1;
      idxl[j] = v;
      if (v >= 0) last = j + 1;
      if ((int64_t)v >= vr) bad = 1;
    }
    if (last) atomicMax(&s_last, last);
    if (bad) atomicOr(&s_bad, 1);
  }
  __syncthreads();
  const int nsel = s_last;  // slots up to the last non-negative index
  if (s_bad && tid == 0) atomicOr(&eb->word, SA_ERR_RANGE | SA_ERR_INDEX_ANY);
  const int nDT = (nd + KT - 1) / KT;
  const int T = nDT + (nsel + KT - 1) / KT;

  // ---- the query slice as three bf16 pieces (B operand of S^T = K . Q^T):
  // lane (head i16, g) holds dims 32 c + 8 g .. + 7 of the wave's slice
  const int head = hg * NH + i16;
  const int64_t qrow = (((int64_t)b * S + s) * H + head) * D;
  u32x4_l qb[3][4];
#pragma unroll
  for (int c = 0; c < 4; c++) {
    const float4 x0 = *(const float4*)(q + qrow + 128 * w + 32 * c + 8 * g);
    const float4 x1 = *(const float4*)(q + qrow + 128 * w + 32 * c + 8 * g + 4);
    const float xv[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    split3x8(xv, qb[0][c], qb[1][c], qb[2][c]);
  }

  // ---- per-lane LDS offsets (within a plane)
  uint32_t kofs[4];  // K: row i16 (+HALF for keys 16..31), chunk 4 c + g
#pragma unroll
  for (int c = 0; c < 4; c++) kofs[c] = (uint32_t)(i16 * ROWB + 16 * csa_swz(i16, 4 * c + g));
  uint32_t vofs[8];  // V^T: lane 4 jj + qq of group g reads row 4 g + jj, dims 16 dt + 4 qq
  {
    const int jj = i16 >> 2, qq = i16 & 3;
    const int R = 4 * g + jj;
#pragma unroll
    for (int dt = 0; dt < 8; dt++) vofs[dt] = (uint32_t)(R * ROWB + 16 * csa_swz(R, 2 * dt + (qq >> 1)) + 8 * (qq & 1));
  }
  const uint32_t slot = (uint32_t)(w * SLOT);
  uint8_t* const slotp = smem + slot;

  // ---- global sources
  const __amdgpu_buffer_rsrc_t krsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(ckv + (int64_t)b * Tcur * D), (short)0, (int)((int64_t)Tcur * D * 4), 0x00020000);
  const __amdgpu_buffer_rsrc_t rrsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(rec + (int64_t)b * rcap * REC), (short)0, (int)(rcap * REC), 0x00020000);
  int64_t bias_row = 0;
  if (BIAS)
    bias_row = ((((int64_t)(bb == 1 ? 0 : b) * bh + (bh == 1 ? 0 : head)) * bs + (bs == 1 ? 0 : s)) * bk);
  const int64_t cand_last = Dn + K - 1;
  const bool tailw = w == 3;  // wave 3's slice is block 6 plus the BF16 tail

  u32x4_l raw[2][RAWN];
  uint32_t rsh[2];
  float braw[2][8];
  float bcur[8];  // the bias of the tile being computed (taken out of braw when staged)

  // issue the global loads of tile t into register set SET
  auto issue = [&](int t, auto setc) {
    constexpr int SET = decltype(setc)::value;
    if (t >= T) return;
    if (t < nDT) {
      // lane: rows (lane >> 4) + 4 gI, 32-byte chunk lane & 15 of the slice
      const int cc = lane & 15;
#pragma unroll
      for (int gI = 0; gI < 8; gI++) {
        const int k = (lane >> 4) + 4 * gI;
        const int c = KT * t + k;
        const uint32_t off = c < nd ? (uint32_t)(((r0 + c) * D + 128 * w + 8 * cc) * 4) : 0x80000000u;
        raw[SET][2 * gI] = __builtin_bit_cast(u32x4_l, __builtin_amdgcn_raw_buffer_load_b128(krsrc, off, 0, 0));
        raw[SET][2 * gI + 1] = __builtin_bit_cast(u32x4_l, __builtin_amdgcn_raw_buffer_load_b128(krsrc, off + 16, 0, 0));
      }
    } else {
      const int k = lane & 31, hb = lane >> 5;
      const int j = KT * (t - nDT) + k;
      const int32_t r = idxl[j];
      const bool ok = r >= 0 && (int64_t)r < vr;
      const bool tail = tailw && hb;
      const int64_t a = (int64_t)r * REC + (tail ? TAILB : 65 * (2 * w + hb));
      rsh[SET] = (uint32_t)(a & 3);
      const uint32_t off = ok ? (uint32_t)(a & ~(int64_t)3) : 0x80000000u;
#pragma unroll
      for (int i = 0; i < 5; i++)
        raw[SET][i] = __builtin_bit_cast(u32x4_l, __builtin_amdgcn_raw_buffer_load_b128(rrsrc, off + 16 * i, 0, 0));
      if (tailw) {
        // the tail's last bytes sit in dword 32 of the window; for the last
        // record of the buffer a 16-byte (or 4-byte) load of it would straddle
        // the buffer end and be dropped by the range check, so its three
        // possibly needed bytes are loaded one by one
#pragma unroll
        for (int i = 5; i < 8; i++)
          raw[SET][i] = __builtin_bit_cast(u32x4_l, __builtin_amdgcn_raw_buffer_load_b128(rrsrc, off + 16 * i, 0, 0));
#pragma unroll
        for (int i = 0; i < 3; i++)
          raw[SET][8][i] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rrsrc, off + 128 + i, 0, 0);
      }
    }
    if (BIAS) {
      // lane (head i16, g): keys 16 hh + 4 g + r of the tile
#pragma unroll
      for (int i = 0; i < 8; i++) {
        const int k = 16 * (i >> 2) + 4 * g + (i & 3);
        int64_t c = t < nDT ? (int64_t)(KT * t + k) : Dn + (int64_t)(KT * (t - nDT) + k);
        c = c < cand_last ? c : cand_last;
        braw[SET][i] = bias[bias_row + (bk == 1 ? 0 : c)];
      }
    }
  };

  // write tile t's slice from register set SET into the wave's LDS slot
  auto stage = [&](int t, auto setc) {
    constexpr int SET = decltype(setc)::value;
    if (BIAS) {
#pragma unroll
      for (int i = 0; i < 8; i++) bcur[i] = braw[SET][i];
    }
    if (t < nDT) {
      const int cc = lane & 15;
#pragma unroll
      for (int gI = 0; gI < 8; gI++) {
        const int k = (lane >> 4) + 4 * gI;
        const u32x4_l lo = raw[SET][2 * gI], hi = raw[SET][2 * gI + 1];
        const float xv[8] = {__uint_as_float(lo[0]), __uint_as_float(lo[1]), __uint_as_float(lo[2]),
                             __uint_as_float(lo[3]), __uint_as_float(hi[0]), __uint_as_float(hi[1]),
                             __uint_as_float(hi[2]), __uint_as_float(hi[3])};
        u32x4_l p1, p2, p3;
        split3x8(xv, p1, p2, p3);
        const uint32_t o = (uint32_t)(k * ROWB + 16 * csa_swz(k, cc));
        *(lds_u32x4*)(slotp + o) = p1;
        *(lds_u32x4*)(slotp + PLANE + o) = p2;
        *(lds_u32x4*)(slotp + 2 * PLANE + o) = p3;
      }
    } else {
      const int k = lane & 31, hb = lane >> 5;
      const uint32_t sh = rsh[SET];
      uint32_t wv[32];
      if (tailw && hb) {
        uint32_t Dw[33];
#pragma unroll
        for (int i = 0; i < 8; i++) {
          Dw[4 * i] = raw[SET][i][0];
          Dw[4 * i + 1] = raw[SET][i][1];
          Dw[4 * i + 2] = raw[SET][i][2];
          Dw[4 * i + 3] = raw[SET][i][3];
        }
        Dw[32] = (raw[SET][8][0] & 0xffu) | ((raw[SET][8][1] & 0xffu) << 8) | ((raw[SET][8][2] & 0xffu) << 16);
#pragma unroll
        for (int i = 0; i < 32; i++) wv[i] = __builtin_amdgcn_alignbyte(Dw[i + 1], Dw[i], sh);
      } else {
        uint32_t Dw[20];
#pragma unroll
        for (int i = 0; i < 5; i++) {
          Dw[4 * i] = raw[SET][i][0];
          Dw[4 * i + 1] = raw[SET][i][1];
          Dw[4 * i + 2] = raw[SET][i][2];
          Dw[4 * i + 3] = raw[SET][i][3];
        }
        const uint32_t e = (Dw[0] >> (8 * sh)) & 0xffu;
        const uint32_t o1 = sh + 1;  // byte offset of the first code, 1..4
#pragma unroll
        for (int i = 0; i < 16; i++) {
          const uint32_t cw = o1 == 4 ? Dw[i + 1] : __builtin_amdgcn_alignbyte(Dw[i + 1], Dw[i], o1);
          fp8x4_to_bf16x4(cw, e, wv[2 * i], wv[2 * i + 1]);
        }
      }
#pragma unroll
      for (int qd = 0; qd < 8; qd++) {
        const uint32_t o = (uint32_t)(k * ROWB + 16 * csa_swz(k, 8 * hb + qd));
        *(lds_u32x4*)(slotp + o) = (u32x4_l){wv[4 * qd], wv[4 * qd + 1], wv[4 * qd + 2], wv[4 * qd + 3]};
      }
    }
  };

  const float fs = scale * kLog2eL;
  f32x4_l o[8];
#pragma unroll
  for (int dt = 0; dt < 8; dt++) o[dt] = (f32x4_l){0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.0f;

  auto compute = [&](int t, auto setc) {
    constexpr int SET = decltype(setc)::value;  // also the exchange buffer
    const bool dense = t < nDT;
    // ---- partial S^T over this wave's dims
    f32x4_l acc[2] = {(f32x4_l){0.f, 0.f, 0.f, 0.f}, (f32x4_l){0.f, 0.f, 0.f, 0.f}};
    if (dense) {
#pragma unroll
      for (int c = 0; c < 4; c++) {
#pragma unroll
        for (int hh = 0; hh < 2; hh++) {
          const uint32_t a = kofs[c] + hh * HALF;
          const u32x4_l k1 = *(const lds_u32x4*)(slotp + a);
          const u32x4_l k2 = *(const lds_u32x4*)(slotp + PLANE + a);
          const u32x4_l k3 = *(const lds_u32x4*)(slotp + 2 * PLANE + a);
          acc[hh] = mfma_bf16(k1, qb[0][c], acc[hh]);
          acc[hh] = mfma_bf16(k1, qb[1][c], acc[hh]);
          acc[hh] = mfma_bf16(k2, qb[0][c], acc[hh]);
          acc[hh] = mfma_bf16(k1, qb[2][c], acc[hh]);
          acc[hh] = mfma_bf16(k2, qb[1][c], acc[hh]);
          acc[hh] = mfma_bf16(k3, qb[0][c], acc[hh]);
        }
      }
    } else {
#pragma unroll
      for (int c = 0; c < 4; c++) {
#pragma unroll
        for (int hh = 0; hh < 2; hh++) {
          const u32x4_l k1 = *(const lds_u32x4*)(slotp + kofs[c] + hh * HALF);
          acc[hh] = mfma_bf16(k1, qb[0][c], acc[hh]);
          acc[hh] = mfma_bf16(k1, qb[1][c], acc[hh]);
          acc[hh] = mfma_bf16(k1, qb[2][c], acc[hh]);
        }
      }
    }
    // ---- sum the four waves' partials (fixed order: identical in every wave)
    uint8_t* ex = smem + EXCH_OFF + SET * EXCH_BUF;
    *(lds_u32x4*)(ex + w * EXCH_WAVE + lane * 32) = __builtin_bit_cast(u32x4_l, acc[0]);
    *(lds_u32x4*)(ex + w * EXCH_WAVE + lane * 32 + 16) = __builtin_bit_cast(u32x4_l, acc[1]);
    lds_barrier();
    float sv[8];
    {
      f32x4_l s0 = __builtin_bit_cast(f32x4_l, *(const lds_u32x4*)(ex + lane * 32));
      f32x4_l s1 = __builtin_bit_cast(f32x4_l, *(const lds_u32x4*)(ex + lane * 32 + 16));
#pragma unroll
      for (int ww = 1; ww < 4; ww++) {
        s0 += __builtin_bit_cast(f32x4_l, *(const lds_u32x4*)(ex + ww * EXCH_WAVE + lane * 32));
        s1 += __builtin_bit_cast(f32x4_l, *(const lds_u32x4*)(ex + ww * EXCH_WAVE + lane * 32 + 16));
      }
#pragma unroll
      for (int r = 0; r < 4; r++) {
        sv[r] = s0[r];
        sv[4 + r] = s1[r];
      }
    }
    // ---- validity, bias, online softmax (log2 units)
    bool valid[8];
    if (dense) {
#pragma unroll
      for (int i = 0; i < 8; i++) valid[i] = KT * t + 16 * (i >> 2) + 4 * g + (i & 3) < nd;
    } else {
      const int j0 = KT * (t - nDT) + 4 * g;
#pragma unroll
      for (int hh = 0; hh < 2; hh++) {
        const u32x4_l iv = *(const __attribute__((address_space(3))) u32x4_l*)(idxl + j0 + 16 * hh);
#pragma unroll
        for (int r = 0; r < 4; r++) {
          const int32_t rr = (int32_t)iv[r];
          valid[4 * hh + r] = rr >= 0 && (int64_t)rr < vr;
        }
      }
    }
    float tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 8; i++) {
      float x = sv[i] * fs;
      if (BIAS) x += bcur[i] * kLog2eL;
      sv[i] = valid[i] ? x : -INFINITY;
      tmax = fmaxf(tmax, sv[i]);
    }
    tmax = max_x32(max_x16(tmax));
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = m_new == -INFINITY ? 1.0f : exp2f(m_run - m_new);
    float pv[8], psum = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; i++) {
      pv[i] = sv[i] == -INFINITY ? 0.0f : exp2f(sv[i] - m_new);
      psum += pv[i];
    }
    psum = sum_x32(sum_x16(psum));
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < 8; dt++) o[dt] *= alpha;
    u32x4_l pb[3];
    split3x8(pv, pb[0], pb[1], pb[2]);
    // ---- O^T += V^T . P^T over this wave's 128 output dims
    typedef __attribute__((address_space(3))) s16x4_l lds_s16x4;
#pragma unroll
    for (int dt = 0; dt < 8; dt++) {
      if (dense) {
        u32x4_l v[3];
#pragma unroll
        for (int pl = 0; pl < 3; pl++) {
          const s16x4_l a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(slotp + pl * PLANE + vofs[dt]));
          const s16x4_l a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(slotp + pl * PLANE + vofs[dt] + HALF));
          const s16x4_l a8[2] = {a0, a1};
          v[pl] = __builtin_bit_cast(u32x4_l, a8);
        }
        o[dt] = mfma_bf16(v[0], pb[0], o[dt]);
        o[dt] = mfma_bf16(v[0], pb[1], o[dt]);
        o[dt] = mfma_bf16(v[1], pb[0], o[dt]);
        o[dt] = mfma_bf16(v[0], pb[2], o[dt]);
        o[dt] = mfma_bf16(v[1], pb[1], o[dt]);
        o[dt] = mfma_bf16(v[2], pb[0], o[dt]);
      } else {
        const s16x4_l a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(slotp + vofs[dt]));
        const s16x4_l a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(slotp + vofs[dt] + HALF));
        const s16x4_l a8[2] = {a0, a1};
        const u32x4_l v = __builtin_bit_cast(u32x4_l, a8);
        o[dt] = mfma_bf16(v, pb[0], o[dt]);
        o[dt] = mfma_bf16(v, pb[1], o[dt]);
        o[dt] = mfma_bf16(v, pb[2], o[dt]);
      }
    }
  };

  issue(0, std::integral_constant<int, 0>{});
  issue(1, std::integral_constant<int, 1>{});
  for (int t = 0; t < T; t += 2) {
    stage(t, std::integral_constant<int, 0>{});
    issue(t + 2, std::integral_constant<int, 0>{});
    compute(t, std::integral_constant<int, 0>{});
    if (t + 1 < T) {
      stage(t + 1, std::integral_constant<int, 1>{});
      issue(t + 3, std::integral_constant<int, 1>{});
      compute(t + 1, std::integral_constant<int, 1>{});
    }
  }

  // ---- Y = O / (l + exp(sink - m)); a head with no candidate gives zeros
  const float den = l_run + exp2f(sink[head] * kLog2eL - m_run);
  const bool none = m_run == -INFINITY;
  const bool bad = !none && !(den > 0.0f && den < INFINITY);
  if (__builtin_amdgcn_ballot_w64(bad) != 0 && lane == 0) atomicOr(&eb->word, SA_ERR_CSA_DENOM);
  const float inv = none ? 0.0f : 1.0f / den;
  float* yrow = y + qrow + 128 * w + 4 * g;
#pragma unroll
  for (int dt = 0; dt < 8; dt++) {
    const f32x4_l r = o[dt] * inv;
    *(float4*)(yrow + 16 * dt) = make_float4(r[0], r[1], r[2], r[3]);
  }
}

sa_status launch_csa_attention(sparse_attn_ctx* c, const CsaArgs& a) {
  using namespace cs;
  const int64_t G = a.batch * a.q_seq * (a.heads / NH);
  const dim3 grid((unsigned)G), block(THREADS);
  static bool attr_set[2] = {false, false};
  const int variant = a.bias ? 1 : 0;
  void* fns[2] = {(void*)csa_attention_kernel<false>, (void*)csa_attention_kernel<true>};
  if (!attr_set[variant]) {
    hipError_t e = hipFuncSetAttribute(fns[variant], hipFuncAttributeMaxDynamicSharedMemorySize, (int)LDS_BYTES);
    if (e != hipSuccess) return check_hip(c, e, "csa attention LDS attribute");
    attr_set[variant] = true;
  }
  prof_begin(c);
#define SA_CSA_LAUNCH(BV)                                                                                     \
  hipLaunchKernelGGL((csa_attention_kernel<BV>), grid, block, LDS_BYTES, c->stream, a.q, a.ckv, a.rec, a.sel, \
                     a.sink, a.bias, a.total, a.y, (int)a.batch, (int)a.q_seq, (int)a.heads, (int)a.cur_len,  \
                     a.record_cap, (int)a.index_heads, (int)a.topk, (int)a.bias_dims[0], (int)a.bias_dims[1], \
                     (int)a.bias_dims[2], (int)a.bias_dims[3], a.scale, c->err)
  if (a.bias)
    SA_CSA_LAUNCH(true);
  else
    SA_CSA_LAUNCH(false);
#undef SA_CSA_LAUNCH
  prof_end(c);
  return check_hip(c, hipGetLastError(), "csa attention");
}

}  // namespace sa
