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
// Work split: one workgroup of eight waves per (batch, query, 16-head group),
// in two streams of four. The candidates are cut into units (16 window rows,
// or 32 selected records); stream z takes units z, z + 2, z + 4, .. and keeps
// its own online softmax, and the two merge at the end. In a stream, wave w
// owns dims 128w .. 128w+127 of every key and of the output: per unit it
// stages its own 128-dim slice into LDS (bf16; a current_kv slice as three
// bf16 planes), computes the partial S^T over its dims, and the four partials
// are summed through LDS (one barrier per pair of units) in a fixed order, so
// the four waves of a stream hold the same scores, maxima and sums. With
// two waves per SIMD, one wave's matrix work and loads overlap the other's
// softmax and waits. Global loads run one unit ahead.
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
constexpr int KT = 32;                  // records per record unit
constexpr int DKT = 16;                 // window rows per dense unit
constexpr int NH = 16;                  // heads per workgroup
constexpr int THREADS = 512;            // two streams of four waves
constexpr int ROWB = 256;               // bytes of one key's 128-dim bf16 slice
constexpr int HALF = 16 * ROWB;         // 16 rows: a dense plane, or records 16..31 of a unit
constexpr int SLOT = 3 * HALF;          // per wave: three dense planes or one record unit
constexpr int KMAX = 2048;              // selected width limit (the index row lives in LDS)
constexpr int EXCH_OFF = 8 * SLOT;      // partial-score exchange, two buffers per stream
constexpr int EXCH_WAVE = 64 * 32;
constexpr int EXCH_BUF = 4 * EXCH_WAVE;
constexpr int IDX_OFF = EXCH_OFF + 4 * EXCH_BUF;
constexpr int MISC_OFF = IDX_OFF + (KMAX + KT) * 4;  // the row plus one unit of padding
constexpr size_t LDS_BYTES = (size_t)MISC_OFF + 16;
static_assert(LDS_BYTES <= 160 * 1024, "one workgroup per CU");
static_assert(SLOT >= 8 * 64 * 16 + 3 * 64 * 4, "a slot holds a stream's end state");
}  // namespace cs

__device__ __forceinline__ int csa_swz(int R, int ch) { return ch ^ (2 * (R & 7)) ^ ((R >> 3) & 1); }

// x = p1 + p2 + p3 exactly for 2N fp32 values: three packed bf16 pieces, each
// the nearest bf16 to the remainder of the previous ones
template <int N, typename V>
__device__ __forceinline__ void split3(const float (&x)[2 * N], V& p1, V& p2, V& p3) {
#pragma unroll
  for (int i = 0; i < N; i++) {
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

typedef unsigned u32x2_l __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4_l mfma_bf16(u32x4_l a, u32x4_l b, f32x4_l c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_l, a), __builtin_bit_cast(bf16x8_l, b),
                                                 c, 0, 0, 0);
}
// the 16-key contraction of a dense unit's O^T update
__device__ __forceinline__ f32x4_l mfma_bf16_k16(s16x4_l a, u32x2_l b, f32x4_l c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, __builtin_bit_cast(s16x4_l, b), c, 0, 0, 0);
}

// The body of one wave. TAILW: a wave whose slice holds the BF16 tail (slice
// 3); the two instantiations issue fixed, different load counts per unit, so
// the compiler's wait counts stay exact across the loop.
template <bool BIAS, bool TAILW>
__device__ __forceinline__ void
csa_wave(const float* __restrict__ q, const float* __restrict__ ckv, const uint8_t* __restrict__ rec,
         const int32_t* __restrict__ sel, const float* __restrict__ sink, const float* __restrict__ bias,
         const int64_t* __restrict__ total_ptr, float* __restrict__ y, int B, int S, int H, int Tcur,
         int64_t rcap, int idx_heads, int K, int bb, int bh, int bs, int bk, float scale,
         ErrorBlock* __restrict__ eb) {
  using namespace cs;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // the wave index as a scalar: the unit loop's branches and the load
  // descriptors derive from the stream, and stay uniform only if the
  // compiler knows it is
  const int wv8 = __builtin_amdgcn_readfirstlane(tid >> 6);
  // dim slice, stream: stream 1's slices are rotated by one, so the two
  // waves of slice 3 (which also decode the BF16 tail) sit on different SIMDs
  const int z = wv8 >> 2, w = (wv8 + z) & 3;
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
  int* const misc = (int*)(smem + MISC_OFF);  // [0] slots up to the last index >= 0, [1] range flag
  if (tid == 0) {
    misc[0] = 0;
    misc[1] = 0;
  }
  if (tid < KT) idxl[KMAX + tid] = -1;  // read by a unit past the end
  __syncthreads();
  {
    const int32_t* srow = sel + ((int64_t)b * idx_heads * S + s) * K;
    int last = 0, bad = 0;
    // stored sanitized: an index that is no candidate (negative, or not a
    // complete record) becomes -1, so a candidate is simply an entry >= 0
    for (int j = tid; j < KMAX; j += THREADS) {
      const int32_t v = j < K ? srow[j] : -1;
      const bool cand = v >= 0 && (int64_t)v < vr;
      idxl[j] = cand ? v : -1;
      if (cand) last = j + 1;
      if ((int64_t)v >= vr) bad = 1;
    }
    // one LDS atomic per wave
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) last = max(last, __shfl_xor(last, off));
    if (lane == 0 && last) atomicMax(&misc[0], last);
    if (__builtin_amdgcn_ballot_w64(bad) != 0 && lane == 0) atomicOr(&misc[1], 1);
  }
  __syncthreads();
  // workgroup-uniform by construction; readfirstlane tells the compiler so,
  // and the unit loop's branches stay scalar (no exec-masked paths)
  const int nsel = __builtin_amdgcn_readfirstlane(misc[0]);  // slots up to the last index >= 0
  if (misc[1] && tid == 0) atomicOr(&eb->word, SA_ERR_RANGE | SA_ERR_INDEX_ANY);
  const int nDU = __builtin_amdgcn_readfirstlane((nd + DKT - 1) / DKT);  // dense units
  const int NU = nDU + (nsel + KT - 1) / KT;                             // all units

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
    split3<4>(xv, qb[0][c], qb[1][c], qb[2][c]);
  }

  // ---- per-lane LDS offsets (within a plane)
  uint32_t kofs[4];  // K: row i16 (+HALF for records 16..31), chunk 4 c + g
#pragma unroll
  for (int c = 0; c < 4; c++) kofs[c] = (uint32_t)(i16 * ROWB + 16 * csa_swz(i16, 4 * c + g));
  uint32_t vofs[8];  // V^T: lane 4 jj + qq of group g reads row 4 g + jj, dims 16 dt + 4 qq
  {
    const int jj = i16 >> 2, qq = i16 & 3;
    const int R = 4 * g + jj;
#pragma unroll
    for (int dt = 0; dt < 8; dt++) vofs[dt] = (uint32_t)(R * ROWB + 16 * csa_swz(R, 2 * dt + (qq >> 1)) + 8 * (qq & 1));
  }
  uint8_t* const slotp = smem + wv8 * SLOT;

  // ---- global sources
  const __amdgpu_buffer_rsrc_t krsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(ckv + (int64_t)b * Tcur * D), (short)0, (int)((int64_t)Tcur * D * 4), 0x00020000);
  const __amdgpu_buffer_rsrc_t rrsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(rec + (int64_t)b * rcap * REC), (short)0, (int)(rcap * REC), 0x00020000);
  int64_t bias_row = 0;
  if (BIAS)
    bias_row = ((((int64_t)(bb == 1 ? 0 : b) * bh + (bh == 1 ? 0 : head)) * bs + (bs == 1 ? 0 : s)) * bk);
  const int64_t cand_last = Dn + K - 1;
  constexpr bool tailw = TAILW;  // slice 3 is block 6 plus the BF16 tail

  // Every unit issues the same instructions (8 x 16 bytes per lane, plus 3
  // single bytes in the tail wave and 8 bias words with a bias), addressed by
  // the unit's kind and out of range where unused, so the compiler's wait
  // counts are exact.
  u32x4_l raw[8];
  uint32_t rby[3];
  uint32_t rsh = 0, rsc = 0;
  float braw[8];
  float bcur[8];  // the bias of the unit being computed (taken out of braw when staged)
  constexpr uint32_t OOB = 0x80000000u;

  auto issue = [&](int u) {
    const bool dn = u < nDU;  // uniform
    // dense unit: lane loads window row 16 u + (lane >> 4) + 4 gI, 32-byte chunk lane & 15
    const int cc = lane & 15;
    uint32_t doff[4];
#pragma unroll
    for (int gI = 0; gI < 4; gI++) {
      const int c = DKT * u + (lane >> 4) + 4 * gI;
      doff[gI] = (dn && c < nd) ? (uint32_t)(((r0 + c) * D + 128 * w + 8 * cc) * 4) : OOB;
    }
    // record unit: lane loads 64 dims (block 2 w + hb, or the tail) of slot k
    const int k = lane & 31, hb = lane >> 5;
    int j = KT * (u - nDU) + k;
    j = j < 0 ? 0 : (j > KMAX - 1 ? KMAX - 1 : j);
    const int32_t r = idxl[j];
    const bool ok = !dn && u < NU && r >= 0;
    const bool tail = tailw && hb;
    // a coded block's window starts at the dword of its first code (the scale
    // byte, one before, is loaded by itself); the tail's at its first byte
    const int64_t a = (int64_t)r * REC + (tail ? TAILB : 65 * (2 * w + hb) + 1);
    const uint32_t a4 = ok ? (uint32_t)(a & ~(int64_t)3) : OOB;
    rsh = (uint32_t)(a & 3);
    rsc = (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rrsrc, ok ? (uint32_t)(a - 1) : OOB, 0, 0);
    const __amdgpu_buffer_rsrc_t rs = dn ? krsrc : rrsrc;
#pragma unroll
    for (int i = 0; i < 8; i++) {
      // records: 80 bytes cover a coded block; the tail wave's lanes take 128
      const uint32_t ro = (i < 5 || tailw) ? (a4 == OOB ? OOB : a4 + 16 * i) : OOB;
      const uint32_t off = dn ? (doff[i >> 1] == OOB ? OOB : doff[i >> 1] + 16 * (i & 1)) : ro;
      raw[i] = __builtin_bit_cast(u32x4_l, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
    }
    if (tailw) {
      // the tail's last bytes sit in dword 32 of the window; for the last
      // record of the buffer a 4- or 16-byte load of it would straddle the
      // buffer end and be dropped by the range check, so its three possibly
      // needed bytes are loaded one by one
#pragma unroll
      for (int i = 0; i < 3; i++)
        rby[i] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rrsrc, a4 == OOB ? OOB : a4 + 128 + i, 0, 0);
    }
    if (BIAS) {
      // lane (head i16, g): keys 16 hh + 4 g + r of a record unit, keys
      // 4 g + r of a dense unit (its words 4..7 repeat 0..3)
#pragma unroll
      for (int i = 0; i < 8; i++) {
        const int kk = 16 * (i >> 2) + 4 * g + (i & 3);
        int64_t c = dn ? (int64_t)(DKT * u + 4 * g + (i & 3)) : Dn + (int64_t)(KT * (u - nDU) + kk);
        c = c < cand_last ? c : cand_last;
        braw[i] = bias[bias_row + (bk == 1 ? 0 : c)];
      }
    }
  };

  // per-lane LDS write offsets of a unit (fixed over the loop)
  uint32_t dwo[4], rwo[8];
#pragma unroll
  for (int gI = 0; gI < 4; gI++) {
    const int kr = (lane >> 4) + 4 * gI;
    dwo[gI] = (uint32_t)(kr * ROWB + 16 * csa_swz(kr, lane & 15));
  }
#pragma unroll
  for (int qd = 0; qd < 8; qd++)
    rwo[qd] = (uint32_t)((lane & 31) * ROWB + 16 * csa_swz(lane & 31, 8 * (lane >> 5) + qd));

  // write unit u from the load registers into the wave's LDS slot
  auto stage = [&](int u) {
    if (BIAS) {
#pragma unroll
      for (int i = 0; i < 8; i++) bcur[i] = braw[i];
    }
    if (u < nDU) {
#pragma unroll
      for (int gI = 0; gI < 4; gI++) {
        const u32x4_l lo = raw[2 * gI], hi = raw[2 * gI + 1];
        const float xv[8] = {__uint_as_float(lo[0]), __uint_as_float(lo[1]), __uint_as_float(lo[2]),
                             __uint_as_float(lo[3]), __uint_as_float(hi[0]), __uint_as_float(hi[1]),
                             __uint_as_float(hi[2]), __uint_as_float(hi[3])};
        u32x4_l p1, p2, p3;
        split3<4>(xv, p1, p2, p3);
        *(lds_u32x4*)(slotp + dwo[gI]) = p1;
        *(lds_u32x4*)(slotp + HALF + dwo[gI]) = p2;
        *(lds_u32x4*)(slotp + 2 * HALF + dwo[gI]) = p3;
      }
    } else {
      const int hb = lane >> 5;
      const uint32_t sh = rsh;
      uint32_t wv[32];
      if (tailw && hb) {
        uint32_t Dw[33];
#pragma unroll
        for (int i = 0; i < 8; i++) {
          Dw[4 * i] = raw[i][0];
          Dw[4 * i + 1] = raw[i][1];
          Dw[4 * i + 2] = raw[i][2];
          Dw[4 * i + 3] = raw[i][3];
        }
        Dw[32] = (rby[0] & 0xffu) | ((rby[1] & 0xffu) << 8) | ((rby[2] & 0xffu) << 16);
#pragma unroll
        for (int i = 0; i < 32; i++) wv[i] = __builtin_amdgcn_alignbyte(Dw[i + 1], Dw[i], sh);
      } else {
        uint32_t Dw[20];  // codes from byte sh of Dw[0]: 64 + 3 bytes fit 17 dwords
#pragma unroll
        for (int i = 0; i < 5; i++) {
          Dw[4 * i] = raw[i][0];
          Dw[4 * i + 1] = raw[i][1];
          Dw[4 * i + 2] = raw[i][2];
          Dw[4 * i + 3] = raw[i][3];
        }
        const uint32_t e = rsc & 0xffu;
        uint32_t cw[16];
#pragma unroll
        for (int i = 0; i < 16; i++) cw[i] = __builtin_amdgcn_alignbyte(Dw[i + 1], Dw[i], sh);
        // scale bytes 10..246: v_cvt_scalef32_pk_bf16_fp8 is exact (every
        // code times 2^(e-127) is a bf16 normal); a lane with another byte
        // redoes its row on the integer path after the stores, in a block
        // of its own so the common path carries none of it
        const bool ext = e < 10u || e > 246u;
        const float sc = __uint_as_float((ext ? 127u : e) << 23);
#pragma unroll
        for (int i = 0; i < 16; i++) {
          wv[2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(cw[i], sc, false));
          wv[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(cw[i], sc, true));
        }
#pragma unroll
        for (int qd = 0; qd < 8; qd++)
          *(lds_u32x4*)(slotp + rwo[qd]) = (u32x4_l){wv[4 * qd], wv[4 * qd + 1], wv[4 * qd + 2], wv[4 * qd + 3]};
        if (__builtin_amdgcn_ballot_w64(ext) != 0) {
          if (ext) {
#pragma unroll
            for (int i = 0; i < 16; i++) fp8x4_to_bf16x4(cw[i], e, wv[2 * i], wv[2 * i + 1]);
#pragma unroll
            for (int qd = 0; qd < 8; qd++)
              *(lds_u32x4*)(slotp + rwo[qd]) = (u32x4_l){wv[4 * qd], wv[4 * qd + 1], wv[4 * qd + 2], wv[4 * qd + 3]};
          }
        }
        return;
      }
#pragma unroll
      for (int qd = 0; qd < 8; qd++)
        *(lds_u32x4*)(slotp + rwo[qd]) = (u32x4_l){wv[4 * qd], wv[4 * qd + 1], wv[4 * qd + 2], wv[4 * qd + 3]};
    }
  };

  const float fs = scale * kLog2eL;
  f32x4_l o[8];
#pragma unroll
  for (int dt = 0; dt < 8; dt++) o[dt] = (f32x4_l){0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, m_ref = -INFINITY, l_run = 0.0f;
  constexpr float kTau = 8.0f;  // p <= 2^8 against the reference

  // exchange buffers of this stream; lane's partial at lane * 16 (+1024 for
  // records 16..31 of a record unit)
  uint8_t* const exs = smem + EXCH_OFF + z * 2 * EXCH_BUF;

  // ---- partial S^T of unit u over this wave's dims, written to the exchange
  auto scores_out = [&](int u, int xb) {
    uint8_t* ex = exs + xb * EXCH_BUF + w * EXCH_WAVE + lane * 16;
    if (u < nDU) {
      // piece products of weight >= 2^-16: (1,1) (1,2) (2,1) (1,3) (2,2) (3,1),
      // one accumulator per query piece so consecutive MFMAs are independent
      f32x4_l acc[3];
#pragma unroll
      for (int pc = 0; pc < 3; pc++) acc[pc] = (f32x4_l){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 4; c++) {
        u32x4_l k[3];
#pragma unroll
        for (int pl = 0; pl < 3; pl++) k[pl] = *(const lds_u32x4*)(slotp + pl * HALF + kofs[c]);
        acc[0] = mfma_bf16(k[0], qb[0][c], acc[0]);
        acc[1] = mfma_bf16(k[0], qb[1][c], acc[1]);
        acc[2] = mfma_bf16(k[1], qb[0][c], acc[2]);
        acc[1] = mfma_bf16(k[0], qb[2][c], acc[1]);
        acc[2] = mfma_bf16(k[1], qb[1][c], acc[2]);
        acc[0] = mfma_bf16(k[2], qb[0][c], acc[0]);
      }
      *(lds_u32x4*)ex = __builtin_bit_cast(u32x4_l, (acc[0] + acc[1]) + acc[2]);
    } else {
      f32x4_l acc[2][3];
#pragma unroll
      for (int hh = 0; hh < 2; hh++)
#pragma unroll
        for (int pc = 0; pc < 3; pc++) acc[hh][pc] = (f32x4_l){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 4; c++) {
        u32x4_l k[2];
#pragma unroll
        for (int hh = 0; hh < 2; hh++) k[hh] = *(const lds_u32x4*)(slotp + kofs[c] + hh * HALF);
#pragma unroll
        for (int pc = 0; pc < 3; pc++)
#pragma unroll
          for (int hh = 0; hh < 2; hh++) acc[hh][pc] = mfma_bf16(k[hh], qb[pc][c], acc[hh][pc]);
      }
#pragma unroll
      for (int hh = 0; hh < 2; hh++)
        *(lds_u32x4*)(ex + 1024 * hh) = __builtin_bit_cast(u32x4_l, (acc[hh][0] + acc[hh][1]) + acc[hh][2]);
    }
  };

  // ---- sum of the stream's four partials (fixed order: identical in its
  // waves), online softmax (log2 units), O^T += V^T . P^T over this wave's
  // 128 output dims. One code path for both kinds of unit, so O stays in
  // place across the loop. Lane (head i16, g) holds 8 scores: keys 4g+r and
  // 16+4g+r of a record unit; of a dense unit only the first four are keys.
  //
  // A k=32 product takes two 4-key operand halves: for a record unit the
  // two key halves of one bf16 plane; for a dense unit two of its planes
  // over the same 4 keys, with the probability pieces doubled to match, so
  // its six piece products (1,1)+(2,1), (1,2)+(2,2), (1,3)+(3,1) also take
  // three products per output tile.
  auto update = [&](int u, int xb) {
    const bool dense = u < nDU;  // uniform
    const uint8_t* ex = exs + xb * EXCH_BUF + lane * 16;
    float sv[8];
#pragma unroll
    for (int hh = 0; hh < 2; hh++) {
      f32x4_l sum = __builtin_bit_cast(f32x4_l, *(const lds_u32x4*)(ex + 1024 * hh));
#pragma unroll
      for (int ww = 1; ww < 4; ww++)
        sum += __builtin_bit_cast(f32x4_l, *(const lds_u32x4*)(ex + ww * EXCH_WAVE + 1024 * hh));
#pragma unroll
      for (int r = 0; r < 4; r++) sv[4 * hh + r] = sum[r];
    }
    bool valid[8];
    if (dense) {
#pragma unroll
      for (int i = 0; i < 8; i++) valid[i] = i < 4 && DKT * u + 4 * g + i < nd;
    } else {
      const int j0 = KT * (u - nDU) + 4 * g;
#pragma unroll
      for (int hh = 0; hh < 2; hh++) {
        const u32x4_l iv = *(const __attribute__((address_space(3))) u32x4_l*)(idxl + j0 + 16 * hh);
#pragma unroll
        for (int r = 0; r < 4; r++) valid[4 * hh + r] = (int32_t)iv[r] >= 0;
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
    // exponents are taken against a reference m_ref that moves only when a
    // score exceeds it by more than 2^TAU (then O and l are rescaled), so O is
    // rarely touched; the true maximum m_run is kept for the final scaling
    m_run = fmaxf(m_run, tmax);
    if (__builtin_amdgcn_ballot_w64(tmax > m_ref + kTau) != 0) {
      const float m_new = tmax > m_ref + kTau ? m_run : m_ref;
      const float alpha = m_new == m_ref ? 1.0f : exp2f(m_ref - m_new);
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < 8; dt++) o[dt] *= alpha;
      m_ref = m_new;
    }
    float pv[8], psum = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; i++) {
      // the hardware exp2: a result below 2^-126 may flush to zero, far
      // below an fp32 ulp of the sum (which holds a term >= 1)
      pv[i] = sv[i] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(sv[i] - m_ref);
      psum += pv[i];
    }
    psum = sum_x32(sum_x16(psum));
    l_run += psum;
#pragma unroll
    for (int i = 0; i < 4; i++) pv[4 + i] = dense ? pv[i] : pv[4 + i];
    u32x4_l pb[3];
    split3<4>(pv, pb[0], pb[1], pb[2]);
    u32x4_l pb2 = pb[2];  // dense: (piece 3, piece 1) of the four keys
    pb2[2] = dense ? pb[0][0] : pb2[2];
    pb2[3] = dense ? pb[0][1] : pb2[3];
    typedef __attribute__((address_space(3))) s16x4_l lds_s16x4;
    auto vload = [&](uint32_t off) { return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(slotp + off)); };
    const uint32_t hi2 = dense ? 2 * HALF : HALF;  // second half of the third product's operand
    u32x4_l va[8], vb[8];
#pragma unroll
    for (int dt = 0; dt < 8; dt++) {
      const s16x4_l lo = vload(vofs[dt]), hi = vload(vofs[dt] + HALF), h2 = vload(vofs[dt] + hi2);
      const s16x4_l a8[2] = {lo, hi}, b8[2] = {lo, h2};
      va[dt] = __builtin_bit_cast(u32x4_l, a8);
      vb[dt] = __builtin_bit_cast(u32x4_l, b8);
    }
#pragma unroll
    for (int dt = 0; dt < 8; dt++) o[dt] = mfma_bf16(va[dt], pb[0], o[dt]);
#pragma unroll
    for (int dt = 0; dt < 8; dt++) o[dt] = mfma_bf16(va[dt], pb[1], o[dt]);
#pragma unroll
    for (int dt = 0; dt < 8; dt++) o[dt] = mfma_bf16(vb[dt], pb2, o[dt]);
  };

  // ---- the unit loop: stream z takes units z, z + 2, ..; both streams run
  // the same number of iterations, one barrier each, so every wave meets
  // every barrier. A stream with no unit left in the last iteration runs a
  // unit past the end: its loads are out of range (zeros), its index slots
  // are padding, so it adds nothing.
  const int NI = (NU + 1) >> 1;
  issue(z);
  for (int it = 0; it < NI; it++) {
    const int u = 2 * it + z;
    const int xb = it & 1;
    stage(u);
    issue(u + 2);
    scores_out(u, xb);
    lds_barrier();
    update(u, xb);
  }

  // ---- merge the streams: stream 1 leaves (O, m_run, m_ref, l) in its slot,
  // stream 0 combines and writes Y = O / (l + exp(sink - m)) against the true
  // maximum m; a head with no candidate gives zeros
  float* const endst = (float*)slotp;
  if (z == 1) {
#pragma unroll
    for (int dt = 0; dt < 8; dt++) *(lds_u32x4*)(slotp + 16 * (8 * lane + dt)) = __builtin_bit_cast(u32x4_l, o[dt]);
    endst[8 * 64 * 4 + lane] = m_run;
    endst[8 * 64 * 4 + 64 + lane] = m_ref;
    endst[8 * 64 * 4 + 128 + lane] = l_run;
  }
  __syncthreads();
  if (z == 1) return;
  const uint8_t* const pslot = smem + (4 + ((w + 3) & 3)) * SLOT;  // stream 1's wave of slice w
  const float* const pend = (const float*)pslot;
  const float m1 = pend[8 * 64 * 4 + lane], mr1 = pend[8 * 64 * 4 + 64 + lane], l1 = pend[8 * 64 * 4 + 128 + lane];
  const float mx = fmaxf(m_run, m1);
  const bool none = mx == -INFINITY;
  // each stream's terms are scaled from its reference to mx (a stream with no
  // candidate has reference -inf and weight 0)
  const float f0 = none ? 0.0f : exp2f(m_ref - mx);
  const float f1 = none ? 0.0f : exp2f(mr1 - mx);
  const float den = l_run * f0 + l1 * f1 + exp2f(sink[head] * kLog2eL - mx);
  const bool bad = !none && !(den > 0.0f && den < INFINITY);
  if (__builtin_amdgcn_ballot_w64(bad) != 0 && lane == 0) atomicOr(&eb->word, SA_ERR_CSA_DENOM);
  const float inv = none ? 0.0f : 1.0f / den;
  float* yrow = y + qrow + 128 * w + 4 * g;
#pragma unroll
  for (int dt = 0; dt < 8; dt++) {
    const f32x4_l o1 = __builtin_bit_cast(f32x4_l, *(const lds_u32x4*)(pslot + 16 * (8 * lane + dt)));
    f32x4_l r = (o[dt] * f0 + o1 * f1) * inv;
    if (none) r = (f32x4_l){0.f, 0.f, 0.f, 0.f};
    *(float4*)(yrow + 16 * dt) = make_float4(r[0], r[1], r[2], r[3]);
  }
}

template <bool BIAS>
__global__ void __launch_bounds__(cs::THREADS, 1)
csa_attention_kernel(const float* __restrict__ q, const float* __restrict__ ckv,
                     const uint8_t* __restrict__ rec, const int32_t* __restrict__ sel,
                     const float* __restrict__ sink, const float* __restrict__ bias,
                     const int64_t* __restrict__ total_ptr, float* __restrict__ y, int B, int S, int H,
                     int Tcur, int64_t rcap, int idx_heads, int K, int bb, int bh, int bs, int bk,
                     float scale, ErrorBlock* __restrict__ eb) {
  const int wv8 = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  if (((wv8 + (wv8 >> 2)) & 3) == 3)
    csa_wave<BIAS, true>(q, ckv, rec, sel, sink, bias, total_ptr, y, B, S, H, Tcur, rcap, idx_heads, K, bb, bh,
                         bs, bk, scale, eb);
  else
    csa_wave<BIAS, false>(q, ckv, rec, sel, sink, bias, total_ptr, y, B, S, H, Tcur, rcap, idx_heads, K, bb, bh,
                          bs, bk, scale, eb);
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
  const ProfEvents pe = prof_next(c);
#define SA_CSA_LAUNCH(BV)                                                                                     \
  SA_MAIN_LAUNCH(pe, (csa_attention_kernel<BV>), grid, block, LDS_BYTES, c->stream, a.q, a.ckv, a.rec, a.sel, \
                     a.sink, a.bias, a.total, a.y, (int)a.batch, (int)a.q_seq, (int)a.heads, (int)a.cur_len,  \
                     a.record_cap, (int)a.index_heads, (int)a.topk, (int)a.bias_dims[0], (int)a.bias_dims[1], \
                     (int)a.bias_dims[2], (int)a.bias_dims[3], a.scale, c->err)
  if (a.bias)
    SA_CSA_LAUNCH(true);
  else
    SA_CSA_LAUNCH(false);
#undef SA_CSA_LAUNCH
  return check_hip(c, hipGetLastError(), "csa attention");
}

}  // namespace sa
