// Shared-latent selected-token attention over fp8_e4m3_block64 records on the
// gfx950 matrix cores, with wave pairs that share the gathered tile.
//
// As in the bf16 shared-latent kernel, all 64 query heads of a (batch, query)
// row read one kv head through one index row, so per 32-key tile the scores
// S^T = K_sel . Q^T and the update O^T += V_sel^T . P^T are dense products on
// v_mfma_f32_16x16x32_bf16 with fp32 accumulation, followed by an online
// softmax per head. The records are decoded to bf16 on the way into LDS (the
// CSA pages' record: per 64-dim block an E8M0 scale byte and 64 E4M3FN codes,
// then the RoPE dims as little-endian BF16), and the query is never
// quantized.
//
// Work split inside the workgroup (4 waves): waves 2p and 2p+1 form pair p and
// own heads 32p .. 32p+31. Wave 2p+h scores keys 16h .. 16h+15 of every tile
// for the pair's 32 heads (all 576 dims) and accumulates dv 256h .. 256h+255
// of the output for all 32 keys. Every K row of a tile is read from LDS by one
// wave per pair and every V element by one wave per pair, half of what a
// one-wave-per-16-heads split reads; the price is one 16-byte exchange of
// probabilities per lane and tile between the two waves of a pair. The pair
// shares one softmax reference per head (the larger of the two waves' maxima
// on the first tile), kept fixed afterwards so O is never rescaled; a score
// more than 2^100 above it restarts the workgroup's key range with the larger
// reference.
//
// Record decode: each lane fetches one 64-dim block of one key (its codes from
// the 4-byte-aligned word holding the first code, the scale byte, and 16 RoPE
// bytes) into registers two tiles ahead, then converts with
// v_cvt_scalef32_pk_bf16_fp8 (E4M3FN code times the power-of-two scale, exact
// in bf16 for scale bytes 10..246; other scale bytes take an exact integer
// path) and writes the bf16 row into a ring of three LDS tiles.
//
// With fused validation each workgroup checks its own columns of the index
// row (IndexShare host-validator rules) while it stages the keys, and the
// finisher of each row records the row's first violation.
#include "sa_mfma_dev.h"
#include "sa_quant_dev.h"
#include "sa_validate_dev.h"

namespace sa {

namespace pk {
constexpr int DK = 576;
constexpr int DV = 512;
constexpr int NH = 64;
constexpr int KT = 32;                          // keys per tile
constexpr int ROWB = DK * 2;                    // bf16 bytes per decoded row in LDS
constexpr int TILE_BYTES = KT * ROWB;           // 36864
constexpr int HALF_ROWS = 16 * ROWB;            // byte offset of keys 16..31 of a tile
constexpr int THREADS = 256;
constexpr int WAVES = THREADS / 64;
constexpr int KSTEPS = DK / 32;                 // 18 k-steps of S^T
constexpr int DVT = DV / 2 / 16;                // 16 dv tiles of O^T per wave
constexpr int REC = 648;                        // record bytes: 8 x (1 + 64) + 64 x 2
constexpr int NOPE = 512;                       // fp8-coded dims
constexpr int NSTAGE = 3;                       // decoded tiles in the LDS ring
constexpr int KEYCAP = 2048;                    // keys staged in LDS at a time
constexpr int RING_BYTES = NSTAGE * TILE_BYTES;
constexpr int PX_BYTES = 2 * WAVES * 64 * 16;   // probability exchange, two tiles
constexpr size_t LDS_BYTES = (size_t)RING_BYTES + PX_BYTES + KEYCAP * 4 + 64;
constexpr int LOADS = 7;                        // global load instructions per lane and tile
constexpr float TAU_HARD = 100.0f;              // largest exponent taken against the reference
constexpr int QB_AGPR = 14;                     // k-steps of head block 1's Q kept in AGPRs
}  // namespace pk

// LDS reads of step j of the interleaved S / PV loop: one K read of k-step j
// (j < 18) and the two transpose reads of dv tile j (j < 16)
__host__ __device__ constexpr int pair_step_reads(int j) {
  return (j < pk::KSTEPS ? 1 : 0) + (j < pk::DVT ? 2 : 0);
}

// one lane's share of one tile's records: 17 words from the aligned word
// holding its block's first code, the scale byte, 16 RoPE bytes
struct PairRaw {
  u32x4_l c0, c1, c2, c3;
  uint32_t c4;
  uint32_t sc;
  u32x4_l rope;
};

// APPEND (with FUSED): the launch also appends the batch's cur_len current
// rows in place (rows past_len[b] ..; bf16 rows quantized when cur_quant,
// else records copied) and writes present_len[b]; every workgroup writes its
// batch's new records itself and waits for them before it loads any, so it
// reads its own writes; with `reset` the launch's last workgroup replaces
// the error word instead of adding to it.
// BIAS: the additive attention bias (bf16, IndexShare `bias_at`) of each
// selected key is added to its scaled (and softcapped) score; its shape,
// right-aligned against [batch, 64, q_seq, cap], is bd0..bd3, each extent 1
// (broadcast) or the full one.
template <bool I64, bool FUSED, bool SOFTCAP, bool APPEND, bool BIAS>
__global__ void __launch_bounds__(pk::THREADS, 1)
pair_forward_kernel(const uint16_t* __restrict__ q, uint8_t* __restrict__ cache,
                    const void* __restrict__ idx, const int32_t* __restrict__ valid_len,
                    uint16_t* __restrict__ y, float* __restrict__ part_o, float* __restrict__ part_ml,
                    int64_t q_seq, int64_t rows, int64_t cap, int64_t width, int splits, float scale,
                    float softcap, ErrorBlock* __restrict__ eb,
                    unsigned long long* __restrict__ row_key, unsigned* __restrict__ row_done,
                    const void* __restrict__ cur, const int32_t* __restrict__ past_len,
                    int32_t* __restrict__ present_len, int64_t cur_len, int reset, int cur_quant,
                    const uint16_t* __restrict__ bias, int64_t bd0, int64_t bd1, int64_t bd2, int64_t bd3) {
  using namespace pk;
  extern __shared__ __attribute__((aligned(1024))) uint8_t lds_raw[];
  lds_u8* ring = (lds_u8*)lds_raw;
  lds_u8* px = ring + RING_BYTES;
  int* keys_s = (int*)(lds_raw + RING_BYTES + PX_BYTES);
  int* misc = keys_s + KEYCAP;  // [1] restart request, [8 + w] wave w's key count
  unsigned long long* minkey_s = (unsigned long long*)(misc + 4);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar LDS bases
  const int pair = wave >> 1;
  const int half = wave & 1;
  const int g = lane >> 4;
  const int c16 = lane & 15;
  const int head0 = 32 * pair + c16;  // this lane's column of S^T / O^T in head block 0 (+16: block 1)

  int split;
  int64_t row;
  if (splits == 1) {
    row = rows - 1 - (int64_t)blockIdx.x;
    split = 0;
  } else {
    row = (int64_t)(blockIdx.x % (unsigned)rows);  // a row's splits share blockIdx % 8 (XCD)
    split = (int)(blockIdx.x / (unsigned)rows);
  }
  const int64_t b = row / q_seq;
  const int64_t qi = row - b * q_seq;
  int64_t bound;
  int64_t app_p = 0;
  bool app_ok = false;
  if constexpr (APPEND) {
    app_p = (int64_t)past_len[b];
    app_ok = app_p >= 0 && app_p + cur_len <= cap;  // else nothing is appended and the word says so
    bound = app_p + cur_len;
  } else {
    bound = valid_len ? (int64_t)valid_len[b] : cap;
  }
  bound = bound < 0 ? 0 : (bound > cap ? cap : bound);
  const int64_t ibase = row * width;
  const uint8_t* cache_b = cache + b * cap * REC;
  // this batch's records as a buffer (raw, byte offsets; the range check
  // returns zeros for the offsets of empty tile slots)
  const __amdgpu_buffer_rsrc_t crsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)cache_b, (short)0, (int)(cap * REC), 0x00020000);

  const int wtiles = (int)((width + KT - 1) / KT);
  const int tps = (wtiles + splits - 1) / splits;
  const int c0 = (int)min((int64_t)split * tps * KT, width);
  const int c1 = (int)min((int64_t)c0 + (int64_t)tps * KT, width);

  // ---- per-lane LDS offsets within a decoded tile (row-major rows of 1152
  // bytes, 16-byte chunk c of row R stored at chunk c ^ (R & 6))
  // K: this wave's keys 16 half + c16, chunk 4S + g -> one base per parity of S
  const int kf = c16 & 6;
  const int kbase = half * HALF_ROWS + c16 * ROWB + ((g ^ (kf & 2)) << 4);
  const int kbase_e = kbase + ((kf >> 2) << 6);
  const int kbase_o = kbase - ((kf >> 2) << 6);
  // V^T: lane 4 jj + qq of group g points at row 4g + jj, dv 16 dt + 4 qq of
  // this wave's dv half; one base per dt mod 4
  int vbase[4];
  {
    const int jj = c16 >> 2, qq = c16 & 3;
    const int R = 4 * g + jj;
    const int fv = (R & 6) >> 1;
#pragma unroll
    for (int k = 0; k < 4; k++)
      vbase[k] = half * (DV / 2) * 2 + R * ROWB + ((k ^ fv) << 5) + ((qq >> 1) << 4) + ((qq & 1) << 3);
  }
  // record staging: lane (key slot dk, block dj) of each tile
  const int dk = tid & 31;
  const int dj = tid >> 5;
  const int dshift = (dj + 1) & 3;               // first code's byte within its word
  const uint32_t dcodes = (uint32_t)(65 * dj + 1 - dshift);
  const uint32_t dscale = (uint32_t)(65 * dj);
  const uint32_t drope = (uint32_t)(NOPE / 64 * 65 + 16 * dj);
  // LDS byte offsets within a tile of the lane's decoded chunks: chunk
  // 8 dj + c of row dk is stored at chunk (8 dj + c) ^ (dk & 6); for
  // c = 4 c2 + 2 c1 + c0 that is dk * ROWB + 128 dj + 64 (c2 ^ s2) + 32 (c1 ^ s1)
  // + 16 c0, one base per (c2, c1) with c0 as an immediate offset
  uint32_t wofs[4];
  {
    const int s1 = (dk >> 1) & 1, s2 = (dk >> 2) & 1;
#pragma unroll
    for (int k = 0; k < 4; k++)
      wofs[k] = (uint32_t)(dk * ROWB + 128 * dj + 64 * ((k >> 1) ^ s2) + 32 * ((k & 1) ^ s1));
  }
  const uint32_t wrope = (uint32_t)(dk * ROWB + 16 * (64 + (dj ^ (dk & 6))));
  const float f = SOFTCAP ? kLog2eL : scale * kLog2eL;  // scores -> log2 units
  // the bias rows of this lane's two heads (element 0 when the key extent is 1)
  const uint16_t* brow0 = bias;
  int64_t bstep = 0;  // head0 + 16 relative to head0
  if constexpr (BIAS) {
    brow0 = bias + (((bd0 == 1 ? 0 : b) * bd1 + (bd1 == 1 ? 0 : head0)) * bd2 + (bd2 == 1 ? 0 : qi)) * bd3;
    bstep = bd1 == 1 ? 0 : 16 * bd2 * bd3;
  }
  const bool bkey = BIAS && bd3 != 1;
  const uint32_t px_own = (uint32_t)(uintptr_t)(px + (wave * 64 + lane) * 16);
  const uint32_t px_peer = (uint32_t)(uintptr_t)(px + ((wave ^ 1) * 64 + lane) * 16);
  constexpr int PXH = WAVES * 64 * 16;  // second exchange buffer

  bf16x8_l qa[KSTEPS], qb[KSTEPS];
  bool q_loaded = false;
  bool first_pass = true;
  float m_floor0 = -INFINITY, m_floor1 = -INFINITY;
  f32x4_l o0[DVT], o1[DVT];
  float m_ref0, m_ref1, l0, l1;
  unsigned long long mk = ~0ull;
  int vhi = c0;  // columns below vhi have been validated

  // Stage columns [st0, st1) of the index row: the keys (clamped into the
  // cache) go to keys_s, each wave's count of keys up to the row's last
  // non-padding entry to misc[8 + wave], and columns not validated before
  // are checked. Called with no reader of keys_s / misc left.
  auto stage_keys = [&](int st0, int st1) {
    constexpr int PER = KEYCAP / THREADS;  // every load in flight at once
    const bool check = FUSED && st0 >= vhi;
    // every load is unconditional (addresses clamped into the stage) so all
    // of them are in flight together; out-of-stage lanes are fixed up after
    int64_t v[PER], u[PER];
#pragma unroll
    for (int k = 0; k < PER; k++) {
      const int c = min(st0 + tid + THREADS * k, st1 - 1);
      v[k] = load_index<I64>(idx, ibase + c);
      if (check) u[k] = load_index<I64>(idx, ibase + max(c - 1, 0));
    }
    int last = 0, fresh = 0;
#pragma unroll
    for (int k = 0; k < PER; k++) {
      const int s = tid + THREADS * k;
      const int c = st0 + s;
      if (c < st1) {
        keys_s[s] = (int)((v[k] >= 0 && v[k] < bound) ? v[k] : 0);  // clamp: a bad row stays in bounds
        if (v[k] != -1) last = s + 1;
        if (APPEND && v[k] >= app_p && v[k] < bound) fresh = 1;     // selects a row this launch appends
        if (check && column_class(c, v[k], u[k], bound))
          mk = min(mk, (unsigned long long)(row * (width + 1) + c));
      }
    }
    if (check) vhi = st1;
    last = wave_max_nonneg(last);
    if (lane == 0) misc[8 + wave] = last;
    if constexpr (APPEND) {
      fresh = wave_max_nonneg(fresh);
      if (lane == 0) misc[12 + wave] = fresh;
    }
    if (tid == 0) misc[1] = 0;
  };
  // the first stage's index loads go out before anything waits on memory
  bool staged = c0 < c1;
  if (staged) stage_keys(c0, min(c0 + KEYCAP, c1));

  // APPEND: the batch's current rows go into the cache (quantized by one
  // wave per row, or copied 8 bytes per lane) from a workgroup that loads one
  // of them (before its loads, and it waits for its stores, so it reads them
  // back from its own L2), and from one workgroup per batch at its end (which
  // also reports the append); no other workgroup touches them
  const bool duty = split == 0 && qi == 0;
  bool app_done = false;  // uniform
  bool app_bad = false;   // a current row held a NaN or an infinity (this wave's rows)
  auto append_rows = [&]() {
    if (app_ok) {
      uint8_t* dst0 = cache + (b * cap + app_p) * REC;
      if (cur_quant) {
        for (int t = wave; t < cur_len; t += WAVES)
          app_bad |= quantize_row_wave((const uint16_t*)cur + (b * cur_len + t) * DK, dst0 + t * REC, DK,
                                       DK - NOPE, lane);
      } else {
        const uint2* src = (const uint2*)((const uint8_t*)cur + b * cur_len * REC);
        for (int u = tid; u < cur_len * (REC / 8); u += THREADS) ((uint2*)dst0)[u] = src[u];
      }
    }
    app_done = true;
  };

  for (;;) {
#pragma unroll
    for (int t = 0; t < DVT; t++) o0[t] = o1[t] = (f32x4_l){0.f, 0.f, 0.f, 0.f};
    m_ref0 = m_floor0;
    m_ref1 = m_floor1;
    l0 = l1 = 0.0f;
    float ms0 = m_floor0, ms1 = m_floor1;  // largest scaled scores seen (this lane)
    bool restart = false;

    for (int st0 = c0; st0 < c1 && !restart; st0 += KEYCAP) {
      const int st1 = min(st0 + KEYCAP, c1);
      const bool need_ref = first_pass && st0 == c0;  // uniform
      if (!staged) {
        __syncthreads();  // the previous stage's readers are done with keys_s / misc / the ring
        stage_keys(st0, st1);
      }
      staged = false;
      __syncthreads();
      const int kcount = max(max(misc[8], misc[9]), max(misc[10], misc[11]));
      const int ntile = (kcount + KT - 1) / KT;
      if constexpr (APPEND) {
        // this stage loads appended records: they are stored and have landed
        // before the loads (the barrier waits for the stores)
        if ((misc[12] | misc[13] | misc[14] | misc[15]) != 0) {
          if (!app_done) append_rows();
          __syncthreads();
        }
      }

      if (ntile == 0) continue;  // uniform: no key in this stage

      auto tile_addr = [&](int tt) { return (uint32_t)(uintptr_t)(ring + (tt % NSTAGE) * TILE_BYTES); };
      // ---- record staging: issue the loads of tile tt (zeros past the keys)
      // byte offset of the lane's record in tile tt (beyond the buffer, so
      // the loads return zeros, for slots past the keys)
      auto rec_base = [&](int tt) {
        const int slot = tt * KT + dk;
        uint32_t base = 0x80000000u;
        if (tt < ntile && slot < kcount) base = (uint32_t)keys_s[slot] * (uint32_t)REC;
        return base;
      };
      auto issue = [&](PairRaw& R, uint32_t base) {
        R.c0 = __builtin_bit_cast(u32x4_l, __builtin_amdgcn_raw_buffer_load_b128(crsrc, base + dcodes, 0, 0));
        R.c1 = __builtin_bit_cast(u32x4_l, __builtin_amdgcn_raw_buffer_load_b128(crsrc, base + dcodes + 16, 0, 0));
        R.c2 = __builtin_bit_cast(u32x4_l, __builtin_amdgcn_raw_buffer_load_b128(crsrc, base + dcodes + 32, 0, 0));
        R.c3 = __builtin_bit_cast(u32x4_l, __builtin_amdgcn_raw_buffer_load_b128(crsrc, base + dcodes + 48, 0, 0));
        R.c4 = __builtin_amdgcn_raw_buffer_load_b32(crsrc, base + dcodes + 64, 0, 0);
        R.sc = (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(crsrc, base + dscale, 0, 0);
        R.rope = __builtin_bit_cast(u32x4_l, __builtin_amdgcn_raw_buffer_load_b128(crsrc, base + drope, 0, 0));
      };
      // decode tile tt from registers into its ring slot
      auto store = [&](const PairRaw& R, int tt) {
        if (tt >= ntile) return;  // uniform: a tile past the keys is never read
        const uint32_t e = R.sc & 0xffu;
        const uint32_t D[17] = {R.c0[0], R.c0[1], R.c0[2], R.c0[3], R.c1[0], R.c1[1], R.c1[2], R.c1[3],
                                R.c2[0], R.c2[1], R.c2[2], R.c2[3], R.c3[0], R.c3[1], R.c3[2], R.c3[3], R.c4};
        uint32_t w[32];
        // empty slots (past the keys) were loaded as zeros: scale 0, codes 0
        if ((e >= 10u && e <= 246u) || tt * KT + dk >= kcount) {
          const float s = __uint_as_float(e << 23);
#pragma unroll
          for (int i = 0; i < 16; i++) {
            const uint32_t cw = __builtin_amdgcn_alignbyte(D[i + 1], D[i], (uint32_t)dshift);
            w[2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(cw, s, false));
            w[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(cw, s, true));
          }
        } else {
#pragma unroll
          for (int i = 0; i < 16; i++) {
            const uint32_t cw = __builtin_amdgcn_alignbyte(D[i + 1], D[i], (uint32_t)dshift);
            w[2 * i] = fp8_code_to_bf16_exact(cw & 0xffu, e) | (fp8_code_to_bf16_exact((cw >> 8) & 0xffu, e) << 16);
            w[2 * i + 1] = fp8_code_to_bf16_exact((cw >> 16) & 0xffu, e) | (fp8_code_to_bf16_exact(cw >> 24, e) << 16);
          }
        }
        const uint32_t T = tile_addr(tt);
#pragma unroll
        for (int k = 0; k < 4; k++) {
          const uint32_t a = T + wofs[k];
          ds_write_b128_off<0>(a, (u32x4_l){w[8 * k], w[8 * k + 1], w[8 * k + 2], w[8 * k + 3]});
          ds_write_b128_off<16>(a, (u32x4_l){w[8 * k + 4], w[8 * k + 5], w[8 * k + 6], w[8 * k + 7]});
        }
        ds_write_b128_off<0>(T + wrope, R.rope);
      };

      // BIAS: the lane's bias values of tile tt (keys of slots 16 half + 4g + i,
      // heads head0 and head0 + 16), loaded ahead of their softmax as ordinary
      // loads issued before the record loads of the same iteration (the
      // compiler's wait at the use leaves those in flight). Staged keys are
      // already clamped into the cache.
      uint16_t bv0[4], bv1[4];
      auto bias_load = [&](int tt) {
        if constexpr (BIAS) {
#pragma unroll
          for (int i = 0; i < 4; i++) {
            const int slot = tt * KT + 16 * half + 4 * g + i;
            const int64_t kc = bkey && slot < kcount ? keys_s[slot] : 0;
            bv0[i] = brow0[kc];
            bv1[i] = brow0[bstep + kc];
          }
        }
      };
      bias_load(0);  // before the record loads: its wait leaves them in flight
      PairRaw ra, rb;
      issue(ra, rec_base(0));
      issue(rb, rec_base(1));
      uint32_t base_next = rec_base(2);
      if (!q_loaded) {
        // Q^T of the pair's heads, loaded while the first records are in
        // flight; lane (c16, g) holds dims 32 s + 8g .. +8 of heads head0 and
        // head0 + 16. The MFMA B operands read Q from AGPRs (all of block 0,
        // most of block 1): the vector registers stay free for the pipeline
        u32x4_l qraw[KSTEPS];
        const uint16_t* qp0 = q + ((b * NH + head0) * q_seq + qi) * DK + 8 * g;
#pragma unroll
        for (int s = 0; s < KSTEPS; s++) qraw[s] = __builtin_bit_cast(u32x4_l, *(const uint4*)(qp0 + s * 32));
#pragma unroll
        for (int s = 0; s < KSTEPS; s++) {
          u32x4_l r = qraw[s];
          asm volatile("" : "+a"(r));
          qa[s] = __builtin_bit_cast(bf16x8_l, r);
        }
        const uint16_t* qp = q + ((b * NH + head0 + 16) * q_seq + qi) * DK + 8 * g;
#pragma unroll
        for (int s = 0; s < KSTEPS; s++) qraw[s] = __builtin_bit_cast(u32x4_l, *(const uint4*)(qp + s * 32));
#pragma unroll
        for (int s = 0; s < KSTEPS; s++) {
          u32x4_l r = qraw[s];
          if (s < QB_AGPR) asm volatile("" : "+a"(r));
          qb[s] = __builtin_bit_cast(bf16x8_l, r);
        }
        q_loaded = true;
      }
      wait_vm<LOADS>();
      store(ra, 0);
      issue(ra, base_next);
      base_next = rec_base(3);  // read one iteration ahead of its loads
      wait_vm<LOADS>();
      store(rb, 1);

      uint32_t ka_e = 0, ka_o = 0, va[4] = {0, 0, 0, 0};
      auto set_k = [&](int tt) {
        const uint32_t T = tile_addr(tt);
        ka_e = T + kbase_e;
        ka_o = T + kbase_o;
      };
      auto set_v = [&](int tt) {
        const uint32_t T = tile_addr(tt);
#pragma unroll
        for (int k = 0; k < 4; k++) va[k] = T + vbase[k];
      };
      u32x4_l kr[KSTEPS];
      s16x4_l vr0[DVT], vr1[DVT];
      f32x4_l sa[2][2];
      auto kread = [&](auto sc) {
        constexpr int S = decltype(sc)::value;
        kr[S] = ds_read_b128_at<64 * S>((S & 1) ? ka_o : ka_e);
      };
      auto kmfma = [&](auto sc) {
        constexpr int S = decltype(sc)::value;
        const bf16x8_l a = __builtin_bit_cast(bf16x8_l, kr[S]);
        sa[0][S & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qa[S], sa[0][S & 1], 0, 0, 0);
        sa[1][S & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qb[S], sa[1][S & 1], 0, 0, 0);
      };
      auto vread = [&](auto dc) {
        constexpr int DT = decltype(dc)::value;
        vr0[DT] = ds_read_tr16_at<32 * (DT & ~3)>(va[DT & 3]);
        vr1[DT] = ds_read_tr16_at<32 * (DT & ~3) + HALF_ROWS>(va[DT & 3]);
      };
      bf16x8_l pb0, pb1;
      auto vmfma = [&](auto dc) {
        constexpr int DT = decltype(dc)::value;
        const s16x4_l a8[2] = {vr0[DT], vr1[DT]};
        const bf16x8_l a = __builtin_bit_cast(bf16x8_l, a8);
        o0[DT] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb0, o0[DT], 0, 0, 0);
        o1[DT] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb1, o1[DT], 0, 0, 0);
      };
      auto zero_s = [&]() {
#pragma unroll
        for (int hb = 0; hb < 2; hb++) sa[hb][0] = sa[hb][1] = (f32x4_l){0.f, 0.f, 0.f, 0.f};
      };
      // softmax of tile tt from sa: lane holds keys 16 half + 4g + r of heads
      // head0 (block 0) and head0 + 16 (block 1). Returns this wave's four
      // probability words and writes them to the exchange buffer of tile tt.
      auto softmax = [&](int tt) {
        const f32x4_l s0 = sa[0][0] + sa[0][1], s1 = sa[1][0] + sa[1][1];
        float x0[4], x1[4];
#pragma unroll
        for (int i = 0; i < 4; i++) {
          x0[i] = s0[i];
          x1[i] = s1[i];
        }
        if constexpr (SOFTCAP) {
#pragma unroll
          for (int i = 0; i < 4; i++) {
            x0[i] = softcap * tanhf(x0[i] * scale / softcap);
            x1[i] = softcap * tanhf(x1[i] * scale / softcap);
          }
        }
        if constexpr (BIAS) {
          // the bias joins the scaled (and softcapped) score, then log2 units
#pragma unroll
          for (int i = 0; i < 4; i++) {
            x0[i] = ((SOFTCAP ? x0[i] : x0[i] * scale) + bf16_to_f32(bv0[i])) * kLog2eL;
            x1[i] = ((SOFTCAP ? x1[i] : x1[i] * scale) + bf16_to_f32(bv1[i])) * kLog2eL;
          }
        }
        if ((tt + 1) * KT > kcount) {  // uniform: only the last tile has empty slots
          const int slot_base = tt * KT + 16 * half + 4 * g;
#pragma unroll
          for (int i = 0; i < 4; i++)
            if (slot_base + i >= kcount) x0[i] = x1[i] = -INFINITY;
        }
        // scores in log2 units, rounded once: the maximum then gives exp2(0)
        // exactly (an FMA against a rounded maximum can overflow for huge scores)
        if constexpr (!BIAS) {
#pragma unroll
          for (int i = 0; i < 4; i++) {
            x0[i] *= f;
            x1[i] *= f;
          }
        }
        const float lm0 = fmaxf(fmaxf(x0[0], x0[1]), fmaxf(x0[2], x0[3]));
        const float lm1 = fmaxf(fmaxf(x1[0], x1[1]), fmaxf(x1[2], x1[3]));
        ms0 = fmaxf(ms0, lm0);
        ms1 = fmaxf(ms1, lm1);
        if (need_ref && tt == 0) {
          // the pair's reference: the larger of both waves' first-tile maxima
          const float t0 = max_x32(max_x16(lm0)), t1 = max_x32(max_x16(lm1));
          ds_write_b64_at(px_own + PXH, (u32x2_l){__float_as_uint(t0), __float_as_uint(t1)});
          lds_barrier();
          u32x2_l pm;
          asm volatile("ds_read_b64 %0, %1 offset:%2\n\ts_waitcnt lgkmcnt(0)" : "=v"(pm) : "v"(px_peer), "n"(PXH) : "memory");
          m_ref0 = fmaxf(t0, __uint_as_float(pm[0]));
          m_ref1 = fmaxf(t1, __uint_as_float(pm[1]));
        }
        // a score more than 2^TAU_HARD above the reference: this pass is
        // discarded and redone (its exp2 may overflow)
        if (lm0 > m_ref0 + TAU_HARD || lm1 > m_ref1 + TAU_HARD) misc[1] = 1;  // every writer stores 1
        const float n0 = m_ref0 == -INFINITY ? 0.0f : -m_ref0;
        const float n1 = m_ref1 == -INFINITY ? 0.0f : -m_ref1;
        float p0[4], p1[4];
#pragma unroll
        for (int i = 0; i < 4; i++) {
          p0[i] = __builtin_amdgcn_exp2f(x0[i] + n0);
          p1[i] = __builtin_amdgcn_exp2f(x1[i] + n1);
        }
        l0 += (p0[0] + p0[1]) + (p0[2] + p0[3]);
        l1 += (p1[0] + p1[1]) + (p1[2] + p1[3]);
        const u32x4_l pw = {pack_bf16x2(p0[0], p0[1]), pack_bf16x2(p0[2], p0[3]), pack_bf16x2(p1[0], p1[1]),
                            pack_bf16x2(p1[2], p1[3])};
        ds_write_b128_at(px_own + (uint32_t)((tt & 1) * PXH), pw);
        return pw;
      };
      // the B operands of PV for tile tt: keys 4g + r from the half-0 wave,
      // then 16 + 4g + r from the half-1 wave (the K order of the V^T reads)
      auto take_peer = [&](int tt, const u32x4_l& own) {
        u32x4_l pw;
        asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(pw) : "v"(px_peer + (uint32_t)((tt & 1) * PXH)) : "memory");
        const u32x4_l lo = half ? pw : own, hi = half ? own : pw;
        pb0 = __builtin_bit_cast(bf16x8_l, (u32x4_l){lo[0], lo[1], hi[0], hi[1]});
        pb1 = __builtin_bit_cast(bf16x8_l, (u32x4_l){lo[2], lo[3], hi[2], hi[3]});
      };

      // ---- tile 0: S alone, the reads KD k-steps ahead of their MFMAs
      lds_barrier();
      set_k(0);
      zero_s();
      {
        constexpr int KD = 6;
        static_for<KD>(kread);
        static_for<KSTEPS>([&](auto sc) {
          constexpr int S = decltype(sc)::value;
          if constexpr (S + KD < KSTEPS) kread(std::integral_constant<int, S + KD>{});
          constexpr int LATER = (KD < KSTEPS - 1 - S ? KD : KSTEPS - 1 - S);
          lgkm_wait_tied1<LATER>(kr[S]);
          kmfma(sc);
          __builtin_amdgcn_sched_barrier(0);
        });
      }
      u32x4_l pown = softmax(0);

      // ---- steady state: S of tile t+1 interleaved with PV of tile t, one
      // k-step and one dv tile per step (4 MFMAs, 2 KB of LDS reads per
      // wave), the reads PL steps ahead; then the softmax of tile t+1 and the
      // decode of tile t+2 (its records were loaded one iteration earlier)
      auto iteration = [&](int t, PairRaw& rnext, PairRaw& rdec) {
        lds_barrier();  // tile t+1 decoded, tile t's exchange visible, tile t-1's slot free
        bias_load(t + 1);         // older than tile t+3's record loads
        issue(rnext, base_next);  // tile t+3
        take_peer(t, pown);
        set_k(t + 1);
        set_v(t);
        zero_s();
        constexpr int PL = 2;
        auto sread = [&](auto jc) {
          constexpr int J = decltype(jc)::value;
          if constexpr (J < KSTEPS) kread(jc);
          if constexpr (J < DVT) vread(jc);
        };
        static_for<PL>(sread);
        static_for<KSTEPS>([&](auto jc) {
          constexpr int J = decltype(jc)::value;
          if constexpr (J + PL < KSTEPS) sread(std::integral_constant<int, J + PL>{});
          constexpr int LATER = pair_step_reads(J + 1) * (J + 1 < KSTEPS) + pair_step_reads(J + 2) * (PL > 1 && J + 2 < KSTEPS);
          if constexpr (J < DVT) {
            lgkm_wait3<LATER>(kr[J], vr0[J], vr1[J]);
            kmfma(jc);
            vmfma(jc);
          } else {
            lgkm_wait_tied1<LATER>(kr[J]);
            kmfma(jc);
          }
          __builtin_amdgcn_sched_barrier(0);
        });
        pown = softmax(t + 1);
        wait_vm<LOADS>();  // tile t+2's records (tile t+3's may stay in flight)
        store(rdec, t + 2);
        base_next = rec_base(t + 4);
      };
      int t = 0;
      for (; t + 2 < ntile; t += 2) {
        iteration(t, rb, ra);      // loads tile t+3 into rb, decodes t+2 from ra
        iteration(t + 1, ra, rb);  // loads tile t+4 into ra, decodes t+3 from rb
      }
      if (t + 1 < ntile) {
        iteration(t, rb, ra);
        t++;
      }

      // ---- the last tile's PV alone
      lds_barrier();
      take_peer(ntile - 1, pown);
      set_v(ntile - 1);
      {
        constexpr int VD = 6;
        static_for<VD>(vread);
        static_for<DVT>([&](auto dc) {
          constexpr int DT = decltype(dc)::value;
          constexpr int AHEAD = (VD - 1 < DVT - 1 - DT ? VD - 1 : DVT - 1 - DT);
          lgkm_wait_tied<2 * AHEAD>(vr0[DT], vr1[DT]);
          vmfma(dc);
          if constexpr (DT + VD < DVT) vread(std::integral_constant<int, DT + VD>{});
          __builtin_amdgcn_sched_barrier(0);
        });
      }
      wait_vm<0>();  // record loads issued past the last tile
      __syncthreads();
      restart = misc[1] != 0;
    }
    if (!restart) break;
    // the next pass starts from the largest scaled score either wave of the
    // pair has seen for each head
    first_pass = false;
    {
      float a0 = max_x32(max_x16(ms0)), a1 = max_x32(max_x16(ms1));
      __syncthreads();
      ds_write_b64_at(px_own, (u32x2_l){__float_as_uint(a0), __float_as_uint(a1)});
      lds_barrier();
      u32x2_l pm;
      asm volatile("ds_read_b64 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(pm) : "v"(px_peer) : "memory");
      m_floor0 = fmaxf(a0, __uint_as_float(pm[0]));
      m_floor1 = fmaxf(a1, __uint_as_float(pm[1]));
      __syncthreads();
    }
  }

  // ---- the workgroup's first violation (fused validation)
  if constexpr (FUSED) {
    if (c0 == 0 && tid == 0 && width > 0 && load_index<I64>(idx, ibase) == -1)
      mk = min(mk, (unsigned long long)(row * (width + 1) + width));  // all -1, unless a column fails
    if (tid == 0) *minkey_s = ~0ull;
    __syncthreads();
    if (mk != ~0ull) atomicMin(minkey_s, mk);
  }

  // ---- epilogue: each head's sum over both waves of its pair
  __syncthreads();
  {
    const float s0 = sum_x32(sum_x16(l0)), s1 = sum_x32(sum_x16(l1));
    ds_write_b64_at(px_own, (u32x2_l){__float_as_uint(s0), __float_as_uint(s1)});
    lds_barrier();
    u32x2_l pl;
    asm volatile("ds_read_b64 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(pl) : "v"(px_peer) : "memory");
    l0 = s0 + __uint_as_float(pl[0]);
    l1 = s1 + __uint_as_float(pl[1]);
  }
  // lane holds O^T[256 half + 16 dt + 4g + r][head0 (+16)]. Every head's
  // output is normalised by its row sum and rounded to bf16 into LDS rows
  // (the ring is free), then each lane stores 16 contiguous bytes of one
  // head's row: to Y when the keys are not split, else to the split's partial
  // (with its fp32 (reference, row sum) pairs, merged by the bf16 merge
  // kernel), written through the L2 so the launch's end has no dirty
  // partials to write back.
  {
    constexpr int YROW = 1024 + 16;
    __syncthreads();
    const float inv0 = l0 > 0.0f ? 1.0f / l0 : 0.0f;
    const float inv1 = l1 > 0.0f ? 1.0f / l1 : 0.0f;
    lds_u8* y0 = ring + head0 * YROW + (DV / 2) * 2 * half + 8 * g;
    lds_u8* y1 = y0 + 16 * YROW;
#pragma unroll
    for (int dt = 0; dt < DVT; dt++) {
      *(__attribute__((address_space(3))) u32x2_l*)(y0 + 32 * dt) =
          (u32x2_l){pack_bf16x2(o0[dt][0] * inv0, o0[dt][1] * inv0), pack_bf16x2(o0[dt][2] * inv0, o0[dt][3] * inv0)};
      *(__attribute__((address_space(3))) u32x2_l*)(y1 + 32 * dt) =
          (u32x2_l){pack_bf16x2(o1[dt][0] * inv1, o1[dt][1] * inv1), pack_bf16x2(o1[dt][2] * inv1, o1[dt][3] * inv1)};
    }
    if (splits > 1 && g == 0 && half == 0) {
      const __amdgpu_buffer_rsrc_t mrsrc = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(part_ml + (row * splits + split) * NH * 2), (short)0, NH * 8, 0x00020000);
      __builtin_amdgcn_raw_buffer_store_b64((u32x2_l){__float_as_uint(m_ref0), __float_as_uint(l0)}, mrsrc,
                                            head0 * 8, 0, kWriteThrough);
      __builtin_amdgcn_raw_buffer_store_b64((u32x2_l){__float_as_uint(m_ref1), __float_as_uint(l1)}, mrsrc,
                                            (head0 + 16) * 8, 0, kWriteThrough);
    }
    __syncthreads();
    if (splits == 1) {
#pragma unroll 4
      for (int hh = 0; hh < 16; hh++) {
        const int h = 16 * wave + hh;
        const u32x4_l v = *(const lds_u32x4*)(ring + h * YROW + 16 * lane);
        *(u32x4_l*)(y + ((b * NH + h) * q_seq + qi) * DV + 8 * lane) = v;
      }
    } else {
      const __amdgpu_buffer_rsrc_t prsrc = __builtin_amdgcn_make_buffer_rsrc(
          (void*)((uint16_t*)part_o + (row * splits + split) * NH * DV), (short)0, NH * DV * 2, 0x00020000);
#pragma unroll 4
      for (int hh = 0; hh < 16; hh++) {
        const int h = 16 * wave + hh;
        const u32x4_l v = *(const lds_u32x4*)(ring + h * YROW + 16 * lane);
        __builtin_amdgcn_raw_buffer_store_b128(v, prsrc, h * (DV * 2) + 16 * lane, 0, kWriteThrough);
      }
    }
  }
  if constexpr (APPEND) {
    if (duty) {
      if (!app_done) append_rows();
      if (app_bad && lane == 0) atomicOr(&eb->call_word, SA_ERR_QUANT_NONFINITE | SA_ERR_APPEND_ANY);
      if (tid == 0) {
        // an atomic store: this launch's finisher may read it
        if (app_ok) atomicExch(&present_len[b], (int32_t)(app_p + cur_len));
        else atomicOr(&eb->call_word, SA_ERR_APPEND_CAPACITY | SA_ERR_APPEND_ANY);
      }
    }
  }
  if constexpr (FUSED) __syncthreads();  // minkey_s is complete

  // ---- error block: with split keys this workgroup's first violation goes
  // to the row's slot, and the merge kernel that follows the launch records
  // each row's first violation and finishes the launch's record; a row's only
  // workgroup records its row and counts it toward the launch's record itself
  if constexpr (FUSED) {
    if (tid == 0) {
      const unsigned long long k = *minkey_s;
      if (splits == 1) {
        if (k != ~0ull) record_row_violation<I64>(eb, idx, row, width, k, bound);
        // present_len is stored atomically above and read atomically there
        finish_launch<I64, false>(eb, idx, width, q_seq, q_seq, APPEND ? present_len : valid_len, cap,
                                  (unsigned)rows, reset != 0);
      } else if (k != ~0ull) {
        atomicMin(&row_key[row], k);
      }
    }
  }
}

bool pair_supported(const sa_config& cfg, int64_t index_heads) {
  return mla_supported(cfg, index_heads) && cfg.cache_format == SA_CACHE_FP8_E4M3_BLOCK64 &&
         cfg.rope_dim == pk::DK - pk::NOPE && cfg.max_cache_len <= (int64_t)(0x7fffffffLL / pk::REC);
}

static bool g_pair_attr[20] = {};

sa_status launch_forward_pair(sparse_attn_ctx* c, const FwdArgs& a, int splits, bool fused, const AppendArgs* app) {
  using namespace pk;
  const int64_t rows = a.batch * a.q_seq;
  if (rows <= 0) return SA_OK;
  if (splits > 1 && rows * splits > c->partial_rows)
    return set_error(c, SA_E_STATE, "forward: split-K partials exceed the context's buffers");
  if (rows > c->rows_cap) return set_error(c, SA_E_STATE, "forward: more rows than the context holds");
  if (a.cap > (int64_t)(0x7fffffffLL / REC)) return set_error(c, SA_E_SHAPE, "forward: cache too long for 32-bit record offsets");
  const int64_t wgs = rows * splits;
  if (wgs > 0x7fffffffLL) return set_error(c, SA_E_SHAPE, "forward: too many rows for one launch");
  const bool cap_on = a.softcap != 0.0f;
  if (app && (!fused || app->cur_len < 0 || app->cur_len > kFusedAppendRows))
    return set_error(c, SA_E_STATE, "forward: in-launch append needs fused validation and at most 8 rows");
  const bool bias_on = a.bias != nullptr;
  if (app && bias_on) return set_error(c, SA_E_STATE, "forward: in-launch append takes no bias");
  const int variant = app ? 8 + (a.idx64 ? 1 : 0) + (cap_on ? 2 : 0)
                          : (bias_on ? 12 : 0) + (a.idx64 ? 1 : 0) + (fused ? 2 : 0) + (cap_on ? 4 : 0);
  const void* fns[20] = {(const void*)pair_forward_kernel<false, false, false, false, false>,
                         (const void*)pair_forward_kernel<true, false, false, false, false>,
                         (const void*)pair_forward_kernel<false, true, false, false, false>,
                         (const void*)pair_forward_kernel<true, true, false, false, false>,
                         (const void*)pair_forward_kernel<false, false, true, false, false>,
                         (const void*)pair_forward_kernel<true, false, true, false, false>,
                         (const void*)pair_forward_kernel<false, true, true, false, false>,
                         (const void*)pair_forward_kernel<true, true, true, false, false>,
                         (const void*)pair_forward_kernel<false, true, false, true, false>,
                         (const void*)pair_forward_kernel<true, true, false, true, false>,
                         (const void*)pair_forward_kernel<false, true, true, true, false>,
                         (const void*)pair_forward_kernel<true, true, true, true, false>,
                         (const void*)pair_forward_kernel<false, false, false, false, true>,
                         (const void*)pair_forward_kernel<true, false, false, false, true>,
                         (const void*)pair_forward_kernel<false, true, false, false, true>,
                         (const void*)pair_forward_kernel<true, true, false, false, true>,
                         (const void*)pair_forward_kernel<false, false, true, false, true>,
                         (const void*)pair_forward_kernel<true, false, true, false, true>,
                         (const void*)pair_forward_kernel<false, true, true, false, true>,
                         (const void*)pair_forward_kernel<true, true, true, false, true>};
  if (!g_pair_attr[variant]) {
    hipError_t e = hipFuncSetAttribute(fns[variant], hipFuncAttributeMaxDynamicSharedMemorySize, (int)LDS_BYTES);
    if (e != hipSuccess) return check_hip(c, e, "forward (fp8 pair) LDS attribute");
    g_pair_attr[variant] = true;
  }
  const dim3 grid((unsigned)wgs), block(THREADS);
  const ProfEvents pe = prof_next(c);
  const void* cur = app ? app->cur : nullptr;
  const int32_t* plen = app ? app->past_len : nullptr;
  int32_t* prlen = app ? app->present_len : nullptr;
  const int64_t clen = app ? app->cur_len : 0;
  const int reset = app ? app->reset : 0;
  const int quant = app ? app->quant : 0;
#define SA_PAIR(I, F, C, A, B)                                                                        \
  SA_MAIN_LAUNCH(pe, (pair_forward_kernel<I, F, C, A, B>), grid, block, LDS_BYTES, c->stream,         \
                     (const uint16_t*)a.q, (uint8_t*)a.k, a.idx, a.valid_len, (uint16_t*)a.y,         \
                     c->partial_o, c->partial_ml, a.q_seq, rows, a.cap, a.width, splits, a.scale,     \
                     a.softcap, c->err, c->row_key, c->row_done, cur, plen, prlen, clen, reset, quant, \
                     (const uint16_t*)a.bias, a.bd[0], a.bd[1], a.bd[2], a.bd[3])
  switch (variant) {
    case 0: SA_PAIR(false, false, false, false, false); break;
    case 1: SA_PAIR(true, false, false, false, false); break;
    case 2: SA_PAIR(false, true, false, false, false); break;
    case 3: SA_PAIR(true, true, false, false, false); break;
    case 4: SA_PAIR(false, false, true, false, false); break;
    case 5: SA_PAIR(true, false, true, false, false); break;
    case 6: SA_PAIR(false, true, true, false, false); break;
    case 7: SA_PAIR(true, true, true, false, false); break;
    case 8: SA_PAIR(false, true, false, true, false); break;
    case 9: SA_PAIR(true, true, false, true, false); break;
    case 10: SA_PAIR(false, true, true, true, false); break;
    case 11: SA_PAIR(true, true, true, true, false); break;
    case 12: SA_PAIR(false, false, false, false, true); break;
    case 13: SA_PAIR(true, false, false, false, true); break;
    case 14: SA_PAIR(false, true, false, false, true); break;
    case 15: SA_PAIR(true, true, false, false, true); break;
    case 16: SA_PAIR(false, false, true, false, true); break;
    case 17: SA_PAIR(true, false, true, false, true); break;
    case 18: SA_PAIR(false, true, true, false, true); break;
    default: SA_PAIR(true, true, true, false, true); break;
  }
#undef SA_PAIR
  sa_status s = check_hip(c, hipGetLastError(), "forward (fp8 pair)");
  if (s != SA_OK || splits == 1) return s;
  return launch_latent_merge(c, a, rows, splits, fused, app);
}

}  // namespace sa
