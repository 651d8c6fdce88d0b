// Shared-latent selected-token attention over bf16 rows on the gfx950 matrix
// cores, fed by a direct-to-LDS gather: the form for rows with an attention
// bias (the eight-wave kernel of k_forward_latent_decode.hip takes the rows
// without one).
//
// All 64 query heads of a (batch, query) row read one kv head through one
// index row (IndexShare with kv_num_heads = 1 and a shared index list; the
// latent row is 576 wide and its first 512 dims are V). Per 32-key tile:
// S^T = K_sel . Q^T and O^T += V_sel^T . P^T on v_mfma_f32_16x16x32_bf16, an
// online softmax per head, and optionally a split of the row's keys over
// several workgroups merged by log-sum-exp (the bf16 merge kernel of the
// eight-wave kernel).
//
// Data movement:
//  * the gathered rows go from HBM straight into LDS (global_load_lds, 16 B
//    per lane) through a ring of NSTAGE tiles of 32 rows x 1152 B; each lane
//    may fetch any 16-byte chunk, so the tile is stored row-major with chunk c
//    of row R at chunk c ^ (R & 6). On gfx950 a ds_read_b128 is served in four
//    passes of four lane quads ({0,3,5,6}, {1,2,4,7} and the same eight quads
//    + 8); under that swizzle the K reads below (16 rows, one chunk) hit 16
//    distinct bank groups per pass, and so do the transposing V reads;
//  * wave w owns heads 16 w .. 16 w + 15: all 576 dims of their scores and
//    all 512 dims of their outputs, so no wave waits for another between the
//    tile barriers;
//  * K (the A operand of S^T) is read as 16-byte rows; V^T (the A operand of
//    O^T) comes from the same row-major tile through ds_read_b64_tr_b16, whose
//    16-lane transpose hands lane i the value of dv i for four keys. Both are
//    inline asm with immediate offsets and counted waits;
//  * each head keeps a fixed softmax reference (its first tile's max), so the
//    O^T accumulators are only ever touched by the MFMAs;
//  * with fused validation each workgroup checks its own columns of the index
//    row (IndexShare host-validator rules) while it stages the keys; a row's
//    first violation is recorded by its only workgroup, or, with split keys,
//    by the merge kernel that follows the launch.
#include "sa_mfma_dev.h"
#include "sa_validate_dev.h"

namespace sa {

namespace lat {
constexpr int DK = 576;
constexpr int DV = 512;
constexpr int NH = 64;
constexpr int KT = 32;                          // keys per tile
constexpr int NSTAGE = 4;                       // tiles in the LDS ring
constexpr int ROWB = DK * 2;                    // 1152 bytes per cache row
constexpr int TILE_BYTES = KT * ROWB;           // 36864
constexpr int HALF_ROWS = 16 * ROWB;            // byte offset of keys 16..31 of a tile
constexpr int THREADS = 256;
constexpr int WAVES = THREADS / 64;
constexpr int WAVE_LOADS = TILE_BYTES / 1024 / WAVES;  // 9 wave-wide 1 KB loads per tile
constexpr int KSTEPS = DK / 32;                 // 18 k-steps of S^T
constexpr int DVT = DV / 16;                    // 32 dv tiles of O^T
constexpr int KEYCAP = 2048;                    // keys staged in LDS at a time
constexpr int RING_BYTES = NSTAGE * TILE_BYTES;
constexpr size_t LDS_BYTES = (size_t)RING_BYTES + KEYCAP * 4 + 64;
constexpr float TAU_HARD = 100.0f;              // largest exponent taken against the reference
static_assert(NSTAGE >= 3, "the steady state keeps tiles t, t+1 and the refill in the ring");
}  // namespace lat

// LDS reads of step j of the interleaved S / PV loop: the two K reads of
// k-step j (j < 18) and the four transpose reads of dv tiles 2j, 2j + 1 (j < 16)
__host__ __device__ constexpr int step_reads(int j) {
  return (j < lat::KSTEPS ? 2 : 0) + (2 * j + 1 < lat::DVT ? 4 : 0);
}

// APPEND (with FUSED): the launch also appends the batch's cur_len current
// rows to the cache in place (rows past_len[b] ..) and writes present_len[b];
// every workgroup writes its batch's new rows itself before it gathers, so it
// reads its own writes whatever other workgroups do; with `reset` the
// launch's last workgroup replaces the error word instead of adding to it.
// BIAS: the additive attention bias (bf16, IndexShare `bias_at`) of each
// selected key is added to its scaled (and softcapped) score; its shape,
// right-aligned against [batch, 64, q_seq, cap], is bd0..bd3, each extent 1
// (broadcast) or the full one.
template <bool I64, bool FUSED, bool SOFTCAP, bool APPEND, bool BIAS>
__global__ void __launch_bounds__(lat::THREADS, 1)
latent_forward_kernel(const uint16_t* __restrict__ q, uint8_t* __restrict__ cache,
                      const void* __restrict__ idx, const int32_t* __restrict__ valid_len,
                      uint16_t* __restrict__ y,
                      float* __restrict__ part_o, float* __restrict__ part_ml, int64_t q_seq,
                      int64_t rows, int64_t cap, int64_t width, int splits, float scale,
                      float softcap, ErrorBlock* __restrict__ eb,
                      unsigned long long* __restrict__ row_key, unsigned* __restrict__ row_done,
                      const uint8_t* __restrict__ cur, const int32_t* __restrict__ past_len,
                      int32_t* __restrict__ present_len, int64_t cur_len, int reset,
                      const uint16_t* __restrict__ bias, int64_t bd0, int64_t bd1, int64_t bd2, int64_t bd3) {
  using namespace lat;
  extern __shared__ __attribute__((aligned(1024))) uint8_t lds_raw[];
  lds_u8* ring = (lds_u8*)lds_raw;
  int* keys_s = (int*)(lds_raw + RING_BYTES);
  int* misc = keys_s + KEYCAP;  // [1] restart request, [8 + w] wave w's key count
  unsigned long long* minkey_s = (unsigned long long*)(misc + 4);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar LDS bases
  const int g = lane >> 4;
  const int c16 = lane & 15;
  const int head = 16 * wave + c16;  // this lane's column of S^T and O^T

  int split;
  int64_t row;
  if (splits == 1) {
    row = rows - 1 - (int64_t)blockIdx.x;  // long (late causal) rows first
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
  const uint8_t* cache_b = cache + b * cap * ROWB;
  // this batch's cache rows as a buffer (raw, byte offsets; dword 3 holds the
  // 32-bit data format the gfx9 buffer loads expect)
  const __amdgpu_buffer_rsrc_t crsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)cache_b, (short)0, (int)(cap * ROWB), 0x00020000);

  // columns of the index row this workgroup owns
  const int wtiles = (int)((width + KT - 1) / KT);
  const int tps = (wtiles + splits - 1) / splits;
  const int c0 = (int)min((int64_t)split * tps * KT, width);
  const int c1 = (int)min((int64_t)c0 + (int64_t)tps * KT, width);

  // ---- per-lane LDS offsets within a tile (see the file comment)
  // K: row c16 (+16 for keys 16..31), chunk 4S + g stored at
  // (4S + g) ^ (c16 & 6) = 4 (S ^ f2) + (g ^ f1): one base per parity of S,
  // 64 S is an immediate.
  const int kf = c16 & 6;
  const int kbase = c16 * ROWB + ((g ^ (kf & 2)) << 4);
  const int kbase_e = kbase + ((kf >> 2) << 6);   // even S: 64 (S + f2)
  const int kbase_o = kbase - ((kf >> 2) << 6);   // odd S:  64 (S - f2)
  // V^T: lane 4 jj + qq of group g points at row 4g + jj, dv 16 dt + 4 qq,
  // i.e. chunk 2 dt + (qq >> 1) stored at 2 (dt ^ f') + (qq >> 1): one base
  // per dt mod 4, 32 (dt & ~3) is an immediate.
  int vbase[4];
  {
    const int jj = c16 >> 2, qq = c16 & 3;
    const int R = 4 * g + jj;
    const int fv = (R & 6) >> 1;
#pragma unroll
    for (int k = 0; k < 4; k++) vbase[k] = R * ROWB + ((k ^ fv) << 5) + ((qq >> 1) << 4) + ((qq & 1) << 3);
  }
  // gather: this wave's 9 loads per tile cover 1 KB blocks 9 wave + i of the
  // tile; lane l of block k fills tile slot 64 k + l = row R, chunk p, which
  // holds logical chunk p ^ (R & 6) of that row
  int ld_row[WAVE_LOADS], ld_off[WAVE_LOADS];
#pragma unroll
  for (int i = 0; i < WAVE_LOADS; i++) {
    const int sl = 64 * (WAVE_LOADS * wave + i) + lane;
    const int R = sl / 72;
    const int p = sl - 72 * R;
    ld_row[i] = R;
    ld_off[i] = (p ^ (R & 6)) << 4;
  }
  const float f = SOFTCAP ? kLog2eL : scale * kLog2eL;  // scores -> log2 units
  // the bias row of this lane's head (element 0 when the key extent is 1)
  const uint16_t* brow = bias;
  if constexpr (BIAS)
    brow = bias + (((bd0 == 1 ? 0 : b) * bd1 + (bd1 == 1 ? 0 : head)) * bd2 + (bd2 == 1 ? 0 : qi)) * bd3;
  const bool bkey = BIAS && bd3 != 1;

  // ---- softmax state. Each head's reference m_ref is its first tile's max
  // and then stays fixed: exp2(x - m_ref) of a later, larger score is a
  // larger power of two, which bf16 P and fp32 O / l hold as well (y = O / l
  // does not depend on the reference), so O is never rescaled. Only a score
  // more than 2^TAU_HARD above the reference could overflow; then the
  // workgroup restarts its key range with the largest maxima seen as
  // references. Each restart moves past at least one more tile.
  bf16x8_l qreg[KSTEPS];
  bool q_loaded = false;
  float m_floor = -INFINITY;
  f32x4_l o[DVT];
  float m_ref, l_run;
  unsigned long long mk = ~0ull;  // first violating column of this workgroup's columns
  int vhi = c0;                   // columns below vhi have been validated

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

  // APPEND: the batch's current rows go into the cache from a workgroup that
  // gathers one of them (before its gathers, and it waits for its stores, so
  // it reads them back from its own L2), and from one workgroup per batch at
  // its end (which also reports the append); no other workgroup touches them
  const bool duty = split == 0 && qi == 0;
  bool app_done = false;  // uniform
  auto append_rows = [&]() {
    if (app_ok) {
      const uint4* src = (const uint4*)(cur + b * cur_len * ROWB);
      uint4* dst = (uint4*)(cache + (b * cap + app_p) * ROWB);
      for (int u = tid; u < cur_len * (ROWB / 16); u += THREADS) dst[u] = src[u];
    }
    app_done = true;
  };

  for (;;) {
#pragma unroll
    for (int t = 0; t < DVT; t++) o[t] = (f32x4_l){0.f, 0.f, 0.f, 0.f};
    m_ref = m_floor;
    l_run = 0.0f;
    float m_seen = m_floor;
    bool restart = false;

    for (int st0 = c0; st0 < c1 && !restart; st0 += KEYCAP) {
      const int st1 = min(st0 + KEYCAP, c1);
      if (!staged) {
        __syncthreads();  // the previous stage's readers are done with keys_s / misc / the ring
        stage_keys(st0, st1);
      }
      staged = false;
      __syncthreads();
      const int kcount = max(max(misc[8], misc[9]), max(misc[10], misc[11]));
      const int ntile = (kcount + KT - 1) / KT;
      if constexpr (APPEND) {
        // this stage gathers appended rows: they are stored and have landed
        // before the gathers (the barrier waits for the stores)
        if ((misc[12] | misc[13] | misc[14] | misc[15]) != 0) {
          if (!app_done) append_rows();
          __syncthreads();
        }
      }
      if (ntile == 0) continue;  // uniform: only padding in these columns
      u32x4_l qraw[KSTEPS];

      // The gather of tile tt: this wave's nine 1 KB loads, buffer loads
      // from the batch's cache rows at byte offsets goff[i]. A slot past the
      // keys gets an offset beyond the buffer's size, for which the range
      // check returns zeros (its V rows must not hold garbage: P = 0 there,
      // and 0 * inf is NaN). goff is filled one LDS round trip ahead of the
      // issue; slot < ntile * KT <= KEYCAP keeps every lane's key read in
      // bounds, and keys fit in 24 bits (the host keeps cap * ROWB < 2^31).
      // A tile past the last one is "gathered" too (all offsets out of range:
      // zeros into a ring slot no later tile uses), so the issue is
      // unconditional; its key reads are clamped into the staged keys.
      uint32_t goff[WAVE_LOADS];
      int gkey[WAVE_LOADS];
      auto gather_keys = [&](int tt) {  // issue the key reads
        const int tk = tt < ntile ? tt : 0;
#pragma unroll
        for (int i = 0; i < WAVE_LOADS; i++) gkey[i] = keys_s[tk * KT + ld_row[i]];
      };
      auto gather_finish = [&](int tt) {  // the LDS round trip ends here
#pragma unroll
        for (int i = 0; i < WAVE_LOADS; i++) {
          goff[i] = tt * KT + ld_row[i] < kcount ? __umul24((uint32_t)gkey[i], (uint32_t)ROWB) + (uint32_t)ld_off[i]
                                                 : 0x80000000u;
          asm volatile("" : "+v"(goff[i]));
        }
      };
      auto gather_offsets = [&](int tt) {
        gather_keys(tt);
        gather_finish(tt);
      };
      auto gather_one = [&](int tt, int i) {
        lds_u8* dst = ring + (tt % NSTAGE) * TILE_BYTES + (WAVE_LOADS * wave + i) * 1024;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(crsrc, (__attribute__((address_space(3))) void*)dst, 16, goff[i], 0, 0, 0);
      };
      if (!q_loaded) {
        // Q^T of this wave's 16 heads, in flight with the first gathers (and
        // older than them, so the gathers' counted waits cover it); lane
        // (c16, g) holds dims 32 s + 8g .. +8 of its head
        const uint16_t* qp = q + ((b * NH + head) * q_seq + qi) * DK + 8 * g;
#pragma unroll
        for (int s = 0; s < KSTEPS; s++) qraw[s] = __builtin_bit_cast(u32x4_l, *(const uint4*)(qp + s * 32));
      }
      // prologue: tiles 0 .. NSTAGE-2 in flight
#pragma unroll
      for (int p = 0; p < NSTAGE - 1; p++) {
        gather_offsets(p);
#pragma unroll
        for (int i = 0; i < WAVE_LOADS; i++) gather_one(p, i);
      }
      gather_offsets(NSTAGE - 1);  // for the first refill

      if (!q_loaded) {
        // Q moves to the accumulation registers (the MFMA B operand reads it
        // there; the vector registers stay free for in-flight LDS reads)
#pragma unroll
        for (int s = 0; s < KSTEPS; s++) {
          u32x4_l raw = qraw[s];
          asm volatile("" : "+a"(raw));
          qreg[s] = __builtin_bit_cast(bf16x8_l, raw);
        }
        q_loaded = true;
      }

      // ---- the pieces of a tile. S^T[key, head] for key halves kh (rows
      // 16 kh + c16) with two accumulator chains per half (even / odd
      // k-steps); O^T[dv, head] += V^T[dv, key] . P^T[key, head].
      auto tile_addr = [&](int tt) { return (uint32_t)(uintptr_t)(ring + (tt % NSTAGE) * TILE_BYTES); };
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
      u32x4_l kr0[KSTEPS], kr1[KSTEPS];
      s16x4_l vr0[DVT], vr1[DVT];
      f32x4_l sa[2][2];
      auto kread = [&](auto sc) {
        constexpr int S = decltype(sc)::value;
        const uint32_t a = (S & 1) ? ka_o : ka_e;
        kr0[S] = ds_read_b128_at<64 * S>(a);
        kr1[S] = ds_read_b128_at<64 * S + HALF_ROWS>(a);
      };
      auto kmfma = [&](auto sc) {
        constexpr int S = decltype(sc)::value;
        const bf16x8_l a0 = __builtin_bit_cast(bf16x8_l, kr0[S]);
        const bf16x8_l a1 = __builtin_bit_cast(bf16x8_l, kr1[S]);
        sa[0][S & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, qreg[S], sa[0][S & 1], 0, 0, 0);
        sa[1][S & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, qreg[S], sa[1][S & 1], 0, 0, 0);
      };
      auto vread = [&](auto dc) {
        constexpr int DT = decltype(dc)::value;
        vr0[DT] = ds_read_tr16_at<32 * (DT & ~3)>(va[DT & 3]);
        vr1[DT] = ds_read_tr16_at<32 * (DT & ~3) + HALF_ROWS>(va[DT & 3]);
      };
      auto vmfma = [&](auto dc, const bf16x8_l& pb) {
        constexpr int DT = decltype(dc)::value;
        const s16x4_l a8[2] = {vr0[DT], vr1[DT]};
        o[DT] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_l, a8), pb, o[DT], 0, 0, 0);
      };
      auto zero_s = [&]() {
#pragma unroll
        for (int kh = 0; kh < 2; kh++) sa[kh][0] = sa[kh][1] = (f32x4_l){0.f, 0.f, 0.f, 0.f};
      };
      // BIAS: the lane's eight bias values of tile tt (its head, the keys of
      // slots 4g + i and 16 + 4g + i), loaded a tile ahead of their softmax as
      // ordinary loads (the compiler places the wait at the use; they are
      // older than the refill's gathers, so the counted gather waits cover
      // them too). Staged keys are already clamped into the cache.
      uint16_t bv[8];
      auto bias_load = [&](int tt) {
        if constexpr (BIAS) {
#pragma unroll
          for (int i = 0; i < 8; i++) {
            const int slot = tt * KT + 4 * g + (i < 4 ? i : 12 + i);
            const int key = slot < kcount ? keys_s[slot] : 0;
            bv[i] = brow[bkey ? key : 0];
          }
        }
      };
      // softmax of tile tt from sa; lane holds keys 4g + r and 16 + 4g + r of
      // its head. Scores are taken to log2 units with one multiply by f.
      // Returns P^T.
      auto softmax = [&](int tt) {
        const f32x4_l s0 = sa[0][0] + sa[0][1], s1 = sa[1][0] + sa[1][1];
        float x[8];
#pragma unroll
        for (int i = 0; i < 4; i++) {
          x[i] = s0[i];
          x[4 + i] = s1[i];
        }
        if constexpr (SOFTCAP) {
#pragma unroll
          for (int i = 0; i < 8; i++) x[i] = softcap * tanhf(x[i] * scale / softcap);
        }
        if constexpr (BIAS) {
          // the bias joins the scaled (and softcapped) score, then log2 units
#pragma unroll
          for (int i = 0; i < 8; i++) x[i] = ((SOFTCAP ? x[i] : x[i] * scale) + bf16_to_f32(bv[i])) * kLog2eL;
        }
        if ((tt + 1) * KT > kcount) {  // uniform: only the last tile has empty slots
          const int slot_base = tt * KT + 4 * g;
#pragma unroll
          for (int i = 0; i < 8; i++)
            if (slot_base + (i < 4 ? i : 12 + i) >= kcount) x[i] = -INFINITY;
        }
        // scores in log2 units, rounded once: the maximum then gives exp2(0)
        // exactly (an FMA against a rounded maximum can overflow for huge scores)
        if constexpr (!BIAS) {
#pragma unroll
          for (int i = 0; i < 8; i++) x[i] *= f;
        }
        float tmax = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])), fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
        tmax = max_x32(max_x16(tmax));
        m_seen = fmaxf(m_seen, tmax);
        if (m_ref == -INFINITY) m_ref = tmax;  // first tile of this head: O and l are still 0
        // a score more than 2^TAU_HARD above the reference: this pass is
        // discarded and redone (its exp2 may overflow)
        if (tmax > m_ref + TAU_HARD) misc[1] = 1;  // benign race: every writer stores 1
        const float nm = m_ref == -INFINITY ? 0.0f : -m_ref;
        float p[8];
#pragma unroll
        for (int i = 0; i < 8; i++) p[i] = __builtin_amdgcn_exp2f(x[i] + nm);
        const float psum = ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
        l_run += sum_x32(sum_x16(psum));
        const u32x4_l pw = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                            pack_bf16x2(p[6], p[7])};
        return __builtin_bit_cast(bf16x8_l, pw);
      };

      // ---- tile 0: S alone, the reads KD k-steps ahead of their MFMAs
      // (tiles 1 .. NSTAGE-2 may stay in flight)
      bias_load(0);
      wait_vm<(NSTAGE - 2) * WAVE_LOADS>();
      lds_barrier();
      set_k(0);
      zero_s();
      {
        constexpr int KD = 5;
        static_for<KD>(kread);
        static_for<KSTEPS>([&](auto sc) {
          constexpr int S = decltype(sc)::value;
          if constexpr (S + KD < KSTEPS) kread(std::integral_constant<int, S + KD>{});
          constexpr int LATER = (KD < KSTEPS - 1 - S ? KD : KSTEPS - 1 - S);
          lgkm_wait_tied<2 * LATER>(kr0[S], kr1[S]);
          kmfma(sc);
          __builtin_amdgcn_sched_barrier(0);
        });
      }
      bf16x8_l pb = softmax(0);

      // ---- steady state: S of tile t+1 interleaved with PV of tile t, one
      // k-step and two dv tiles per step (4 MFMAs and 4 KB of LDS reads per
      // wave), the reads PL steps ahead; then the softmax of tile t+1
      for (int t = 0; t + 1 < ntile; t++) {
        wait_vm<(NSTAGE - 3) * WAVE_LOADS>();  // tile t+1 has landed for this wave (later ones may stay in flight)
        lds_barrier();          // and for everyone; tile t-1's slot is free
        const int tn = t + NSTAGE - 1;  // refills tile t-1's slot; offsets read last iteration
        gather_keys(tn + 1);  // in order ahead of the step reads; consumed after the softmax
        bias_load(t + 1);
        set_k(t + 1);
        set_v(t);
        zero_s();
        constexpr int PL = 2;
        auto sread = [&](auto jc) {
          constexpr int J = decltype(jc)::value;
          if constexpr (J < KSTEPS) kread(jc);
          if constexpr (2 * J + 1 < DVT) {
            vread(std::integral_constant<int, 2 * J>{});
            vread(std::integral_constant<int, 2 * J + 1>{});
          }
        };
        static_for<PL>(sread);
        static_for<KSTEPS>([&](auto jc) {
          constexpr int J = decltype(jc)::value;
          if constexpr (J + PL < KSTEPS) sread(std::integral_constant<int, J + PL>{});
          if constexpr (J < WAVE_LOADS) gather_one(tn, J);  // one 1 KB load per step
          // LDS reads issued after step J's: those of steps J+1 .. J+PL
          constexpr int LATER = step_reads(J + 1) * (J + 1 < KSTEPS) + step_reads(J + 2) * (PL > 1 && J + 2 < KSTEPS);
          if constexpr (2 * J + 1 < DVT) {
            lgkm_wait6<LATER>(kr0[J], kr1[J], vr0[2 * J], vr1[2 * J], vr0[2 * J + 1], vr1[2 * J + 1]);
            kmfma(jc);
            vmfma(std::integral_constant<int, 2 * J>{}, pb);
            vmfma(std::integral_constant<int, 2 * J + 1>{}, pb);
          } else {
            lgkm_wait_tied<LATER>(kr0[J], kr1[J]);
            kmfma(jc);
          }
          __builtin_amdgcn_sched_barrier(0);
        });
        pb = softmax(t + 1);
        gather_finish(tn + 1);
      }

      // ---- the last tile's PV alone, the reads VD tiles ahead
      set_v(ntile - 1);
      {
        constexpr int VD = 8;
        static_for<VD>(vread);
        static_for<DVT>([&](auto dc) {
          constexpr int DT = decltype(dc)::value;
          constexpr int AHEAD = (VD - 1 < DVT - 1 - DT ? VD - 1 : DVT - 1 - DT);
          lgkm_wait_tied<2 * AHEAD>(vr0[DT], vr1[DT]);
          vmfma(dc, pb);
          if constexpr (DT + VD < DVT) vread(std::integral_constant<int, DT + VD>{});
          __builtin_amdgcn_sched_barrier(0);
        });
      }
      // a restart request is acted on once the stage's tiles are done (only
      // inputs whose scores jump by more than 2^TAU_HARD ever raise one)
      __syncthreads();
      restart = misc[1] != 0;
    }
    if (!restart) break;
    m_floor = m_seen;
  }

  // ---- the workgroup's first violation (fused validation)
  if constexpr (FUSED) {
    if (c0 == 0 && tid == 0 && width > 0 && load_index<I64>(idx, ibase) == -1)
      mk = min(mk, (unsigned long long)(row * (width + 1) + width));  // all -1, unless a column fails
    if (tid == 0) *minkey_s = ~0ull;
    __syncthreads();
    if (mk != ~0ull) atomicMin(minkey_s, mk);
  }

  // ---- epilogue: lane holds O^T[16 dt + 4g + r][16 wave + c16]. Every
  // head's output is normalised by its row sum and rounded to bf16 into LDS
  // rows (the ring is free), then each lane stores 16 contiguous bytes of one
  // head's row: to Y when the keys are not split, else to the split's partial
  // (with its fp32 (reference, row sum) pairs, merged by the bf16 merge
  // kernel), written through the L2 so the launch's end has no dirty
  // partials to write back.
  {
    constexpr int YROW = 1024 + 16;  // padded: the 16 heads of one write hit distinct banks
    __syncthreads();
    const float inv = l_run > 0.0f ? 1.0f / l_run : 0.0f;
    lds_u8* yl = ring + head * YROW + 8 * g;
#pragma unroll
    for (int dt = 0; dt < DVT; dt++) {
      const uint32_t lo = pack_bf16x2(o[dt][0] * inv, o[dt][1] * inv);
      const uint32_t hi = pack_bf16x2(o[dt][2] * inv, o[dt][3] * inv);
      *(__attribute__((address_space(3))) u32x2_l*)(yl + 32 * dt) = (u32x2_l){lo, hi};
    }
    if (splits > 1 && g == 0) {
      const __amdgpu_buffer_rsrc_t mrsrc = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(part_ml + (row * splits + split) * NH * 2), (short)0, NH * 8, 0x00020000);
      __builtin_amdgcn_raw_buffer_store_b64((u32x2_l){__float_as_uint(m_ref), __float_as_uint(l_run)}, mrsrc,
                                            head * 8, 0, kWriteThrough);
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

bool latent_supported(const sa_config& cfg, int64_t index_heads) {
  return mla_supported(cfg, index_heads) && cfg.cache_format == SA_CACHE_DENSE &&
         cfg.max_cache_len <= (int64_t)(0x7fffffffLL / lat::ROWB);
}

static bool g_latent_attr[20] = {};

sa_status launch_forward_latent(sparse_attn_ctx* c, const FwdArgs& a, int splits, bool fused, const AppendArgs* app) {
  using namespace lat;
  const int64_t rows = a.batch * a.q_seq;
  if (rows <= 0) return SA_OK;
  if (splits > 1 && rows * splits > c->partial_rows)
    return set_error(c, SA_E_STATE, "forward: split-K partials exceed the context's buffers");
  if (rows > c->rows_cap) return set_error(c, SA_E_STATE, "forward: more rows than the context holds");
  const int64_t wgs = rows * splits;
  if (wgs > 0x7fffffffLL) return set_error(c, SA_E_SHAPE, "forward: too many rows for one launch");
  const bool cap_on = a.softcap != 0.0f;
  if (app && (!fused || app->cur_len < 0 || app->cur_len > kFusedAppendRows))
    return set_error(c, SA_E_STATE, "forward: in-launch append needs fused validation and at most 8 rows");
  const bool bias_on = a.bias != nullptr;
  if (app && bias_on) return set_error(c, SA_E_STATE, "forward: in-launch append takes no bias");
  const int variant = app ? 8 + (a.idx64 ? 1 : 0) + (cap_on ? 2 : 0)
                          : (bias_on ? 12 : 0) + (a.idx64 ? 1 : 0) + (fused ? 2 : 0) + (cap_on ? 4 : 0);
  const void* fns[20] = {(const void*)latent_forward_kernel<false, false, false, false, false>,
                         (const void*)latent_forward_kernel<true, false, false, false, false>,
                         (const void*)latent_forward_kernel<false, true, false, false, false>,
                         (const void*)latent_forward_kernel<true, true, false, false, false>,
                         (const void*)latent_forward_kernel<false, false, true, false, false>,
                         (const void*)latent_forward_kernel<true, false, true, false, false>,
                         (const void*)latent_forward_kernel<false, true, true, false, false>,
                         (const void*)latent_forward_kernel<true, true, true, false, false>,
                         (const void*)latent_forward_kernel<false, true, false, true, false>,
                         (const void*)latent_forward_kernel<true, true, false, true, false>,
                         (const void*)latent_forward_kernel<false, true, true, true, false>,
                         (const void*)latent_forward_kernel<true, true, true, true, false>,
                         (const void*)latent_forward_kernel<false, false, false, false, true>,
                         (const void*)latent_forward_kernel<true, false, false, false, true>,
                         (const void*)latent_forward_kernel<false, true, false, false, true>,
                         (const void*)latent_forward_kernel<true, true, false, false, true>,
                         (const void*)latent_forward_kernel<false, false, true, false, true>,
                         (const void*)latent_forward_kernel<true, false, true, false, true>,
                         (const void*)latent_forward_kernel<false, true, true, false, true>,
                         (const void*)latent_forward_kernel<true, true, true, false, true>};
  if (!g_latent_attr[variant]) {
    hipError_t e = hipFuncSetAttribute(fns[variant], hipFuncAttributeMaxDynamicSharedMemorySize, (int)LDS_BYTES);
    if (e != hipSuccess) return check_hip(c, e, "forward (latent) LDS attribute");
    g_latent_attr[variant] = true;
  }
  const dim3 grid((unsigned)wgs), block(THREADS);
  const ProfEvents pe = prof_next(c);
  const uint8_t* cur = app ? (const uint8_t*)app->cur : nullptr;
  const int32_t* plen = app ? app->past_len : nullptr;
  int32_t* prlen = app ? app->present_len : nullptr;
  const int64_t clen = app ? app->cur_len : 0;
  const int reset = app ? app->reset : 0;
#define SA_LAT(I, F, C, A, B)                                                                         \
  SA_MAIN_LAUNCH(pe, (latent_forward_kernel<I, F, C, A, B>), grid, block, LDS_BYTES, c->stream,       \
                     (const uint16_t*)a.q, (uint8_t*)a.k, a.idx, a.valid_len, (uint16_t*)a.y,         \
                     c->partial_o, c->partial_ml, a.q_seq, rows, a.cap, a.width, splits, a.scale,     \
                     a.softcap, c->err, c->row_key, c->row_done, cur, plen, prlen, clen, reset,       \
                     (const uint16_t*)a.bias, a.bd[0], a.bd[1], a.bd[2], a.bd[3])
  switch (variant) {
    case 0: SA_LAT(false, false, false, false, false); break;
    case 1: SA_LAT(true, false, false, false, false); break;
    case 2: SA_LAT(false, true, false, false, false); break;
    case 3: SA_LAT(true, true, false, false, false); break;
    case 4: SA_LAT(false, false, true, false, false); break;
    case 5: SA_LAT(true, false, true, false, false); break;
    case 6: SA_LAT(false, true, true, false, false); break;
    case 7: SA_LAT(true, true, true, false, false); break;
    case 8: SA_LAT(false, true, false, true, false); break;
    case 9: SA_LAT(true, true, false, true, false); break;
    case 10: SA_LAT(false, true, true, true, false); break;
    case 11: SA_LAT(true, true, true, true, false); break;
    case 12: SA_LAT(false, false, false, false, true); break;
    case 13: SA_LAT(true, false, false, false, true); break;
    case 14: SA_LAT(false, true, false, false, true); break;
    case 15: SA_LAT(true, true, false, false, true); break;
    case 16: SA_LAT(false, false, true, false, true); break;
    case 17: SA_LAT(true, false, true, false, true); break;
    case 18: SA_LAT(false, true, true, false, true); break;
    default: SA_LAT(true, true, true, false, true); break;
  }
#undef SA_LAT
  sa_status s = check_hip(c, hipGetLastError(), "forward (latent)");
  if (s != SA_OK || splits == 1) return s;
  return launch_latent_merge(c, a, rows, splits, fused, app);
}

}  // namespace sa
