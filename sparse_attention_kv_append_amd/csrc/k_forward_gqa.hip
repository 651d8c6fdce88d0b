// Grouped-query selected-token attention on the gfx950 matrix cores, with the
// gathered key tile shared by several query rows.
//
// Semantics are IndexShare's `index_share_row` for separate K and V caches,
// bf16 rows of 128 dims, and one index list per (batch, query) shared by all
// query heads (the standard Attention page's softcap applies when set). In a
// grouped-query layout the `group` heads of one kv head read the same K and V
// rows, so a workgroup takes one (batch, kv head) and R = min(32, 128 / group)
// consecutive queries: up to 128 (query, head) rows, 16 per wave (eight
// waves, two per SIMD, so one wave's softmax overlaps the other's MFMAs). Walking the index rows 32 columns at a time, a tile is
// shared when every one of the R rows holds, in each column, either the same
// key or padding (-1): then the tile's 32 K and V rows are gathered once and
// S^T = K_tile . Q^T and O^T += V_tile^T . P^T run for all the rows on
// v_mfma_f32_16x16x32_bf16. Dense causal selections - the degenerate case where every
// query selects a prefix of the keys - share every tile. A tile that is not
// shared is redone row by row (R small passes, each gathering that row's own
// keys and updating only its rows), so any valid index rows give IndexShare's
// result, only more slowly.
//
// The optional additive bias (IndexShare `bias_at`, read at each selected
// key's cache position, after the softcap) is loaded per lane for its eight
// (row, column) scores of a tile, one iteration before that tile's softmax.
//
// Per row the softmax is the usual online form (running maximum and sum in
// log2 units, the accumulators rescaled when the maximum grows). A row's
// key count n is its number of entries before the first -1; a workgroup stops
// at the first tile in which every one of its rows is padding.
//
// Data movement per 32-column tile: the R index rows' 32 columns are copied
// into LDS six tiles ahead (direct-to-LDS, one dword per lane); four tiles
// ahead every thread folds its share of them into per-column partial maxima
// and minima (and the first -1 of each row); three tiles ahead each wave
// combines the partials into the tile's keys and flags and issues the tile's
// K and V gathers (direct-to-LDS, 16 bytes per lane) into a four-tile ring.
// LDS rows of 256 bytes are stored with 16-byte chunk c of row R at chunk
// c ^ (R & 15) for K (the K reads of 16 rows x one chunk hit 16 distinct
// bank groups per pass) and c ^ 2 (R & 7) for V (the transposing V reads of
// 8 rows x 32 bytes hit 64 distinct banks).
#include "sa_mfma_dev.h"
#include "sa_validate_dev.h"

namespace sa {

namespace gq {
constexpr int D = 128;                           // head dim of Q, K and V
constexpr int ROWB = D * 2;                      // 256 bytes per cache row
constexpr int KT = 32;                           // columns (keys) per tile
constexpr int MROWS = 128;                       // (query, head) rows per workgroup
constexpr int RB = 1;                            // 16-row blocks per wave
constexpr int WAVES = MROWS / (16 * RB);         // 8 waves, two per SIMD
constexpr int THREADS = 64 * WAVES;
constexpr int RMAX = 32;                         // queries per workgroup at most
constexpr int KSTEPS = D / 32;                   // 4 k-steps of S^T
constexpr int DVT = D / 16;                      // 8 dv tiles of O^T
constexpr int NSTAGE = 4;                        // K/V tiles in the ring
constexpr int KV_TILE = 2 * KT * ROWB;           // K rows then V rows: 16 KB
constexpr int RING_BYTES = NSTAGE * KV_TILE;
constexpr int SPARE_OFF = RING_BYTES;            // one more K/V tile for row-by-row passes
constexpr int GLOADS = KV_TILE / 1024 / WAVES;   // 4 one-KB K/V loads per wave and tile
constexpr int IDX_SLOTS = 4;                     // index tiles in flight or being folded
template <bool I64> constexpr int idx_tile_bytes() { return RMAX * KT * (I64 ? 8 : 4); }
template <bool I64> constexpr int ILOADS = idx_tile_bytes<I64>() / 256 / WAVES;  // dword loads per wave
constexpr int IDX_OFF = SPARE_OFF + KV_TILE;
template <bool I64> constexpr int part_off() { return IDX_OFF + IDX_SLOTS * idx_tile_bytes<I64>(); }
constexpr int PART_BYTES = 2 * KT * WAVES * 4;   // per slot: max, min [32 columns][wave] (int32)
template <bool I64> constexpr int nrow_off() { return part_off<I64>() + 2 * PART_BYTES; }
template <bool I64> constexpr int flag_off() { return nrow_off<I64>() + RMAX * 4; }
template <bool I64> constexpr int rmin_off() { return flag_off<I64>() + WAVES * 8 * 4; }
template <bool I64> constexpr size_t lds_bytes() { return (size_t)rmin_off<I64>() + RMAX * 8; }
static_assert(flag_off<false>() % 8 == 0 && flag_off<true>() % 8 == 0, "8-byte row minima");
}  // namespace gq

// LDS reads of step j of the interleaved S / PV loop: the K read of (k-step
// j >> 1, key half j & 1) and the two transposing V reads of dv tile j
__host__ __device__ constexpr int gqa_step_reads(int j) { return j < 8 ? 3 : 0; }

// FUSED: the launch validates its index rows (IndexShare host-validator
// rules, each column against its left neighbour): the kv heads of a
// (batch, query block, split) share its columns out, every workgroup counts
// one arrival per query row it covers, and the last arrival of a row records
// the row's first violation, then counts toward the launch's last-arrival
// record of the error block (with `reset` that record replaces the word).
// APPEND (with FUSED): the launch also appends the current K/V rows in place
// (rows past_len[b] ..): every workgroup writes its (batch, kv head)'s rows
// itself and waits for the stores before any gather, so it reads its own
// writes; the workgroup of kv head 0, query block 0 and split 0 writes
// present_len[b] (or flags a row count that does not fit the capacity).
template <bool I64, bool SOFTCAP, bool BIAS, bool FUSED, bool APPEND>
__global__ void __launch_bounds__(gq::THREADS, 1)
gqa_forward_kernel(const uint16_t* __restrict__ q, uint8_t* __restrict__ kc, uint8_t* __restrict__ vc,
                   const void* __restrict__ idx, const int32_t* __restrict__ valid_len, uint16_t* __restrict__ y,
                   int64_t batch, int64_t hkv, int64_t q_seq, int64_t cap, int64_t width, int group, int nqb,
                   float scale, float softcap, const uint16_t* __restrict__ bias, int64_t bd0, int64_t bd1,
                   int64_t bd2, int64_t bd3, int splits, float* __restrict__ part_o,
                   float* __restrict__ part_ml, ErrorBlock* __restrict__ eb,
                   unsigned long long* __restrict__ row_key, unsigned* __restrict__ row_done,
                   const uint8_t* __restrict__ cur_k, const uint8_t* __restrict__ cur_v,
                   const int32_t* __restrict__ past_len, int32_t* __restrict__ present_len, int64_t cur_len,
                   int reset) {
  static_assert(FUSED || !APPEND, "the in-launch append reports through the fused error record");
  static_assert(gq::RB == 1, "the bias prefetch holds one row block per wave");
  using namespace gq;
  constexpr int ITB = idx_tile_bytes<I64>();
  constexpr int IL = ILOADS<I64>;
  constexpr int ISZ = I64 ? 8 : 4;
  extern __shared__ __attribute__((aligned(1024))) uint8_t lds_raw[];
  lds_u8* lds = (lds_u8*)lds_raw;
  int* part = (int*)(lds_raw + part_off<I64>());          // [2 slots][max | min][32 columns][wave]
  int* n_s = (int*)(lds_raw + nrow_off<I64>());          // [RMAX] first -1 column of each query row
  int* flag_s = (int*)(lds_raw + flag_off<I64>());       // [wave][8] tile flags, per wave
  // [RMAX] fused validation: each query row's smallest failing key
  unsigned long long* rmin = (unsigned long long*)(lds_raw + rmin_off<I64>());

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4;
  const int c16 = lane & 15;

  // ---- workgroup -> (batch, kv head, query block); the query blocks of one
  // (batch, kv head) share blockIdx % 8 (one XCD, one L2)
  const int xcd = (int)(blockIdx.x & 7u);
  const int rest0 = (int)(blockIdx.x >> 3);
  const int sp = rest0 % splits;  // split-KV: this workgroup's share of the index columns
  const int rest = rest0 / splits;
  const int qb = rest % nqb;
  const int64_t pr = (int64_t)(rest / nqb) * 8 + xcd;  // (batch, kv head) pair
  if (pr >= batch * hkv) return;                       // grid padding (uniform)
  const int64_t b = pr / hkv;
  const int64_t kvh = pr - b * hkv;
  const int R = group >= MROWS ? 1 : min(RMAX, MROWS / group);  // queries of this workgroup
  const int64_t q0 = (int64_t)qb * R;
  const int rlive = (int)min((int64_t)R, q_seq - q0);  // queries that exist
  const int hq = (int)(hkv * group);
  int64_t bound = valid_len ? (int64_t)valid_len[b] : cap;
  int64_t app_p = 0;
  bool app_ok = false;
  if constexpr (APPEND) {
    app_p = (int64_t)past_len[b];
    app_ok = app_p >= 0 && app_p + cur_len <= cap;  // else nothing is appended and the word says so
    bound = app_p + cur_len;
  }
  bound = bound < 0 ? 0 : (bound > cap ? cap : bound);
  // tiles [xo, xo + ntile_w) of the index rows; the kernel numbers them from 0
  const int ntile_all = (int)((width + KT - 1) / KT);
  const int tps = (ntile_all + splits - 1) / splits;
  const int xo = min(ntile_all, sp * tps);
  const int ntile_w = min(ntile_all, xo + tps) - xo;

  // this lane's rows: block rb holds row m = 16 (RB wave + rb) + c16
  int row_q[RB], row_h[RB];
  bool row_on[RB];
#pragma unroll
  for (int rb = 0; rb < RB; rb++) {
    const int m = 16 * (RB * wave + rb) + c16;
    const int r = m / group;
    row_q[rb] = r;
    row_h[rb] = (int)(kvh * group) + (m - r * group);
    row_on[rb] = m < R * group && r < rlive;
  }
  // live rows are a prefix of the workgroup's rows: a wave with none (decode
  // leaves most of the 128 rows empty) only gathers, folds and syncs
  const bool wlive = 16 * RB * wave < rlive * group;

  // ---- the optional bias (IndexShare `bias_at`): each row's element at key
  // 0 (an extent of 1 broadcasts); rows that do not exist read element 0
  const uint16_t* brow[RB];
  const bool bkey = bd3 != 1;
#pragma unroll
  for (int rb = 0; rb < RB; rb++) {
    int64_t off = 0;
    if (BIAS && row_on[rb])
      off = (((bd0 == 1 ? 0 : b) * bd1 + (bd1 == 1 ? 0 : row_h[rb])) * bd2 + (bd2 == 1 ? 0 : q0 + row_q[rb])) * bd3;
    brow[rb] = bias + off;
  }

  // ---- buffers: this (batch, kv head)'s K and V rows; the index rows of the
  // workgroup's queries (reads past the live queries return zeros)
  const int64_t kv_base = (b * hkv + kvh) * cap * ROWB;
  if constexpr (APPEND) {
    // this (batch, kv head)'s current rows, written before any gather and
    // waited for (every workgroup that may read them writes them itself)
    if (app_ok) {
      const int64_t n16 = cur_len * (ROWB / 16);
      const uint4* sk = (const uint4*)(cur_k + pr * cur_len * ROWB);
      const uint4* sv = (const uint4*)(cur_v + pr * cur_len * ROWB);
      uint4* dk = (uint4*)(kc + kv_base + app_p * ROWB);
      uint4* dv = (uint4*)(vc + kv_base + app_p * ROWB);
      for (int64_t u = tid; u < n16; u += THREADS) {
        dk[u] = sk[u];
        dv[u] = sv[u];
      }
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's stores have completed
    __syncthreads();
  }
  const __amdgpu_buffer_rsrc_t krsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)(kc + kv_base), (short)0, (int)(cap * ROWB), 0x00020000);
  const __amdgpu_buffer_rsrc_t vrsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)(vc + kv_base), (short)0, (int)(cap * ROWB), 0x00020000);
  const uint8_t* ibase = (const uint8_t*)idx + (b * q_seq + q0) * width * ISZ;
  const __amdgpu_buffer_rsrc_t irsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)ibase, (short)0, (int)min((int64_t)0x7fffffff, (int64_t)rlive * width * ISZ), 0x00020000);

  for (int i = tid; i < RMAX; i += THREADS) {
    n_s[i] = 0x7fffffff;
    if constexpr (FUSED) rmin[i] = ~0ull;
  }
  const int64_t irow0 = b * q_seq + q0;  // index row of query q0 (one index head)
  constexpr int FR = RMAX / (THREADS / 32);  // rows each folding thread visits
  // FUSED: the index columns this workgroup validates at its end (kv head h
  // takes the h-th slice of the block's columns, for every query row); when
  // they fit two per thread they are loaded here, in flight with the rest of
  // the launch, so the check at the end does not wait on memory
  int64_t vmb = 0, vme = 0;
  int64_t pv[2] = {-1, -1}, pu[2] = {0, 0};
  bool pre = false;
  if constexpr (FUSED) {
    const int64_t cb = (int64_t)xo * KT;
    const int64_t ce = min((int64_t)(xo + ntile_w) * KT, width);
    const int64_t ncols = ce > cb ? ce - cb : 0;
    const int64_t chunk = (ncols + hkv - 1) / hkv;
    vmb = cb + min(ncols, kvh * chunk);
    vme = min(cb + ncols, vmb + chunk);
    const int64_t mc = vme - vmb;
    pre = mc > 0 && (int64_t)rlive * mc <= 2 * THREADS;  // uniform
    if (pre) {
#pragma unroll
      for (int k = 0; k < 2; k++) {
        const int64_t e = tid + (int64_t)THREADS * k;
        if (e < (int64_t)rlive * mc) {
          const int64_t r = e / mc, c = vmb + (e - r * mc);
          const int64_t off = (irow0 + r) * width + c;
          pv[k] = load_index<I64>(idx, off);
          pu[k] = c > 0 ? load_index<I64>(idx, off - 1) : 0;
        }
      }
    }
  }

  // ---- index tiles: lane l of load i of wave w copies dword d = 64 (IL w + i) + l
  // of the tile's [RMAX][32] block (row r = d / (32 ISZ / 4), column j)
  auto issue_idx = [&](int x) {
    lds_u8* slot = lds + IDX_OFF + (x % IDX_SLOTS) * ITB;
#pragma unroll
    for (int i = 0; i < IL; i++) {
      const int d = 64 * (IL * wave + i) + lane;
      const int r = d / (KT * ISZ / 4);
      const int wj = d - r * (KT * ISZ / 4);  // dword within the row's 32 columns
      const int64_t col = (int64_t)(xo + x) * KT + wj / (ISZ / 4);
      uint32_t off = 0x80000000u;  // past the buffer: zeros
      if (r < rlive && col < width) off = (uint32_t)(((int64_t)r * width + col) * ISZ + (wj % (ISZ / 4)) * 4);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(irsrc, (__attribute__((address_space(3))) void*)(slot + 256 * (IL * wave + i)),
                                              4, off, 0, 0, 0);
    }
  };
  auto idx_at = [&](const lds_u8* slot, int r, int j) -> int64_t {
    if constexpr (I64) return *(const __attribute__((address_space(3))) int64_t*)(slot + (r * KT + j) * 8);
    else return *(const __attribute__((address_space(3))) int32_t*)(slot + (r * KT + j) * 4);
  };
  // fold index tile x: thread (column j = tid & 31, group tg = tid >> 5)
  // over rows tg, tg + THREADS / 32, ...: maximum and minimum over the
  // non-padding entries (values taken as int32: below -1 -> -2, from the
  // cache length up -> the cache length, which keeps every valid row exact),
  // and the first -1 of each row; the two halves of a wave are merged, and
  // lanes 0..31 store the wave's partials
  auto fold = [&](int x) {
    const lds_u8* slot = lds + IDX_OFF + (x % IDX_SLOTS) * ITB;
    const int j = tid & 31, tg = tid >> 5;
    const int64_t col = (int64_t)(xo + x) * KT + j;
    int mx = -1, mn = 0x7fffffff;
#pragma unroll
    for (int k = 0; k < FR; k++) {
      const int r = tg + (THREADS / 32) * k;
      if (r < rlive) {
        const int64_t v = col < width ? idx_at(slot, r, j) : -1;
        const int v32 = v == -1 ? -1 : (v < -1 ? -2 : (v >= bound ? (int)bound : (int)v));
        mx = max(mx, v32);
        if (v32 != -1) mn = min(mn, v32);
        else ds_min_i32_at((uint32_t)(uintptr_t)(lds + nrow_off<I64>()) + 4u * (uint32_t)r, (int)col);
      }
    }
    {
      const auto sx = __builtin_amdgcn_permlane32_swap((unsigned)mx, (unsigned)mx, false, false);
      const auto sn = __builtin_amdgcn_permlane32_swap((unsigned)mn, (unsigned)mn, false, false);
      mx = max((int)sx[0], (int)sx[1]);
      mn = min((int)sn[0], (int)sn[1]);
    }
    int* pp = part + (x & 1) * (2 * KT * WAVES);
    if (lane < 32) {
      pp[j * WAVES + wave] = mx;
      pp[KT * WAVES + j * WAVES + wave] = mn;
    }
  };

  // ---- K/V gather of a tile: lane l of load i of wave w fills 16-byte
  // chunk 64 (4 w + i) + l of the slot: waves 0, 1 the K rows, waves 2, 3 the V rows
  int ld_row[GLOADS], ld_off[GLOADS];
  const bool kwave = wave < WAVES / 2;  // the first half of the waves loads K rows
#pragma unroll
  for (int i = 0; i < GLOADS; i++) {
    const int ci = (64 * (GLOADS * wave + i) + lane) & 511;
    const int Rr = ci >> 4, pc = ci & 15;
    ld_row[i] = Rr;
    ld_off[i] = (kwave ? (pc ^ (Rr & 15)) : (pc ^ (2 * (Rr & 7)))) << 4;
  }
  const __amdgpu_buffer_rsrc_t grsrc = kwave ? krsrc : vrsrc;
  uint32_t goff[GLOADS];
  auto gather_issue = [&](lds_u8* slot) {
#pragma unroll
    for (int i = 0; i < GLOADS; i++)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(grsrc, (__attribute__((address_space(3))) void*)(slot + 1024 * (GLOADS * wave + i)),
                                              16, goff[i], 0, 0, 0);
  };
  // gather offsets from each lane's column key (column lane & 31); keys
  // outside the cache read zeros
  auto key_offsets = [&](int64_t kfor_lane) {
    const int kc32 = kfor_lane >= 0 && kfor_lane < bound ? (int)kfor_lane : -1;
#pragma unroll
    for (int i = 0; i < GLOADS; i++) {
      const int kk = __shfl(kc32, ld_row[i], 64);
      goff[i] = kk >= 0 ? (uint32_t)kk * ROWB + (uint32_t)ld_off[i] : 0x80000000u;
    }
  };
  // combine the partials of tile x (every wave for itself): this lane's
  // column key, and the tile's flags (bit 0 shared, bit 1 all padding) in
  // this wave's flag slot
  int ntile = ntile_w;
  auto finalize = [&](int x) -> int64_t {
    const int* pp = part + (x & 1) * (2 * KT * WAVES) + (lane & 31) * WAVES;
    int mx = -1, mn = 0x7fffffff;
#pragma unroll
    for (int w4 = 0; w4 < WAVES; w4 += 4) {
      const u32x4_l a = *(const lds_u32x4*)(pp + w4);
      const u32x4_l c = *(const lds_u32x4*)(pp + KT * WAVES + w4);
#pragma unroll
      for (int e = 0; e < 4; e++) {
        mx = max(mx, (int)a[e]);
        mn = min(mn, (int)c[e]);
      }
    }
    const bool pad = mx == -1;
    const bool shared = pad || mn == mx;
    const uint64_t sh = __ballot(shared), pd = __ballot(pad);
    const int flags = (sh == ~0ull ? 1 : 0) | (pd == ~0ull ? 2 : 0);
    if (x < ntile_w && (flags & 2) && x < ntile) ntile = x;  // every row has ended
    if (lane == 0) flag_s[wave * 8 + (x & 7)] = flags;
    return mx;
  };

  // ---- Q^T as the B operand: lane (c16, g) holds dims 32 S + 8 g .. +8 of
  // row c16 of each block
  bf16x8_l qreg[RB][KSTEPS];
#pragma unroll
  for (int rb = 0; rb < RB; rb++) {
    const uint16_t* qp = q + (((b * hq + row_h[rb]) * q_seq + q0 + row_q[rb]) * D) + 8 * g;
#pragma unroll
    for (int s = 0; s < KSTEPS; s++) {
      u32x4_l raw = {0u, 0u, 0u, 0u};
      if (row_on[rb]) raw = __builtin_bit_cast(u32x4_l, *(const uint4*)(qp + 32 * s));
      qreg[rb][s] = __builtin_bit_cast(bf16x8_l, raw);
    }
  }

  // ---- per-lane LDS addresses within a K/V tile
  // K: row c16 (+16 for keys 16..31), chunk 4 S + g stored at (4 S + g) ^ c16
  uint32_t kofs[KSTEPS];
#pragma unroll
  for (int s = 0; s < KSTEPS; s++) kofs[s] = (uint32_t)(c16 * ROWB + 16 * ((4 * s + g) ^ c16));
  // V^T: lane 4 jj + qq of group g reads row 4 g + jj (+16), dv 16 dt + 4 qq:
  // chunk 2 dt + (qq >> 1) stored at 2 (dt ^ fr) + (qq >> 1), fr = row & 7
  uint32_t vofs[DVT];
  {
    const int jj = c16 >> 2, qq = c16 & 3;
    const int Rr = 4 * g + jj;
    const int fr = Rr & 7;
#pragma unroll
    for (int dt = 0; dt < DVT; dt++)
      vofs[dt] = (uint32_t)(KT * ROWB + Rr * ROWB + 16 * (2 * (dt ^ fr) + (qq >> 1)) + 8 * (qq & 1));
  }
  constexpr int HALF = 16 * ROWB;  // keys 16..31 of a tile

  // scores in log2 units: raw dot product times scale * log2 e; with a softcap
  // c, c tanh(s / c) log2 e with tanh(x) = 1 - 2 / (exp(2x) + 1) on the
  // hardware exp2 and reciprocal (a few fp32 ulps of tanh, exact limits +-1)
  const float f = scale * kLog2eL;
  const float cap_k = SOFTCAP ? 2.0f * scale * kLog2eL / softcap : 0.0f;  // exp2 argument per raw dot unit
  const float cap_a = SOFTCAP ? softcap * kLog2eL : 0.0f;
  const float cap_b = 2.0f * cap_a;
  f32x4_l o[RB][DVT];
  float m_run[RB], l_run[RB];
#pragma unroll
  for (int rb = 0; rb < RB; rb++) {
#pragma unroll
    for (int dt = 0; dt < DVT; dt++) o[rb][dt] = (f32x4_l){0.f, 0.f, 0.f, 0.f};
    m_run[rb] = -INFINITY;
    l_run[rb] = 0.0f;
  }

  f32x4_l sa[RB][2];  // [row block][key half]
  auto zero_s = [&]() {
#pragma unroll
    for (int rb = 0; rb < RB; rb++) sa[rb][0] = sa[rb][1] = (f32x4_l){0.f, 0.f, 0.f, 0.f};
  };
  u32x4_l kr[8];
  s16x4_l vr0[DVT], vr1[DVT];
  uint32_t kslot = 0, vslot = 0;
  auto kread = [&](auto jc) {
    constexpr int J = decltype(jc)::value;  // k-step J >> 1, key half J & 1
    kr[J] = ds_read_b128_at<(J & 1) * HALF>(kslot + kofs[J >> 1]);
  };
  auto kmfma = [&](auto jc) {
    constexpr int J = decltype(jc)::value;
    const bf16x8_l a = __builtin_bit_cast(bf16x8_l, kr[J]);
#pragma unroll
    for (int rb = 0; rb < RB; rb++)
      sa[rb][J & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qreg[rb][J >> 1], sa[rb][J & 1], 0, 0, 0);
  };
  auto vread = [&](auto dc) {
    constexpr int DT = decltype(dc)::value;
    vr0[DT] = ds_read_tr16_at<0>(vslot + vofs[DT]);
    vr1[DT] = ds_read_tr16_at<HALF>(vslot + vofs[DT]);
  };
  bf16x8_l pb[RB];
  auto vmfma = [&](auto dc) {
    constexpr int DT = decltype(dc)::value;
    const s16x4_l a8[2] = {vr0[DT], vr1[DT]};
    const bf16x8_l a = __builtin_bit_cast(bf16x8_l, a8);
#pragma unroll
    for (int rb = 0; rb < RB; rb++)
      o[rb][DT] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[rb], o[rb][DT], 0, 0, 0);
  };
  // S of the tile at kslot alone (reads two steps ahead)
  auto s_alone = [&]() {
    zero_s();
    static_for<2>(kread);
    static_for<8>([&](auto jc) {
      constexpr int J = decltype(jc)::value;
      if constexpr (J + 2 < 8) kread(std::integral_constant<int, J + 2>{});
      constexpr int LATER = (J + 2 < 8) ? 2 : 7 - J;
      lgkm_wait_tied1<LATER>(kr[J]);
      kmfma(jc);
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  // PV of the tile at vslot alone
  auto pv_alone = [&]() {
    static_for<4>(vread);
    static_for<DVT>([&](auto dc) {
      constexpr int DT = decltype(dc)::value;
      constexpr int AHEAD = (3 < DVT - 1 - DT ? 3 : DVT - 1 - DT);
      lgkm_wait_tied<2 * AHEAD>(vr0[DT], vr1[DT]);
      vmfma(dc);
      if constexpr (DT + 4 < DVT) vread(std::integral_constant<int, DT + 4>{});
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  // bias of this lane's eight (row, column) scores of a tile: columns 4 g + i
  // and 16 + 4 g + i, whose keys lanes 0..31 hold (one column each). The
  // steady state loads a tile's values one iteration before its softmax, so
  // they land behind that iteration's gathers (ordinary loads: the compiler
  // places the wait at the use).
  float bvf[8];
  auto bias_load = [&](int64_t colkey, uint16_t (&dst)[8]) {
    if constexpr (BIAS) {
      const int kc32 = (bkey && colkey >= 0 && colkey < bound) ? (int)colkey : 0;  // clamp as the gather does
#pragma unroll
      for (int i = 0; i < 8; i++) {
        const int kcol = __shfl(kc32, i < 4 ? 4 * g + i : 16 + 4 * g + i - 4, 64);
        dst[i] = brow[0][row_on[0] ? kcol : 0];
      }
    }
  };
  auto bias_use = [&](const uint16_t (&src)[8]) {
    if constexpr (BIAS) {
#pragma unroll
      for (int i = 0; i < 8; i++) bvf[i] = bf16_to_f32(src[i]) * kLog2eL;
    }
  };
  // online softmax of the scores in sa for tile x; `only` < 0: every row,
  // else only the rows of query `only`; `none`: every row masked (the
  // tile is redone row by row). Rescales O and returns P^T in pb.
  auto softmax = [&](int x, int only, bool none) {
    const int64_t c0 = (int64_t)(xo + x) * KT;
#pragma unroll
    for (int rb = 0; rb < RB; rb++) {
      float xs[8];
#pragma unroll
      for (int i = 0; i < 4; i++) {
        xs[i] = sa[rb][0][i];
        xs[4 + i] = sa[rb][1][i];
      }
#pragma unroll
      for (int i = 0; i < 8; i++) {
        if constexpr (SOFTCAP) xs[i] = cap_a - cap_b * __builtin_amdgcn_rcpf(__builtin_amdgcn_exp2f(xs[i] * cap_k) + 1.0f);
        else xs[i] *= f;
        if constexpr (BIAS) xs[i] += bvf[i];  // after the softcap, in log2 units
      }
      const bool live = row_on[rb] && !none && (only < 0 || only == row_q[rb]);
      const int64_t n = live ? (int64_t)n_s[row_q[rb]] : 0;
#pragma unroll
      for (int i = 0; i < 8; i++) {
        const int64_t col = c0 + (i < 4 ? 4 * g + i : 16 + 4 * g + i - 4);
        xs[i] = col < n ? xs[i] : -INFINITY;
      }
      float tmax = fmaxf(fmaxf(fmaxf(xs[0], xs[1]), fmaxf(xs[2], xs[3])), fmaxf(fmaxf(xs[4], xs[5]), fmaxf(xs[6], xs[7])));
      tmax = max_x32(max_x16(tmax));
      const float mn = fmaxf(m_run[rb], tmax);
      const float alpha = mn == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m_run[rb] - mn);
      m_run[rb] = mn;
      const float nm = mn == -INFINITY ? 0.0f : -mn;
      float p[8];
#pragma unroll
      for (int i = 0; i < 8; i++) p[i] = __builtin_amdgcn_exp2f(xs[i] + nm);
      const float ps = ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
      l_run[rb] = l_run[rb] * alpha + sum_x32(sum_x16(ps));
      if (__ballot(alpha != 1.0f)) {
#pragma unroll
        for (int dt = 0; dt < DVT; dt++) o[rb][dt] *= alpha;
      }
      const u32x4_l pw = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                          pack_bf16x2(p[6], p[7])};
      pb[rb] = __builtin_bit_cast(bf16x8_l, pw);
    }
  };
  auto slot_of = [&](int x) { return (uint32_t)(uintptr_t)(lds + (x % NSTAGE) * KV_TILE); };
  auto tile_flags = [&](int x) { return flag_s[wave * 8 + (x & 7)]; };

  // A tile that is not shared, redone one query at a time through the spare
  // slot: that query's own keys are gathered (clamped into the cache), its
  // rows updated, every other row masked. Waits for every load in flight.
  auto row_by_row = [&](int x) {
    const uint32_t spare = (uint32_t)(uintptr_t)(lds + SPARE_OFF);
    for (int r = 0; r < rlive; r++) {
      if ((int64_t)n_s[r] <= (int64_t)(xo + x) * KT) continue;  // uniform: the row ended before this tile
      const int64_t col = (int64_t)(xo + x) * KT + (lane & 31);
      int64_t kl = -1;
      if (col < width) kl = load_index<I64>(ibase, (int64_t)r * width + col);
      key_offsets(kl);
      uint16_t brr[8];
      bias_load(kl, brr);
      wait_vm<0>();
      __syncthreads();  // every wave is done with the spare slot
      gather_issue(lds + SPARE_OFF);
      wait_vm<0>();
      bias_use(brr);
      __syncthreads();
      kslot = spare;
      vslot = spare;
      if (wlive) {
        s_alone();
        softmax(x, r, false);
        pv_alone();
      }
    }
    // the tile's PV in the pipeline must add nothing
#pragma unroll
    for (int rb = 0; rb < RB; rb++) pb[rb] = __builtin_bit_cast(bf16x8_l, (u32x4_l){0u, 0u, 0u, 0u});
  };

  // ---- prologue: index tiles 0..3 folded, keys of tiles 0..2 gathered,
  // index tiles 4, 5 in flight
#pragma unroll 1
  for (int x = 0; x < 4; x++) issue_idx(x);
  wait_vm<0>();
  __syncthreads();  // n_s initialised, index tiles 0..3 in LDS
  fold(0);
  fold(1);
  __syncthreads();
  int64_t kk = finalize(0);
  const int64_t key0 = kk;
  key_offsets(kk);
  gather_issue(lds + 0 * KV_TILE);
  issue_idx(4);
  kk = finalize(1);
  const int64_t key_n1 = kk;  // keys of tile 1, then of the tile two after the one being scored
  key_offsets(kk);
  lds_barrier();  // partial slots of tiles 0, 1 are read
  fold(2);
  fold(3);
  gather_issue(lds + 1 * KV_TILE);
  lds_barrier();
  kk = finalize(2);
  int64_t key_n2 = kk;
  key_offsets(kk);
  gather_issue(lds + 2 * KV_TILE);
  issue_idx(5);
  // the iteration-0 fold reads tile 4's index slot: everything but the last
  // tile's loads has landed
  if (ntile > 0) {
    wait_vm<GLOADS + IL>();  // tile 0 and index tile 4 have landed for this wave
    lds_barrier();
    kslot = slot_of(0);
    if (tile_flags(0) & 1) {
      if (wlive) {
        s_alone();
        uint16_t br0[8];
        bias_load(key0, br0);
        bias_use(br0);
        softmax(0, -1, false);
      }
    } else {
      if (wlive) {
        zero_s();
        softmax(0, -1, true);
      }
      row_by_row(0);
    }
  }

  // ---- steady state: iteration t scores tile t+1 interleaved with the PV
  // of tile t, issues the gather of tile t+3 and the index load of tile t+6,
  // folds index tile t+4 and finalizes tile t+3. With a bias it also loads
  // tile t+2's bias (into bload) and uses tile t+1's, loaded one iteration
  // earlier (buse).
  // With a bias, two iterations per trip with the bias registers alternating,
  // so a tile's values stay in the same registers from their load to their use.
  constexpr int UN = BIAS ? 2 : 1;
  uint16_t ba[8], bb[8];
  if (!wlive) {
    // a wave with no live row: the same gathers, index loads, folds and
    // barriers, no reads, products or softmax
    for (int t = 0; t + 1 < ntile; t++) {
      wait_vm<GLOADS + IL>();
      lds_barrier();
      kk = finalize(t + 3);
      key_offsets(kk);
      const bool shared_next = (tile_flags(t + 1) & 1) != 0;
#pragma unroll
      for (int j = 0; j < GLOADS; j++)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(grsrc, (__attribute__((address_space(3))) void*)(lds + ((t + 3) % NSTAGE) * KV_TILE + 1024 * (GLOADS * wave + j)),
                                                16, goff[j], 0, 0, 0);
      issue_idx(t + 6);
      fold(t + 4);
      if (!shared_next) row_by_row(t + 1);
    }
  } else {
  bias_load(key_n1, ba);
  for (int t0 = 0; t0 + 1 < ntile; t0 += UN) {
#pragma unroll
   for (int u = 0; u < UN; u++) {
    const int t = t0 + u;
    if (u > 0 && t + 1 >= ntile) break;
    const uint16_t(&buse)[8] = u == 0 ? ba : bb;
    uint16_t(&bload)[8] = u == 0 ? bb : ba;
    wait_vm<GLOADS + IL>();  // tile t+1 and index tile t+4 have landed (the last iteration's loads may not)
    lds_barrier();           // for every wave; tile t-1's slot and partial slot t+3 & 1 are free
    kk = finalize(t + 3);    // partials folded in the last iteration
    key_offsets(kk);
    const bool shared_next = (tile_flags(t + 1) & 1) != 0;
    bias_load(key_n2, bload);  // unused when tile t+2 is not shared
    kslot = slot_of(t + 1);
    vslot = slot_of(t);
    zero_s();
    constexpr int PL = 2;
    auto sread = [&](auto jc) {
      kread(jc);
      vread(jc);
    };
    static_for<PL>(sread);
    static_for<8>([&](auto jc) {
      constexpr int J = decltype(jc)::value;
      if constexpr (J + PL < 8) sread(std::integral_constant<int, J + PL>{});
      if constexpr (J < GLOADS) {  // the gather of tile t+3, one load per step
        __builtin_amdgcn_raw_ptr_buffer_load_lds(grsrc, (__attribute__((address_space(3))) void*)(lds + ((t + 3) % NSTAGE) * KV_TILE + 1024 * (GLOADS * wave + J)),
                                                16, goff[J], 0, 0, 0);
      }
      constexpr int LATER = gqa_step_reads(J + 1) * (J + 1 < 8) + gqa_step_reads(J + 2) * (J + 2 < 8);
      lgkm_wait3<LATER>(kr[J], vr0[J], vr1[J]);
      kmfma(jc);
      vmfma(jc);
      __builtin_amdgcn_sched_barrier(0);
    });
    issue_idx(t + 6);
    fold(t + 4);
    if (shared_next) {
      bias_use(buse);
      softmax(t + 1, -1, false);
    } else {
      softmax(t + 1, -1, true);
      row_by_row(t + 1);
    }
    key_n2 = kk;
   }
  }
  }

  // ---- the last tile's PV alone
  if (ntile > 0 && wlive) {
    vslot = slot_of(ntile - 1);
    pv_alone();
  }
  wait_vm<0>();  // loads issued past the last tile

  // ---- store: lane holds O^T[16 dt + 4 g + r][row c16] of each block
  if (splits > 1) {
    // split-KV: the unnormalised O, the running maximum (log2 units) and sum
    // of each row for the combine
#pragma unroll
    for (int rb = 0; rb < RB; rb++) {
      if (!row_on[rb]) continue;
      const int64_t prow = ((b * hq + row_h[rb]) * q_seq + q0 + row_q[rb]) * splits + sp;
      float* op = part_o + prow * D + 4 * g;
#pragma unroll
      for (int dt = 0; dt < DVT; dt++) *(f32x4_l*)(op + 16 * dt) = o[rb][dt];
      if (g == 0) *(float2*)(part_ml + prow * 2) = make_float2(m_run[rb], l_run[rb]);
    }
  } else {
#pragma unroll
    for (int rb = 0; rb < RB; rb++) {
      if (!row_on[rb]) continue;
      const float inv = l_run[rb] > 0.0f ? 1.0f / l_run[rb] : 0.0f;
      uint16_t* yp = y + (((b * hq + row_h[rb]) * q_seq + q0 + row_q[rb]) * D) + 4 * g;
#pragma unroll
      for (int dt = 0; dt < DVT; dt++) {
        const u32x2_l w2 = {pack_bf16x2(o[rb][dt][0] * inv, o[rb][dt][1] * inv),
                            pack_bf16x2(o[rb][dt][2] * inv, o[rb][dt][3] * inv)};
        *(u32x2_l*)(yp + 16 * dt) = w2;
      }
    }
  }
  if constexpr (!FUSED) return;

  // ---- fused validation (launched with the in-launch append, for
  // decode-like blocks, where most waves hold no row): the kv heads of this (batch, query block, split) share its
  // columns out; kv head h checks the h-th slice for every query row of the
  // block, from memory (the index rows are in L2), each column against its
  // left neighbour. A failing column, or a first column of -1 (a row of
  // padding only), lowers its row's minimum key in LDS.
  const bool duty = kvh == 0 && qb == 0 && sp == 0;
  if constexpr (APPEND) {
    if (duty && tid == 0) {
      // a device-scope atomic store: the launch's record reads it without a fence
      if (app_ok) atomicExch(&present_len[b], (int32_t)(app_p + cur_len));
      else atomicOr(&eb->call_word, SA_ERR_APPEND_CAPACITY | SA_ERR_APPEND_ANY);
    }
  }
  {
    const int64_t mb = vmb, me = vme;
    const uint32_t rmin_a = (uint32_t)(uintptr_t)(lds + rmin_off<I64>());
    if (pre) {  // the values loaded at the start
      const int64_t mc = me - mb;
#pragma unroll
      for (int k = 0; k < 2; k++) {
        const int64_t e = tid + (int64_t)THREADS * k;
        if (e < (int64_t)rlive * mc) {
          const int64_t r = e / mc, c = mb + (e - r * mc);
          if (column_class(c, pv[k], pu[k], bound))
            ds_min_u64_at(rmin_a + 8u * (uint32_t)r, (unsigned long long)((irow0 + r) * (width + 1) + c));
        }
      }
    }
    for (int r = 0; r < rlive && me > mb && !pre; r++) {  // uniform
      const int64_t rb0 = (irow0 + r) * width;
      for (int64_t c0 = mb + tid; c0 < me; c0 += 2 * THREADS) {
        const int64_t c1 = c0 + THREADS;
        const int64_t v0 = load_index<I64>(idx, rb0 + c0);
        const int64_t u0 = c0 > 0 ? load_index<I64>(idx, rb0 + c0 - 1) : 0;
        const int64_t v1 = c1 < me ? load_index<I64>(idx, rb0 + c1) : -1;
        const int64_t u1 = c1 < me ? load_index<I64>(idx, rb0 + c1 - 1) : 0;
        if (column_class(c0, v0, u0, bound))
          ds_min_u64_at(rmin_a + 8u * (uint32_t)r, (unsigned long long)((irow0 + r) * (width + 1) + c0));
        if (column_class(c1, v1, u1, bound))
          ds_min_u64_at(rmin_a + 8u * (uint32_t)r, (unsigned long long)((irow0 + r) * (width + 1) + c1));
      }
    }
    // a row whose first entry is -1 holds only padding (unless a column fails)
    if (xo == 0 && kvh == 0 && width > 0 && tid < rlive && load_index<I64>(idx, (irow0 + tid) * width) == -1)
      ds_min_u64_at(rmin_a + 8u * (uint32_t)tid, (unsigned long long)((irow0 + tid) * (width + 1) + width));
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this thread's LDS minima have landed
  __syncthreads();
  // ---- arrivals: the splits x kv heads workgroups of a query row each count
  // one; the last records the row's first violation and counts toward the
  // launch's record
  if (tid < rlive) {
    const int64_t irow = irow0 + tid;
    unsigned long long k = rmin[tid];
    if (k != ~0ull) atomicMin(&row_key[irow], k);
    // the row minimum (and present_len) are device-scope atomics: waiting for
    // them to complete orders them before the count
    __builtin_amdgcn_s_waitcnt(0);
    if (atomicAdd(&row_done[irow], 1u) == (unsigned)(splits * hkv) - 1) {
      atomicExch(&row_done[irow], 0u);        // re-armed for the next launch
      k = atomicExch(&row_key[irow], ~0ull);  // every workgroup's minimum, re-armed
      if (k != ~0ull) {
        const int64_t col = (int64_t)(k % (unsigned long long)(width + 1));
        int cls = 6;
        if (col < width) {
          const int64_t v = load_index<I64>(idx, irow * width + col);
          const int64_t u = col > 0 ? load_index<I64>(idx, irow * width + col - 1) : 0;
          cls = column_class(col, v, u, bound);
        }
        atomicOr(&eb->call_word, (1u << (cls - 1)) | SA_ERR_INDEX_ANY);
        atomicMin((unsigned long long*)&eb->call_key, k);
      }
      finish_launch<I64, false>(eb, idx, width, q_seq, q_seq, APPEND ? present_len : valid_len, cap,
                                (unsigned)(batch * q_seq), reset != 0);
    }
  }
}

// Split-KV combine: per output row, y = sum_j O_j 2^(m_j - M) / sum_j l_j 2^(m_j - M)
// over the splits j (M the largest m_j), stored as bf16; a row no split saw gives zeros.
// 32 lanes per row, 4 dims each.
__global__ void __launch_bounds__(256)
gqa_combine_kernel(const float* __restrict__ part_o, const float* __restrict__ part_ml,
                   uint16_t* __restrict__ y, int64_t rows, int splits) {
  constexpr int SMAX = 16;  // the most splits gqa_splits takes
  const int64_t row = (int64_t)blockIdx.x * 8 + (threadIdx.x >> 5);
  if (row >= rows) return;
  const int d = (threadIdx.x & 31) * 4;
  // every split's values loaded at once (indices clamped, extra ones ignored)
  float2 ml[SMAX];
  float4 v[SMAX];
#pragma unroll
  for (int j = 0; j < SMAX; j++) {
    const int64_t pj = row * splits + min(j, splits - 1);
    ml[j] = *(const float2*)(part_ml + pj * 2);
    v[j] = *(const float4*)(part_o + pj * gq::D + d);
  }
  float M = -INFINITY;
#pragma unroll
  for (int j = 0; j < SMAX; j++)
    if (j < splits) M = fmaxf(M, ml[j].x);
  float L = 0.0f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  if (M != -INFINITY) {
#pragma unroll
    for (int j = 0; j < SMAX; j++) {
      if (j >= splits || ml[j].x == -INFINITY) continue;  // past the splits, or a split that saw no key of the row
      const float w = exp2f(ml[j].x - M);
      L += ml[j].y * w;
      acc.x += v[j].x * w;
      acc.y += v[j].y * w;
      acc.z += v[j].z * w;
      acc.w += v[j].w * w;
    }
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  const uint32_t lo = (uint32_t)f32_to_bf16_rne(acc.x * inv) | ((uint32_t)f32_to_bf16_rne(acc.y * inv) << 16);
  const uint32_t hi = (uint32_t)f32_to_bf16_rne(acc.z * inv) | ((uint32_t)f32_to_bf16_rne(acc.w * inv) << 16);
  *(uint2*)(y + row * gq::D + d) = make_uint2(lo, hi);
}

// (row, split) units the split-KV buffers hold: splits are only taken while
// (batch, kv head, query block) units number fewer than the CUs, and a unit
// holds at most 128 rows, so rows x splits < 128 x (2 x 256)
int64_t gqa_partial_rows(const sa_config& cfg) {
  const int64_t rows_max = cfg.max_batch * cfg.max_q_seq * cfg.num_heads;
  return std::min<int64_t>(rows_max * 16, (int64_t)gq::MROWS * 2 * kNumCUs);
}

// Splits per (batch, kv head, query block) so that the launch covers the CUs,
// at least four 32-key tiles per split (the pipeline's prologue is six tiles
// deep), at most 16; 1 when the buffers cannot hold the partials.
int gqa_splits(const sparse_attn_ctx* c, int64_t batch, int64_t q_seq, int64_t width) {
  using namespace gq;
  const sa_config& k = c->cfg;
  const int64_t group = k.num_heads / k.kv_num_heads;
  const int64_t R = group >= MROWS ? 1 : std::min<int64_t>(RMAX, MROWS / group);
  const int64_t units = batch * k.kv_num_heads * ((q_seq + R - 1) / R);
  if (units <= 0 || units >= kNumCUs) return 1;
  const int64_t want = (kNumCUs + units - 1) / units;
  const int64_t by_tiles = std::max<int64_t>(1, ((width + KT - 1) / KT) / 4);
  const int64_t s = std::min<int64_t>(std::min<int64_t>(want, by_tiles), 16);
  if (s <= 1 || batch * q_seq * k.num_heads * s > c->gpart_rows) return 1;
  return (int)s;
}

// The launch validates its own index rows (and may append) when a workgroup's
// rows fill at most half of its waves (decode-like blocks): the idle waves
// leave room for the check at the end. Larger blocks keep the standalone
// validation kernel, which reads the rows once for all kv heads.
bool gqa_fuses(const sa_config& cfg, int64_t q_seq) {
  using namespace gq;
  const int64_t group = cfg.num_heads / cfg.kv_num_heads;
  const int64_t R = group >= MROWS ? 1 : std::min<int64_t>(RMAX, MROWS / group);
  return std::min<int64_t>(R, q_seq) * group <= MROWS / 2;
}

bool gqa_supported(const sa_config& cfg, int64_t index_heads) {
  if (cfg.dtype != SA_BF16 || cfg.kv_layout != SA_KV_SEPARATE || cfg.cache_format != SA_CACHE_DENSE) return false;
  if (index_heads != 1 || cfg.head_dim_qk != gq::D || cfg.head_dim_v != gq::D) return false;
  if (cfg.kv_num_heads <= 0 || cfg.num_heads % cfg.kv_num_heads != 0) return false;
  const int64_t group = cfg.num_heads / cfg.kv_num_heads;
  if (group > gq::MROWS) return false;
  return cfg.max_cache_len <= (int64_t)(0x7fffffffLL / gq::ROWB);
}

static bool g_gqa_attr[16] = {};

sa_status launch_forward_gqa(sparse_attn_ctx* c, const FwdArgs& a, bool fused, const AppendArgs* app) {
  using namespace gq;
  const int group = (int)(a.hq / a.hkv);
  const int R = group >= MROWS ? 1 : std::min(RMAX, MROWS / group);
  const int64_t nqb = (a.q_seq + R - 1) / R;
  const int64_t pairs = a.batch * a.hkv;
  if (pairs <= 0 || nqb <= 0) return SA_OK;
  const int splits = gqa_splits(c, a.batch, a.q_seq, a.width);
  const int64_t wgs = (pairs + 7) / 8 * 8 * nqb * splits;
  if (wgs > 0x7fffffffLL || nqb > 0x7fffffffLL) return set_error(c, SA_E_SHAPE, "forward: too many rows for one launch");
  if (a.cap > (int64_t)(0x7fffffffLL / ROWB)) return set_error(c, SA_E_SHAPE, "forward: cache too long for 32-bit row offsets");
  if ((int64_t)R * a.width * (a.idx64 ? 8 : 4) > 0x7fffffffLL)
    return set_error(c, SA_E_SHAPE, "forward: index rows too wide for 32-bit offsets");
  const bool cap_on = a.softcap != 0.0f;
  const bool bias_on = a.bias != nullptr;
  // the launch validates itself only together with the in-launch append (a
  // plain forward keeps the standalone validation kernel, which measured
  // faster than the check at the end of every workgroup)
  if (fused != (app != nullptr)) return set_error(c, SA_E_STATE, "forward: in-launch validation comes with the append");
  if (fused && (!c->row_key || !c->row_done))
    return set_error(c, SA_E_STATE, "forward: fused validation needs the context's row buffers");
  if (fused && a.batch * a.q_seq > c->rows_cap)
    return set_error(c, SA_E_STATE, "forward: more index rows than the context holds");
  const int mode = app ? 1 : 0;
  const int variant = (a.idx64 ? 1 : 0) + (cap_on ? 2 : 0) + (bias_on ? 4 : 0) + 8 * mode;
#define SA_GQA_FN(M)                                                                                        \
  (const void*)gqa_forward_kernel<false, false, false, M, M>, (const void*)gqa_forward_kernel<true, false, false, M, M>, \
      (const void*)gqa_forward_kernel<false, true, false, M, M>, (const void*)gqa_forward_kernel<true, true, false, M, M>, \
      (const void*)gqa_forward_kernel<false, false, true, M, M>, (const void*)gqa_forward_kernel<true, false, true, M, M>, \
      (const void*)gqa_forward_kernel<false, true, true, M, M>, (const void*)gqa_forward_kernel<true, true, true, M, M>
  const void* fns[16] = {SA_GQA_FN(false), SA_GQA_FN(true)};
#undef SA_GQA_FN
  const size_t lds = a.idx64 ? lds_bytes<true>() : lds_bytes<false>();
  if (!g_gqa_attr[variant]) {
    hipError_t e = hipFuncSetAttribute(fns[variant], hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return check_hip(c, e, "forward (gqa) LDS attribute");
    g_gqa_attr[variant] = true;
  }
  const dim3 grid((unsigned)wgs), block(THREADS);
  const ProfEvents pe = prof_next(c);
  const uint8_t* cur_k = app ? (const uint8_t*)app->cur : nullptr;
  const uint8_t* cur_v = app ? (const uint8_t*)app->cur_v : nullptr;
  const int32_t* plen = app ? app->past_len : nullptr;
  int32_t* prlen = app ? app->present_len : nullptr;
  const int64_t clen = app ? app->cur_len : 0;
  const int reset = app ? app->reset : 0;
#define SA_GQA(I, C, BI, F, A)                                                                                \
  SA_MAIN_LAUNCH(pe, (gqa_forward_kernel<I, C, BI, F, A>), grid, block, lds, c->stream, (const uint16_t*)a.q, \
                     (uint8_t*)a.k, (uint8_t*)a.v, a.idx, a.valid_len, (uint16_t*)a.y, a.batch, a.hkv,        \
                     a.q_seq, a.cap, a.width, group, (int)nqb, a.scale, a.softcap, (const uint16_t*)a.bias,    \
                     a.bd[0], a.bd[1], a.bd[2], a.bd[3], splits, c->gpart_o, c->gpart_ml, c->err, c->row_key,  \
                     c->row_done, cur_k, cur_v, plen, prlen, clen, reset)
#define SA_GQA_M(F, A)                                   \
  switch (variant & 7) {                                 \
    case 0: SA_GQA(false, false, false, F, A); break;    \
    case 1: SA_GQA(true, false, false, F, A); break;     \
    case 2: SA_GQA(false, true, false, F, A); break;     \
    case 3: SA_GQA(true, true, false, F, A); break;      \
    case 4: SA_GQA(false, false, true, F, A); break;     \
    case 5: SA_GQA(true, false, true, F, A); break;      \
    case 6: SA_GQA(false, true, true, F, A); break;      \
    default: SA_GQA(true, true, true, F, A); break;      \
  }
  if (mode == 0) {
    SA_GQA_M(false, false)
  } else {
    SA_GQA_M(true, true)
  }
#undef SA_GQA_M
#undef SA_GQA
  sa_status st = check_hip(c, hipGetLastError(), "forward (gqa)");
  if (st != SA_OK || splits == 1) return st;
  const int64_t rows = a.batch * a.hq * a.q_seq;
  hipLaunchKernelGGL(gqa_combine_kernel, dim3((unsigned)((rows + 7) / 8)), dim3(256), 0, c->stream, c->gpart_o,
                     c->gpart_ml, (uint16_t*)a.y, rows, splits);
  return check_hip(c, hipGetLastError(), "forward (gqa combine)");
}

}  // namespace sa
