// Shared-latent selected-token attention, bf16 rows, on the gfx950 matrix
// cores with a direct-to-LDS gather pipeline.
//
// Same contraction as the first shared-latent kernel (all 64 query heads read
// one kv head through one index row; S^T = K_sel . Q^T and O^T += V_sel^T . P^T
// on v_mfma_f32_16x16x32_bf16, an online softmax per head, optional split of a
// row's keys with a log-sum-exp combine), with the data movement rebuilt for
// gfx950:
//  * gathered rows go from HBM straight into LDS (16-byte global_load_lds per
//    lane), no registers in between, through a ring of NSTAGE 32-key tiles, so
//    up to three tiles (108 KB) are in flight per CU while one is computed;
//  * a tile holds dims 0..511 of its 32 rows as [32][64 chunks] (one wave load
//    per row) and the 64 rope dims as [32][8 chunks]; 16-byte chunk c of row r
//    sits at chunk c ^ f(r) (c ^ f2(r) in the rope part), with f, f2 chosen so
//    both LDS read patterns below are free of bank conflicts;
//  * K (A operand of S^T) is read as 16-byte rows; V^T (A operand of O^T) is
//    read from the same row-major tile with ds_read_b64_tr_b16, whose
//    16-lane transpose hands lane i the value of dv i for four keys;
//  * the softmax reference max only moves when a tile's max exceeds it by more
//    than 2^8, so the O^T accumulators are rarely rescaled;
//  * with fused validation each workgroup checks its own columns of the index
//    row (IndexShare host-validator rules) and the per-row / per-launch first
//    failure is gathered with atomics, so no separate validation launch runs;
//  * blocks are numbered so all splits of a row share an XCD (and its L2).
#include "sa_validate_dev.h"

namespace sa {

namespace lat {
constexpr int DK = 576;
constexpr int DV = 512;
constexpr int NH = 64;
constexpr int KT = 32;                          // keys per tile
constexpr int NSTAGE = 4;                       // tiles in the LDS ring
constexpr int ROWB = DK * 2;                    // 1152 bytes per cache row
constexpr int MROW = 1024 + 64;                 // LDS stride of a tile row's dims 0..511
constexpr int MAIN_BYTES = KT * MROW;           // 34816
constexpr int ROPE_BYTES = KT * 128;            // dims 512..575 of the 32 rows
constexpr int TILE_BYTES = MAIN_BYTES + ROPE_BYTES;  // 38912
constexpr int WAVE_LOADS = 9;                   // per wave per tile: 8 main rows + 1 rope load
constexpr int KSTEPS = DK / 32;                 // 18
constexpr int DVT = DV / 16;                    // 32
constexpr int KEYCAP = 1024;                    // keys staged in LDS at a time
constexpr int THREADS = 256;
constexpr float TAU = 8.0f;                     // lazy-rescale threshold (log2 units)
constexpr size_t LDS_BYTES = (size_t)NSTAGE * TILE_BYTES + KEYCAP * 4 + 32;
}  // namespace lat

typedef __bf16 bf16x8_l __attribute__((ext_vector_type(8)));
typedef float f32x4_l __attribute__((ext_vector_type(4)));
typedef short s16x4_l __attribute__((ext_vector_type(4)));
typedef unsigned u32x4_l __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;

constexpr float kLog2eL = 1.4426950408889634f;

// Chunk swizzles. Main part: rows of 64 16-byte chunks at a 1088-byte stride
// (so row r starts 4r slots into the 16-slot bank cycle); chunk c of row r
// sits at c ^ f(r), f(r) in 0..3. For the K reads (16 rows, one chunk) the
// slots 4r + (c ^ f(r)) mod 16 are distinct because f(4a + b) is distinct
// over a; for the V^T transpose reads (8 rows 4a + b, a in {0,1} or {2,3},
// two adjacent chunks) bit 1 of f separates the two a's. Rope part: rows of 8
// chunks at 128 bytes, chunk c at c ^ f2(r), distinct over the 8 even and the
// 8 odd rows of any aligned 16.
__device__ __forceinline__ int swz(int r) { return (((r >> 2) & 1) << 1) | ((r >> 3) & 1); }
__device__ __forceinline__ int swz2(int r) { return (r >> 1) & 7; }

// vmcnt-only wait (gfx9 encoding: expcnt and lgkmcnt left at their maxima)
template <int N>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// 16-lane transposing LDS read (see the file comment). Issued as inline asm:
// the compiler would otherwise wait for every outstanding LDS DMA before it.
// The caller waits for the result with lgkm_wait_tied.
__device__ __forceinline__ s16x4_l ds_read_tr16(const lds_u8* p) {
  s16x4_l r;
  asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(r) : "v"((uint32_t)(uintptr_t)p) : "memory");
  return r;
}

// Wait until at most N LDS/scalar-memory operations are outstanding, and make
// the two values depend on the wait. LDS operations complete in issue order,
// so every LDS read issued more than N LDS operations ago has landed.
template <int N>
__device__ __forceinline__ void lgkm_wait_tied(s16x4_l& a, s16x4_l& b) {
  static_assert(N >= 0 && N <= 15, "lgkmcnt range");
  asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(a), "+v"(b) : "n"(N) : "memory");
}

// Issue this wave's share of one tile (9 wave-wide loads of 64 x 16 bytes):
// main rows r = wave + 4i (lane l takes logical chunk l ^ f(r) of the row's
// dims 0..511) and rope load k = wave (8 rows: lane l takes row 8k + l/8,
// rope chunk (l % 8) ^ f2(row)). Slots past kcount load zeros.
__device__ __forceinline__ void issue_tile(const uint8_t* __restrict__ cache_b,
                                           const uint8_t* __restrict__ zeros,
                                           const int* __restrict__ keys_s, int slot0, int kcount,
                                           lds_u8* tile, int wave, int lane) {
  using namespace lat;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const int r = wave + 4 * i;
    const int slot = slot0 + r;
    const uint8_t* src = slot < kcount ? cache_b + (int64_t)keys_s[slot] * ROWB + ((lane ^ swz(r)) << 4)
                                       : zeros;
    __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)src,
                                     (__attribute__((address_space(3))) void*)(tile + r * MROW), 16, 0, 0);
  }
  {
    const int r = 8 * wave + (lane >> 3);
    const int slot = slot0 + r;
    const uint8_t* src = slot < kcount
        ? cache_b + (int64_t)keys_s[slot] * ROWB + 1024 + (((lane & 7) ^ swz2(r)) << 4)
        : zeros;
    __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)src,
                                     (__attribute__((address_space(3))) void*)(tile + MAIN_BYTES + wave * 1024),
                                     16, 0, 0);
  }
}

template <bool I64, bool FUSED, bool SOFTCAP>
__global__ void __launch_bounds__(lat::THREADS, 1)
latent_forward_kernel(const uint16_t* __restrict__ q, const uint8_t* __restrict__ cache,
                      const void* __restrict__ idx, const int32_t* __restrict__ valid_len,
                      const uint8_t* __restrict__ zeros, uint16_t* __restrict__ y,
                      float* __restrict__ part_o, float* __restrict__ part_ml, int64_t q_seq,
                      int64_t rows, int64_t cap, int64_t width, int splits, float scale,
                      float softcap, ErrorBlock* __restrict__ eb,
                      unsigned long long* __restrict__ row_key, unsigned* __restrict__ row_done) {
  using namespace lat;
  extern __shared__ __attribute__((aligned(1024))) uint8_t lds_raw[];
  lds_u8* ring = (lds_u8*)lds_raw;
  int* keys_s = (int*)(lds_raw + NSTAGE * TILE_BYTES);
  int* misc = keys_s + KEYCAP;  // [0] kcount, [2..3] block min key (u64)
  unsigned long long* minkey_s = (unsigned long long*)(misc + 2);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 4;
  const int c16 = lane & 15;

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
  int64_t bound = valid_len ? (int64_t)valid_len[b] : cap;
  bound = bound < 0 ? 0 : (bound > cap ? cap : bound);
  const int64_t ibase = row * width;
  const uint8_t* cache_b = cache + b * cap * ROWB;

  // columns of the index row this workgroup owns
  const int wtiles = (int)((width + KT - 1) / KT);
  const int tps = (wtiles + splits - 1) / splits;
  const int c0 = min((int64_t)split * tps * KT, width);
  const int c1 = (int)min((int64_t)c0 + (int64_t)tps * KT, width);

  // ---- fused validation of columns [c0, c1)
  if constexpr (FUSED) {
    if (tid == 0) *minkey_s = ~0ull;
    __syncthreads();
    unsigned long long mk = ~0ull;
    for (int c = c0 + tid; c < c1; c += THREADS) {
      const int64_t v = load_index<I64>(idx, ibase + c);
      const int64_t u = c > 0 ? load_index<I64>(idx, ibase + c - 1) : 0;
      if (column_class(c, v, u, bound)) mk = min(mk, (unsigned long long)(row * (width + 1) + c));
    }
    if (c0 == 0 && tid == 0 && load_index<I64>(idx, ibase) == -1)
      mk = min(mk, (unsigned long long)(row * (width + 1) + width));  // all -1, unless a column fails
    if (mk != ~0ull) atomicMin(minkey_s, mk);
    __syncthreads();
    if (tid == 0) {
      unsigned long long k = *minkey_s;
      bool finish_row = true;
      if (splits > 1) {
        if (k != ~0ull) atomicMin(&row_key[row], k);
        __threadfence();
        finish_row = atomicAdd(&row_done[row], 1u) == (unsigned)splits - 1;
        if (finish_row) {
          k = atomicMin(&row_key[row], ~0ull);
          row_key[row] = ~0ull;
          row_done[row] = 0u;
        }
      }
      if (finish_row && k != ~0ull) {
        const int64_t col = (int64_t)(k % (unsigned long long)(width + 1));
        int cls = 6;
        if (col < width) {
          const int64_t v = load_index<I64>(idx, ibase + col);
          const int64_t u = col > 0 ? load_index<I64>(idx, ibase + col - 1) : 0;
          cls = column_class(col, v, u, bound);
        }
        atomicOr(&eb->word, (1u << (cls - 1)) | SA_ERR_INDEX_ANY);
        atomicMin((unsigned long long*)&eb->call_key, k);
      }
      finish_launch<I64>(eb, idx, width, q_seq, q_seq, valid_len, cap);
    }
  }

  // ---- Q^T of this wave's 16 heads in registers: lane (c16, g) holds dims 32s + 8g .. +8
  const int head = wave * 16 + c16;
  bf16x8_l qreg[KSTEPS];
  {
    const uint16_t* qp = q + ((b * NH + head) * q_seq + qi) * DK + 8 * g;
#pragma unroll
    for (int s = 0; s < KSTEPS; s++) {
      u32x4_l raw = __builtin_bit_cast(u32x4_l, *(const uint4*)(qp + s * 32));
      // Q lives in the accumulation registers (MFMA reads its B operand from
      // them); the vector registers stay free for O and in-flight LDS reads
      asm volatile("" : "+a"(raw));
      qreg[s] = __builtin_bit_cast(bf16x8_l, raw);
    }
  }
  // per-lane LDS read offsets within a tile; the per-step parts are immediates
  const int fk = swz(c16);                               // rows c16 and 16 + c16 share f, f2
  const int kbase = c16 * MROW + ((g ^ fk) << 4);        // + 64 s (s < 16), + 16 MROW for keys 16..31
  const int fk2 = swz2(c16);
  const int rbase0 = MAIN_BYTES + c16 * 128 + ((g ^ fk2) << 4);        // rope step s = 16
  const int rbase1 = MAIN_BYTES + c16 * 128 + (((4 + g) ^ fk2) << 4);  // rope step s = 17
  const int vrow = 4 * g + (c16 >> 2);                   // V^T rows vrow, vrow + 16
  const int fv = swz(vrow);
  const int vq = (c16 & 3) >> 1;
  // chunk (2 dt + vq) ^ fv = 2 dt + vlo + (dt even ? vhi : -vhi)
  const int vlo = (vq ^ fv) & 1, vhi = fv & 2;
  const int vbase_e = vrow * MROW + ((vlo + vhi) << 4) + 8 * (c16 & 1);
  const int vbase_o = vrow * MROW + ((vlo - vhi) << 4) + 8 * (c16 & 1);
  const float sl2 = scale * kLog2eL;

  // Softmax reference. Each head's reference m_ref is its first tile's max
  // and then stays fixed: exp2(x - m_ref) of a later, larger score is just a
  // larger power of two, which bf16 P and fp32 O / l hold exactly as well
  // (y = O / l does not depend on the reference), so O is never rescaled and
  // only ever touched by the MFMAs. Only a score more than 2^TAU_HARD above
  // the reference could overflow; then the workgroup restarts its key range
  // with the largest maxima seen as references. Every restart moves past at
  // least one more tile, so there are at most as many restarts as tiles.
  constexpr float TAU_HARD = 100.0f;
  float m_floor = -INFINITY;  // reference to start from
  f32x4_l o[DVT];
  float m_ref, l_run;
  for (;;) {
#pragma unroll
    for (int t = 0; t < DVT; t++) o[t] = (f32x4_l){0.f, 0.f, 0.f, 0.f};
    m_ref = m_floor;
    l_run = 0.0f;
    float m_seen = m_floor;
    bool restart = false;

    for (int st0 = c0; st0 < c1 && !restart; st0 += KEYCAP) {
      const int st1 = min(st0 + KEYCAP, c1);
      __syncthreads();  // previous stage's readers are done with keys_s / the ring
      if (tid == 0) {
        misc[0] = 0;
        misc[1] = 0;  // restart request
      }
      __syncthreads();
      int last = 0;
      for (int s = tid; s < st1 - st0; s += THREADS) {
        const int64_t key = load_index<I64>(idx, ibase + st0 + s);
        keys_s[s] = (int)((key >= 0 && key < bound) ? key : 0);  // clamp: a bad row stays in bounds
        if (key != -1) last = s + 1;
      }
      if (last) atomicMax(&misc[0], last);
      __syncthreads();
      const int kcount = misc[0];
      const int ntile = (kcount + KT - 1) / KT;
      // prologue: tiles 0 .. NSTAGE-2 in flight (tiles past the end load zeros)
#pragma unroll
      for (int p = 0; p < NSTAGE - 1; p++)
        issue_tile(cache_b, zeros, keys_s, p * KT, kcount, ring + p * TILE_BYTES, wave, lane);

      for (int t = 0; t < ntile; t++) {
        wait_vm<(NSTAGE - 2) * WAVE_LOADS>();  // this wave's loads of tile t have landed
        __syncthreads();                       // everyone's have; tile t-1 is consumed
        issue_tile(cache_b, zeros, keys_s, (t + NSTAGE - 1) * KT, kcount,
                   ring + ((t + NSTAGE - 1) % NSTAGE) * TILE_BYTES, wave, lane);
        const lds_u8* T = ring + (t % NSTAGE) * TILE_BYTES;

        // ---- S^T[key, head] for the tile's two 16-key halves; four
        // independent accumulator chains (even / odd k-steps per half)
        f32x4_l sa0 = {0.f, 0.f, 0.f, 0.f}, sa1 = sa0, sb0 = sa0, sb1 = sa0;
        const lds_u8* TK = T + kbase;
        // operands of step s: rows c16 and 16 + c16, chunk 4s + g (rope steps 16, 17)
        auto kread = [&](int s, u32x4_l& a0, u32x4_l& a1) {
          const lds_u8* p0 = s < 16 ? TK + 64 * s : T + (s == 16 ? rbase0 : rbase1);
          const lds_u8* p1 = s < 16 ? p0 + 16 * MROW : p0 + 16 * 128;
          a0 = *(const __attribute__((address_space(3))) u32x4_l*)p0;
          a1 = *(const __attribute__((address_space(3))) u32x4_l*)p1;
        };
        // reads run KD steps ahead of the MFMAs that consume them
        constexpr int KD = 4;
        u32x4_l kr0[KSTEPS], kr1[KSTEPS];
#pragma unroll
        for (int s = 0; s < KD; s++) kread(s, kr0[s], kr1[s]);
#pragma unroll
        for (int s = 0; s < KSTEPS; s++) {
          if (s + KD < KSTEPS) kread(s + KD, kr0[s + KD], kr1[s + KD]);
          if (s & 1) {
            sb0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_l, kr0[s]), qreg[s], sb0, 0, 0, 0);
            sb1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_l, kr1[s]), qreg[s], sb1, 0, 0, 0);
          } else {
            sa0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_l, kr0[s]), qreg[s], sa0, 0, 0, 0);
            sa1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_l, kr1[s]), qreg[s], sa1, 0, 0, 0);
          }
          __builtin_amdgcn_sched_barrier(0);  // keep the read window at KD steps
        }
        const f32x4_l sacc0 = sa0 + sb0, sacc1 = sa1 + sb1;
        // ---- scores; lane holds keys 4g + r (half 0) and 16 + 4g + r (half 1) of head c16
        const int slot_base = t * KT + 4 * g;
        float x[8];
        float tmax = -INFINITY;
#pragma unroll
        for (int i = 0; i < 8; i++) {
          float sc = i < 4 ? sacc0[i] : sacc1[i - 4];
          if constexpr (SOFTCAP) sc = softcap * tanhf(sc * scale / softcap) * kLog2eL;
          else sc = sc * sl2;
          const int slot = slot_base + (i < 4 ? i : 12 + i);
          sc = slot < kcount ? sc : -INFINITY;
          x[i] = sc;
          tmax = fmaxf(tmax, sc);
        }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
        m_seen = fmaxf(m_seen, tmax);
        if (m_ref == -INFINITY) m_ref = tmax;  // first tile of this head: O and l are still 0
        if (tmax > m_ref + TAU_HARD) misc[1] = 1;  // benign race: every writer stores 1
        float psum = 0.0f;
        bf16x8_l pb;
#pragma unroll
        for (int i = 0; i < 8; i++) {
          const float p = (m_ref == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(fminf(x[i] - m_ref, TAU_HARD));
          psum += p;
          pb[i] = (__bf16)p;
        }
        psum += __shfl_xor(psum, 16, 64);
        psum += __shfl_xor(psum, 32, 64);
        l_run += psum;
        // ---- O^T[dv, head] += V^T[dv, key] . P^T[key, head]; transpose reads
        // run VD dv tiles ahead of the MFMA that consumes them
        constexpr int VD = 8;
        const lds_u8* TVe = T + vbase_e;
        const lds_u8* TVo = T + vbase_o;
        s16x4_l vr0[DVT], vr1[DVT];
        auto vread = [&](int dt) {
          const lds_u8* pv = (dt & 1 ? TVo : TVe) + 32 * dt;
          vr0[dt] = ds_read_tr16(pv);
          vr1[dt] = ds_read_tr16(pv + 16 * MROW);
        };
#pragma unroll
        for (int dt = 0; dt < VD; dt++) vread(dt);
#pragma unroll
        for (int dt = 0; dt < DVT; dt++) {
          // reads of tiles dt+1 .. min(dt+VD-1, DVT-1) may stay in flight
          constexpr int dummy = 0;
          (void)dummy;
          if (DVT - 1 - dt >= VD - 1) lgkm_wait_tied<2 * (VD - 1)>(vr0[dt], vr1[dt]);
          else if (DVT - 1 - dt == 6) lgkm_wait_tied<12>(vr0[dt], vr1[dt]);
          else if (DVT - 1 - dt == 5) lgkm_wait_tied<10>(vr0[dt], vr1[dt]);
          else if (DVT - 1 - dt == 4) lgkm_wait_tied<8>(vr0[dt], vr1[dt]);
          else if (DVT - 1 - dt == 3) lgkm_wait_tied<6>(vr0[dt], vr1[dt]);
          else if (DVT - 1 - dt == 2) lgkm_wait_tied<4>(vr0[dt], vr1[dt]);
          else if (DVT - 1 - dt == 1) lgkm_wait_tied<2>(vr0[dt], vr1[dt]);
          else lgkm_wait_tied<0>(vr0[dt], vr1[dt]);
          const s16x4_l a8[2] = {vr0[dt], vr1[dt]};
          o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_l, a8), pb, o[dt], 0, 0, 0);
          if (dt + VD < DVT) vread(dt + VD);
          __builtin_amdgcn_sched_barrier(0);  // keep the read window at VD tiles
        }
      }
      // a restart request is acted on once the stage's tiles are done (only
      // inputs whose scores jump by more than 2^TAU_HARD ever raise one)
      __syncthreads();
      restart = misc[1] != 0;
      wait_vm<0>();  // outstanding ring loads have landed before the ring is reused
    }
    if (!restart) break;
    m_floor = m_seen;
  }

  // ---- epilogue: lane holds O^T[16 dt + 4g + r][head]
  if (splits == 1) {
    const float inv = l_run > 0.0f ? 1.0f / l_run : 0.0f;
    uint16_t* yp = y + ((b * NH + head) * q_seq + qi) * DV + 4 * g;
#pragma unroll
    for (int dt = 0; dt < DVT; dt++) {
      const uint32_t lo = (uint32_t)f32_to_bf16_rne(o[dt][0] * inv) | ((uint32_t)f32_to_bf16_rne(o[dt][1] * inv) << 16);
      const uint32_t hi = (uint32_t)f32_to_bf16_rne(o[dt][2] * inv) | ((uint32_t)f32_to_bf16_rne(o[dt][3] * inv) << 16);
      *(uint2*)(yp + 16 * dt) = make_uint2(lo, hi);
    }
  } else {
    const int64_t pr = (row * splits + split) * NH + head;
    float* op = part_o + pr * DV + 4 * g;
#pragma unroll
    for (int dt = 0; dt < DVT; dt++) *(float4*)(op + 16 * dt) = make_float4(o[dt][0], o[dt][1], o[dt][2], o[dt][3]);
    if (g == 0) {
      part_ml[pr * 2] = m_ref;
      part_ml[pr * 2 + 1] = l_run;
    }
  }
}

static bool g_latent_attr[8] = {false, false, false, false, false, false, false, false};

sa_status launch_forward_latent(sparse_attn_ctx* c, const FwdArgs& a, int splits, bool fused) {
  using namespace lat;
  const int64_t rows = a.batch * a.q_seq;
  if (rows <= 0) return SA_OK;
  if (splits > 1 && rows * splits > c->partial_rows)
    return set_error(c, SA_E_STATE, "forward: split-K partials exceed the context's buffers");
  if (rows > c->rows_cap) return set_error(c, SA_E_STATE, "forward: more rows than the context holds");
  const int64_t wgs = rows * splits;
  if (wgs > 0x7fffffffLL) return set_error(c, SA_E_SHAPE, "forward: too many rows for one launch");
  const bool cap_on = a.softcap != 0.0f;
  const int variant = (a.idx64 ? 1 : 0) + (fused ? 2 : 0) + (cap_on ? 4 : 0);
  const void* fns[8] = {(const void*)latent_forward_kernel<false, false, false>,
                        (const void*)latent_forward_kernel<true, false, false>,
                        (const void*)latent_forward_kernel<false, true, false>,
                        (const void*)latent_forward_kernel<true, true, false>,
                        (const void*)latent_forward_kernel<false, false, true>,
                        (const void*)latent_forward_kernel<true, false, true>,
                        (const void*)latent_forward_kernel<false, true, true>,
                        (const void*)latent_forward_kernel<true, true, true>};
  if (!g_latent_attr[variant]) {
    hipError_t e = hipFuncSetAttribute(fns[variant], hipFuncAttributeMaxDynamicSharedMemorySize, (int)LDS_BYTES);
    if (e != hipSuccess) return check_hip(c, e, "forward (latent) LDS attribute");
    g_latent_attr[variant] = true;
  }
  const dim3 grid((unsigned)wgs), block(THREADS);
  prof_begin(c);
#define SA_LAT(I, F, C)                                                                              \
  hipLaunchKernelGGL((latent_forward_kernel<I, F, C>), grid, block, LDS_BYTES, c->stream,            \
                     (const uint16_t*)a.q, (const uint8_t*)a.k, a.idx, a.valid_len, c->zeros,        \
                     (uint16_t*)a.y, c->partial_o, c->partial_ml, a.q_seq, rows, a.cap, a.width,    \
                     splits, a.scale, a.softcap, c->err, c->row_key, c->row_done)
  switch (variant) {
    case 0: SA_LAT(false, false, false); break;
    case 1: SA_LAT(true, false, false); break;
    case 2: SA_LAT(false, true, false); break;
    case 3: SA_LAT(true, true, false); break;
    case 4: SA_LAT(false, false, true); break;
    case 5: SA_LAT(true, false, true); break;
    case 6: SA_LAT(false, true, true); break;
    default: SA_LAT(true, true, true); break;
  }
#undef SA_LAT
  prof_end(c);
  sa_status s = check_hip(c, hipGetLastError(), "forward (latent)");
  if (s != SA_OK || splits == 1) return s;
  return launch_mla_combine(c, rows, a.q_seq, splits, (uint16_t*)a.y);
}

}  // namespace sa
