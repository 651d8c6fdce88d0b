// Shared-latent selected-token attention over bf16 rows without an attention
// bias: gfx950 matrix cores fed by a direct-to-LDS gather, two waves per
// SIMD, with the value half of each gathered tile read from LDS once. Decode
// rows split their keys over several workgroups (merged by a second kernel);
// prefill rows take one workgroup each, the longest rows first.
//
// The operation is IndexShare's `index_share_row` with one kv head shared by
// all 64 query heads and one index list per (batch, query); the 576-wide
// latent row is the key and its first 512 dims are the value (the CSA pages'
// record that is both key and value). Per 32-key tile a workgroup computes
// S^T = K_sel . Q^T and O^T += V_sel^T . P^T on v_mfma_f32_16x16x32_bf16.
//
// Eight waves, w = 2 hb + kh, play two roles per tile:
//  * scores and softmax of head block hb (heads 16 hb .. 16 hb + 15) over the
//    tile's keys 16 kh .. 16 kh + 15 (all 576 dims; the block's Q in
//    registers), probabilities rounded to bf16 into an LDS exchange (two
//    4 KB buffers, by tile parity);
//  * PV of dv 64 w .. 64 w + 63 for all 64 heads over the tile's 32 keys,
//    reading both key halves of all four head blocks from the exchange.
// The value half of a tile is read from LDS once (with the transposing
// ds_read_b64_tr_b16, the slower of the two reads) and the key half four
// times. Every wave holds about 200 registers, so two share a SIMD and one
// issues MFMAs while the other waits on memory or LDS. The scores of tile
// t+1 are interleaved with the PV of tile t, so a tile needs one workgroup
// barrier, and the ring keeps two tiles in flight while two are read. The two
// waves of a head block agree on one softmax reference per head (the maximum
// of its first tile over both key halves, through LDS) and keep it fixed, so
// the O^T accumulators are only touched by the MFMAs; a score more than
// 2^TAU_HARD above it restarts the workgroup's key range with the maxima seen
// as references.
//
// Gather: rows go from HBM straight into LDS (global_load_lds, 16 B per lane),
// chunk c of ring row R stored at chunk c ^ (R & 6); under that swizzle the K
// reads (16 rows, one chunk) and the transposing V reads are bank-conflict
// free. The workgroup's Q rows (64 x 1152 bytes) come in through the same
// path into two ring slots before the first tiles, as whole cache lines.
#include <type_traits>

#include "sa_mfma_dev.h"
#include "sa_validate_dev.h"

namespace sa {

namespace lhd {
constexpr int DK = 576;
constexpr int DV = 512;
constexpr int NH = 64;
constexpr int KT = 32;                          // keys per tile
constexpr int NSTAGE = 4;                       // tiles in the LDS ring: two read, two in flight
constexpr int ROWB = DK * 2;                    // 1152 bytes per cache row
constexpr int TILE_BYTES = KT * ROWB;           // 36864
constexpr int HALF_ROWS = 16 * ROWB;            // byte offset of keys 16..31 of a tile
constexpr int THREADS = 512;
constexpr int WAVES = THREADS / 64;
constexpr int TILE_LOADS = TILE_BYTES / 1024;   // 36 wave-wide 1 KB loads per tile:
constexpr int MAX_LOADS = 5;                    //   waves 0-3 issue 5, waves 4-7 issue 4
constexpr int KSTEPS = DK / 32;                 // 18 k-steps of S^T
constexpr int DVW = DV / WAVES / 16;            // 4 dv tiles of O^T per wave
constexpr int KEYCAP = 1696;                    // keys staged in LDS at a time (what the LDS leaves)
constexpr int RING_BYTES = NSTAGE * TILE_BYTES; // 147456
constexpr int P_OFF = RING_BYTES;               // bf16 probabilities [buffer][head block][lane][kh] x 8 B
constexpr int P_BYTES = 2 * 4 * 64 * 16;        // 8192: two buffers, alternating by tile
constexpr int KEYS_OFF = P_OFF + P_BYTES;
constexpr int MISC_OFF = KEYS_OFF + KEYCAP * 4;
constexpr int MISC_BYTES = 1408;
constexpr size_t LDS_BYTES = (size_t)MISC_OFF + MISC_BYTES;  // 163840
constexpr float TAU_HARD = 100.0f;              // largest exponent taken against the reference
static_assert(LDS_BYTES <= 163840, "one workgroup per CU");
static_assert(4 * MAX_LOADS + 4 * (MAX_LOADS - 1) == TILE_LOADS, "gather split over the waves");
// misc layout (4-byte words): [0] restart request, [8 + w] wave w's key count,
// [16 + w] wave w saw a freshly appended key, [24..25] workgroup first
// violation (8 bytes), [32 + h] head h's floor for the reference (the maxima
// of an abandoned pass), [96 ..] per-wave exchange of 16 floats (w * 16 + c16)
// and, at the end, each wave's (reference, row sum) per head, 2 x 128 floats
constexpr int M_RESTART = 0, M_LAST = 8, M_FRESH = 16, M_MINKEY = 24, M_FLOOR = 32, M_XCH = 96;
static_assert((M_XCH + 256) * 4 <= MISC_BYTES, "misc layout");
}  // namespace lhd

// APPEND (with FUSED): the launch also appends the batch's cur_len current
// rows to the cache in place (rows past_len[b] ..) and writes present_len[b];
// a workgroup that gathers one of them writes the batch's new rows itself
// before it gathers, so it reads its own writes whatever other workgroups do;
// with `reset` the launch's last finisher replaces the error word instead of
// adding to it.
template <bool I64, bool FUSED, bool SOFTCAP, bool APPEND>
__global__ void __launch_bounds__(lhd::THREADS, 1)
latent_decode_kernel(const uint16_t* __restrict__ q, uint8_t* __restrict__ cache,
                     const void* __restrict__ idx, const int32_t* __restrict__ valid_len,
                     uint16_t* __restrict__ y, float* __restrict__ part_o, float* __restrict__ part_ml,
                     int64_t q_seq, int64_t rows, int64_t cap, int64_t width, int splits, float scale,
                     float softcap, ErrorBlock* __restrict__ eb, unsigned long long* __restrict__ row_key,
                     unsigned* __restrict__ row_done, const uint8_t* __restrict__ cur,
                     const int32_t* __restrict__ past_len, int32_t* __restrict__ present_len, int64_t cur_len,
                     int reset) {
  using namespace lhd;
  extern __shared__ __attribute__((aligned(1024))) uint8_t lds_raw[];
  lds_u8* ring = (lds_u8*)lds_raw;
  int* keys_s = (int*)(lds_raw + KEYS_OFF);
  int* misc = (int*)(lds_raw + MISC_OFF);
  float* xch = (float*)(misc + M_XCH);
  float* floor_s = (float*)(misc + M_FLOOR);
  unsigned long long* minkey_s = (unsigned long long*)(misc + M_MINKEY);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hb = wave >> 1;  // head block of the scores
  const int kh = wave & 1;   // key half of the scores
  const int g = lane >> 4;
  const int c16 = lane & 15;
  // this wave's share of a tile's 36 gather loads
  const int nload = wave < 4 ? MAX_LOADS : MAX_LOADS - 1;
  const int block0 = wave < 4 ? MAX_LOADS * wave : (MAX_LOADS - 1) * wave + 4;

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
  const uint8_t* cache_b = cache + b * cap * ROWB;
  const __amdgpu_buffer_rsrc_t crsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)cache_b, (short)0, (int)(cap * ROWB), 0x00020000);

  // columns of the index row this workgroup owns
  const int wtiles = (int)((width + KT - 1) / KT);
  const int tps = (wtiles + splits - 1) / splits;
  const int c0 = (int)min((int64_t)split * tps * KT, width);
  const int c1 = (int)min((int64_t)c0 + (int64_t)tps * KT, width);

  // ---- per-lane LDS offsets within a tile
  // K (A operand of S^T): row 16 kh + c16, logical chunk 4 S + g, stored at
  // (4 S + g) ^ (c16 & 6) = 4 (S ^ f2) + (g ^ (kf & 2)); one base per parity
  // of S, 64 S an immediate.
  const int kf = c16 & 6;
  const int kbase = kh * HALF_ROWS + c16 * ROWB + ((g ^ (kf & 2)) << 4);
  const int kbase_e = kbase + ((kf >> 2) << 6);
  const int kbase_o = kbase - ((kf >> 2) << 6);
  // V^T (A operand of O^T): lane 4 jj + qq of group g points at row 4 g + jj,
  // dv 16 dt + 4 qq, i.e. chunk 2 dt + (qq >> 1) stored at 2 (dt ^ f') +
  // (qq >> 1); this wave's dv tiles are dt = 4 wave + d, at
  // vcommon + ((d ^ vflip) << 5), keys 16..31 at + HALF_ROWS.
  int vcommon, vflip;
  {
    const int jj = c16 >> 2, qq = c16 & 3;
    const int R = 4 * g + jj;
    vflip = (R & 6) >> 1;
    vcommon = R * ROWB + 128 * wave + ((qq >> 1) << 4) + ((qq & 1) << 3);
  }
  // probability exchange: [buffer][head block][lane][kh] x 8 bytes; a PV read
  // of 16 bytes at [buffer][h][lane] is the B operand of head block h as the
  // MFMA takes it (lane (c16, g): head c16, keys 4 g .. 4 g + 3, then
  // 16 + 4 g .. 16 + 4 g + 3)
  const uint32_t p_base = (uint32_t)(uintptr_t)(lds_raw + P_OFF);
  const uint32_t p_wr = p_base + (uint32_t)((hb * 64 + lane) * 16 + kh * 8);
  const uint32_t p_rd = p_base + (uint32_t)(lane * 16);
  // gather: this wave's loads cover 1 KB blocks block0 + i of the tile; lane
  // l of block k fills tile slot 64 k + l = row R, chunk p, which holds
  // logical chunk p ^ (R & 6) of that row
  auto ld_row = [&](int i) { return (64 * (block0 + i) + lane) / 72; };
  auto ld_off = [&](int i) {
    const int sl = 64 * (block0 + i) + lane;
    const int R = sl / 72;
    return ((sl - 72 * R) ^ (R & 6)) << 4;
  };
  const float f = SOFTCAP ? kLog2eL : scale * kLog2eL;  // scores -> log2 units

  bf16x8_l qreg[KSTEPS];
  f32x4_l o[DVW][4];
  float m_ref, l_run, m_seen;
  unsigned long long mk = ~0ull;
  int vhi = c0;

  // Stage columns [st0, st1): keys (clamped into the cache) to keys_s, each
  // wave's count of keys up to its last non-padding column to misc, and the
  // columns not validated before checked. load_keys issues the index loads
  // (the raw words are widened where they are used); keys_to_lds, called with
  // no reader of keys_s / misc left, consumes them.
  constexpr int PER = (KEYCAP + THREADS - 1) / THREADS;
  using IdxT = typename std::conditional<I64, int64_t, int32_t>::type;
  IdxT kv[PER], ku[PER];
  auto load_keys = [&](int st0, int st1) {
    const int need = (st1 - st0 + THREADS - 1) / THREADS;  // uniform
    const bool check = FUSED && st0 >= vhi;
    const IdxT* ip = (const IdxT*)idx + ibase;
#pragma unroll
    for (int k = 0; k < PER; k++) {
      if (k == 0 || k < need) {
        const int c = min(st0 + tid + THREADS * k, st1 - 1);
        kv[k] = ip[c];
        if (check) ku[k] = ip[max(c - 1, 0)];
      }
    }
  };
  auto keys_to_lds = [&](int st0, int st1) {
    const int need = (st1 - st0 + THREADS - 1) / THREADS;
    const bool check = FUSED && st0 >= vhi;
    int last = 0, fresh = 0;
#pragma unroll
    for (int k = 0; k < PER; k++) {
      const int s = tid + THREADS * k;
      const int c = st0 + s;
      if ((k == 0 || k < need) && c < st1) {
        const int64_t vk = (int64_t)kv[k];
        keys_s[s] = (int)((vk >= 0 && vk < bound) ? vk : 0);  // clamp: a bad row stays in bounds
        if (vk != -1) last = s + 1;
        if (APPEND && vk >= app_p && vk < bound) fresh = 1;
        if (check && column_class(c, vk, (int64_t)ku[k], bound))
          mk = min(mk, (unsigned long long)(row * (width + 1) + c));
      }
    }
    if (check) vhi = st1;
    last = wave_max_nonneg(last);
    if (lane == 0) misc[M_LAST + wave] = last;
    if constexpr (APPEND) {
      fresh = wave_max_nonneg(fresh);
      if (lane == 0) misc[M_FRESH + wave] = fresh;
    }
    if (tid == 0) misc[M_RESTART] = 0;
  };
  const bool duty = split == 0 && qi == 0;
  bool app_done = false;
  auto append_rows = [&]() {
    if (app_ok) {
      const uint4* src = (const uint4*)(cur + b * cur_len * ROWB);
      uint4* dst = (uint4*)(cache + (b * cap + app_p) * ROWB);
      for (int u = tid; u < cur_len * (ROWB / 16); u += THREADS) dst[u] = src[u];
    }
    app_done = true;
  };

  // ---- the current stage: its key count, tile count and gathers
  int kcount = 0, ntile = 0;
  // After the staged keys are visible: the stage's key and tile counts; with
  // APPEND, a stage that gathers a freshly appended row first stores the
  // batch's current rows.
  auto stage_counts = [&]() {
    int kc = 0;
#pragma unroll
    for (int w = 0; w < WAVES; w++) kc = max(kc, misc[M_LAST + w]);
    kcount = kc;
    ntile = (kcount + KT - 1) / KT;
    if constexpr (APPEND) {
      int fr = 0;
#pragma unroll
      for (int w = 0; w < WAVES; w++) fr |= misc[M_FRESH + w];
      if (fr != 0) {
        if (!app_done) append_rows();
        __syncthreads();  // the stores have landed before the gathers
      }
    }
  };
  // The gather of tile tt: this wave's loads, buffer loads from the batch's
  // cache rows at byte offsets goff[i]. A slot past the keys gets an offset
  // beyond the buffer's size, for which the range check returns zeros (its V
  // rows must not hold garbage: P = 0 there, and 0 * inf is NaN). A tile past
  // the last one is "gathered" too (all offsets out of range), so the issue
  // is unconditional and the counted waits stay exact; its key reads are
  // clamped into the staged keys.
  uint32_t goff[MAX_LOADS];
  // (the slot geometry is recomputed from the lane id each time rather than
  // held in ten registers across the kernel)
  auto gather_offsets = [&](int tt) {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int tk = tt < ntile ? tt : 0;
    int gkey[MAX_LOADS], grow[MAX_LOADS];
#pragma unroll
    for (int i = 0; i < MAX_LOADS; i++) {
      grow[i] = (64 * (block0 + i) + ln) / 72;
      gkey[i] = keys_s[tk * KT + min(grow[i], KT - 1)];
    }
#pragma unroll
    for (int i = 0; i < MAX_LOADS; i++) {
      const int sl = 64 * (block0 + i) + ln;
      const int lo = ((sl - 72 * grow[i]) ^ (grow[i] & 6)) << 4;
      goff[i] = tt * KT + grow[i] < kcount ? __umul24((uint32_t)gkey[i], (uint32_t)ROWB) + (uint32_t)lo : 0x80000000u;
      asm volatile("" : "+v"(goff[i]));
    }
  };
  auto gather_one = [&](int tt, int i) {
    lds_u8* dst = ring + (tt % NSTAGE) * TILE_BYTES + (block0 + i) * 1024;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(crsrc, (__attribute__((address_space(3))) void*)dst, 16, goff[i], 0, 0,
                                             0);
  };
  auto gather_issue = [&](int tt) {
#pragma unroll
    for (int i = 0; i < MAX_LOADS; i++)
      if (i < nload) gather_one(tt, i);
  };
  // counted waits: this wave's loads of `tiles` later tiles may stay in flight
  auto wait_tiles = [&](auto tiles) {
    constexpr int T = decltype(tiles)::value;
    if (wave < 4) wait_vm<T * MAX_LOADS>();
    else wait_vm<T * (MAX_LOADS - 1)>();
  };

  // ---- the first stage. The index loads go out first; the workgroup's Q (64
  // head rows of 1152 bytes: two tiles' worth) follows into ring slots 2 and
  // 3 with the tiles' own gather pattern and swizzle (whole cache lines, each
  // row fetched once). Tiles 0 and 1 are gathered as soon as the keys are
  // staged, while Q is still landing; then each wave reads its head block's B
  // operands with the K-read pattern (lane (c16, g) holds dims 32 S + 8 g ..
  // + 8 of head 16 hb + c16) by counted reads (a compiler-visible read of the
  // ring would wait for the tile gathers too), and slots 2 and 3 return to
  // the ring.
  if (tid < NH) floor_s[tid] = -INFINITY;  // read after the first stage's barrier
  bool pro_done = false;
  if (c0 < c1) {
    const int st1 = min(c0 + KEYCAP, c1);
    load_keys(c0, st1);
    const uint16_t* qrow0 = q + ((b * NH) * q_seq + qi) * DK;
    const int qstride = (int)(q_seq * ROWB);  // bytes between heads (63 strides fit 32 bits: checked at launch)
    const __amdgpu_buffer_rsrc_t qrsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)qrow0, (short)0, (NH - 1) * qstride + ROWB, 0x00020000);
#pragma unroll
    for (int u = 0; u < 2; u++)
#pragma unroll
      for (int i = 0; i < MAX_LOADS; i++)
        if (i < nload)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              qrsrc, (__attribute__((address_space(3))) void*)(ring + (2 + u) * TILE_BYTES + (block0 + i) * 1024), 16,
              (uint32_t)((32 * u + ld_row(i)) * qstride + ld_off(i)), 0, 0, 0);
    keys_to_lds(c0, st1);
    lds_barrier();
    stage_counts();
    gather_offsets(0);
    gather_issue(0);
    gather_offsets(1);
    gather_issue(1);
    wait_tiles(std::integral_constant<int, 2>{});  // this wave's Q loads have landed (tiles 0, 1 in flight)
    lds_barrier();                                 // and everyone's
    {
      // head 16 hb + c16 is row 16 (hb & 1) + c16 of slot 2 + (hb >> 1)
      const uint32_t qa_e = (uint32_t)(uintptr_t)(ring + (2 + (hb >> 1)) * TILE_BYTES + (hb & 1) * HALF_ROWS) +
                            (uint32_t)(kbase_e - kh * HALF_ROWS);
      const uint32_t qa_o = qa_e + (uint32_t)(kbase_o - kbase_e);
      u32x4_l qraw[KSTEPS];
      static_for<KSTEPS>([&](auto sc) {
        constexpr int S = decltype(sc)::value;
        qraw[S] = ds_read_b128_at<64 * S>((S & 1) ? qa_o : qa_e);
      });
      static_for<KSTEPS / 2>([&](auto pc) {
        constexpr int P = decltype(pc)::value;
        constexpr int LATER = KSTEPS - 2 * P - 2;
        lgkm_wait_tied<(LATER > 15 ? 15 : LATER)>(qraw[2 * P], qraw[2 * P + 1]);
      });
#pragma unroll
      for (int s = 0; s < KSTEPS; s++) qreg[s] = __builtin_bit_cast(bf16x8_l, qraw[s]);
    }
    lds_barrier();  // every wave has its Q: slots 2 and 3 return to the ring
    gather_offsets(2);
    gather_issue(2);
    gather_offsets(NSTAGE - 1);
    pro_done = true;
  }

  const uint32_t p_buf = 4096;  // the two probability buffers alternate by tile parity
  f32x4_l sacc;
  // ---- softmax of tile tt from sacc into probability buffer pb: lane holds
  // keys 16 kh + 4 g + r of head 16 hb + c16, in log2 units rounded once (the
  // maximum then gives exp2(0) exactly); the pass's first tile fixes the
  // reference of both waves of the head block
  auto softmax_write = [&](bool first, int tt, uint32_t pb) {
    // the scores come straight from the last matrix instruction, sometimes
    // across a branch, where the compiler has been seen to leave too little
    // padding before the first read: eight slots here, tied to the values
    asm volatile("s_nop 7" : "+v"(sacc));
    float x[4];
    {
#pragma unroll
      for (int r = 0; r < 4; r++) x[r] = sacc[r];
    }
    if constexpr (SOFTCAP) {
#pragma unroll
      for (int r = 0; r < 4; r++) x[r] = softcap * tanhf(x[r] * scale / softcap);
    }
    if ((tt + 1) * KT > kcount) {  // uniform: only the last tile has empty slots
      const int slot_base = tt * KT + 16 * kh + 4 * g;
#pragma unroll
      for (int r = 0; r < 4; r++)
        if (slot_base + r >= kcount) x[r] = -INFINITY;
    }
#pragma unroll
    for (int r = 0; r < 4; r++) x[r] *= f;
    const float tmax = max_x32(max_x16(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]))));
    m_seen = fmaxf(m_seen, tmax);
    if (first) {  // uniform
      int ln = lane;  // the exchange addresses are recomputed rather than held
      asm volatile("" : "+v"(ln));
      const int cc = ln & 15;
      if (ln < 16) xch[16 * wave + cc] = tmax;
      lds_barrier();
      const float other = xch[16 * (wave ^ 1) + cc];
      const float both = kh == 0 ? fmaxf(tmax, other) : fmaxf(other, tmax);
      m_ref = fmaxf(both, floor_s[16 * hb + cc]);
    }
    // a score more than 2^TAU_HARD above the reference: the pass is redone
    if (tmax > m_ref + TAU_HARD) misc[M_RESTART] = 1;  // benign race: every writer stores 1
    const float nm = m_ref == -INFINITY ? 0.0f : -m_ref;
    float pv[4];
#pragma unroll
    for (int r = 0; r < 4; r++) pv[r] = __builtin_amdgcn_exp2f(x[r] + nm);
    l_run += sum_x32(sum_x16((pv[0] + pv[1]) + (pv[2] + pv[3])));
    ds_write_b64_at(p_wr + pb, (u32x2_l){pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3])});
  };
  auto tile_addr = [&](int tt) { return (uint32_t)(uintptr_t)(ring + (tt % NSTAGE) * TILE_BYTES); };
  u32x4_l kr[KSTEPS];
  s16x4_l vr0[DVW], vr1[DVW];
  uint32_t ka_e = 0, ka_o = 0, va[DVW] = {0, 0, 0, 0};
  auto set_k = [&](int tt) {
    const uint32_t T = tile_addr(tt);
    ka_e = T + kbase_e;
    ka_o = T + kbase_o;
  };
  auto set_v = [&](int tt) {
    const uint32_t T = tile_addr(tt);
#pragma unroll
    for (int d = 0; d < DVW; d++) va[d] = T + vcommon + ((d ^ vflip) << 5);
  };
  auto kread = [&](auto sc) {
    constexpr int S = decltype(sc)::value;
    kr[S] = ds_read_b128_at<64 * S>((S & 1) ? ka_o : ka_e);
  };
  auto kmfma = [&](auto sc) {
    constexpr int S = decltype(sc)::value;
    sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_l, kr[S]), qreg[S], sacc, 0, 0, 0);
  };
  auto vread = [&](auto dc) {
    constexpr int D = decltype(dc)::value;
    vr0[D] = ds_read_tr16_at<0>(va[D]);
    vr1[D] = ds_read_tr16_at<HALF_ROWS>(va[D]);
  };
  // PV of dv tile D for head block H
  auto vmfma = [&](auto dc, auto hc, const bf16x8_l* pb) {
    constexpr int D = decltype(dc)::value;
    constexpr int H = decltype(hc)::value;
    const s16x4_l a8[2] = {vr0[D], vr1[D]};
    o[D][H] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_l, a8), pb[H], o[D][H], 0, 0, 0);
  };
  // the four head blocks' probabilities of tile tt (buffer by parity)
  auto pread = [&](int tt, u32x4_l* pr) {
    const uint32_t a = p_rd + ((tt & 1) ? p_buf : 0u);
    pr[0] = ds_read_b128_at<0>(a);
    pr[1] = ds_read_b128_at<1024>(a);
    pr[2] = ds_read_b128_at<2048>(a);
    pr[3] = ds_read_b128_at<3072>(a);
  };
  // the same, returned complete: reads and wait in one statement, so no copy
  // of a register still being written can be placed between them
  auto pread_now = [&](int tt, u32x4_l* pr) {
    const uint32_t a = p_rd + ((tt & 1) ? p_buf : 0u);
    asm volatile(
        "ds_read_b128 %0, %4\n\tds_read_b128 %1, %4 offset:1024\n\t"
        "ds_read_b128 %2, %4 offset:2048\n\tds_read_b128 %3, %4 offset:3072\n\ts_waitcnt lgkmcnt(0)"
        : "=&v"(pr[0]), "=&v"(pr[1]), "=&v"(pr[2]), "=&v"(pr[3])
        : "v"(a)
        : "memory");
  };

  bool first_tile = true;
  for (;;) {
#pragma unroll
    for (int d = 0; d < DVW; d++)
#pragma unroll
      for (int h = 0; h < 4; h++) o[d][h] = (f32x4_l){0.f, 0.f, 0.f, 0.f};
    l_run = 0.0f;
    m_seen = -INFINITY;
    m_ref = -INFINITY;
    bool restart = false;
    first_tile = true;

    for (int st0 = c0; st0 < c1 && !restart; st0 += KEYCAP) {
      const int st1 = min(st0 + KEYCAP, c1);
      if (!pro_done) {
        __syncthreads();  // the previous stage's readers are done with keys_s / misc / the ring
        load_keys(st0, st1);
        keys_to_lds(st0, st1);
        lds_barrier();
        stage_counts();
#pragma unroll
        for (int p = 0; p < NSTAGE - 1; p++) {
          gather_offsets(p);
          gather_issue(p);
        }
        gather_offsets(NSTAGE - 1);
      }
      pro_done = false;
      if (ntile == 0) continue;  // uniform: only padding in these columns

      // ---- tile 0: S alone, the K reads KD k-steps ahead of their MFMAs
      // (tiles 1 .. NSTAGE-2 may stay in flight)
      wait_tiles(std::integral_constant<int, NSTAGE - 2>{});
      lds_barrier();
      set_k(0);
      sacc = (f32x4_l){0.f, 0.f, 0.f, 0.f};
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
      softmax_write(first_tile, 0, 0u);
      first_tile = false;

      // ---- steady state: S of tile t+1 interleaved with PV of tile t. Step
      // J does k-step J of the scores (1 K read, 1 MFMA) and, for J < 16, the
      // PV of dv tile J / 4 for head block J % 4 (1 MFMA; the tile's 2 V reads
      // at J % 4 == 0), the reads PL steps ahead; then the softmax of tile t+1
      // into the other probability buffer. This wave's gather of tile t+3 goes
      // out one load per step.
      for (int t = 0; t < ntile; t++) {
        wait_tiles(std::integral_constant<int, NSTAGE - 3>{});  // tile t+1 has landed for this wave
        lds_barrier();  // and for everyone; P(t) is complete; tile t-1's slot is free
        const int tn = t + NSTAGE - 1;
        u32x4_l pr[4];
        set_v(t);
        bf16x8_l pb[4];
        if (t + 1 < ntile) {
          pread(t, pr);
          set_k(t + 1);
          sacc = (f32x4_l){0.f, 0.f, 0.f, 0.f};
          constexpr int PL = 3;
          auto step_reads = [](int j) { return j < KSTEPS ? 1 + ((j < 4 * DVW && j % 4 == 0) ? 2 : 0) : 0; };
          auto sread = [&](auto jc) {
            constexpr int J = decltype(jc)::value;
            if constexpr (J < KSTEPS) kread(jc);
            if constexpr (J < 4 * DVW && J % 4 == 0) vread(std::integral_constant<int, J / 4>{});
          };
          static_for<PL>(sread);
          static_for<KSTEPS>([&](auto jc) {
            constexpr int J = decltype(jc)::value;
            if constexpr (J + PL < KSTEPS) sread(std::integral_constant<int, J + PL>{});
            if constexpr (J < MAX_LOADS) {
              if (J < nload) gather_one(tn, J);
            }
            // LDS reads issued after step J's: those of steps J+1 .. J+PL
            constexpr int LATER = step_reads(J + 1) + step_reads(J + 2) + step_reads(J + 3);
            if constexpr (J == 0) {
              // the probability reads were issued before every step read
              constexpr int AFTER_P = LATER + step_reads(0);
              lgkm_wait_tied<AFTER_P + 2>(pr[0], pr[1]);
              lgkm_wait_tied<AFTER_P>(pr[2], pr[3]);
#pragma unroll
              for (int h = 0; h < 4; h++) pb[h] = __builtin_bit_cast(bf16x8_l, pr[h]);
            }
            if constexpr (J < 4 * DVW && J % 4 == 0) {
              lgkm_wait3<LATER>(kr[J], vr0[J / 4], vr1[J / 4]);
            } else {
              lgkm_wait_tied1<LATER>(kr[J]);
            }
            kmfma(jc);
            if constexpr (J < 4 * DVW)
              vmfma(std::integral_constant<int, J / 4>{}, std::integral_constant<int, J % 4>{}, pb);
            __builtin_amdgcn_sched_barrier(0);
          });
          softmax_write(false, t + 1, ((t + 1) & 1) ? p_buf : 0u);
        } else {
          // the last tile's PV alone: its probabilities, then all of its V
          // reads ahead
          pread_now(t, pr);
#pragma unroll
          for (int h = 0; h < 4; h++) pb[h] = __builtin_bit_cast(bf16x8_l, pr[h]);
          static_for<DVW>(vread);
          static_for<DVW>([&](auto dc) {
            constexpr int D = decltype(dc)::value;
            lgkm_wait_tied<2 * (DVW - 1 - D)>(vr0[D], vr1[D]);
            static_for<4>([&](auto hc) { vmfma(dc, hc, pb); });
            __builtin_amdgcn_sched_barrier(0);
          });
          gather_issue(tn);
        }
        gather_offsets(t + NSTAGE);  // offsets of the next iteration's gather
      }
      __syncthreads();
      restart = misc[M_RESTART] != 0;
    }
    if (!restart) break;
    // both waves of a head block restart from the same maxima
    __syncthreads();
    if (g == 0) xch[16 * wave + c16] = m_seen;
    __syncthreads();
    if (kh == 0 && g == 0) {
      const float other = xch[16 * (wave ^ 1) + c16];
      floor_s[16 * hb + c16] = fmaxf(floor_s[16 * hb + c16], fmaxf(m_seen, other));
    }
  }

  // ---- each head's reference and both key halves' row sums, to the waves
  // that hold its outputs: xch[w * 16 + c16] = reference, xch[128 + ...] = sum
  __syncthreads();
  if (g == 0) {
    xch[16 * wave + c16] = m_ref;
    xch[128 + 16 * wave + c16] = l_run;
  }
  if constexpr (FUSED) {
    if (c0 == 0 && tid == 0 && width > 0 && load_index<I64>(idx, ibase) == -1)
      mk = min(mk, (unsigned long long)(row * (width + 1) + width));  // all -1, unless a column fails
    if (tid == 0) *minkey_s = ~0ull;
  }
  __syncthreads();
  if constexpr (FUSED) {
    if (mk != ~0ull) atomicMin(minkey_s, mk);
  }
  // the row sum of head 16 h + c16, key halves added in order
  auto l_total = [&](int h) { return xch[128 + 32 * h + c16] + xch[128 + 32 * h + 16 + c16]; };

  // ---- epilogue: lane holds O^T[64 wave + 16 d + 4 g + r][16 h + c16]. Every
  // head's output is normalised by its row sum and rounded to bf16, then
  // written as whole 1 KB rows through LDS: to Y when the keys are not split,
  // else to the split's partial (the merge kernel combines the splits with
  // their (reference, row sum) pairs, which stay fp32). The partials are
  // written through the L2 as they are stored, so the end of the launch has
  // no 16 MB of dirty partials to write back before the merge can start.
  {
    constexpr int YROW = 1024 + 16;  // padded: the 16 heads of one write hit distinct banks
    __syncthreads();                 // the ring is free
#pragma unroll
    for (int h = 0; h < 4; h++) {
      const float lt = l_total(h);
      const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
      lds_u8* yl = ring + (16 * h + c16) * YROW + 128 * wave + 8 * g;
#pragma unroll
      for (int d = 0; d < DVW; d++) {
        const uint32_t lo = pack_bf16x2(o[d][h][0] * inv, o[d][h][1] * inv);
        const uint32_t hi = pack_bf16x2(o[d][h][2] * inv, o[d][h][3] * inv);
        *(__attribute__((address_space(3))) u32x2_l*)(yl + 32 * d) = (u32x2_l){lo, hi};
      }
    }
    if (splits > 1 && kh == 0 && g == 0) {
      const __amdgpu_buffer_rsrc_t mrsrc = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(part_ml + ((row * splits + split) * NH) * 2), (short)0, NH * 8, 0x00020000);
      const u32x2_l ml = {__float_as_uint(m_ref), __float_as_uint(l_total(hb))};
      __builtin_amdgcn_raw_buffer_store_b64(ml, mrsrc, (16 * hb + c16) * 8, 0, kWriteThrough);
    }
    __syncthreads();
    if (splits == 1) {
      uint16_t* dst = y + (b * NH * q_seq + qi) * DV;
#pragma unroll 4
      for (int hq = 0; hq < 8; hq++) {
        const int hd = 8 * wave + hq;
        const u32x4_l v = *(const lds_u32x4*)(ring + hd * YROW + 16 * lane);
        *(u32x4_l*)(dst + hd * q_seq * DV + 8 * lane) = v;
      }
    } else {
      const __amdgpu_buffer_rsrc_t prsrc = __builtin_amdgcn_make_buffer_rsrc(
          (void*)((uint16_t*)part_o + (row * splits + split) * NH * DV), (short)0, NH * DV * 2, 0x00020000);
#pragma unroll 4
      for (int hq = 0; hq < 8; hq++) {
        const int hd = 8 * wave + hq;
        const u32x4_l v = *(const lds_u32x4*)(ring + hd * YROW + 16 * lane);
        __builtin_amdgcn_raw_buffer_store_b128(v, prsrc, hd * (DV * 2) + 16 * lane, 0, kWriteThrough);
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

  // ---- error block: with split keys this workgroup's first violation goes
  // to the row's slot, and the merge kernel that follows the launch records
  // each row's first violation and finishes the launch's record; a row's only
  // workgroup records its row and counts it toward the launch's record itself
  if constexpr (FUSED) {
    __syncthreads();  // every wave's LDS minimum is in
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

// Log-sum-exp merge of the split partials (standard Attention page,
// `attention_combine`; m in log2 units): M = max_j m_j and
// y = sum_j l_j 2^(m_j - M) o_j / sum_j l_j 2^(m_j - M), o_j the split's
// output normalised by its own row sum l_j and stored as bf16 (Y's own
// precision: the merge adds at most one bf16 rounding of each split's output). One 128-thread workgroup
// per (row, head), each thread 4 channels; block i serves row i % rows, on
// the XCD that wrote that row's partials. Each round loads 8 splits before
// using any. With FIN (fused validation) the workgroup of head 0 of each row
// then turns the row's first violation (the minimum the split workgroups left
// in row_key) into its class bit and counts the row toward the launch's
// record: the finish that would otherwise cost the attention launch a
// device-wide round trip per workgroup at its end.
template <bool FIN, bool I64>
__global__ void __launch_bounds__(128)
latent_merge_kernel(const uint16_t* __restrict__ part_o, const float* __restrict__ part_ml, uint16_t* __restrict__ y,
                    int64_t rows, int64_t q_seq, int splits, ErrorBlock* __restrict__ eb,
                    unsigned long long* __restrict__ row_key, const void* __restrict__ idx, int64_t width,
                    const int32_t* __restrict__ valid_len, const int32_t* __restrict__ past_len,
                    const int32_t* __restrict__ present_len, int64_t cur_len, int64_t cap, int reset) {
  using namespace lhd;
  constexpr int CH = 8;
  const int64_t row = (int64_t)(blockIdx.x % (unsigned)rows);
  const int head = (int)(blockIdx.x / (unsigned)rows);
  const int64_t b = row / q_seq, qi = row - b * q_seq;
  const int d = threadIdx.x * 4;
  // y = sum_j w_j o_j / sum_j w_j with w_j = l_j 2^(m_j - M) and o_j the
  // split's normalised output; M is raised as later splits come in
  float M = -INFINITY, L = 0.0f;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int j0 = 0; j0 < splits; j0 += CH) {
    float2 ml[CH];
    uint2 v[CH];
#pragma unroll
    for (int j = 0; j < CH; j++) {
      const int64_t pr = (row * splits + j0 + j) * NH + head;
      if (j0 + j < splits) {
        ml[j] = *(const float2*)(part_ml + pr * 2);
        v[j] = *(const uint2*)(part_o + pr * DV + d);
      } else {
        ml[j] = make_float2(-INFINITY, 0.0f);
        v[j] = make_uint2(0u, 0u);
      }
    }
    float Mn = M;
#pragma unroll
    for (int j = 0; j < CH; j++) Mn = fmaxf(Mn, ml[j].x);
    if (Mn == -INFINITY) continue;  // no key in these splits yet
    const float r = M == -INFINITY ? 0.0f : exp2f(M - Mn);
    L *= r;
#pragma unroll
    for (int e = 0; e < 4; e++) acc[e] *= r;
#pragma unroll
    for (int j = 0; j < CH; j++) {
      const float w = ml[j].x == -INFINITY ? 0.0f : ml[j].y * exp2f(ml[j].x - Mn);
      L += w;
      acc[0] += w * __uint_as_float(v[j].x << 16);
      acc[1] += w * __uint_as_float(v[j].x & 0xffff0000u);
      acc[2] += w * __uint_as_float(v[j].y << 16);
      acc[3] += w * __uint_as_float(v[j].y & 0xffff0000u);
    }
    M = Mn;
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  *(uint2*)(y + ((b * NH + head) * q_seq + qi) * DV + d) =
      make_uint2(pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv));

  if constexpr (FIN) {
    if (head != 0 || threadIdx.x != 0) return;
    const unsigned long long k = atomicExch(&row_key[row], ~0ull);
    if (k != ~0ull) {
      int64_t bound = past_len ? (int64_t)past_len[b] + cur_len : (valid_len ? (int64_t)valid_len[b] : cap);
      bound = bound < 0 ? 0 : (bound > cap ? cap : bound);
      record_row_violation<I64>(eb, idx, row, width, k, bound);
    }
    // the launch's other inputs were written before it began: no cache fences
    finish_launch<I64, false>(eb, idx, width, q_seq, q_seq, past_len ? present_len : valid_len, cap,
                              (unsigned)rows, reset != 0);
  }
}

sa_status launch_latent_merge(sparse_attn_ctx* c, const FwdArgs& a, int64_t rows, int splits, bool fused,
                                     const AppendArgs* app) {
  const dim3 grid((unsigned)(rows * lhd::NH)), block(lhd::DV / 4);
  const int32_t* plen = app ? app->past_len : nullptr;
  int32_t* prlen = app ? app->present_len : nullptr;
  const int64_t clen = app ? app->cur_len : 0;
  const int reset = app ? app->reset : 0;
#define SA_MERGE(F, I)                                                                                     \
  hipLaunchKernelGGL((latent_merge_kernel<F, I>), grid, block, 0, c->stream, (const uint16_t*)c->partial_o,      \
                     c->partial_ml,                                                                         \
                     (uint16_t*)a.y, rows, a.q_seq, splits, c->err, c->row_key, a.idx, a.width, a.valid_len, \
                     plen, prlen, clen, a.cap, reset)
  if (!fused) SA_MERGE(false, false);
  else if (a.idx64) SA_MERGE(true, true);
  else SA_MERGE(true, false);
#undef SA_MERGE
  return check_hip(c, hipGetLastError(), "forward (merge)");
}

static bool g_lhd_attr[12] = {};

// The kernel addresses a row's 64 query heads from one buffer resource:
// 63 head strides of q_seq rows plus one row must fit its 32-bit range.
bool latent_decode_fits(int64_t q_seq) {
  return q_seq >= 1 && (lhd::NH - 1) * q_seq * lhd::ROWB + lhd::ROWB <= 0x7fffffffLL;
}

sa_status launch_forward_latent_decode(sparse_attn_ctx* c, const FwdArgs& a, int splits, bool fused,
                                       const AppendArgs* app) {
  using namespace lhd;
  const int64_t rows = a.batch * a.q_seq;
  if (rows <= 0) return SA_OK;
  if (!latent_decode_fits(a.q_seq)) return set_error(c, SA_E_STATE, "forward: q_seq too large for the decode kernel");
  if (splits > 1 && rows * splits > c->partial_rows)
    return set_error(c, SA_E_STATE, "forward: split-K partials exceed the context's buffers");
  if (rows > c->rows_cap) return set_error(c, SA_E_STATE, "forward: more rows than the context holds");
  const int64_t wgs = rows * splits;
  if (wgs > 0x7fffffffLL) return set_error(c, SA_E_SHAPE, "forward: too many rows for one launch");
  const bool cap_on = a.softcap != 0.0f;
  if (app && (!fused || app->cur_len < 0 || app->cur_len > kFusedAppendRows))
    return set_error(c, SA_E_STATE, "forward: in-launch append needs fused validation and at most 8 rows");
  const int variant = app ? 8 + (a.idx64 ? 1 : 0) + (cap_on ? 2 : 0)
                          : (a.idx64 ? 1 : 0) + (fused ? 2 : 0) + (cap_on ? 4 : 0);
  const void* fns[12] = {(const void*)latent_decode_kernel<false, false, false, false>,
                         (const void*)latent_decode_kernel<true, false, false, false>,
                         (const void*)latent_decode_kernel<false, true, false, false>,
                         (const void*)latent_decode_kernel<true, true, false, false>,
                         (const void*)latent_decode_kernel<false, false, true, false>,
                         (const void*)latent_decode_kernel<true, false, true, false>,
                         (const void*)latent_decode_kernel<false, true, true, false>,
                         (const void*)latent_decode_kernel<true, true, true, false>,
                         (const void*)latent_decode_kernel<false, true, false, true>,
                         (const void*)latent_decode_kernel<true, true, false, true>,
                         (const void*)latent_decode_kernel<false, true, true, true>,
                         (const void*)latent_decode_kernel<true, true, true, true>};
  if (!g_lhd_attr[variant]) {
    hipError_t e = hipFuncSetAttribute(fns[variant], hipFuncAttributeMaxDynamicSharedMemorySize, (int)LDS_BYTES);
    if (e != hipSuccess) return check_hip(c, e, "forward (latent decode) LDS attribute");
    g_lhd_attr[variant] = true;
  }
  const dim3 grid((unsigned)wgs), block(THREADS);
  const ProfEvents pe = prof_next(c);
  const uint8_t* cur = app ? (const uint8_t*)app->cur : nullptr;
  const int32_t* plen = app ? app->past_len : nullptr;
  int32_t* prlen = app ? app->present_len : nullptr;
  const int64_t clen = app ? app->cur_len : 0;
  const int reset = app ? app->reset : 0;
#define SA_LHD(I, F, C, A)                                                                            \
  SA_MAIN_LAUNCH(pe, (latent_decode_kernel<I, F, C, A>), grid, block, LDS_BYTES, c->stream,           \
                     (const uint16_t*)a.q, (uint8_t*)a.k, a.idx, a.valid_len, (uint16_t*)a.y,         \
                     c->partial_o, c->partial_ml, a.q_seq, rows, a.cap, a.width, splits, a.scale,     \
                     a.softcap, c->err, c->row_key, c->row_done, cur, plen, prlen, clen, reset)
  switch (variant) {
    case 0: SA_LHD(false, false, false, false); break;
    case 1: SA_LHD(true, false, false, false); break;
    case 2: SA_LHD(false, true, false, false); break;
    case 3: SA_LHD(true, true, false, false); break;
    case 4: SA_LHD(false, false, true, false); break;
    case 5: SA_LHD(true, false, true, false); break;
    case 6: SA_LHD(false, true, true, false); break;
    case 7: SA_LHD(true, true, true, false); break;
    case 8: SA_LHD(false, true, false, true); break;
    case 9: SA_LHD(true, true, false, true); break;
    case 10: SA_LHD(false, true, true, true); break;
    default: SA_LHD(true, true, true, true); break;
  }
#undef SA_LHD
  sa_status s = check_hip(c, hipGetLastError(), "forward (latent decode)");
  if (s != SA_OK || splits == 1) return s;
  return launch_latent_merge(c, a, rows, splits, fused, app);
}

}  // namespace sa
