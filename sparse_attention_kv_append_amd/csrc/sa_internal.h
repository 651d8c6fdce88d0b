// Internal declarations shared by the library's translation units (host
// launchers, the context, small device helpers). Not part of the ABI.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <string>
#include <vector>

#include "../../include/sparse_attn.h"

namespace sa {

constexpr int kNumCUs = 256;  // MI355X: 8 XCDs x 32 CUs

struct ErrorBlock {  // device layout of the context's error state
  uint32_t word;        // OR-latched error bits
  uint32_t done_blocks; // validation blocks finished in the current launch
  uint64_t first_bad;   // row*(W+1)+col of the first failing call's first violation
  uint64_t call_key;    // the same, within the current validation launch
  int64_t detail_value; // index at first_bad
  int64_t detail_prev;  // index left of it (column > 0)
  int64_t detail_bound; // cache length of its batch
  int64_t detail_b, detail_h, detail_q, detail_col;  // where it is
  int32_t detail_class; // 1..6, 0 = no detail recorded
  uint32_t call_word;   // bits latched by the current forward launch, merged into word by its last arrival
};

}  // namespace sa

struct sparse_attn_ctx {
  uint32_t magic;
  sa_config cfg;
  hipStream_t stream;
  int device;
  sa::ErrorBlock* err;  // device
  float* partial_o;     // device: split-K unnormalised outputs
  float* partial_ml;    // device: split-K (max, sum) pairs
  int64_t partial_rows; // capacity of the partial buffers in (row, split) units
  float* gpart_o;       // device: grouped-query split-KV unnormalised outputs [(row, split)][128]
  float* gpart_ml;      // device: grouped-query split-KV (max, sum) pairs
  int64_t gpart_rows;   // capacity of those in (row, split) units
  uint8_t* zeros;       // device: 1 KB of zeros (source of padded tile slots)
  unsigned long long* row_key;  // device [rows_cap]: per-row first violation, fused validation
  unsigned* row_done;           // device [rows_cap]: splits of a row that finished validation
  int64_t rows_cap;
  std::string last_error;
  // optional timing of the main forward kernel
  std::vector<hipEvent_t> prof_start, prof_stop;
  int64_t prof_n;
};

namespace sa {

constexpr uint32_t kMagic = 0x53504154u;  // "SPAT"

// ---- device helpers ------------------------------------------------------

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t w = __float_as_uint(f);
  if ((w & 0x7f800000u) == 0x7f800000u && (w & 0x007fffffu)) return (uint16_t)((w >> 16) | 0x40u);
  w += 0x7fffu + ((w >> 16) & 1u);
  return (uint16_t)(w >> 16);
}

// the state of a reset error block (no bit latched, no violation recorded,
// the per-launch slots and counter armed); written by one thread
__device__ __forceinline__ void clear_error_block(ErrorBlock* e) {
  e->word = 0u;
  e->done_blocks = 0u;
  e->first_bad = ~0ull;
  e->call_key = ~0ull;
  e->detail_class = 0;
  e->call_word = 0u;
}

template <int DT>
__device__ __forceinline__ float load_elem(const void* p, int64_t i) {
  if constexpr (DT == SA_F32) {
    return ((const float*)p)[i];
  } else if constexpr (DT == SA_F16) {
    return (float)((const _Float16*)p)[i];
  } else {
    return bf16_to_f32(((const uint16_t*)p)[i]);
  }
}

template <int DT>
__device__ __forceinline__ void store_elem(void* p, int64_t i, float v) {
  if constexpr (DT == SA_F32) {
    ((float*)p)[i] = v;
  } else if constexpr (DT == SA_F16) {
    ((_Float16*)p)[i] = (_Float16)v;  // round to nearest even
  } else {
    ((uint16_t*)p)[i] = f32_to_bf16_rne(v);
  }
}

template <bool I64>
__device__ __forceinline__ int64_t load_index(const void* p, int64_t i) {
  if constexpr (I64) {
    return ((const int64_t*)p)[i];
  } else {
    return (int64_t)((const int32_t*)p)[i];
  }
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// ---- host launchers (one per translation unit) ---------------------------

sa_status launch_reset_error(sparse_attn_ctx* c);
constexpr int PEAK_READ_BLOCKS = 1024;  // workgroups (of 256 threads) of the read probe
sa_status launch_peak_copy(sparse_attn_ctx* c, void* dst, const void* src, int64_t bytes, void* sink);
sa_status launch_peak_mfma(sparse_attn_ctx* c, float* out, int64_t blocks, int iters);
sa_status launch_append_copy(sparse_attn_ctx* c, int64_t batch, int64_t heads, int64_t row_bytes,
                             const void* past, int64_t past_cap, const int32_t* past_len,
                             const void* cur, int64_t cur_len, void* present, int64_t present_cap,
                             bool copy_past, int32_t* present_len, const void* past2 = nullptr,
                             const void* cur2 = nullptr, void* present2 = nullptr);
sa_status launch_append_quantize(sparse_attn_ctx* c, int64_t batch, int64_t heads, int64_t dk,
                                 int64_t rope, const void* cur_bf16, int64_t cur_len,
                                 const int32_t* past_len, int64_t past_cap, void* present,
                                 int64_t present_cap, int32_t* present_len);
sa_status launch_validate(sparse_attn_ctx* c, const void* idx, int64_t batch, int64_t heads,
                          int64_t q_seq, int64_t width, const int32_t* valid_len,
                          int64_t cache_len, uint32_t* word, uint8_t* row_class,
                          uint64_t* first_bad);

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* idx;
  const int32_t* valid_len;
  void* y;
  int64_t batch, hq, hkv, q_seq, dk, dv, rope, cap, index_heads, width;
  float scale, softcap;
  int dtype, cache_format, kv_layout, idx64;
  // optional additive bias (config dtype), its shape right-aligned against
  // [B, Hq, Sq, cap] and padded with 1 on the left
  const void* bias = nullptr;
  int64_t bd[4] = {1, 1, 1, 1};
};

// the in-launch append of the shared-latent LDS-ring kernel: current rows
// already in the cache's storage format, written in place
struct AppendArgs {
  const void* cur;
  const void* cur_v = nullptr;  // separate K/V caches: the current V rows (cur holds K)
  const int32_t* past_len;
  int32_t* present_len;
  int64_t cur_len;
  int reset;  // the launch replaces the error word (reset, then this launch)
  int quant;  // fp8 records: cur holds bf16 rows to quantize (else packed records)
};
constexpr int64_t kFusedAppendRows = 8;  // current rows per batch the in-launch append takes

bool mla_supported(const sa_config& cfg, int64_t index_heads);
// the LDS-ring kernel: bf16 shared-latent rows, per-batch cache below 2 GiB
// (its gathers use 32-bit offsets from the batch's cache base)
bool latent_supported(const sa_config& cfg, int64_t index_heads);
// the wave-pair kernel: fp8_e4m3_block64 shared-latent records (64 RoPE dims),
// per-batch cache below 2 GiB (32-bit record offsets from the batch's base)
bool pair_supported(const sa_config& cfg, int64_t index_heads);
// the grouped-query kernel: bf16 separate K/V caches of 128 dims, one index
// list per (batch, query), group size up to 128, per-head cache below 2 GiB
bool gqa_supported(const sa_config& cfg, int64_t index_heads);
// split-KV count of the grouped-query kernel for these sizes (1 = no split)
int gqa_splits(const sparse_attn_ctx* c, int64_t batch, int64_t q_seq, int64_t width);
// (row, split) capacity of the grouped-query split-KV buffers a config needs
int64_t gqa_partial_rows(const sa_config& cfg);
int mla_splits(int64_t rows, int64_t width);
sa_status launch_forward_generic(sparse_attn_ctx* c, const FwdArgs& a);
// capacity-mode length recovery from the bias frontier: per batch entry,
// valid = 1 + the last key column with a finite bias, write = valid - cur_len
// (0 below cur_len); bd is the bias shape padded to rank 4
sa_status launch_capacity_lengths(sparse_attn_ctx* c, const void* bias, int dtype, const int64_t* bd,
                                  int64_t batch, int64_t keys, int64_t cur_len, int32_t* valid_len,
                                  int32_t* write_pos);
// the same, then each batch entry's current K and V rows (row_bytes, a
// multiple of 16; 16-byte aligned tensors) written in place at its write position
// (with reset_eb: the launch also resets that error block, as
// launch_reset_error would just before it)
sa_status launch_capacity_append(sparse_attn_ctx* c, const void* bias, int dtype, const int64_t* bd, int64_t batch,
                                 int64_t keys, int64_t cur_len, int32_t* valid_len, int32_t* write_pos,
                                 const void* cur_k, const void* cur_v, void* cache_k, void* cache_v, int64_t heads,
                                 int64_t row_bytes, ErrorBlock* reset_eb = nullptr);
sa_status launch_forward_mla(sparse_attn_ctx* c, const FwdArgs& a, int splits);
sa_status launch_forward_latent(sparse_attn_ctx* c, const FwdArgs& a, int splits, bool fused,
                                const AppendArgs* app = nullptr);
// the same rows without a bias on the eight-wave kernel: each wave scores one
// 16-head block over one key half and does the PV of one dv eighth for all
// heads, exchanging bf16 probabilities through LDS; split keys are merged by
// a second kernel
// whether a launch over q_seq queries fits the eight-wave kernel's addressing
bool latent_decode_fits(int64_t q_seq);
// log-sum-exp merge of split partials written as normalised bf16 rows with
// their fp32 (reference, row sum) pairs; with fused validation it also records
// each row's first violation and finishes the launch's record
sa_status launch_latent_merge(sparse_attn_ctx* c, const FwdArgs& a, int64_t rows, int splits, bool fused,
                              const AppendArgs* app);
sa_status launch_forward_latent_decode(sparse_attn_ctx* c, const FwdArgs& a, int splits, bool fused,
                                       const AppendArgs* app = nullptr);
sa_status launch_forward_pair(sparse_attn_ctx* c, const FwdArgs& a, int splits, bool fused,
                              const AppendArgs* app = nullptr);
// whether a grouped-query launch over q_seq queries validates (and appends) itself
bool gqa_fuses(const sa_config& cfg, int64_t q_seq);
// fused (exactly when app is given): the launch validates its index columns,
// records the error block itself and appends the current K/V rows in place
sa_status launch_forward_gqa(sparse_attn_ctx* c, const FwdArgs& a, bool fused, const AppendArgs* app);
// CSA ratio-4 selected sink attention (512-dim rows, 583-byte records)
struct CsaArgs {
  const float* q;          // [B, S, H, 512]
  const float* ckv;        // [B, Tcur, 512]
  const uint8_t* rec;      // [B, record_cap, 583]
  const int32_t* sel;      // [B, index_heads, S, topk]
  const float* sink;       // [H]
  const float* bias;       // NULL or right-aligned [bias_dims]
  const int64_t* total;    // device: total_sequence_length
  float* y;                // [B, S, H, 512]
  int64_t batch, q_seq, heads, cur_len, record_cap, index_heads, topk;
  int64_t bias_dims[4];
  float scale;
};
sa_status launch_csa_attention(sparse_attn_ctx* c, const CsaArgs& a);
// CSA ratio-4 selection producer (index head dim 128, RoPE 64, 68-byte FP4 keys)
struct CsaIndexArgs {
  const float* iq;         // [B, S, H, 128]
  const float* iw;         // [B, S, H]
  const uint8_t* keys;     // [B, key_cap, 68]
  const int64_t* total;    // device: total_sequence_length
  int32_t* selected;       // [B, out_heads, S, topk]
  void* workspace;         // csa_index_workspace_bytes(B S, H, key_cap)
  int64_t batch, q_seq, heads, key_cap, topk, out_heads;
};
size_t csa_index_workspace_bytes(int64_t rows, int64_t H, int64_t kcap);
sa_status launch_csa_index_select(sparse_attn_ctx* c, const CsaIndexArgs& a);
sa_status launch_mla_combine(sparse_attn_ctx* c, int64_t rows, int64_t q_seq, int splits, uint16_t* y);

sa_status set_error(sparse_attn_ctx* c, sa_status s, const std::string& msg);
void free_buffers(sparse_attn_ctx* c);
// Optional timing of a call's main kernel: the event pair the next launch
// carries (null when timing is off or its slots are used up). The launch
// takes the events with hipExtLaunchKernel, which stamps them with the
// dispatch's own start and end, so the time is the kernel's alone.
struct ProfEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};
ProfEvents prof_next(sparse_attn_ctx* c);
#define SA_MAIN_LAUNCH(pe, kernel, grid, block, shmem, stream, ...)                                        \
  do {                                                                                                     \
    if ((pe).start)                                                                                        \
      hipExtLaunchKernelGGL(kernel, grid, block, shmem, stream, (pe).start, (pe).stop, 0u, __VA_ARGS__);  \
    else                                                                                                   \
      hipLaunchKernelGGL(kernel, grid, block, shmem, stream, __VA_ARGS__);                                \
  } while (0)
sa_status check_hip(sparse_attn_ctx* c, hipError_t e, const char* what);

}  // namespace sa
