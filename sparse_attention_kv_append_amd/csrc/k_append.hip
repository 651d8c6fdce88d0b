// KV append (IndexShare `build_present` / `build_present_capacity`), the
// fp8_e4m3_block64 quantize-on-append (CSA CPU page, `finalize_attention_record`
// pack loop) and the error-word reset.
//
// The append is a pure byte copy. For one (batch, kv head) both the past rows
// [0, P) and the new rows land in one contiguous byte range of the present
// buffer, so each launch copies flat ranges with the widest vector the row
// width and pointer alignment allow; there is no per-element index math.
#include "sa_quant_dev.h"

#include <algorithm>

namespace sa {

__global__ void reset_error_kernel(ErrorBlock* err) {
  if (threadIdx.x == 0) clear_error_block(err);
}

sa_status launch_reset_error(sparse_attn_ctx* c) {
  hipLaunchKernelGGL(reset_error_kernel, dim3(1), dim3(64), 0, c->stream, c->err);
  return check_hip(c, hipGetLastError(), "reset_error");
}

constexpr int kCopyBlock = 256;
constexpr int kCopyUnroll = 4;

// grid.x = (batch * heads) * chunks; each block copies kCopyBlock*kCopyUnroll
// vector units of one (batch, head) segment. grid.y = 2 copies a second
// tensor of the same geometry (V beside K) in the same launch.
template <typename V>
__global__ void __launch_bounds__(kCopyBlock)
append_copy_kernel(const char* __restrict__ past_a, const char* __restrict__ past_b, int64_t past_cap,
                   const int32_t* __restrict__ past_len, const char* __restrict__ cur_a,
                   const char* __restrict__ cur_b, int64_t cur_len, char* __restrict__ present_a,
                   char* __restrict__ present_b, int64_t present_cap,
                   int64_t heads, int64_t row_bytes, int64_t chunks, int copy_past,
                   int32_t* __restrict__ present_len, ErrorBlock* __restrict__ err) {
  const bool second = blockIdx.y != 0;
  const char* __restrict__ past = second ? past_b : past_a;
  const char* __restrict__ cur = second ? cur_b : cur_a;
  char* __restrict__ present = second ? present_b : present_a;
  if (second) present_len = nullptr;
  const int64_t bh = blockIdx.x / chunks;
  const int64_t chunk = blockIdx.x - bh * chunks;
  const int64_t b = bh / heads;
  const int64_t P = past_len ? (int64_t)past_len[b] : past_cap;
  if (P < 0 || P > past_cap || P + cur_len > present_cap) {
    if (!second && chunk == 0 && threadIdx.x == 0) atomicOr(&err->word, SA_ERR_APPEND_CAPACITY | SA_ERR_APPEND_ANY);
    return;
  }
  if (present_len && chunk == 0 && threadIdx.x == 0 && bh % heads == 0) {
    present_len[b] = (int32_t)(P + cur_len);
  }
  const int64_t ru = row_bytes / (int64_t)sizeof(V);
  const int64_t past_units = copy_past ? P * ru : 0;
  const int64_t cur_units = cur_len * ru;
  const V* __restrict__ sp = (const V*)(past + bh * past_cap * row_bytes);
  const V* __restrict__ sc = (const V*)(cur + bh * cur_len * row_bytes);
  V* __restrict__ d = (V*)(present + bh * present_cap * row_bytes);
  const int64_t dst_cur = P * ru;
  const int64_t u0 = chunk * (kCopyBlock * kCopyUnroll) + threadIdx.x;
  V vals[kCopyUnroll];
#pragma unroll
  for (int k = 0; k < kCopyUnroll; k++) {
    const int64_t u = u0 + (int64_t)k * kCopyBlock;
    if (u < past_units) {
      vals[k] = sp[u];
    } else if (u - past_units < cur_units) {
      vals[k] = sc[u - past_units];
    }
  }
#pragma unroll
  for (int k = 0; k < kCopyUnroll; k++) {
    const int64_t u = u0 + (int64_t)k * kCopyBlock;
    if (u < past_units) {
      d[u] = vals[k];
    } else if (u - past_units < cur_units) {
      d[dst_cur + (u - past_units)] = vals[k];
    }
  }
}

static int pick_vec(int64_t row_bytes, const void* a, const void* b, const void* c) {
  const uintptr_t mis = (uintptr_t)a | (uintptr_t)b | (uintptr_t)c;
  for (int v = 16; v > 1; v >>= 1) {
    if (row_bytes % v == 0 && (mis % (uintptr_t)v) == 0) return v;
  }
  return 1;
}

sa_status launch_append_copy(sparse_attn_ctx* c, int64_t batch, int64_t heads, int64_t row_bytes,
                             const void* past, int64_t past_cap, const int32_t* past_len,
                             const void* cur, int64_t cur_len, void* present, int64_t present_cap,
                             bool copy_past, int32_t* present_len, const void* past2, const void* cur2,
                             void* present2) {
  const bool two = present2 != nullptr;
  int vec = pick_vec(row_bytes, copy_past ? past : nullptr, cur, present);
  if (two) vec = std::min(vec, pick_vec(row_bytes, copy_past ? past2 : nullptr, cur2, present2));
  const int64_t max_rows = (copy_past ? past_cap : 0) + cur_len;
  const int64_t units = max_rows * (row_bytes / vec);
  const int64_t per_block = (int64_t)kCopyBlock * kCopyUnroll;
  const int64_t chunks = units > 0 ? (units + per_block - 1) / per_block : 1;
  const int64_t blocks = batch * heads * chunks;
  if (blocks <= 0) return SA_OK;
  if (blocks > 0x7fffffffLL) return set_error(c, SA_E_SHAPE, "kv_append: cache too large for one launch");
  const dim3 grid((unsigned)blocks, two ? 2u : 1u), block(kCopyBlock);
#define SA_COPY(T)                                                                                      \
  hipLaunchKernelGGL(append_copy_kernel<T>, grid, block, 0, c->stream, (const char*)past,               \
                     (const char*)past2, past_cap, past_len, (const char*)cur, (const char*)cur2, cur_len, \
                     (char*)present, (char*)present2, present_cap, heads, row_bytes, chunks,              \
                     copy_past ? 1 : 0, present_len, c->err)
  switch (vec) {
    case 16: SA_COPY(uint4); break;
    case 8: SA_COPY(uint2); break;
    case 4: SA_COPY(uint32_t); break;
    case 2: SA_COPY(uint16_t); break;
    default: SA_COPY(uint8_t); break;
  }
#undef SA_COPY
  return check_hip(c, hipGetLastError(), "kv_append copy");
}

// ---- fp8_e4m3_block64 quantize-on-append -----------------------------------

// One wave per new row; lane l owns element l of every 64-value block.
__global__ void __launch_bounds__(256)
append_quantize_kernel(const uint16_t* __restrict__ cur, int64_t cur_len,
                       const int32_t* __restrict__ past_len, int64_t past_cap,
                       uint8_t* __restrict__ present, int64_t present_cap, int64_t heads,
                       int64_t total_rows, int dk, int rope, int64_t rec_bytes,
                       int32_t* __restrict__ present_len, ErrorBlock* __restrict__ err) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= total_rows) return;
  const int64_t t = row % cur_len;
  const int64_t bh = row / cur_len;
  const int64_t b = bh / heads;
  const int64_t P = past_len ? (int64_t)past_len[b] : past_cap;
  if (P < 0 || P > past_cap || P + cur_len > present_cap) {
    if (lane == 0) atomicOr(&err->word, SA_ERR_APPEND_CAPACITY | SA_ERR_APPEND_ANY);
    return;
  }
  if (present_len && lane == 0 && t == 0 && bh % heads == 0) present_len[b] = (int32_t)(P + cur_len);
  const uint16_t* src = cur + row * dk;
  uint8_t* dst = present + (bh * present_cap + P + t) * rec_bytes;
  // a row holding a NaN or an infinity is latched and left unwritten
  if (quantize_row_wave(src, dst, dk, rope, lane) && lane == 0)
    atomicOr(&err->word, SA_ERR_QUANT_NONFINITE | SA_ERR_APPEND_ANY);
}

sa_status launch_append_quantize(sparse_attn_ctx* c, int64_t batch, int64_t heads, int64_t dk,
                                 int64_t rope, const void* cur_bf16, int64_t cur_len,
                                 const int32_t* past_len, int64_t past_cap, void* present,
                                 int64_t present_cap, int32_t* present_len) {
  const int64_t rows = batch * heads * cur_len;
  const int64_t rec = (dk - rope) / 64 * 65 + 2 * rope;
  // no current rows: present_len (and the capacity check) as the copy path does
  if (rows <= 0)
    return launch_append_copy(c, batch, heads, rec, nullptr, past_cap, past_len, nullptr, 0, present, present_cap,
                              false, present_len);
  const int64_t blocks = (rows + 3) / 4;
  if (blocks > 0x7fffffffLL) return set_error(c, SA_E_SHAPE, "kv_append: too many rows");
  hipLaunchKernelGGL(append_quantize_kernel, dim3((unsigned)blocks), dim3(256), 0, c->stream,
                     (const uint16_t*)cur_bf16, cur_len, past_len, past_cap, (uint8_t*)present,
                     present_cap, heads, rows, (int)dk, (int)rope, rec, present_len, c->err);
  return check_hip(c, hipGetLastError(), "kv_append quantize");
}

}  // namespace sa
