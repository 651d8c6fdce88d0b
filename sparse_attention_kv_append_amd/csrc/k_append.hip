// KV append (IndexShare `build_present` / `build_present_capacity`), the
// fp8_e4m3_block64 quantize-on-append (CSA CPU page, `finalize_attention_record`
// pack loop) and the error-word reset.
//
// The append is a pure byte copy. For one (batch, kv head) both the past rows
// [0, P) and the new rows land in one contiguous byte range of the present
// buffer, so each launch copies flat ranges with the widest vector the row
// width and pointer alignment allow; there is no per-element index math.
#include "sa_internal.h"

namespace sa {

__global__ void reset_error_kernel(ErrorBlock* err) {
  if (threadIdx.x == 0) {
    err->word = 0u;
    err->done_blocks = 0u;
    err->first_bad = ~0ull;
    err->call_key = ~0ull;
    err->detail_class = 0;
    err->call_word = 0u;
  }
}

sa_status launch_reset_error(sparse_attn_ctx* c) {
  hipLaunchKernelGGL(reset_error_kernel, dim3(1), dim3(64), 0, c->stream, c->err);
  return check_hip(c, hipGetLastError(), "reset_error");
}

constexpr int kCopyBlock = 256;
constexpr int kCopyUnroll = 4;

// grid.x = (batch * heads) * chunks; each block copies kCopyBlock*kCopyUnroll
// vector units of one (batch, head) segment.
template <typename V>
__global__ void __launch_bounds__(kCopyBlock)
append_copy_kernel(const char* __restrict__ past, int64_t past_cap,
                   const int32_t* __restrict__ past_len, const char* __restrict__ cur,
                   int64_t cur_len, char* __restrict__ present, int64_t present_cap,
                   int64_t heads, int64_t row_bytes, int64_t chunks, int copy_past,
                   int32_t* __restrict__ present_len, ErrorBlock* __restrict__ err) {
  const int64_t bh = blockIdx.x / chunks;
  const int64_t chunk = blockIdx.x - bh * chunks;
  const int64_t b = bh / heads;
  const int64_t P = past_len ? (int64_t)past_len[b] : past_cap;
  if (P < 0 || P > past_cap || P + cur_len > present_cap) {
    if (chunk == 0 && threadIdx.x == 0) atomicOr(&err->word, SA_ERR_APPEND_CAPACITY | SA_ERR_APPEND_ANY);
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
                             bool copy_past, int32_t* present_len) {
  const int vec = pick_vec(row_bytes, copy_past ? past : nullptr, cur, present);
  const int64_t max_rows = (copy_past ? past_cap : 0) + cur_len;
  const int64_t units = max_rows * (row_bytes / vec);
  const int64_t per_block = (int64_t)kCopyBlock * kCopyUnroll;
  const int64_t chunks = units > 0 ? (units + per_block - 1) / per_block : 1;
  const int64_t blocks = batch * heads * chunks;
  if (blocks <= 0) return SA_OK;
  if (blocks > 0x7fffffffLL) return set_error(c, SA_E_SHAPE, "kv_append: cache too large for one launch");
  const dim3 grid((unsigned)blocks), block(kCopyBlock);
#define SA_COPY(T)                                                                          \
  hipLaunchKernelGGL(append_copy_kernel<T>, grid, block, 0, c->stream, (const char*)past,   \
                     past_cap, past_len, (const char*)cur, cur_len, (char*)present,          \
                     present_cap, heads, row_bytes, chunks, copy_past ? 1 : 0, present_len,   \
                     c->err)
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

// E4M3FN code of x * 2^(127 - e), x given by its fp32 bits: round to nearest
// even, saturate at 448 (code 0x7E), sign kept (a negative value that rounds
// to zero gives 0x80). Integer-exact: x = sig * 2^ex, and the quantum of the
// target binade is 2^q with q = max(floor(log2 v), -6) - 3 (the subnormal
// quantum 2^-9 below 2^-6). The code bits are (max(lg,-6)+7)*8 + n - 8, which
// runs continuously across the subnormal/normal seam and binade carries.
__device__ __forceinline__ uint32_t e4m3fn_encode_scaled(uint32_t w, int e) {
  const uint32_t sign = (w >> 31) << 7;
  const uint32_t a = w & 0x7fffffffu;
  if (a == 0) return sign;
  const int E = (int)(a >> 23);
  const uint32_t sig = E ? ((a & 0x7fffffu) | 0x800000u) : (a & 0x7fffffu);
  const int ex = (E ? E - 150 : -149) + 127 - e;
  const int lg = (31 - __clz((int)sig)) + ex;
  const int lgc = lg < -6 ? -6 : lg;
  const int shift = (lgc - 3) - ex;
  uint32_t n;
  if (shift <= 0) {
    n = sig << (-shift);
  } else if (shift >= 32) {
    n = 0;
  } else {
    n = sig >> shift;
    const uint32_t rem = sig & ((1u << shift) - 1u);
    const uint32_t half = 1u << (shift - 1);
    if (rem > half || (rem == half && (n & 1u))) n += 1u;
  }
  int code = ((lgc + 7) << 3) + (int)n - 8;
  if (code > 0x7e) code = 0x7e;
  return sign | (uint32_t)code;
}

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
  const int nblk = (dk - rope) / 64;
  // non-finite values anywhere in the row: latch and leave the row unwritten
  bool bad = false;
  for (int d = lane; d < dk; d += 64) bad |= ((src[d] & 0x7f80u) == 0x7f80u);
  if (__ballot(bad) != 0ull) {
    if (lane == 0) atomicOr(&err->word, SA_ERR_QUANT_NONFINITE | SA_ERR_APPEND_ANY);
    return;
  }
  for (int j = 0; j < nblk; j++) {
    const uint32_t w = (uint32_t)src[64 * j + lane] << 16;
    uint32_t amax = w & 0x7fffffffu;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) amax = max(amax, (uint32_t)__shfl_xor((int)amax, o, 64));
    uint32_t code = 0;
    int e = 127;
    if (amax != 0) {
      const int E = (int)(amax >> 23);
      const int k = E ? E - 127 : (31 - __clz((int)(amax & 0x7fffffu))) - 149;
      e = k - 8 + 127;
      e = e < 0 ? 0 : (e > 254 ? 254 : e);
      code = e4m3fn_encode_scaled(w, e);
    }
    if (lane == 0) dst[65 * j] = (uint8_t)e;
    dst[65 * j + 1 + lane] = (uint8_t)code;
  }
  uint8_t* tail = dst + 65 * nblk;
  for (int i = lane; i < rope; i += 64) {
    const uint16_t bits = src[dk - rope + i];
    tail[2 * i] = (uint8_t)(bits & 0xff);
    tail[2 * i + 1] = (uint8_t)(bits >> 8);
  }
}

sa_status launch_append_quantize(sparse_attn_ctx* c, int64_t batch, int64_t heads, int64_t dk,
                                 int64_t rope, const void* cur_bf16, int64_t cur_len,
                                 const int32_t* past_len, int64_t past_cap, void* present,
                                 int64_t present_cap, int32_t* present_len) {
  const int64_t rows = batch * heads * cur_len;
  if (rows <= 0) return SA_OK;
  const int64_t rec = (dk - rope) / 64 * 65 + 2 * rope;
  const int64_t blocks = (rows + 3) / 4;
  if (blocks > 0x7fffffffLL) return set_error(c, SA_E_SHAPE, "kv_append: too many rows");
  hipLaunchKernelGGL(append_quantize_kernel, dim3((unsigned)blocks), dim3(256), 0, c->stream,
                     (const uint16_t*)cur_bf16, cur_len, past_len, past_cap, (uint8_t*)present,
                     present_cap, heads, rows, (int)dk, (int)rope, rec, present_len, c->err);
  return check_hip(c, hipGetLastError(), "kv_append quantize");
}

}  // namespace sa
