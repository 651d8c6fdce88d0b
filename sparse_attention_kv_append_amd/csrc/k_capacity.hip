// Capacity-mode length recovery (IndexShare page, kernel `capacity_write_pos`).
//
// When the present cache aliases a fixed-capacity past, its shape no longer
// tells how many rows are live; the additive bias's causal/padding frontier
// does. For batch entry b: valid = 1 + the largest key column k with a finite
// bias(b, h, q, k) for some head h and query q (0 if none), and the current
// rows go to write = valid - cur_len (0 when valid < cur_len).
//
// The pages give one thread per batch entry looping over every broadcast
// (h, q, k). Here one 256-thread workgroup per batch entry reads the entry's
// slice of the bias coalesced: in 16-byte vectors (four per thread in
// flight) when the rows are whole vectors, else each row from its end down in
// batches of aligned 16-byte vectors (sixteen per thread in flight), stopping
// at the first batch that holds a finite element. An extent of 1
// along heads or queries is not expanded, and an extent of 1 along keys
// makes a finite element stand for every column. Finiteness is read from the
// exponent bits (vector path). The per-thread maxima are reduced with wave
// shuffles and one LDS atomic per wave.
#include "sa_internal.h"
#include "sa_mfma_dev.h"

namespace sa {

constexpr int kCapThreads = 256;
constexpr int kCapUnroll = 4;  // 16-byte loads per thread in flight at once
constexpr int kRowUnroll = 16;  // the same, scanning one row that is not whole vectors

// finite test on the raw bits of one element (exponent not all ones)
template <int DT>
__device__ __forceinline__ bool bits_finite(uint32_t bits) {
  if constexpr (DT == SA_F32) return (bits & 0x7f800000u) != 0x7f800000u;
  else if constexpr (DT == SA_F16) return (bits & 0x7c00u) != 0x7c00u;
  else return (bits & 0x7f80u) != 0x7f80u;
}

// 1 + the largest in-row column (e % bd3, or keys - 1 when bd3 == 1) over the
// finite elements of one 16-byte vector starting at element e0 (the vector
// lies within one row: bd3 is a multiple of its element count)
template <int DT>
__device__ __forceinline__ int vec_best(uint4 v, int64_t e0, int64_t bd3, int64_t keys) {
  constexpr int PER = DT == SA_F32 ? 4 : 8;
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  int last = -1;  // last finite element of the vector
#pragma unroll
  for (int j = 0; j < PER; j++) {
    const uint32_t bits = PER == 4 ? w[j] : ((w[j >> 1] >> (16 * (j & 1))) & 0xffffu);
    if (bits_finite<DT>(bits)) last = j;
  }
  if (last < 0) return 0;
  return bd3 == 1 ? (int)keys : (int)(e0 % bd3) + last + 1;
}

// 1 + the largest finite column of batch entry b's bias slice, reduced over
// the workgroup (every thread returns it)
template <int DT, bool VEC>
__device__ __forceinline__ int capacity_scan(const void* __restrict__ bias, int64_t b, int64_t bd0, int64_t bd1,
                                             int64_t bd2, int64_t bd3, int64_t keys, int* best_s) {
  const int64_t n = bd1 * bd2 * bd3;  // elements of one batch entry's slice
  const int64_t base = (bd0 == 1 ? 0 : b) * n;
  if (threadIdx.x == 0) *best_s = 0;
  __syncthreads();
  int best = 0;  // 1 + largest finite column seen by this thread
  if constexpr (VEC) {
    // n and bd3 are multiples of the vector width, the slice is 16-byte aligned
    constexpr int PER = DT == SA_F32 ? 4 : 8;
    const uint4* __restrict__ vp = (const uint4*)((const char*)bias + base * (DT == SA_F32 ? 4 : 2));
    const int64_t nv = n / PER;
    for (int64_t v0 = threadIdx.x; v0 < nv; v0 += (int64_t)kCapThreads * kCapUnroll) {
      uint4 vals[kCapUnroll];
#pragma unroll
      for (int u = 0; u < kCapUnroll; u++) {
        const int64_t v = v0 + (int64_t)u * kCapThreads;
        vals[u] = v < nv ? vp[v] : make_uint4(0xffffffffu, 0xffffffffu, 0xffffffffu, 0xffffffffu);  // NaN: skipped
      }
#pragma unroll
      for (int u = 0; u < kCapUnroll; u++)
        best = max(best, vec_best<DT>(vals[u], (v0 + (int64_t)u * kCapThreads) * PER, bd3, keys));
    }
  } else {
    // rows that are not whole vectors: each (h, q) row is scanned from its
    // last column down in batches of kCapThreads x kRowUnroll 16-byte
    // vectors (aligned to their own address; the at most 2 x (PER - 1)
    // elements before the first and after the last whole vector by single
    // loads, in the first batch), all of a batch's loads in flight at once;
    // the row ends at the first batch holding a finite element, since no
    // lower column can raise the row's maximum
    constexpr int ES = DT == SA_F32 ? 4 : 2;
    constexpr int PER = 16 / ES;
    constexpr int64_t BATCH = (int64_t)kCapThreads * kRowUnroll;  // vectors per batch
    const int64_t rows = bd1 * bd2;
    for (int64_t r = 0; r < rows; r++) {
      const int64_t rb = base + r * bd3;
      if (bd3 == 1) {  // one element stands for every key
        if (threadIdx.x == 0 && isfinite(load_elem<DT>(bias, rb))) best = (int)keys;
        continue;
      }
      const uintptr_t addr = (uintptr_t)bias + (uintptr_t)(rb * ES);
      const int64_t ka = min((int64_t)(((addr + 15) & ~(uintptr_t)15) - addr) / ES, bd3);  // first aligned column
      const int64_t nvec = (bd3 - ka) / PER;
      const int64_t kt = ka + nvec * PER;  // first column after the last whole vector
      const uint4* __restrict__ vp = (const uint4*)(addr + (uintptr_t)(ka * ES));
      // the loose elements: threads 0 .. PER-2 take those before the first
      // whole vector (the row's lowest columns: they count only when nothing
      // above them is finite), threads PER .. 2 PER - 2 those after the last
      // (its highest: they count with the first batch)
      int found = 0;  // 1 + the largest finite column at or above the current batch
      int low = 0;    // 1 + the largest finite column before the first whole vector
      {
        const int t = (int)threadIdx.x;
        if (t < PER - 1 && t < ka && isfinite(load_elem<DT>(bias, rb + t))) low = t + 1;
        if (t >= PER && t < 2 * PER - 1 && kt + (t - PER) < bd3 &&
            isfinite(load_elem<DT>(bias, rb + kt + (t - PER))))
          found = (int)(kt + (t - PER) + 1);
      }
      for (int64_t top = nvec; ; top -= BATCH) {
        uint4 vals[kRowUnroll];
#pragma unroll
        for (int u = 0; u < kRowUnroll; u++) {
          const int64_t v = top - 1 - (threadIdx.x + (int64_t)u * kCapThreads);
          vals[u] = v >= 0 ? vp[v] : make_uint4(0xffffffffu, 0xffffffffu, 0xffffffffu, 0xffffffffu);  // NaN: skipped
        }
#pragma unroll
        for (int u = 0; u < kRowUnroll; u++) {
          const int64_t v = top - 1 - (threadIdx.x + (int64_t)u * kCapThreads);
          if (v >= 0) {
            const int c = vec_best<DT>(vals[u], 0, (int64_t)1 << 62, keys);  // 1 + its last finite lane, or 0
            if (c > 0) found = max(found, (int)(ka + v * PER + c));
          }
        }
        if (__syncthreads_or(found > 0) || top <= BATCH) break;  // uniform
      }
      best = max(best, max(found, low));
    }
  }
  best = wave_max_nonneg(best);
  if ((threadIdx.x & 63) == 0) atomicMax(best_s, best);
  __syncthreads();
  return *best_s;
}

template <int DT, bool VEC>
__global__ void __launch_bounds__(kCapThreads)
capacity_lengths_kernel(const void* __restrict__ bias, int64_t bd0, int64_t bd1, int64_t bd2, int64_t bd3,
                        int64_t keys, int64_t cur_len, int32_t* __restrict__ valid_len,
                        int32_t* __restrict__ write_pos) {
  __shared__ int best_s;
  const int64_t b = blockIdx.x;
  const int v = capacity_scan<DT, VEC>(bias, b, bd0, bd1, bd2, bd3, keys, &best_s);
  if (threadIdx.x == 0) {
    valid_len[b] = v;
    write_pos[b] = v >= cur_len ? (int32_t)(v - cur_len) : 0;
  }
}

// The lengths, then this batch entry's current K and V rows written in place
// at the write position (IndexShare's `capacity_write_pos` followed by its
// two `build_present_capacity` launches, as one): rows of `row_bytes`, a
// multiple of 16, for every kv head.
template <int DT, bool VEC>
__global__ void __launch_bounds__(kCapThreads)
capacity_append_kernel(const void* __restrict__ bias, int64_t bd0, int64_t bd1, int64_t bd2, int64_t bd3,
                       int64_t keys, int64_t cur_len, int32_t* __restrict__ valid_len,
                       int32_t* __restrict__ write_pos, const uint4* __restrict__ cur_k,
                       const uint4* __restrict__ cur_v, uint4* __restrict__ cache_k, uint4* __restrict__ cache_v,
                       int64_t heads, int64_t row_bytes, ErrorBlock* __restrict__ reset_eb) {
  __shared__ int best_s;
  const int64_t b = blockIdx.x;
  // the step's error reset (no other work of the launch touches the block)
  if (reset_eb && b == 0 && threadIdx.x == 0) clear_error_block(reset_eb);
  const int v = capacity_scan<DT, VEC>(bias, b, bd0, bd1, bd2, bd3, keys, &best_s);
  const int64_t wp = v >= cur_len ? (int64_t)v - cur_len : 0;  // wp + cur_len <= keys
  if (threadIdx.x == 0) {
    valid_len[b] = v;
    write_pos[b] = (int32_t)wp;
  }
  const int64_t ru = row_bytes / 16;     // 16-byte units per row
  const int64_t per = heads * cur_len * ru;  // units of one tensor for this batch entry
  const int64_t units = cache_v ? 2 * per : per;  // a shared-latent cache has no V tensor
  for (int64_t u = threadIdx.x; u < units; u += kCapThreads) {
    const bool second = u >= per;
    const int64_t e = second ? u - per : u;
    const int64_t h = e / (cur_len * ru);
    const int64_t rem = e - h * cur_len * ru;  // (row t, unit) of the current rows
    const int64_t t = rem / ru, k = rem - t * ru;
    const int64_t src = ((b * heads + h) * cur_len + t) * ru + k;
    const int64_t dst = ((b * heads + h) * keys + wp + t) * ru + k;
    if (second) cache_v[dst] = cur_v[src];
    else cache_k[dst] = cur_k[src];
  }
}

sa_status launch_capacity_lengths(sparse_attn_ctx* c, const void* bias, int dtype, const int64_t* bd,
                                  int64_t batch, int64_t keys, int64_t cur_len, int32_t* valid_len,
                                  int32_t* write_pos) {
  const dim3 grid((unsigned)batch), block(kCapThreads);
  // 16-byte vectors when every slice and row is a whole number of them
  const int per = dtype == SA_F32 ? 4 : 8;
  const bool vec = bd[3] % per == 0 && ((uintptr_t)bias & 15) == 0;
#define SA_CAP(DT, V)                                                                                      \
  hipLaunchKernelGGL((capacity_lengths_kernel<DT, V>), grid, block, 0, c->stream, bias, bd[0], bd[1], bd[2], \
                     bd[3], keys, cur_len, valid_len, write_pos)
#define SA_CAP_V(DT) \
  if (vec) { SA_CAP(DT, true); } else { SA_CAP(DT, false); }
  if (dtype == SA_F32) {
    SA_CAP_V(SA_F32);
  } else if (dtype == SA_F16) {
    SA_CAP_V(SA_F16);
  } else {
    SA_CAP_V(SA_BF16);
  }
#undef SA_CAP_V
#undef SA_CAP
  return check_hip(c, hipGetLastError(), "capacity_lengths");
}

}  // namespace sa

namespace sa {

sa_status launch_capacity_append(sparse_attn_ctx* c, const void* bias, int dtype, const int64_t* bd, int64_t batch,
                                 int64_t keys, int64_t cur_len, int32_t* valid_len, int32_t* write_pos,
                                 const void* cur_k, const void* cur_v, void* cache_k, void* cache_v, int64_t heads,
                                 int64_t row_bytes, ErrorBlock* reset_eb) {
  const dim3 grid((unsigned)batch), block(kCapThreads);
  const int per = dtype == SA_F32 ? 4 : 8;
  const bool vec = bd[3] % per == 0 && ((uintptr_t)bias & 15) == 0;
#define SA_CAPA(DT, V)                                                                                      \
  hipLaunchKernelGGL((capacity_append_kernel<DT, V>), grid, block, 0, c->stream, bias, bd[0], bd[1], bd[2], \
                     bd[3], keys, cur_len, valid_len, write_pos, (const uint4*)cur_k, (const uint4*)cur_v,   \
                     (uint4*)cache_k, (uint4*)cache_v, heads, row_bytes, reset_eb)
#define SA_CAPA_V(DT) \
  if (vec) { SA_CAPA(DT, true); } else { SA_CAPA(DT, false); }
  if (dtype == SA_F32) {
    SA_CAPA_V(SA_F32);
  } else if (dtype == SA_F16) {
    SA_CAPA_V(SA_F16);
  } else {
    SA_CAPA_V(SA_BF16);
  }
#undef SA_CAPA_V
#undef SA_CAPA
  return check_hip(c, hipGetLastError(), "capacity append");
}

}  // namespace sa
