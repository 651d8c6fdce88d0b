// Measurement aids: the attainable HBM copy rate and bf16 matrix-core rate of
// the device, against which the attention kernels' roofline fractions are
// also reported (beside the vendor figures). Neither is part of the attention
// path.
#include "sa_internal.h"
#include "sa_mfma_dev.h"

#pragma clang fp contract(off)

namespace sa {

namespace {

constexpr int COPY_THREADS = 256;
constexpr int COPY_UNROLL = 4;  // 16-byte vectors in flight per thread

// Grid-stride copy of n 16-byte vectors with streaming (non-temporal) loads
// and stores, so neither L2 nor the last-level cache keeps the data.
__global__ void __launch_bounds__(COPY_THREADS)
peak_copy_kernel(const u32x4_l* __restrict__ src, u32x4_l* __restrict__ dst, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * COPY_THREADS * COPY_UNROLL;
  for (int64_t base = (int64_t)blockIdx.x * COPY_THREADS * COPY_UNROLL + threadIdx.x; base < n; base += stride) {
    u32x4_l v[COPY_UNROLL];
#pragma unroll
    for (int u = 0; u < COPY_UNROLL; u++) {
      const int64_t i = base + (int64_t)u * COPY_THREADS;
      if (i < n) v[u] = __builtin_nontemporal_load(src + i);
    }
#pragma unroll
    for (int u = 0; u < COPY_UNROLL; u++) {
      const int64_t i = base + (int64_t)u * COPY_THREADS;
      if (i < n) __builtin_nontemporal_store(v[u], dst + i);
    }
  }
}

// Grid-stride streaming read of n 16-byte vectors, folded with xor into one
// word per thread (stored, so the loads are not dead).
__global__ void __launch_bounds__(COPY_THREADS)
peak_read_kernel(const u32x4_l* __restrict__ src, uint32_t* __restrict__ out, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * COPY_THREADS * COPY_UNROLL;
  uint32_t acc = 0u;
  for (int64_t base = (int64_t)blockIdx.x * COPY_THREADS * COPY_UNROLL + threadIdx.x; base < n; base += stride) {
    u32x4_l v[COPY_UNROLL];
#pragma unroll
    for (int u = 0; u < COPY_UNROLL; u++) {
      const int64_t i = base + (int64_t)u * COPY_THREADS;
      v[u] = i < n ? __builtin_nontemporal_load(src + i) : (u32x4_l){0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < COPY_UNROLL; u++) acc ^= (v[u][0] ^ v[u][1]) ^ (v[u][2] ^ v[u][3]);
  }
  out[(int64_t)blockIdx.x * COPY_THREADS + threadIdx.x] = acc;
}

static_assert(PEAK_READ_BLOCKS * COPY_THREADS == SA_PEAK_READ_SINK_WORDS, "read probe sink size");

constexpr int MFMA_THREADS = 256;
constexpr int MFMA_CHAINS = 8;  // independent accumulators per wave

// Each wave issues `iters` rounds of MFMA_CHAINS independent
// v_mfma_f32_16x16x32_bf16 (16 x 16 x 32 x 2 = 16384 flops each); the sums
// are stored so that nothing is dead.
__global__ void __launch_bounds__(MFMA_THREADS)
peak_mfma_kernel(float* __restrict__ out, int iters) {
  const int lane = threadIdx.x & 63;
  bf16x8_l a, b;
#pragma unroll
  for (int j = 0; j < 8; j++) {
    a[j] = (__bf16)(0.001f * (float)(lane + j));
    b[j] = (__bf16)(0.002f * (float)(lane - j));
  }
  f32x4_l acc[MFMA_CHAINS];
#pragma unroll
  for (int c = 0; c < MFMA_CHAINS; c++) {  // distinct chains (equal ones would be merged)
    const float v = (float)(c + 1) * (float)(lane + 1);
    acc[c] = (f32x4_l){v, v + 1.f, v + 2.f, v + 3.f};
  }
  int i = 0;
  do {
#pragma unroll
    for (int c = 0; c < MFMA_CHAINS; c++) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[c], 0, 0, 0);
  } while (++i < iters);
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < MFMA_CHAINS; c++) s = s + ((acc[c][0] + acc[c][1]) + (acc[c][2] + acc[c][3]));
  out[(int64_t)blockIdx.x * MFMA_THREADS + threadIdx.x] = s;
}

}  // namespace

sa_status launch_peak_copy(sparse_attn_ctx* c, void* dst, const void* src, int64_t bytes, void* sink) {
  const int64_t n = bytes / 16;
  const int64_t per_block = (int64_t)COPY_THREADS * COPY_UNROLL;
  if (dst) {  // copy: 64 workgroups per CU measured best
    const int64_t blocks = std::min<int64_t>((n + per_block - 1) / per_block, 256 * 64);
    hipLaunchKernelGGL(peak_copy_kernel, dim3((unsigned)blocks), dim3(COPY_THREADS), 0, c->stream,
                       (const u32x4_l*)src, (u32x4_l*)dst, n);
  } else {  // read: 4 workgroups per CU measured best
    const int64_t blocks = std::min<int64_t>((n + per_block - 1) / per_block, PEAK_READ_BLOCKS);
    hipLaunchKernelGGL(peak_read_kernel, dim3((unsigned)blocks), dim3(COPY_THREADS), 0, c->stream,
                       (const u32x4_l*)src, (uint32_t*)sink, n);
  }
  return check_hip(c, hipGetLastError(), "peak copy");
}

sa_status launch_peak_mfma(sparse_attn_ctx* c, float* out, int64_t blocks, int iters) {
  hipLaunchKernelGGL(peak_mfma_kernel, dim3((unsigned)blocks), dim3(MFMA_THREADS), 0, c->stream, out, iters);
  return check_hip(c, hipGetLastError(), "peak mfma");
}

}  // namespace sa
