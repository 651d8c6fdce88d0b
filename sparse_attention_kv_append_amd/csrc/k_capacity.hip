// Capacity-mode length recovery (IndexShare page, kernel `capacity_write_pos`).
//
// When the present cache aliases a fixed-capacity past, its shape no longer
// tells how many rows are live; the additive bias's causal/padding frontier
// does. For batch entry b: valid = 1 + the largest key column k with a finite
// bias(b, h, q, k) for some head h and query q (0 if none), and the current
// rows go to write = valid - cur_len (0 when valid < cur_len).
//
// The pages give one thread per batch entry looping over every broadcast
// (h, q, k). Here one 256-thread workgroup per batch entry reads each element
// of the entry's slice of the bias exactly once, coalesced: an extent of 1
// along heads or queries is not expanded, and an extent of 1 along keys makes
// a finite element stand for every column. The per-thread maxima are reduced
// with wave shuffles and one LDS atomic per wave.
#include "sa_internal.h"
#include "sa_mfma_dev.h"

namespace sa {

constexpr int kCapThreads = 256;

template <int DT>
__global__ void __launch_bounds__(kCapThreads)
capacity_lengths_kernel(const void* __restrict__ bias, int64_t bd0, int64_t bd1, int64_t bd2, int64_t bd3,
                        int64_t keys, int64_t cur_len, int32_t* __restrict__ valid_len,
                        int32_t* __restrict__ write_pos) {
  __shared__ int best_s;
  const int64_t b = blockIdx.x;
  const int64_t n = bd1 * bd2 * bd3;  // elements of one batch entry's slice
  const int64_t base = (bd0 == 1 ? 0 : b) * n;
  if (threadIdx.x == 0) best_s = 0;
  __syncthreads();
  int best = 0;  // 1 + largest finite column seen by this thread
  for (int64_t e = threadIdx.x; e < n; e += kCapThreads) {
    const float v = load_elem<DT>(bias, base + e);
    if (isfinite(v)) {
      const int64_t k = bd3 == 1 ? keys - 1 : e % bd3;
      best = max(best, (int)(k + 1));
    }
  }
  best = wave_max_nonneg(best);
  if ((threadIdx.x & 63) == 0) atomicMax(&best_s, best);
  __syncthreads();
  if (threadIdx.x == 0) {
    const int v = best_s;
    valid_len[b] = v;
    write_pos[b] = v >= cur_len ? (int32_t)(v - cur_len) : 0;
  }
}

sa_status launch_capacity_lengths(sparse_attn_ctx* c, const void* bias, int dtype, const int64_t* bd,
                                  int64_t batch, int64_t keys, int64_t cur_len, int32_t* valid_len,
                                  int32_t* write_pos) {
  const dim3 grid((unsigned)batch), block(kCapThreads);
#define SA_CAP(DT)                                                                                     \
  hipLaunchKernelGGL((capacity_lengths_kernel<DT>), grid, block, 0, c->stream, bias, bd[0], bd[1], bd[2], \
                     bd[3], keys, cur_len, valid_len, write_pos)
  if (dtype == SA_F32) {
    SA_CAP(SA_F32);
  } else if (dtype == SA_F16) {
    SA_CAP(SA_F16);
  } else {
    SA_CAP(SA_BF16);
  }
#undef SA_CAP
  return check_hip(c, hipGetLastError(), "capacity_lengths");
}

}  // namespace sa
