// Device-side pieces of index validation shared by the standalone validation
// kernel and the fused validation inside the shared-latent forward kernel.
// The rules are the IndexShare host `validate_indices` checks, applied to one
// column given its left neighbour (valid whenever every column before it
// passed, which is all the first violation needs).
#pragma once

#include "sa_internal.h"

namespace sa {

// Class of column c holding v, with left neighbour u and cache bound
// (0 = no violation at c). Check order: sentinel, padding, range, duplicate,
// order.
__device__ __forceinline__ int column_class(int64_t c, int64_t v, int64_t u, int64_t bound) {
  if (v == -1) return 0;
  if (v < -1) return 1;                 // invalid sentinel
  if (c > 0 && u == -1) return 2;       // follows trailing padding
  if (v >= bound) return 3;             // out of range
  if (c > 0 && v == u) return 4;        // duplicate
  if (c > 0 && v < u) return 5;         // not strictly increasing
  return 0;
}

// A row's first violation k (row * (width + 1) + column; column == width:
// the row holds only -1) turned into its class bit in the launch's word and
// offered as the launch's first key.
template <bool I64>
__device__ __forceinline__ void record_row_violation(ErrorBlock* __restrict__ eb, const void* __restrict__ idx,
                                                     int64_t row, int64_t width, unsigned long long k,
                                                     int64_t bound) {
  const int64_t col = (int64_t)(k % (unsigned long long)(width + 1));
  int cls = 6;
  if (col < width) {
    const int64_t v = load_index<I64>(idx, row * width + col);
    const int64_t u = col > 0 ? load_index<I64>(idx, row * width + col - 1) : 0;
    cls = column_class(col, v, u, bound);
  }
  atomicOr(&eb->call_word, (1u << (cls - 1)) | SA_ERR_INDEX_ANY);
  atomicMin((unsigned long long*)&eb->call_key, k);
}

// Called by one thread of each of the `expected` participants of a launch
// that gathers into the context's error block (every block of the validation
// kernel; the finisher of every row in the forward kernel), after its
// contributions to eb->call_key / eb->call_word are visible. The last one to
// arrive merges the launch's bits into the word (with `reset`, the word and
// the recorded first violation are cleared first: the launch then stands for
// a reset followed by itself), records the launch's first violation (class,
// values, position) if no earlier launch since the reset failed, then re-arms
// the per-launch slots and counter for the next launch on the stream.
// FENCE = false: every value the participants read was written before the
// launch began or by device-scope atomics, which a plain wait for completion
// orders; the whole-cache fences are then left out.
template <bool I64, bool FENCE = true>
__device__ __forceinline__ void finish_launch(ErrorBlock* __restrict__ eb, const void* __restrict__ idx,
                                              int64_t width, int64_t q_seq, int64_t rows_per_batch,
                                              const int32_t* __restrict__ valid_len, int64_t cache_len,
                                              unsigned expected, bool reset = false) {
  if constexpr (FENCE) __threadfence();
  else __builtin_amdgcn_s_waitcnt(0);  // this thread's atomics have completed
  const unsigned done = atomicAdd(&eb->done_blocks, 1u);
  if (done != expected - 1) return;
  if constexpr (FENCE) __threadfence();
  const unsigned bits = atomicExch(&eb->call_word, 0u);
  if (reset) {
    eb->word = bits;
    eb->first_bad = ~0ull;
    eb->detail_class = 0;
  } else if (bits) {
    atomicOr(&eb->word, bits);
  }
  const unsigned long long key = atomicMin((unsigned long long*)&eb->call_key, ~0ull);
  if (key != ~0ull && eb->detail_class == 0) {
    const int64_t r = (int64_t)(key / (unsigned long long)(width + 1));
    const int64_t c = (int64_t)(key % (unsigned long long)(width + 1));
    const int64_t b = r / rows_per_batch;
    // an atomic load: a length stored (atomically) in this launch is seen
    const int64_t bound =
        valid_len ? (int64_t)__hip_atomic_load(&valid_len[b], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : cache_len;
    int64_t v = -1, u = 0;
    int k = 6;  // column == width: the row holds only -1
    if (c < width) {
      v = load_index<I64>(idx, r * width + c);
      u = c > 0 ? load_index<I64>(idx, r * width + c - 1) : 0;
      k = column_class(c, v, u, bound);
    }
    eb->detail_value = v;
    eb->detail_prev = u;
    eb->detail_bound = bound;
    eb->detail_b = b;
    eb->detail_h = (r - b * rows_per_batch) / q_seq;
    eb->detail_q = (r - b * rows_per_batch) % q_seq;
    eb->detail_col = c;
    eb->first_bad = key;
    if constexpr (FENCE) __threadfence();
    eb->detail_class = k;
  }
  eb->call_key = ~0ull;
  eb->done_blocks = 0u;
}

}  // namespace sa
