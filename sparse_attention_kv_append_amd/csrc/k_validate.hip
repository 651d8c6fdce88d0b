// On-device selected_indices validation (IndexShare `validate_index_rows`,
// with the per-row verdict of the host `validate_indices`).
//
// The host rule scans a row left to right. Its first violation can be found
// in parallel: while the prefix before column c is valid, the scanner's state
// at c is fixed by column c-1 alone (padding has started iff c-1 holds -1; the
// previous valid index is c-1's value otherwise). So every column is checked
// against its left neighbour at once, and the row's verdict is the violation
// with the smallest column; a row with no violation and -1 in column 0 is
// all padding. One wave owns one row and walks it 64 columns at a time; when
// there are few rows and they are long, a workgroup owns one row and each of
// its four waves walks a quarter of the columns, the first quarter with a
// violation giving the row's verdict.
//
// Into the context's error block, the launch's smallest failing (row, col)
// is gathered with an atomic minimum; the last block to finish then records
// that violation's class and values (for the host message) if no earlier
// launch since the last reset has failed, and re-arms the per-launch slot.
#include "sa_validate_dev.h"

namespace sa {

template <bool I64>
__device__ __forceinline__ int64_t shfl_up1(int64_t v) {
  if constexpr (I64) {
    const int lo = __shfl_up((int)(v & 0xffffffff), 1, 64);
    const int hi = __shfl_up((int)(v >> 32), 1, 64);
    return (int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
  } else {
    return (int64_t)__shfl_up((int)v, 1, 64);
  }
}

template <bool I64>
__device__ __forceinline__ int64_t shfl_from(int64_t v, int src) {
  if constexpr (I64) {
    const int lo = __shfl((int)(v & 0xffffffff), src, 64);
    const int hi = __shfl((int)(v >> 32), src, 64);
    return (int64_t)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
  } else {
    return (int64_t)__shfl((int)v, src, 64);
  }
}

template <bool I64>
__global__ void __launch_bounds__(256)
validate_kernel(const void* __restrict__ idx, int64_t rows, int64_t q_seq, int64_t rows_per_batch,
                int64_t width,
                const int32_t* __restrict__ valid_len, int64_t cache_len,
                uint32_t* __restrict__ word, uint8_t* __restrict__ row_class,
                uint64_t* __restrict__ first_bad, ErrorBlock* __restrict__ eb, int wide) {
  // wide == 0: one wave per row (4 rows per block); wide != 0: one block per
  // row, wave w scanning the w-th quarter of its columns (few, long rows)
  __shared__ int w_cls[4];
  __shared__ long long w_col[4];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int64_t row = wide ? (int64_t)blockIdx.x : (int64_t)blockIdx.x * 4 + wv;
  int cls = 0;
  int64_t col = -1;
  int64_t first_val = 0;
  if (row < rows) {
    const int64_t b = row / rows_per_batch;
    const int64_t bound = valid_len ? (int64_t)valid_len[b] : cache_len;
    const int64_t base = row * width;
    const int64_t seg = wide ? (width + 3) / 4 : width;
    const int64_t cbeg = wide ? min(width, (int64_t)wv * seg) : 0;
    const int64_t cend = min(width, cbeg + seg);
    first_val = load_index<I64>(idx, base);
    // value of the column left of the current chunk (column 0 has none)
    int64_t carry = cbeg > 0 ? load_index<I64>(idx, base + cbeg - 1) : 0;
    // 8 chunks of 64 columns per round trip: their loads are all in flight
    // before the first chunk is checked
    for (int64_t c0 = cbeg; c0 < cend && cls == 0; c0 += 8 * 64) {
      // unconditional loads (addresses clamped into the range) so all eight
      // are issued before the first wait; columns past it are fixed up after
      int64_t vals[8];
#pragma unroll
      for (int k = 0; k < 8; k++) {
        const int64_t c = c0 + 64 * k + lane;
        vals[k] = load_index<I64>(idx, base + (c < cend ? c : cend - 1));
      }
#pragma unroll
      for (int k = 0; k < 8; k++)
        if (c0 + 64 * k + lane >= cend) vals[k] = -1;
#pragma unroll
      for (int k = 0; k < 8; k++) {
        const int64_t c = c0 + 64 * k + lane;
        if (c0 + 64 * k >= cend || cls != 0) break;
        const int64_t v = vals[k];
        int64_t u = shfl_up1<I64>(v);
        if (lane == 0) u = carry;
        const int kc = c < cend ? column_class(c, v, u, bound) : 0;
        const uint64_t m = __ballot(kc != 0);
        if (m != 0ull) {
          const int src = __ffsll((long long)m) - 1;
          cls = __shfl(kc, src, 64);
          col = c0 + 64 * k + src;
        }
        carry = shfl_from<I64>(v, 63);
      }
    }
  }
  if (wide) {
    // the row's verdict: the first quarter holding a violation (the prefix
    // before it is valid, so its local verdict is the row's)
    if (lane == 0) {
      w_cls[wv] = cls;
      w_col[wv] = col;
    }
    __syncthreads();
    cls = 0;
    for (int w = 0; w < 4 && cls == 0; w++) {
      cls = w_cls[w];
      col = w_col[w];
    }
  }
  if (row < rows && (!wide || wv == 0)) {
    if (cls == 0 && first_val == -1) {
      cls = 6;  // the row holds only -1
      col = width;
    }
    if (lane == 0) {
      if (row_class) row_class[row] = (uint8_t)cls;
      if (cls) {
        atomicOr(word, (1u << (cls - 1)) | SA_ERR_INDEX_ANY);
        const unsigned long long key = (unsigned long long)(row * (width + 1) + col);
        atomicMin((unsigned long long*)(eb ? &eb->call_key : first_bad), key);
      }
    }
  }
  if (eb == nullptr) return;
  __syncthreads();
  if (threadIdx.x == 0)
    finish_launch<I64>(eb, idx, width, q_seq, rows_per_batch, valid_len, cache_len, gridDim.x);
}

sa_status launch_validate(sparse_attn_ctx* c, const void* idx, int64_t batch, int64_t heads,
                          int64_t q_seq, int64_t width, const int32_t* valid_len,
                          int64_t cache_len, uint32_t* word, uint8_t* row_class,
                          uint64_t* first_bad) {
  const int64_t rows = batch * heads * q_seq;
  if (rows <= 0) return SA_OK;
  // few long rows: a block per row (four waves on its columns); else a wave per row
  const int wide = (rows < 4 * kNumCUs && width >= 1024) ? 1 : 0;
  const int64_t blocks = wide ? rows : (rows + 3) / 4;
  if (blocks > 0x7fffffffLL) return set_error(c, SA_E_SHAPE, "validate_indices: too many rows");
  // the context's block gathers the first failure's detail; caller-owned
  // words and slots only get the OR and the atomic minimum
  ErrorBlock* eb = (word == &c->err->word && first_bad == &c->err->first_bad) ? c->err : nullptr;
  if (c->cfg.index_dtype == SA_IDX_I64) {
    hipLaunchKernelGGL(validate_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, c->stream, idx,
                       rows, q_seq, heads * q_seq, width, valid_len, cache_len, word, row_class,
                       first_bad, eb, wide);
  } else {
    hipLaunchKernelGGL(validate_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, c->stream,
                       idx, rows, q_seq, heads * q_seq, width, valid_len, cache_len, word,
                       row_class, first_bad, eb, wide);
  }
  return check_hip(c, hipGetLastError(), "validate_indices");
}

}  // namespace sa
