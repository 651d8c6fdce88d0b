// C ABI entry points: argument and shape checks (before any launch), the
// context, dispatch to the kernels, and error reporting. Messages for index
// errors use the IndexShare host validator's wording (`validate_indices`,
// `index_error`).
#include <math.h>
#include <stdio.h>

#include <algorithm>
#include <mutex>
#include <set>
#include <string>

#include "sa_internal.h"

namespace {

std::mutex g_reg_mu;
std::set<const sparse_attn_ctx*> g_live;

bool live(const sparse_attn_ctx* c) {
  if (!c) return false;
  std::lock_guard<std::mutex> lk(g_reg_mu);
  return g_live.count(c) != 0 && c->magic == sa::kMagic;
}

int64_t elem_bytes(int dt) { return dt == SA_F32 ? 4 : 2; }

int64_t record_bytes(int64_t dk, int64_t rope) { return (dk - rope) / 64 * 65 + 2 * rope; }

std::string fmt(const char* f, long long a = 0, long long b = 0, long long c = 0, long long d = 0) {
  char buf[256];
  snprintf(buf, sizeof buf, f, a, b, c, d);
  return buf;
}

// ---- scratch of the allocation-free forward: the split-K partials of
// sparse_attn_forward_latent_static live here, one copy per GPU the library
// runs on, held until the process ends. Host code never passes `scratch`
// itself (on the host it names a stand-in, not device memory): it passes the
// address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) uint8_t scratch[SA_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
thread_local std::string g_static_error;

// The device address of this device's scratch, looked up once per device
// with that device current.
hipError_t scratch_address(int dev, void** out) {
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

namespace sa {

sa_status set_error(sparse_attn_ctx* c, sa_status s, const std::string& msg) {
  if (c) c->last_error = msg;
  return s;
}

sa_status check_hip(sparse_attn_ctx* c, hipError_t e, const char* what) {
  if (e == hipSuccess) return SA_OK;
  return set_error(c, SA_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

ProfEvents prof_next(sparse_attn_ctx* c) {
  ProfEvents pe;
  if (c->prof_n < (int64_t)c->prof_start.size()) {
    pe.start = c->prof_start[c->prof_n];
    pe.stop = c->prof_stop[c->prof_n];
    c->prof_n++;
  }
  return pe;
}

void free_buffers(sparse_attn_ctx* c) {
  void* bufs[] = {c->err, c->partial_o, c->partial_ml, c->zeros, c->row_key, c->row_done, c->gpart_o, c->gpart_ml};
  for (void* p : bufs)
    if (p) (void)hipFree(p);
  c->err = nullptr;
  c->partial_o = c->partial_ml = nullptr;
  c->gpart_o = c->gpart_ml = nullptr;
  c->zeros = nullptr;
  c->row_key = nullptr;
  c->row_done = nullptr;
}

static void prof_release(sparse_attn_ctx* c) {
  for (hipEvent_t e : c->prof_start) (void)hipEventDestroy(e);
  for (hipEvent_t e : c->prof_stop) (void)hipEventDestroy(e);
  c->prof_start.clear();
  c->prof_stop.clear();
  c->prof_n = 0;
}

}  // namespace sa

using sa::check_hip;
using sa::set_error;

extern "C" {

const char* sparse_attn_version(void) { return "sparse_attn 0.1.0 gfx950"; }

sa_status sparse_attn_create(const sa_config* cfg, void* hip_stream, sparse_attn_ctx** out) {
  if (!cfg || !out) return SA_E_ARG;
  *out = nullptr;
  const sa_config& k = *cfg;
  if (k.num_heads <= 0 || k.kv_num_heads <= 0 || k.num_heads % k.kv_num_heads != 0) return SA_E_ARG;
  if (k.head_dim_qk <= 0 || k.head_dim_v <= 0) return SA_E_ARG;
  if (k.dtype < SA_F32 || k.dtype > SA_BF16) return SA_E_DTYPE;
  if (k.kv_layout != SA_KV_SEPARATE && k.kv_layout != SA_KV_SHARED_LATENT) return SA_E_ARG;
  if (k.index_dtype != SA_IDX_I32 && k.index_dtype != SA_IDX_I64) return SA_E_DTYPE;
  if (k.cache_format != SA_CACHE_DENSE && k.cache_format != SA_CACHE_FP8_E4M3_BLOCK64) return SA_E_ARG;
  if (k.kv_layout == SA_KV_SEPARATE && k.head_dim_v != k.head_dim_qk) return SA_E_SHAPE;
  if (k.kv_layout == SA_KV_SHARED_LATENT && k.head_dim_v > k.head_dim_qk) return SA_E_SHAPE;
  if (k.cache_format == SA_CACHE_FP8_E4M3_BLOCK64) {
    if (k.kv_layout != SA_KV_SHARED_LATENT || k.dtype != SA_BF16) return SA_E_DTYPE;
    if (k.rope_dim < 0 || k.rope_dim > k.head_dim_qk || (k.head_dim_qk - k.rope_dim) % 64 != 0)
      return SA_E_SHAPE;
  }
  if (!isfinite(k.scale) || k.scale < 0.0f) return SA_E_ARG;
  if (!isfinite(k.softcap) || k.softcap < 0.0f) return SA_E_ARG;
  if (k.max_batch <= 0 || k.max_q_seq <= 0 || k.max_index_width <= 0 || k.max_cache_len <= 0)
    return SA_E_ARG;
  if (k.max_cache_len > 0x7fffffffLL || k.max_index_width > 0x7fffffffLL) return SA_E_UNSUPPORTED;
  const bool mla = sa::mla_supported(k, 1);
  // the generic kernel holds up to 8 heads x Dv/2 channel pairs per 256 threads
  if (!mla && (k.head_dim_v % 2 != 0 || k.head_dim_v > 512 || k.head_dim_qk > 1024))
    return SA_E_UNSUPPORTED;

  sparse_attn_ctx* c = new sparse_attn_ctx();
  c->magic = sa::kMagic;
  c->cfg = k;
  if (c->cfg.scale == 0.0f) c->cfg.scale = 1.0f / sqrtf((float)k.head_dim_qk);
  c->stream = (hipStream_t)hip_stream;
  c->err = nullptr;
  c->partial_o = nullptr;
  c->partial_ml = nullptr;
  c->gpart_o = nullptr;
  c->gpart_ml = nullptr;
  c->gpart_rows = 0;
  c->partial_rows = 0;
  c->zeros = nullptr;
  c->row_key = nullptr;
  c->row_done = nullptr;
  c->rows_cap = k.max_batch * k.max_q_seq;
  c->prof_n = 0;
  hipError_t e = hipGetDevice(&c->device);
  if (e == hipSuccess) e = hipMalloc((void**)&c->err, sizeof(sa::ErrorBlock));
  if (e == hipSuccess && mla) {
    const int64_t rows_max = k.max_batch * k.max_q_seq;
    int64_t need = 0;
    for (int64_t r = 1; r <= std::min<int64_t>(rows_max, sa::kNumCUs); r++) {
      const int s = sa::mla_splits(r, k.max_index_width);
      if (s > 1) need = std::max<int64_t>(need, r * s);
    }
    c->partial_rows = need;
    if (need > 0) {
      e = hipMalloc((void**)&c->partial_o, (size_t)need * k.num_heads * k.head_dim_v * sizeof(float));
      if (e == hipSuccess)
        e = hipMalloc((void**)&c->partial_ml, (size_t)need * k.num_heads * 2 * sizeof(float));
    }
  }
  if (e == hipSuccess && sa::gqa_supported(k, 1)) {
    const int64_t need = sa::gqa_partial_rows(k);
    e = hipMalloc((void**)&c->gpart_o, (size_t)need * 128 * sizeof(float));
    if (e == hipSuccess) e = hipMalloc((void**)&c->gpart_ml, (size_t)need * 2 * sizeof(float));
    if (e == hipSuccess) c->gpart_rows = need;
  }
  if (e == hipSuccess) e = hipMalloc((void**)&c->zeros, 1024);
  if (e == hipSuccess) e = hipMemset(c->zeros, 0, 1024);
  if (e == hipSuccess && (mla || sa::gqa_supported(k, 1))) {
    e = hipMalloc((void**)&c->row_key, (size_t)c->rows_cap * sizeof(unsigned long long));
    if (e == hipSuccess) e = hipMemset(c->row_key, 0xff, (size_t)c->rows_cap * sizeof(unsigned long long));
    if (e == hipSuccess) e = hipMalloc((void**)&c->row_done, (size_t)c->rows_cap * sizeof(unsigned));
    if (e == hipSuccess) e = hipMemset(c->row_done, 0, (size_t)c->rows_cap * sizeof(unsigned));
  }
  if (e == hipSuccess) {
    sa::launch_reset_error(c);
    e = hipStreamSynchronize(c->stream);
  }
  if (e != hipSuccess) {
    sa::free_buffers(c);
    delete c;
    return SA_E_HIP;
  }
  {
    std::lock_guard<std::mutex> lk(g_reg_mu);
    g_live.insert(c);
  }
  *out = c;
  return SA_OK;
}

sa_status sparse_attn_destroy(sparse_attn_ctx* c) {
  if (!c) return SA_OK;
  {
    std::lock_guard<std::mutex> lk(g_reg_mu);
    if (!g_live.count(c)) return SA_E_STATE;
    g_live.erase(c);
  }
  (void)hipStreamSynchronize(c->stream);
  sa::prof_release(c);
  sa::free_buffers(c);
  c->magic = 0;
  delete c;
  return SA_OK;
}

sa_status sparse_attn_set_stream(sparse_attn_ctx* c, void* hip_stream) {
  if (!live(c)) return SA_E_STATE;
  c->stream = (hipStream_t)hip_stream;
  return SA_OK;
}

sa_status sparse_attn_reset_error_async(sparse_attn_ctx* c) {
  if (!live(c)) return SA_E_STATE;
  return sa::launch_reset_error(c);
}

sa_status sparse_attn_measure_copy(sparse_attn_ctx* c, void* dst, const void* src, int64_t bytes) {
  if (!live(c)) return SA_E_STATE;
  if (!dst || !src || bytes < 16 || bytes % 16 || ((uintptr_t)dst | (uintptr_t)src) % 16)
    return set_error(c, SA_E_ARG, "measure_copy: NULL buffer, or size or address not a positive multiple of 16");
  const uintptr_t d = (uintptr_t)dst, s = (uintptr_t)src;
  if (d < s + (uintptr_t)bytes && s < d + (uintptr_t)bytes)
    return set_error(c, SA_E_ARG, "measure_copy: buffers overlap");
  return sa::launch_peak_copy(c, dst, src, bytes, nullptr);
}

sa_status sparse_attn_measure_read(sparse_attn_ctx* c, uint32_t* sink, const void* src, int64_t bytes) {
  if (!live(c)) return SA_E_STATE;
  if (!sink || !src || bytes < 16 || bytes % 16 || (uintptr_t)src % 16)
    return set_error(c, SA_E_ARG, "measure_read: NULL buffer, or size or address not a positive multiple of 16");
  return sa::launch_peak_copy(c, nullptr, src, bytes, sink);
}

sa_status sparse_attn_measure_mfma(sparse_attn_ctx* c, float* out, int64_t workgroups, int32_t iters) {
  if (!live(c)) return SA_E_STATE;
  if (!out || workgroups < 1 || workgroups > 65536 || iters < 1 || iters > (1 << 20))
    return set_error(c, SA_E_ARG, "measure_mfma: NULL output, workgroups outside 1..65536 or iters outside 1..2^20");
  return sa::launch_peak_mfma(c, out, workgroups, iters);
}

sa_status sparse_attn_kv_append(sparse_attn_ctx* c, int64_t batch, const void* past_k,
                                const void* past_v, int64_t past_capacity, const int32_t* past_len,
                                const void* cur_k, const void* cur_v, int64_t cur_len,
                                int32_t cur_is_unquantized_bf16, void* present_k, void* present_v,
                                int64_t present_capacity, int32_t* present_len) {
  if (!live(c)) return SA_E_STATE;
  const sa_config& k = c->cfg;
  c->last_error.clear();
  if (batch <= 0 || batch > k.max_batch)
    return set_error(c, SA_E_STATE, fmt("kv_append: batch %lld outside [1, max_batch %lld]", batch, k.max_batch));
  if (cur_len < 0 || past_capacity < 0 || present_capacity <= 0)
    return set_error(c, SA_E_ARG, "kv_append: negative length or non-positive present capacity");
  if (!cur_k || !present_k) return set_error(c, SA_E_ARG, "kv_append: cur_k and present_k are required");
  const bool latent = k.kv_layout == SA_KV_SHARED_LATENT;
  if (latent && (past_v || cur_v || present_v))
    return set_error(c, SA_E_ARG, "kv_append: shared-latent caches take no value tensors");
  if (!latent && (!cur_v || !present_v))
    return set_error(c, SA_E_ARG, "kv_append: cur_v and present_v are required");
  if (past_capacity > 0 && (!past_k || (!latent && !past_v)))
    return set_error(c, SA_E_ARG, "kv_append: past tensors are required when past_capacity > 0");
  const bool fp8 = k.cache_format == SA_CACHE_FP8_E4M3_BLOCK64;
  if (cur_is_unquantized_bf16 && !fp8)
    return set_error(c, SA_E_DTYPE, "kv_append: cur_is_unquantized_bf16 needs an fp8_e4m3_block64 cache");
  if (!past_len && past_capacity + cur_len > present_capacity)
    return set_error(c, SA_E_CAPACITY,
                     fmt("kv_append: past %lld + current %lld rows exceed present capacity %lld",
                         past_capacity, cur_len, present_capacity));
  if (cur_len > present_capacity)
    return set_error(c, SA_E_CAPACITY, "kv_append: current rows exceed present capacity");
  // in place (present aliases past): both views must use the one row stride
  if (past_capacity > 0 && past_capacity != present_capacity &&
      (present_k == past_k || (!latent && present_v == past_v)))
    return set_error(c, SA_E_ARG,
                     fmt("kv_append: in place (present aliases past) needs past_capacity %lld == present_capacity %lld",
                         past_capacity, present_capacity));
  const int64_t heads = k.kv_num_heads;
  const int64_t krow = fp8 ? record_bytes(k.head_dim_qk, k.rope_dim) : k.head_dim_qk * elem_bytes(k.dtype);
  const bool copy_past = past_capacity > 0 && present_k != past_k;
  sa_status s;
  if (fp8 && cur_is_unquantized_bf16) {
    if (copy_past) {
      s = sa::launch_append_copy(c, batch, heads, krow, past_k, past_capacity, past_len, nullptr, 0,
                                 present_k, present_capacity, true, nullptr);
      if (s != SA_OK) return s;
    }
    s = sa::launch_append_quantize(c, batch, heads, k.head_dim_qk, k.rope_dim, cur_k, cur_len,
                                   past_len, past_capacity, present_k, present_capacity, present_len);
    return s;
  }
  if (latent)
    return sa::launch_append_copy(c, batch, heads, krow, past_k, past_capacity, past_len, cur_k, cur_len,
                                  present_k, present_capacity, copy_past, present_len);
  const int64_t vrow = k.head_dim_v * elem_bytes(k.dtype);
  const bool copy_past_v = past_capacity > 0 && present_v != past_v;
  if (vrow == krow && copy_past_v == copy_past)  // K and V in one launch
    return sa::launch_append_copy(c, batch, heads, krow, past_k, past_capacity, past_len, cur_k, cur_len,
                                  present_k, present_capacity, copy_past, present_len, past_v, cur_v, present_v);
  s = sa::launch_append_copy(c, batch, heads, krow, past_k, past_capacity, past_len, cur_k, cur_len,
                             present_k, present_capacity, copy_past, present_len);
  if (s != SA_OK) return s;
  return sa::launch_append_copy(c, batch, heads, vrow, past_v, past_capacity, past_len, cur_v,
                                cur_len, present_v, present_capacity, copy_past_v, nullptr);
}

static sa_status check_index_geometry(sparse_attn_ctx* c, int64_t batch, int64_t index_heads,
                                      int64_t q_seq, int64_t width) {
  const sa_config& k = c->cfg;
  if (batch <= 0 || batch > k.max_batch)
    return set_error(c, SA_E_STATE, fmt("batch %lld outside [1, max_batch %lld]", batch, k.max_batch));
  if (q_seq <= 0 || q_seq > k.max_q_seq)
    return set_error(c, SA_E_STATE, fmt("q_seq %lld outside [1, max_q_seq %lld]", q_seq, k.max_q_seq));
  if (width <= 0) return set_error(c, SA_E_SHAPE, "selected_indices K dimension must be nonzero");
  if (width > k.max_index_width)
    return set_error(c, SA_E_STATE, fmt("index width %lld above max_index_width %lld", width, k.max_index_width));
  if (index_heads != 1 && index_heads != k.num_heads)
    return set_error(c, SA_E_SHAPE, fmt("selected_indices must have shape [B, 1|N, S_q, K] (N = %lld), got %lld heads",
                                         k.num_heads, index_heads));
  return SA_OK;
}

sa_status sparse_attn_validate_indices(sparse_attn_ctx* c, const void* indices, int64_t batch,
                                       int64_t index_heads, int64_t q_seq, int64_t width,
                                       const int32_t* valid_len, int64_t cache_len,
                                       uint32_t* error_word, uint8_t* row_class,
                                       uint64_t* first_bad) {
  if (!live(c)) return SA_E_STATE;
  c->last_error.clear();
  if (!indices) return set_error(c, SA_E_ARG, "validate_indices: indices is NULL");
  sa_status s = check_index_geometry(c, batch, index_heads, q_seq, width);
  if (s != SA_OK) return s;
  if (!valid_len && cache_len < 0) return set_error(c, SA_E_ARG, "validate_indices: negative cache_len");
  if (!error_word) error_word = &c->err->word;
  if (!first_bad) first_bad = &c->err->first_bad;
  return sa::launch_validate(c, indices, batch, index_heads, q_seq, width, valid_len, cache_len,
                             error_word, row_class, first_bad);
}

namespace sa {
// The kernel that runs a forward launch: 0 = generic, 1 = register-staged
// shared-latent fallback, 2 = shared-latent LDS-ring kernel over bf16 rows,
// 3 = wave-pair kernel over fp8 records, 4 = grouped-query kernel.
static int forward_path(const sa_config& k, int64_t index_heads) {
  if (gqa_supported(k, index_heads)) return 4;
  if (!mla_supported(k, index_heads)) return 0;
  if (latent_supported(k, index_heads)) return 2;
  if (pair_supported(k, index_heads)) return 3;
  return 1;
}
}  // namespace sa

sa_status sparse_attn_query_plan(const sparse_attn_ctx* c, int64_t batch, int64_t q_seq,
                                 int64_t index_heads, int64_t width, int32_t* path, int32_t* splits) {
  if (!live(c) || !path || !splits) return SA_E_STATE;
  *path = sa::forward_path(c->cfg, index_heads);
  *splits = (*path >= 1 && *path <= 3) ? sa::mla_splits(batch * q_seq, width)
            : (*path == 4 ? sa::gqa_splits(c, batch, q_seq, width) : 1);
  return SA_OK;
}

// forward, optionally with the in-launch append of the shared-latent kernel
static sa_status forward_impl(sparse_attn_ctx* c, const void* q, int64_t batch, int64_t q_seq,
                              const void* present_k, const void* present_v, int64_t cache_capacity,
                              const int32_t* valid_len, const void* indices, int64_t index_heads,
                              int64_t width, void* y, int32_t fused_validate, const sa::AppendArgs* app,
                              const void* bias = nullptr, const int64_t* bd = nullptr) {
  const sa_config& k = c->cfg;
  if (!q || !present_k || !indices || !y) return set_error(c, SA_E_ARG, "forward: q, present_k, indices and y are required");
  const bool latent = k.kv_layout == SA_KV_SHARED_LATENT;
  if (latent && present_v) return set_error(c, SA_E_ARG, "forward: shared-latent caches take no present_v");
  if (!latent && !present_v) return set_error(c, SA_E_ARG, "forward: present_v is required");
  if (cache_capacity <= 0 || cache_capacity > k.max_cache_len)
    return set_error(c, SA_E_STATE, fmt("forward: cache capacity %lld outside [1, max_cache_len %lld]",
                                        cache_capacity, k.max_cache_len));
  sa_status s = check_index_geometry(c, batch, index_heads, q_seq, width);
  if (s != SA_OK) return s;
  // the shared-latent MFMA kernels validate their own columns; other paths
  // run the validation kernel first on the same stream
  // a biased forward runs on the MFMA kernel of its layout where there is one
  // (a bf16 shared-latent cache takes the general latent kernel with its
  // split-K combine, not the decode kernel), else on the generic kernel
  const int path = !bias                                 ? sa::forward_path(k, index_heads)
                   : sa::gqa_supported(k, index_heads)    ? 4
                   : sa::latent_supported(k, index_heads) ? 2
                   : sa::pair_supported(k, index_heads)   ? 3
                                                          : 0;
  const bool gqa_fused = path == 4 && app && sa::gqa_fuses(k, q_seq);
  if (fused_validate && path != 2 && path != 3 && !gqa_fused) {
    s = sparse_attn_validate_indices(c, indices, batch, index_heads, q_seq, width, valid_len,
                                     cache_capacity, nullptr, nullptr, nullptr);
    if (s != SA_OK) return s;
  }
  sa::FwdArgs a;
  a.q = q;
  a.k = present_k;
  a.v = present_v;
  a.idx = indices;
  a.valid_len = valid_len;
  a.y = y;
  a.batch = batch;
  a.hq = k.num_heads;
  a.hkv = k.kv_num_heads;
  a.q_seq = q_seq;
  a.dk = k.head_dim_qk;
  a.dv = k.head_dim_v;
  a.rope = k.rope_dim;
  a.cap = cache_capacity;
  a.index_heads = index_heads;
  a.width = width;
  a.scale = k.scale;
  a.softcap = k.softcap;
  a.dtype = k.dtype;
  a.cache_format = k.cache_format;
  a.kv_layout = k.kv_layout;
  a.idx64 = k.index_dtype == SA_IDX_I64;
  if (bias) {
    a.bias = bias;
    for (int i = 0; i < 4; i++) a.bd[i] = bd[i];
  }
  if (app && (path == 4 ? (!app->cur_v || !gqa_fused) : (path != 2 && path != 3)))
    return set_error(c, SA_E_UNSUPPORTED, "step: the in-launch append needs an MFMA path of the cache's layout");
  switch (path) {
    case 2: {
      const int splits = sa::mla_splits(batch * q_seq, width);
      return !bias && sa::latent_decode_fits(q_seq)
                 ? sa::launch_forward_latent_decode(c, a, splits, fused_validate != 0, app)
                 : sa::launch_forward_latent(c, a, splits, fused_validate != 0, app);
    }
    case 3: return sa::launch_forward_pair(c, a, sa::mla_splits(batch * q_seq, width), fused_validate != 0, app);
    case 1: return sa::launch_forward_mla(c, a, sa::mla_splits(batch * q_seq, width));
    case 4: return sa::launch_forward_gqa(c, a, gqa_fused, gqa_fused ? app : nullptr);
    default: return sa::launch_forward_generic(c, a);
  }
}

sa_status sparse_attn_forward(sparse_attn_ctx* c, const void* q, int64_t batch, int64_t q_seq,
                              const void* present_k, const void* present_v,
                              int64_t cache_capacity, const int32_t* valid_len,
                              const void* indices, int64_t index_heads, int64_t width, void* y,
                              int32_t fused_validate) {
  if (!live(c)) return SA_E_STATE;
  c->last_error.clear();
  return forward_impl(c, q, batch, q_seq, present_k, present_v, cache_capacity, valid_len, indices,
                      index_heads, width, y, fused_validate, nullptr);
}

// A bias shape of rank <= 4, right-aligned against `target` and padded with
// 1 on the left into bd; every extent must be 1 or the target's (IndexShare
// `validate_bias_shape`).
static sa_status bias_dims(sparse_attn_ctx* c, const char* who, const int64_t* shape, int32_t rank,
                           const int64_t target[4], int64_t bd[4]) {
  if (rank < 0 || rank > 4)
    return set_error(c, SA_E_SHAPE, std::string(who) + fmt(": attention_bias rank %lld exceeds 4", rank));
  if (rank > 0 && !shape) return set_error(c, SA_E_ARG, std::string(who) + ": attention_bias shape is NULL");
  for (int a = 0; a < 4; a++) bd[a] = 1;
  for (int i = 0; i < rank; i++) bd[4 - rank + i] = shape[i];
  for (int a = 0; a < 4; a++)
    if (bd[a] != 1 && bd[a] != target[a])
      return set_error(c, SA_E_SHAPE,
                       std::string(who) + fmt(": attention_bias dimension %lld is not broadcastable to ", bd[a]) +
                           fmt("[%lld, %lld, %lld, %lld]", target[0], target[1], target[2], target[3]));
  return SA_OK;
}

sa_status sparse_attn_forward_bias(sparse_attn_ctx* c, const void* q, int64_t batch, int64_t q_seq,
                                   const void* present_k, const void* present_v, int64_t cache_capacity,
                                   const int32_t* valid_len, const void* indices, int64_t index_heads,
                                   int64_t width, const void* bias, const int64_t* bias_shape,
                                   int32_t bias_rank, void* y, int32_t fused_validate) {
  if (!live(c)) return SA_E_STATE;
  c->last_error.clear();
  if (!bias)
    return forward_impl(c, q, batch, q_seq, present_k, present_v, cache_capacity, valid_len, indices,
                        index_heads, width, y, fused_validate, nullptr);
  const int64_t target[4] = {batch, c->cfg.num_heads, q_seq, cache_capacity};
  int64_t bd[4];
  sa_status s = bias_dims(c, "forward", bias_shape, bias_rank, target, bd);
  if (s != SA_OK) return s;
  return forward_impl(c, q, batch, q_seq, present_k, present_v, cache_capacity, valid_len, indices,
                      index_heads, width, y, fused_validate, nullptr, bias, bd);
}

sa_status sparse_attn_capacity_lengths(sparse_attn_ctx* c, const void* bias, const int64_t* bias_shape,
                                       int32_t bias_rank, int64_t batch, int64_t q_seq,
                                       int64_t cache_capacity, int64_t cur_len, int32_t* valid_len,
                                       int32_t* write_pos) {
  if (!live(c)) return SA_E_STATE;
  const sa_config& k = c->cfg;
  c->last_error.clear();
  if (!bias)
    return set_error(c, SA_E_ARG,
                     "capacity_lengths: capacity-mode IndexShare requires attention_bias to derive the valid length");
  if (!valid_len || !write_pos) return set_error(c, SA_E_ARG, "capacity_lengths: valid_len and write_pos are required");
  if (batch <= 0 || batch > k.max_batch)
    return set_error(c, SA_E_STATE, fmt("capacity_lengths: batch %lld outside [1, max_batch %lld]", batch, k.max_batch));
  if (q_seq <= 0 || cur_len < 0 || cache_capacity <= 0 || cache_capacity > 0x7fffffffLL)
    return set_error(c, SA_E_ARG, "capacity_lengths: q_seq and cache_capacity must be positive (capacity below "
                                  "2^31) and cur_len non-negative");
  const int64_t target[4] = {batch, k.num_heads, q_seq, cache_capacity};
  int64_t bd[4];
  sa_status s = bias_dims(c, "capacity_lengths", bias_shape, bias_rank, target, bd);
  if (s != SA_OK) return s;
  return sa::launch_capacity_lengths(c, bias, k.dtype, bd, batch, cache_capacity, cur_len, valid_len, write_pos);
}

sa_status sparse_attn_capacity_step(sparse_attn_ctx* c, const void* q, int64_t batch, int64_t q_seq, void* cache_k,
                                    void* cache_v, int64_t cache_capacity, const void* cur_k, const void* cur_v,
                                    int64_t cur_len, const void* indices, int64_t index_heads, int64_t width,
                                    const void* bias, const int64_t* bias_shape, int32_t bias_rank, void* y,
                                    int32_t* valid_len, int32_t* write_pos, int32_t reset_error) {
  if (!live(c)) return SA_E_STATE;
  const sa_config& k = c->cfg;
  c->last_error.clear();
  const bool latent = k.kv_layout == SA_KV_SHARED_LATENT;
  if (!latent && k.cache_format != SA_CACHE_DENSE)
    return set_error(c, SA_E_UNSUPPORTED, "capacity_step: separate K and V caches must be dense");
  if (latent ? (!cache_k || !cur_k || cache_v || cur_v) : (!cache_k || !cache_v || !cur_k || !cur_v))
    return set_error(c, SA_E_ARG, latent ? "capacity_step: a shared-latent cache takes cache_k and cur_k only"
                                         : "capacity_step: cache_k, cache_v, cur_k and cur_v are required");
  if (cur_len <= 0 || cur_len > cache_capacity)
    return set_error(c, SA_E_CAPACITY, "capacity_step: cur_len must be in [1, cache_capacity]");
  if (cache_capacity > k.max_cache_len)
    return set_error(c, SA_E_STATE, fmt("capacity_step: cache capacity %lld above max_cache_len %lld", cache_capacity,
                                        k.max_cache_len));
  // argument checks of the three calls, before anything is launched
  sa_status s = check_index_geometry(c, batch, index_heads, q_seq, width);
  if (s != SA_OK) return s;
  if (!q || !indices || !y) return set_error(c, SA_E_ARG, "capacity_step: q, indices and y are required");
  if (!bias)
    return set_error(c, SA_E_ARG,
                     "capacity_step: capacity-mode IndexShare requires attention_bias to derive the valid length");
  if (!valid_len || !write_pos) return set_error(c, SA_E_ARG, "capacity_step: valid_len and write_pos are required");
  if (cache_capacity > 0x7fffffffLL) return set_error(c, SA_E_ARG, "capacity_step: cache capacity must be below 2^31");
  const int64_t target[4] = {batch, k.num_heads, q_seq, cache_capacity};
  int64_t bd[4];
  s = bias_dims(c, "capacity_step", bias_shape, bias_rank, target, bd);
  if (s != SA_OK) return s;
  const int64_t row = k.head_dim_qk * elem_bytes(k.dtype);
  const uintptr_t mis = (uintptr_t)cache_k | (uintptr_t)cache_v | (uintptr_t)cur_k | (uintptr_t)cur_v;
  // fp8 records (648 bytes, not whole 16-byte units) go through kv_append
  if (k.cache_format == SA_CACHE_DENSE && (latent || k.head_dim_v == k.head_dim_qk) && row % 16 == 0 &&
      (mis & 15) == 0) {
    // the reset, the lengths and the in-place append in one launch
    s = sa::launch_capacity_append(c, bias, k.dtype, bd, batch, cache_capacity, cur_len, valid_len, write_pos, cur_k,
                                   cur_v, cache_k, cache_v, k.kv_num_heads, row, reset_error ? c->err : nullptr);
  } else {
    if (reset_error) {
      s = sa::launch_reset_error(c);
      if (s != SA_OK) return s;
    }
    s = sa::launch_capacity_lengths(c, bias, k.dtype, bd, batch, cache_capacity, cur_len, valid_len, write_pos);
    if (s == SA_OK)
      s = sparse_attn_kv_append(c, batch, cache_k, cache_v, cache_capacity, write_pos, cur_k, cur_v, cur_len, 0,
                                cache_k, cache_v, cache_capacity, nullptr);
  }
  if (s != SA_OK) return s;
  return forward_impl(c, q, batch, q_seq, cache_k, cache_v, cache_capacity, valid_len, indices, index_heads, width, y,
                      1, nullptr, bias, bd);
}

sa_status sparse_attn_step(sparse_attn_ctx* c, const void* q, int64_t batch, int64_t q_seq, void* cache,
                           int64_t cache_capacity, const int32_t* past_len, const void* cur, int64_t cur_len,
                           int32_t cur_is_unquantized_bf16, int32_t* present_len, const void* indices,
                           int64_t index_heads, int64_t width, void* y, int32_t reset_error) {
  if (!live(c)) return SA_E_STATE;
  c->last_error.clear();
  const sa_config& k = c->cfg;
  if (k.kv_layout != SA_KV_SHARED_LATENT)
    return set_error(c, SA_E_UNSUPPORTED, "step: shared-latent caches only (use kv_append + forward)");
  if (!cache || !cur || !past_len || !present_len)
    return set_error(c, SA_E_ARG, "step: cache, cur, past_len and present_len are required");
  if (batch <= 0 || batch > k.max_batch)
    return set_error(c, SA_E_STATE, fmt("step: batch %lld outside [1, max_batch %lld]", batch, k.max_batch));
  if (cur_len < 0 || cache_capacity <= 0 || cache_capacity > k.max_cache_len)
    return set_error(c, SA_E_ARG, "step: negative cur_len or cache capacity outside [1, max_cache_len]");
  if (cur_len > cache_capacity)
    return set_error(c, SA_E_CAPACITY, "step: current rows exceed the cache capacity");
  if (cur_is_unquantized_bf16 && k.cache_format != SA_CACHE_FP8_E4M3_BLOCK64)
    return set_error(c, SA_E_DTYPE, "step: cur_is_unquantized_bf16 needs an fp8_e4m3_block64 cache");
  // the forward's argument checks too, before the reset or the append is launched
  if (!q || !indices || !y) return set_error(c, SA_E_ARG, "step: q, indices and y are required");
  sa_status gs = check_index_geometry(c, batch, index_heads, q_seq, width);
  if (gs != SA_OK) return gs;
  const int path = sa::forward_path(k, index_heads);
  if ((path == 2 || path == 3) && cur_len <= sa::kFusedAppendRows) {
    sa::AppendArgs app;
    app.cur = cur;
    app.past_len = past_len;
    app.present_len = present_len;
    app.cur_len = cur_len;
    app.reset = reset_error != 0;
    app.quant = cur_is_unquantized_bf16 != 0;
    return forward_impl(c, q, batch, q_seq, cache, nullptr, cache_capacity, present_len, indices, index_heads,
                        width, y, 1, &app);
  }
  sa_status s = SA_OK;
  if (reset_error) s = sa::launch_reset_error(c);
  if (s == SA_OK)
    s = sparse_attn_kv_append(c, batch, cache, nullptr, cache_capacity, past_len, cur, nullptr, cur_len,
                              cur_is_unquantized_bf16, cache, nullptr, cache_capacity, present_len);
  if (s == SA_OK)
    s = sparse_attn_forward(c, q, batch, q_seq, cache, nullptr, cache_capacity, present_len, indices,
                            index_heads, width, y, 1);
  return s;
}

sa_status sparse_attn_step_kv(sparse_attn_ctx* c, const void* q, int64_t batch, int64_t q_seq, void* cache_k,
                              void* cache_v, int64_t cache_capacity, const int32_t* past_len, const void* cur_k,
                              const void* cur_v, int64_t cur_len, int32_t* present_len, const void* indices,
                              int64_t index_heads, int64_t width, void* y, int32_t reset_error) {
  if (!live(c)) return SA_E_STATE;
  c->last_error.clear();
  const sa_config& k = c->cfg;
  if (k.kv_layout != SA_KV_SEPARATE)
    return set_error(c, SA_E_UNSUPPORTED, "step_kv: separate K and V caches only (use sparse_attn_step)");
  if (!cache_k || !cache_v || !cur_k || !cur_v || !past_len || !present_len)
    return set_error(c, SA_E_ARG, "step_kv: cache_k, cache_v, cur_k, cur_v, past_len and present_len are required");
  if (batch <= 0 || batch > k.max_batch)
    return set_error(c, SA_E_STATE, fmt("step_kv: batch %lld outside [1, max_batch %lld]", batch, k.max_batch));
  if (cur_len < 0 || cache_capacity <= 0 || cache_capacity > k.max_cache_len)
    return set_error(c, SA_E_ARG, "step_kv: negative cur_len or cache capacity outside [1, max_cache_len]");
  if (cur_len > cache_capacity) return set_error(c, SA_E_CAPACITY, "step_kv: current rows exceed the cache capacity");
  if (!q || !indices || !y) return set_error(c, SA_E_ARG, "step_kv: q, indices and y are required");
  sa_status gs = check_index_geometry(c, batch, index_heads, q_seq, width);
  if (gs != SA_OK) return gs;
  const int path = sa::forward_path(k, index_heads);
  const uintptr_t mis = (uintptr_t)cache_k | (uintptr_t)cache_v | (uintptr_t)cur_k | (uintptr_t)cur_v;
  if (path == 4 && sa::gqa_fuses(k, q_seq) && (mis & 15) == 0) {
    sa::AppendArgs app;
    app.cur = cur_k;
    app.cur_v = cur_v;
    app.past_len = past_len;
    app.present_len = present_len;
    app.cur_len = cur_len;
    app.reset = reset_error != 0;
    app.quant = 0;
    return forward_impl(c, q, batch, q_seq, cache_k, cache_v, cache_capacity, present_len, indices, index_heads,
                        width, y, 1, &app);
  }
  sa_status s = SA_OK;
  if (reset_error) s = sa::launch_reset_error(c);
  if (s == SA_OK)
    s = sparse_attn_kv_append(c, batch, cache_k, cache_v, cache_capacity, past_len, cur_k, cur_v, cur_len, 0,
                              cache_k, cache_v, cache_capacity, present_len);
  if (s == SA_OK)
    s = sparse_attn_forward(c, q, batch, q_seq, cache_k, cache_v, cache_capacity, present_len, indices,
                            index_heads, width, y, 1);
  return s;
}

sa_status sparse_attn_csa_forward(sparse_attn_ctx* c, const float* query, int64_t batch, int64_t q_seq,
                                  int64_t heads, const float* current_kv, int64_t cur_len,
                                  const uint8_t* records, int64_t record_cap, const int32_t* selected,
                                  int64_t index_heads, int64_t topk, const float* head_sink,
                                  const float* bias, const int64_t* bias_dims, const int64_t* total_len,
                                  float scale, float* y) {
  if (!live(c)) return SA_E_STATE;
  c->last_error.clear();
  if (!query || !current_kv || !records || !selected || !head_sink || !total_len || !y)
    return set_error(c, SA_E_ARG, "csa_forward: a required pointer is NULL");
  if (batch < 1 || q_seq < 1 || heads < 1 || cur_len < 1 || record_cap < 1 || index_heads < 1 || topk < 1)
    return set_error(c, SA_E_ARG, "csa_forward: every size must be at least 1");
  if (!isfinite(scale) || scale < 0.0f) return set_error(c, SA_E_ARG, "csa_forward: scale must be finite and >= 0");
  if (heads % 16 != 0) return set_error(c, SA_E_UNSUPPORTED, "csa_forward: heads must be a multiple of 16");
  if (topk > 2048) return set_error(c, SA_E_UNSUPPORTED, "csa_forward: selected width above 2048");
  if (cur_len * 2048 >= (1LL << 31) || record_cap * 583 >= (1LL << 31))
    return set_error(c, SA_E_UNSUPPORTED, "csa_forward: current_kv or record buffer of a batch entry >= 2 GiB");
  if (batch * q_seq * (heads / 16) >= (1LL << 31) || batch * index_heads * q_seq * topk >= (1LL << 40))
    return set_error(c, SA_E_UNSUPPORTED, "csa_forward: grid too large");
  sa::CsaArgs a;
  a.q = query;
  a.ckv = current_kv;
  a.rec = records;
  a.sel = selected;
  a.sink = head_sink;
  a.bias = bias;
  a.total = total_len;
  a.y = y;
  a.batch = batch;
  a.q_seq = q_seq;
  a.heads = heads;
  a.cur_len = cur_len;
  a.record_cap = record_cap;
  a.index_heads = index_heads;
  a.topk = topk;
  a.scale = scale == 0.0f ? 1.0f / sqrtf(512.0f) : scale;
  for (int i = 0; i < 4; i++) a.bias_dims[i] = 1;
  if (bias) {
    if (!bias_dims) return set_error(c, SA_E_ARG, "csa_forward: bias needs bias_dims");
    const int64_t full[3] = {batch, heads, q_seq};
    for (int i = 0; i < 3; i++)
      if (bias_dims[i] != 1 && bias_dims[i] != full[i])
        return set_error(c, SA_E_SHAPE, fmt("csa_forward: bias extent %d is %lld, not 1 or %lld", i,
                                            (long long)bias_dims[i], (long long)full[i]));
    if (bias_dims[3] != 1 && (bias_dims[3] < topk + 1 || bias_dims[3] > topk + 128))
      return set_error(c, SA_E_SHAPE, "csa_forward: bias last extent is neither 1 nor (window candidates + K)");
    for (int i = 0; i < 4; i++) a.bias_dims[i] = bias_dims[i];
  }
  return sa::launch_csa_attention(c, a);
}

size_t sparse_attn_csa_index_workspace_bytes(int64_t batch, int64_t q_seq, int64_t heads, int64_t key_cap) {
  if (batch < 1 || q_seq < 1 || heads < 1 || key_cap < 1) return 0;
  return sa::csa_index_workspace_bytes(batch * q_seq, heads, key_cap);
}

sa_status sparse_attn_csa_index_select(sparse_attn_ctx* c, const float* index_query, const float* index_weight,
                                       const uint8_t* index_keys, int64_t batch, int64_t q_seq, int64_t heads,
                                       int64_t key_cap, const int64_t* total_len, int64_t topk,
                                       int64_t out_heads, int32_t* selected, void* workspace) {
  if (!live(c)) return SA_E_STATE;
  c->last_error.clear();
  if (!index_query || !index_weight || !index_keys || !total_len || !selected || !workspace)
    return set_error(c, SA_E_ARG, "csa_index_select: a required pointer is NULL");
  if (batch < 1 || q_seq < 1 || heads < 1 || key_cap < 1 || topk < 1 || out_heads < 1)
    return set_error(c, SA_E_ARG, "csa_index_select: every size must be at least 1");
  if (heads % 16 != 0 || heads > 64)
    return set_error(c, SA_E_UNSUPPORTED, "csa_index_select: index heads must be 16, 32, 48 or 64");
  if (topk > 2048) return set_error(c, SA_E_UNSUPPORTED, "csa_index_select: selected width above 2048");
  if (key_cap > 32768) return set_error(c, SA_E_UNSUPPORTED, "csa_index_select: more than 32768 index keys");
  if (batch * q_seq >= 65536) return set_error(c, SA_E_UNSUPPORTED, "csa_index_select: batch * q_seq >= 65536");
  sa::CsaIndexArgs a;
  a.iq = index_query;
  a.iw = index_weight;
  a.keys = index_keys;
  a.total = total_len;
  a.selected = selected;
  a.workspace = workspace;
  a.batch = batch;
  a.q_seq = q_seq;
  a.heads = heads;
  a.key_cap = key_cap;
  a.topk = topk;
  a.out_heads = out_heads;
  return sa::launch_csa_index_select(c, a);
}

sa_status sparse_attn_read_error(sparse_attn_ctx* c, uint32_t* word, uint64_t* first_bad) {
  if (!live(c)) return SA_E_STATE;
  sa::ErrorBlock eb;
  hipError_t e = hipStreamSynchronize(c->stream);
  if (e == hipSuccess) e = hipMemcpy(&eb, c->err, sizeof eb, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return check_hip(c, e, "read_error");
  if (word) *word = eb.word;
  if (first_bad) *first_bad = eb.first_bad;
  if (eb.word == 0) {
    c->last_error.clear();
    return SA_OK;
  }
  std::string msg;
  if ((eb.word & SA_ERR_INDEX_ANY) && eb.detail_class != 0) {
    const long long b = eb.detail_b, h = eb.detail_h, q = eb.detail_q, col = eb.detail_col;
    const long long v = eb.detail_value, u = eb.detail_prev, bound = eb.detail_bound;
    const std::string head =
        fmt("selected_indices [batch=%lld, head=%lld, query=%lld, column=%lld]: ", b, h, q, col);
    switch (eb.detail_class) {
      case 1: msg = head + fmt("invalid sentinel %lld", v); break;
      case 2: msg = head + fmt("index %lld follows trailing -1 padding", v); break;
      case 3: msg = head + fmt("index %lld is out of range for cache length %lld", v, bound); break;
      case 4: msg = head + fmt("duplicate index %lld", v); break;
      case 5: msg = head + fmt("indices are not strictly increasing: %lld then %lld", u, v); break;
      default: msg = fmt("selected_indices row [batch=%lld, head=%lld, query=%lld] is all -1", b, h, q);
    }
  }
  if (eb.word & SA_ERR_APPEND_CAPACITY) {
    if (!msg.empty()) msg += "; ";
    msg += "kv_append: a batch's past_len + cur_len does not fit its capacity";
  }
  if (eb.word & SA_ERR_QUANT_NONFINITE) {
    if (!msg.empty()) msg += "; ";
    msg += "kv_append: non-finite value in a row given to the fp8 quantizer";
  }
  if ((eb.word & SA_ERR_RANGE) && eb.detail_class == 0) {
    if (!msg.empty()) msg += "; ";
    msg += "csa_forward: a selected record index is not yet complete (>= total_len / 4)";
  }
  if (eb.word & SA_ERR_CSA_GEOMETRY) {
    if (!msg.empty()) msg += "; ";
    msg += "csa_forward: total_len does not fit the query, current_kv, record or bias sizes";
  }
  if (eb.word & SA_ERR_INDEX_NONFINITE) {
    if (!msg.empty()) msg += "; ";
    msg += "csa_index_select: a record's score is not finite";
  }
  if (eb.word & SA_ERR_CSA_DENOM) {
    if (!msg.empty()) msg += "; ";
    msg += "csa_forward: a softmax denominator is not finite and positive";
  }
  if (msg.empty()) msg = fmt("device error word 0x%llx", (long long)eb.word);
  c->last_error = msg;
  return SA_E_INDEX;
}

sa_status sparse_attn_profile_enable(sparse_attn_ctx* c, int32_t max_launches) {
  if (!live(c)) return SA_E_STATE;
  if (max_launches < 0) return set_error(c, SA_E_ARG, "profile_enable: negative max_launches");
  hipError_t e = hipStreamSynchronize(c->stream);
  if (e != hipSuccess) return check_hip(c, e, "profile_enable");
  sa::prof_release(c);
  for (int32_t i = 0; i < max_launches; i++) {
    hipEvent_t a, b;
    e = hipEventCreate(&a);
    if (e == hipSuccess) {
      e = hipEventCreate(&b);
      if (e != hipSuccess) (void)hipEventDestroy(a);
    }
    if (e != hipSuccess) {
      sa::prof_release(c);
      return check_hip(c, e, "profile_enable");
    }
    c->prof_start.push_back(a);
    c->prof_stop.push_back(b);
  }
  return SA_OK;
}

sa_status sparse_attn_profile_read(sparse_attn_ctx* c, double* total_ms, int64_t* launches) {
  if (!live(c)) return SA_E_STATE;
  hipError_t e = hipStreamSynchronize(c->stream);
  if (e != hipSuccess) return check_hip(c, e, "profile_read");
  double sum = 0.0;
  for (int64_t i = 0; i < c->prof_n; i++) {
    float ms = 0.0f;
    e = hipEventElapsedTime(&ms, c->prof_start[i], c->prof_stop[i]);
    if (e != hipSuccess) return check_hip(c, e, "profile_read");
    sum += ms;
  }
  if (total_ms) *total_ms = sum;
  if (launches) *launches = c->prof_n;
  c->prof_n = 0;
  return SA_OK;
}

const char* sparse_attn_last_error(const sparse_attn_ctx* c) {
  if (!c) return g_static_error.c_str();
  if (!live(c)) return "invalid or destroyed sparse_attn context";
  return c->last_error.c_str();
}

sa_status sparse_attn_forward_latent_static(const void* q, int64_t batch, int64_t q_seq, const void* cache,
                                            int64_t cache_capacity, const int32_t* valid_len,
                                            const void* indices, int32_t index_dtype, int64_t width,
                                            float scale, float softcap, void* y, void* hip_stream) {
  g_static_error.clear();
  auto fail = [](sa_status st, const std::string& m) {
    g_static_error = "forward_latent_static: " + m;
    return st;
  };
  if (!q || !cache || !indices || !y) return fail(SA_E_ARG, "q, cache, indices and y are required");
  if (batch <= 0 || q_seq <= 0 || width <= 0 || cache_capacity <= 0)
    return fail(SA_E_ARG, "batch, q_seq, width and cache_capacity must be positive");
  if (index_dtype != SA_IDX_I32 && index_dtype != SA_IDX_I64) return fail(SA_E_DTYPE, "index_dtype must be SA_IDX_I32 or SA_IDX_I64");
  if (!isfinite(scale) || scale < 0.0f || !isfinite(softcap) || softcap < 0.0f)
    return fail(SA_E_ARG, "scale and softcap must be finite and >= 0");
  if (width > 0x7fffffffLL) return fail(SA_E_UNSUPPORTED, "index width above 2^31 - 1");
  // a context on the stack: the same configuration checks and kernels as
  // sparse_attn_forward on a shared-latent bf16 context, with no device memory
  // of its own
  sparse_attn_ctx sh;
  sh.magic = sa::kMagic;
  sa_config& k = sh.cfg;
  k = sa_config{};
  k.num_heads = 64;
  k.kv_num_heads = 1;
  k.head_dim_qk = 576;
  k.head_dim_v = 512;
  k.rope_dim = 64;
  k.dtype = SA_BF16;
  k.cache_format = SA_CACHE_DENSE;
  k.kv_layout = SA_KV_SHARED_LATENT;
  k.index_dtype = index_dtype;
  k.scale = scale == 0.0f ? 1.0f / sqrtf(576.0f) : scale;
  k.softcap = softcap;
  k.max_batch = batch;
  k.max_q_seq = q_seq;
  k.max_index_width = width;
  k.max_cache_len = cache_capacity;
  if (sa::forward_path(k, 1) != 2)
    return fail(SA_E_UNSUPPORTED, fmt("cache capacity %lld is beyond the shared-latent kernels' reach", cache_capacity));
  sh.stream = (hipStream_t)hip_stream;
  sh.err = nullptr;  // the unvalidated kernels never touch the error block
  sh.gpart_o = sh.gpart_ml = nullptr;
  sh.gpart_rows = 0;
  sh.zeros = nullptr;
  sh.row_key = nullptr;
  sh.row_done = nullptr;
  sh.prof_n = 0;
  const int64_t rows = batch * q_seq;
  sh.rows_cap = rows;
  const int splits = sa::mla_splits(rows, width);
  sh.partial_o = sh.partial_ml = nullptr;
  sh.partial_rows = 0;
  if (splits > 1) {
    const int64_t parts = rows * splits;
    const int64_t o_bytes = (parts * 64 * 512 * 4 + 255) / 256 * 256;
    const int64_t need = o_bytes + parts * 64 * 2 * 4;
    if (need > (int64_t)SA_STATIC_SCRATCH_BYTES)
      return fail(SA_E_CAPACITY, fmt("%lld rows in %lld splits need %lld bytes of split-K partials; the static scratch holds %lld",
                                     rows, splits, need, (long long)SA_STATIC_SCRATCH_BYTES));
    hipError_t e = hipGetDevice(&sh.device);
    if (e != hipSuccess) return fail(SA_E_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
    if (sh.device < 0 || sh.device >= kMaxDevices) return fail(SA_E_UNSUPPORTED, fmt("device %lld beyond the first 64", sh.device));
    void* base = nullptr;
    e = scratch_address(sh.device, &base);
    if (e != hipSuccess) return fail(SA_E_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    sh.partial_o = (float*)base;
    sh.partial_ml = (float*)((uint8_t*)base + o_bytes);
    sh.partial_rows = parts;
  }
  sa::FwdArgs a;
  a.q = q;
  a.k = cache;
  a.v = nullptr;
  a.idx = indices;
  a.valid_len = valid_len;
  a.y = y;
  a.batch = batch;
  a.hq = k.num_heads;
  a.hkv = k.kv_num_heads;
  a.q_seq = q_seq;
  a.dk = k.head_dim_qk;
  a.dv = k.head_dim_v;
  a.rope = k.rope_dim;
  a.cap = cache_capacity;
  a.index_heads = 1;
  a.width = width;
  a.scale = k.scale;
  a.softcap = k.softcap;
  a.dtype = k.dtype;
  a.cache_format = k.cache_format;
  a.kv_layout = k.kv_layout;
  a.idx64 = index_dtype == SA_IDX_I64;
  const sa_status st = sa::latent_decode_fits(q_seq) ? sa::launch_forward_latent_decode(&sh, a, splits, false, nullptr)
                                                     : sa::launch_forward_latent(&sh, a, splits, false, nullptr);
  if (st != SA_OK) g_static_error = "forward_latent_static: " + sh.last_error;
  return st;
}

}  // extern "C"
