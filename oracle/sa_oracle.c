/*
 * Selected-token sparse attention with KV append: the CPU ORACLE.
 *
 * This file is test infrastructure. It is the plain, slow, obviously-correct
 * statement of what the hot path computes, and only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg may load it. The product library
 * never links, calls or includes anything from here, and nothing here includes
 * the product's headers: the constants, codecs and rules below are written
 * out independently.
 *
 * Sources (docs.rs source pages):
 *   [IS]  onnx-runtime-ep-cuda, src/kernels/index_share.rs (IndexShare):
 *         module doc "Determinism / bit-parity", kernels `build_present`,
 *         `build_present_capacity`, `validate_index_rows`, `index_share_row`,
 *         host `validate_indices` / `index_error`, `launch_rows` (default scale),
 *         `bias_at` and `capacity_write_pos` (the optional additive bias and
 *         the capacity-mode length it carries).
 *   [CPU] onnx-runtime-ep-cpu, src/kernels/compressed_sparse_attention.rs
 *         (CSA CPU oracle): `CacheFormat` (record layout, `stored_width`),
 *         `dequantize_cache`, `finalize_attention_record` (pack loop),
 *         `dot` / `accumulate_value` (strict ascending fp32 folds).
 *   [CSA] onnx-runtime-ep-cuda, src/kernels/compressed_sparse_attention.rs:
 *         the sink-attention kernels' in-line record decode (E8M0 scale times
 *         E4M3FN code; BF16 tail read as bits << 16), exp via double.
 *   [ATT] onnx-runtime-ep-cuda, src/kernels/standard_attention.rs: module doc
 *         "Semantics" (softcap after the scaled scores, before the softmax).
 *
 * Arithmetic rules: every float operation is a single fp32 operation, in the
 * order written, with no FMA contraction and no reassociation (build with
 * -O2 -ffp-contract=off -fno-fast-math). exp and tanh are evaluated in double
 * and rounded to fp32 once, as the CSA kernels do for exp.
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *  - K and V may be one shared-latent cache (V = first Dv dims of the K row).
 *  - The E8M0 scale of the fp8 quantizer is floor(log2(amax)) - 8 + 127
 *    (OCP MX rule); E4M3FN codes round to nearest even and saturate to 448.
 *  - A row whose scores are all -inf yields zeros ([IS] `index_share_row`).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

/* ---- storage codes (oracle-local numbering) ----------------------------- */
enum { OR_F32 = 0, OR_F16 = 1, OR_BF16 = 2, OR_FP8_BLOCK64 = 3 };
enum { OR_LAYOUT_SEPARATE = 0, OR_LAYOUT_SHARED_LATENT = 1 };

/* validation classes, in the pages' check order ([IS] `validate_indices`) */
enum {
  OR_OK = 0,
  OR_SENTINEL = 1,   /* index < -1                                   */
  OR_AFTER_PAD = 2,  /* a non-(-1) index after trailing -1 padding    */
  OR_RANGE = 3,      /* index >= cache length of the batch            */
  OR_DUPLICATE = 4,  /* index == previous valid index                 */
  OR_ORDER = 5,      /* index <  previous valid index                 */
  OR_ALL_PAD = 6     /* no valid index in the row                     */
};

/* ---- bf16 / f16 widening and bf16 narrowing ----------------------------- */

/* bf16 -> fp32 is exact: the bf16 bits are the high half of the fp32 bits. */
static float or_bf16_to_f32(uint16_t bits) {
  uint32_t w = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &w, 4);
  return f;
}

/* IEEE binary16 -> fp32, exact, written from the format definition. */
static float or_f16_to_f32(uint16_t h) {
  int sign = (h >> 15) & 1;
  int exp = (h >> 10) & 0x1f;
  int man = h & 0x3ff;
  double v;
  if (exp == 0) {
    v = ldexp((double)man, -24); /* subnormal: man * 2^-24 */
  } else if (exp == 31) {
    v = man ? NAN : INFINITY;
  } else {
    v = ldexp((double)(man + 1024), exp - 25); /* (1 + man/1024) * 2^(exp-15) */
  }
  return (float)(sign ? -v : v);
}

/* The same widening, exported so that tests can check it over every bit pattern. */
float oracle_f16_to_f32(uint16_t h) { return or_f16_to_f32(h); }

/* fp32 -> bf16 round to nearest, ties to even; NaN stays a quiet NaN. */
uint16_t oracle_bf16_from_f32(float x) {
  uint32_t w;
  memcpy(&w, &x, 4);
  if ((w & 0x7f800000u) == 0x7f800000u && (w & 0x007fffffu)) {
    return (uint16_t)((w >> 16) | 0x0040u);
  }
  uint32_t upper = w >> 16;
  uint32_t lower = w & 0xffffu;
  if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u))) upper += 1u;
  return (uint16_t)upper;
}

static float or_load(const void* base, int64_t i, int dtype) {
  switch (dtype) {
    case OR_F32: return ((const float*)base)[i];
    case OR_F16: return or_f16_to_f32(((const uint16_t*)base)[i]);
    default: return or_bf16_to_f32(((const uint16_t*)base)[i]);
  }
}

/* ---- fp8_e4m3_block64 record codec ([CPU] `CacheFormat`) ----------------- */

/* E8M0 scale byte: 2^(e-127); 255 is NaN. */
double oracle_e8m0_value(uint8_t e) { return e == 255 ? NAN : ldexp(1.0, (int)e - 127); }

/* E4M3FN code: 1 sign, 4 exponent bits (bias 7), 3 mantissa bits; no
 * infinities; S.1111.111 is NaN; exponent 0 encodes subnormals M * 2^-9. */
double oracle_e4m3fn_value(uint8_t code) {
  int s = code >> 7, E = (code >> 3) & 0xf, M = code & 7;
  double v;
  if (E == 15 && M == 7) return NAN;
  if (E == 0) v = ldexp((double)M, -9);
  else v = ldexp(1.0 + M / 8.0, E - 7);
  return s ? -v : v;
}

/* Round a non-negative double to the nearest integer, ties to even. */
static double or_rne(double q) {
  double f = floor(q), r = q - f;
  if (r > 0.5 || (r == 0.5 && fmod(f, 2.0) != 0.0)) f += 1.0;
  return f;
}

/* Encode one already-scaled value into E4M3FN: nearest-even, saturate at 448. */
static uint8_t or_e4m3fn_encode(double v) {
  uint8_t s = (v < 0 || (v == 0 && signbit(v))) ? 0x80 : 0x00;
  double a = fabs(v);
  uint8_t mag;
  if (a >= 448.0) {
    mag = 0x7e; /* 1.75 * 2^8, the largest finite code */
  } else if (a < ldexp(1.0, -6)) {
    /* subnormal range: spacing 2^-9; 8 * 2^-9 is the smallest normal, whose
     * code 0x08 follows code 0x07 in the bit pattern, so m == 8 needs no case */
    mag = (uint8_t)or_rne(a / ldexp(1.0, -9));
  } else {
    int e = (int)floor(log2(a));
    /* guard log2 rounding at exact powers of two */
    if (ldexp(1.0, e) > a) e -= 1;
    if (ldexp(1.0, e + 1) <= a) e += 1;
    double m = or_rne(a / ldexp(1.0, e - 3)); /* in [8, 16] */
    if (m == 16.0) { e += 1; m = 8.0; }
    int code = ((e + 7) << 3) | ((int)m - 8);
    mag = (uint8_t)(code > 0x7e ? 0x7e : code);
  }
  return (uint8_t)(s | mag);
}

/* Quantize one 64-value block: returns 0, or -1 if a value is not finite
 * (the CSA oracle rejects non-finite inputs before packing).
 * amax == 0 -> scale byte 127 and all-zero codes. Otherwise
 * e = clamp(floor(log2 amax) - 8 + 127, 0, 254) and
 * code_i = E4M3FN_RNE_sat(x_i * 2^-(e-127)); the scaling is exact in double. */
int oracle_fp8_quantize_block64(const float* x, uint8_t* scale_out, uint8_t* codes) {
  float amax = 0.0f;
  for (int i = 0; i < 64; i++) {
    if (!isfinite(x[i])) return -1;
    float a = fabsf(x[i]);
    if (a > amax) amax = a;
  }
  if (amax == 0.0f) {
    *scale_out = 127;
    memset(codes, 0, 64);
    return 0;
  }
  int k;
  frexp((double)amax, &k); /* amax = f * 2^k with f in [0.5, 1) */
  k -= 1;                  /* floor(log2(amax)) */
  int e = k - 8 + 127;
  if (e < 0) e = 0;
  if (e > 254) e = 254;
  *scale_out = (uint8_t)e;
  for (int i = 0; i < 64; i++) codes[i] = or_e4m3fn_encode(ldexp((double)x[i], 127 - e));
  return 0;
}

/* Width in bytes of one record holding `dk` logical dims whose last `rope`
 * dims are a BF16 tail: (dk - rope)/64 blocks of 65 bytes + 2 * rope. */
int64_t oracle_fp8_record_bytes(int64_t dk, int64_t rope) {
  if (rope < 0 || rope > dk || (dk - rope) % 64 != 0) return -1;
  return (dk - rope) / 64 * 65 + 2 * rope;
}

/* Pack one logical row (fp32 values; the tail values must already be bf16
 * representable or they are rounded RNE) into a record. Returns 0 or -1. */
int oracle_fp8_pack_record(const float* row, int64_t dk, int64_t rope, uint8_t* rec) {
  int64_t blocks = (dk - rope) / 64;
  for (int64_t j = 0; j < blocks; j++) {
    if (oracle_fp8_quantize_block64(row + 64 * j, rec + 65 * j, rec + 65 * j + 1) != 0) return -1;
  }
  uint8_t* tail = rec + 65 * blocks;
  for (int64_t i = 0; i < rope; i++) {
    float v = row[dk - rope + i];
    if (!isfinite(v)) return -1;
    uint16_t b = oracle_bf16_from_f32(v);
    tail[2 * i] = (uint8_t)(b & 0xff); /* little-endian */
    tail[2 * i + 1] = (uint8_t)(b >> 8);
  }
  return 0;
}

/* Decode one record to `dk` fp32 values ([CPU] `dequantize_cache`).
 * Returns 0, or -1 if a scale byte or a code is NaN. */
int oracle_fp8_decode_record(const uint8_t* rec, int64_t dk, int64_t rope, float* out) {
  int64_t blocks = (dk - rope) / 64;
  for (int64_t j = 0; j < blocks; j++) {
    double s = oracle_e8m0_value(rec[65 * j]);
    if (isnan(s)) return -1;
    for (int i = 0; i < 64; i++) {
      double c = oracle_e4m3fn_value(rec[65 * j + 1 + i]);
      if (isnan(c)) return -1;
      out[64 * j + i] = (float)(c * s);
    }
  }
  const uint8_t* tail = rec + 65 * blocks;
  for (int64_t i = 0; i < rope; i++) {
    uint16_t b = (uint16_t)(tail[2 * i] | (tail[2 * i + 1] << 8));
    out[dk - rope + i] = or_bf16_to_f32(b);
  }
  return 0;
}

/* ---- A1: KV append ([IS] `build_present` / `build_present_capacity`) ---- */

/* present[b,h,t,:] = past[b,h,t,:] for t < past_len[b];
 *                  = cur[b,h,t-past_len[b],:] for past_len[b] <= t < past_len[b]+cur_len.
 * Rows are `row_bytes` wide and copied as bytes (the concat is a pure copy).
 * When present == past (in-place, capacity layout) only the new rows are
 * written. Rows of present at or beyond past_len[b]+cur_len are untouched.
 * Returns 0, or -1 if a length does not fit its capacity. */
int oracle_kv_append(const uint8_t* past, int64_t past_cap, const int64_t* past_len,
                     const uint8_t* cur, int64_t cur_len, uint8_t* present,
                     int64_t present_cap, int64_t batch, int64_t heads, int64_t row_bytes) {
  for (int64_t b = 0; b < batch; b++) {
    if (past_len[b] < 0 || past_len[b] > past_cap || past_len[b] + cur_len > present_cap) return -1;
  }
  for (int64_t b = 0; b < batch; b++) {
    for (int64_t h = 0; h < heads; h++) {
      uint8_t* dst = present + (b * heads + h) * present_cap * row_bytes;
      if (present != past) {
        const uint8_t* src = past + (b * heads + h) * past_cap * row_bytes;
        for (int64_t t = 0; t < past_len[b]; t++)
          memcpy(dst + t * row_bytes, src + t * row_bytes, (size_t)row_bytes);
      }
      const uint8_t* c = cur + (b * heads + h) * cur_len * row_bytes;
      for (int64_t t = 0; t < cur_len; t++)
        memcpy(dst + (past_len[b] + t) * row_bytes, c + t * row_bytes, (size_t)row_bytes);
    }
  }
  return 0;
}

/* ---- A3: index validation ([IS] host `validate_indices`) ---------------- */

static int64_t or_load_index(const void* idx, int64_t i, int is_i64) {
  return is_i64 ? ((const int64_t*)idx)[i] : (int64_t)((const int32_t*)idx)[i];
}

/* Scan one row's columns in ascending order, exactly as the host validator
 * does, and return its class (OR_OK if valid). *bad_col receives the column
 * of the first violation, or `width` for an all-padding row. */
static int or_validate_row(const void* idx, int is_i64, int64_t base, int64_t width,
                           int64_t bound, int64_t* bad_col) {
  int padding = 0;
  int64_t count = 0, previous = 0;
  for (int64_t col = 0; col < width; col++) {
    int64_t v = or_load_index(idx, base + col, is_i64);
    if (v == -1) { padding = 1; continue; }
    int cls = OR_OK;
    if (v < -1) cls = OR_SENTINEL;
    else if (padding) cls = OR_AFTER_PAD;
    else if (v >= bound) cls = OR_RANGE;
    else if (count > 0 && v == previous) cls = OR_DUPLICATE;
    else if (count > 0 && v < previous) cls = OR_ORDER;
    if (cls != OR_OK) { *bad_col = col; return cls; }
    previous = v;
    count += 1;
  }
  if (count == 0) { *bad_col = width; return OR_ALL_PAD; }
  *bad_col = -1;
  return OR_OK;
}

/* Validate all rows in (batch, index_head, query) order. row_class[r] gets
 * each row's class. Returns the OR of (1 << (class-1)) over invalid rows,
 * plus 512 if any row is invalid (the IndexShare capture-error bit); the
 * first failing row/column/class and the pages' message are reported. */
uint32_t oracle_validate_indices(const void* idx, int is_i64, int64_t batch, int64_t index_heads,
                                 int64_t q_seq, int64_t width, const int64_t* bound,
                                 uint8_t* row_class, int64_t* first_row, int64_t* first_col,
                                 int* first_class, char* msg, int64_t msg_len) {
  uint32_t word = 0;
  *first_row = -1;
  *first_col = -1;
  *first_class = OR_OK;
  if (msg && msg_len > 0) msg[0] = 0;
  for (int64_t b = 0; b < batch; b++) {
    for (int64_t h = 0; h < index_heads; h++) {
      for (int64_t q = 0; q < q_seq; q++) {
        int64_t row = (b * index_heads + h) * q_seq + q;
        int64_t col;
        int cls = or_validate_row(idx, is_i64, row * width, width, bound[b], &col);
        row_class[row] = (uint8_t)cls;
        if (cls == OR_OK) continue;
        word |= (1u << (cls - 1)) | 512u;
        if (*first_row >= 0) continue;
        *first_row = row;
        *first_col = col;
        *first_class = cls;
        if (!msg || msg_len <= 0) continue;
        int64_t v = cls == OR_ALL_PAD ? -1 : or_load_index(idx, row * width + col, is_i64);
        int64_t prev = col > 0 ? or_load_index(idx, row * width + col - 1, is_i64) : 0;
        char head[160];
        snprintf(head, sizeof head, "selected_indices [batch=%lld, head=%lld, query=%lld, column=%lld]: ",
                 (long long)b, (long long)h, (long long)q, (long long)col);
        switch (cls) {
          case OR_SENTINEL:
            snprintf(msg, (size_t)msg_len, "%sinvalid sentinel %lld", head, (long long)v);
            break;
          case OR_AFTER_PAD:
            snprintf(msg, (size_t)msg_len, "%sindex %lld follows trailing -1 padding", head, (long long)v);
            break;
          case OR_RANGE:
            snprintf(msg, (size_t)msg_len, "%sindex %lld is out of range for cache length %lld", head,
                     (long long)v, (long long)bound[b]);
            break;
          case OR_DUPLICATE:
            snprintf(msg, (size_t)msg_len, "%sduplicate index %lld", head, (long long)v);
            break;
          case OR_ORDER:
            snprintf(msg, (size_t)msg_len, "%sindices are not strictly increasing: %lld then %lld", head,
                     (long long)prev, (long long)v);
            break;
          default:
            snprintf(msg, (size_t)msg_len, "selected_indices row [batch=%lld, head=%lld, query=%lld] is all -1",
                     (long long)b, (long long)h, (long long)q);
        }
      }
    }
  }
  return word;
}

/* ---- A4-A8, A10: the forward ([IS] `index_share_row`) ------------------- */

/* The additive bias at logical (b, h, q, k) ([IS] `bias_at`; the CPU page's
 * `AttentionBias::at`): dims[4] is the bias shape right-aligned against
 * [B, Hq, Sq, keys] and padded with 1; an extent of 1 broadcasts (index 0),
 * any other extent takes the coordinate; the offset is row-major. */
static float or_bias_at(const void* bias, int dtype, const int64_t* dims, int64_t b, int64_t h,
                        int64_t q, int64_t k) {
  const int64_t coord[4] = {b, h, q, k};
  int64_t off = 0;
  for (int a = 0; a < 4; a++) off = off * dims[a] + (dims[a] == 1 ? 0 : coord[a]);
  return or_load(bias, off, dtype);
}

/* Capacity-mode length recovery ([IS] `capacity_write_pos`): when the present
 * cache aliases a fixed-capacity past, its shape no longer says how many rows
 * are live, and the bias frontier does. For each batch b:
 *   valid[b]     = 1 + the largest k < keys with bias(b, h, q, k) finite for
 *                  some (h, q); 0 when there is none
 *   write_pos[b] = valid[b] - cur_len, or 0 when valid[b] < cur_len
 * (the row where this step's cur_len rows go). */
void oracle_capacity_lengths(const void* bias, int dtype, const int64_t* dims, int64_t batch,
                             int64_t hq, int64_t sq, int64_t keys, int64_t cur_len, int64_t* valid,
                             int64_t* write_pos) {
  for (int64_t b = 0; b < batch; b++) {
    int64_t v = 0;
    for (int64_t h = 0; h < hq; h++)
      for (int64_t q = 0; q < sq; q++)
        for (int64_t k = 0; k < keys; k++)
          if (isfinite(or_bias_at(bias, dtype, dims, b, h, q, k)) && k + 1 > v) v = k + 1;
    valid[b] = v;
    write_pos[b] = v >= cur_len ? v - cur_len : 0;
  }
}

/* Load logical dim d of cache row (b, h, t) as fp32. For fp8 records the
 * whole row is decoded into `scratch` once per (row, key) by the caller. */
static const float* or_cache_row(const void* cache, int fmt, int64_t row_index, int64_t row_elems,
                                 int64_t dk, int64_t rope, int64_t record_bytes, float* scratch) {
  if (fmt == OR_FP8_BLOCK64) {
    if (oracle_fp8_decode_record((const uint8_t*)cache + row_index * record_bytes, dk, rope, scratch) != 0)
      return NULL;
    return scratch;
  }
  for (int64_t d = 0; d < row_elems; d++) scratch[d] = or_load(cache, row_index * row_elems + d, fmt);
  return scratch;
}

/*
 * Output rows [row_begin, row_end) of the flattened (b, h, q) order.
 *   q      [B, Hq, Sq, Dk]   in q_dtype (0 f32, 1 f16, 2 bf16)
 *   kcache [B, Hkv, cap, Dk] in cache_fmt (0/1/2, or 3 = fp8 records)
 *   vcache [B, Hkv, cap, Dv] (SEPARATE) or NULL (SHARED_LATENT: V = K[..., :Dv])
 *   idx    [B, Hi, Sq, W]    i32 or i64, rows already valid
 *   y      [B, Hq, Sq, Dv]   fp32 (the caller rounds to its storage dtype)
 *   bias   NULL, or the additive attention bias in bias_dtype (0/1/2) whose
 *          shape, right-aligned against [B, Hq, Sq, cap] and padded with 1 on
 *          the left, is bias_dims[4]; each extent is 1 (broadcast) or the
 *          target's
 * scale == 0 means 1/sqrtf(Dk); softcap == 0 means off.
 * work: 2*Dk + W floats of scratch.
 * Returns 0, or -1 on a record that decodes to NaN or an index out of range.
 */
int oracle_forward_rows(const void* q, int q_dtype, const void* kcache, const void* vcache,
                        int cache_fmt, int kv_layout, int64_t cap, const void* idx, int idx_is_i64,
                        int64_t batch, int64_t hq, int64_t hkv, int64_t sq, int64_t index_heads,
                        int64_t width, int64_t dk, int64_t dv, int64_t rope, float scale,
                        float softcap, const void* bias, int bias_dtype, const int64_t* bias_dims,
                        int64_t row_begin, int64_t row_end, float* y, float* work) {
  (void)batch;
  const int64_t group = hq / hkv;
  const int64_t record_bytes = cache_fmt == OR_FP8_BLOCK64 ? oracle_fp8_record_bytes(dk, rope) : 0;
  if (scale == 0.0f) scale = 1.0f / sqrtf((float)dk); /* [IS] `launch_rows` default */
  const float ss = sqrtf(scale);
  float* krow = work;
  float* vrow = work + dk;
  float* p = work + 2 * dk;
  for (int64_t row = row_begin; row < row_end; row++) {
    const int64_t qi = row % sq;
    const int64_t h = (row / sq) % hq;
    const int64_t b = row / (sq * hq);
    const int64_t kvh = h / group;
    const int64_t ih = index_heads == 1 ? 0 : h;
    const int64_t ibase = ((b * index_heads + ih) * sq + qi) * width;
    const int64_t qbase = row * dk;
    float* yrow = y + row * dv;
    /* A4: n = entries before the first -1 */
    int64_t n = 0;
    while (n < width && or_load_index(idx, ibase + n, idx_is_i64) != -1) n++;
    /* A5 + A6: gather each selected key, scaled dot product, then softcap */
    for (int64_t s = 0; s < n; s++) {
      int64_t key = or_load_index(idx, ibase + s, idx_is_i64);
      if (key < 0 || key >= cap) return -1;
      int64_t kr = (b * hkv + kvh) * cap + key;
      if (!or_cache_row(kcache, cache_fmt, kr, dk, dk, rope, record_bytes, krow)) return -1;
      float acc = 0.0f;
      for (int64_t d = 0; d < dk; d++) {
        float qd = or_load(q, qbase + d, q_dtype) * ss;
        float kd = krow[d] * ss;
        float prod = qd * kd;
        acc = acc + prod;
      }
      if (softcap != 0.0f) acc = softcap * (float)tanh((double)(acc / softcap));
      /* [IS] `index_share_row`: the bias of (b, h, q, key) is added to the
       * scaled score; with a softcap it comes after it, as the standard
       * Attention page applies the softcap before its masks */
      if (bias) acc = acc + or_bias_at(bias, bias_dtype, bias_dims, b, h, qi, key);
      p[s] = acc;
    }
    /* A7: max, exp, ascending sum, multiply by the reciprocal */
    float m = -INFINITY;
    for (int64_t s = 0; s < n; s++) m = fmaxf(m, p[s]);
    if (m == -INFINITY) {
      for (int64_t d = 0; d < dv; d++) yrow[d] = 0.0f;
      continue;
    }
    float l = 0.0f;
    for (int64_t s = 0; s < n; s++) {
      float e = (float)exp((double)(p[s] - m));
      p[s] = e;
      l = l + e;
    }
    const float inv = 1.0f / l;
    for (int64_t s = 0; s < n; s++) p[s] = p[s] * inv;
    /* A8: y_d = sum_s p_s * v_{key_s, d}, ascending over s */
    for (int64_t d = 0; d < dv; d++) yrow[d] = 0.0f;
    for (int64_t s = 0; s < n; s++) {
      int64_t key = or_load_index(idx, ibase + s, idx_is_i64);
      int64_t kr = (b * hkv + kvh) * cap + key;
      const float* v;
      if (kv_layout == OR_LAYOUT_SHARED_LATENT) {
        v = or_cache_row(kcache, cache_fmt, kr, dk, dk, rope, record_bytes, vrow);
      } else {
        v = or_cache_row(vcache, cache_fmt, kr, dv, dv, rope, record_bytes, vrow);
      }
      if (!v) return -1;
      for (int64_t d = 0; d < dv; d++) {
        float prod = p[s] * v[d];
        yrow[d] = yrow[d] + prod;
      }
    }
  }
  return 0;
}

/* ---- CSA ratio-4 selected sink attention ---------------------------------
 * [CPU] `ratio4_attention` (and the driver that derives its cursors from
 * total_sequence_length), [CSA] `csa_ratio4_sink_attention`, the head sink of
 * [CPU] `CompressedSparseAttentionKernel::execute`, and [CPU] `AttentionBias`.
 *
 *   q        [B, S, H, 512] fp32
 *   ckv      [B, Tcur, 512] fp32: the dense rows at absolute positions
 *            total - Tcur .. total - 1
 *   records  [B, Rcap, 583] fp8_e4m3_block64 records (448 coded dims + 64
 *            BF16 tail dims); the first total/4 of each batch are complete
 *   selected [B, Hidx, S, K] int32; every index-head row holds the same
 *            selection, index head 0 is read
 *   sink     [H] fp32, bias NULL or fp32 of the right-aligned shape
 *            bias_dims[4] (each 1 or the full extent of [B, H, S, Cand])
 *   y        [B, S, H, 512] fp32
 * For query s at position p = total - S + s the candidates are the dense
 * positions max(total - Tcur, p + 1 - 128) .. p (Cd of them counted from the
 * window start, Cd = min(Tcur, 128) when total == S, else 128), then the K
 * selected records; Cand = Cd + K. Scores are the ascending fp32 dot times
 * scale (0 -> 1/sqrtf(512)) plus the bias; a negative index is skipped; the
 * softmax denominator adds exp(sink[h] - max) after the candidates' max; a
 * row with no candidate gives zeros.
 *
 * Readings (the pages' CPU path raises an error where their device kernel
 * skips; these are the readings taken here):
 *  - a selected record >= total/4 is skipped and flagged OR_CSA_RANGE;
 *  - a denominator that is not a finite positive fp32 flags OR_CSA_DENOM
 *    (that row's outputs are then meaningless);
 *  - total < S, total < Tcur, total - Tcur > max(0, total - S + 1 - 128),
 *    total/4 > Rcap or a bias extent that does not fit flags
 *    OR_CSA_GEOMETRY and nothing is computed.
 * Returns the flags; -1 cast to uint32 on an allocation failure.
 */
#define OR_CSA_DIM 512
#define OR_CSA_ROPE 64
#define OR_CSA_WINDOW 128
#define OR_CSA_RANGE 1u
#define OR_CSA_DENOM 2u
#define OR_CSA_GEOMETRY 4u

uint32_t oracle_csa_sink_attention(const float* q, int64_t batch, int64_t seq, int64_t heads,
                                   const float* ckv, int64_t cur_len, const uint8_t* records,
                                   int64_t record_cap, const int32_t* selected, int64_t index_heads,
                                   int64_t topk, const float* sink, const float* bias,
                                   const int64_t* bias_dims, int64_t total, float scale, float* y) {
  const int64_t D = OR_CSA_DIM;
  const int64_t rec_bytes = oracle_fp8_record_bytes(D, OR_CSA_ROPE); /* 583 */
  if (total < seq || total < cur_len) return OR_CSA_GEOMETRY;
  const int64_t start = total - seq;           /* position of query 0 */
  const int64_t base = total - cur_len;        /* position of ckv row 0 */
  const int64_t earliest = start + 1 - OR_CSA_WINDOW > 0 ? start + 1 - OR_CSA_WINDOW : 0;
  if (base > earliest) return OR_CSA_GEOMETRY;
  const int64_t valid_records = total / 4;
  if (valid_records > record_cap) return OR_CSA_GEOMETRY;
  const int64_t dense = start == 0 ? (cur_len < OR_CSA_WINDOW ? cur_len : OR_CSA_WINDOW) : OR_CSA_WINDOW;
  const int64_t cand = dense + topk;
  const int64_t target[4] = {batch, heads, seq, cand};
  if (bias) {
    for (int a = 0; a < 4; a++)
      if (bias_dims[a] != 1 && bias_dims[a] != target[a]) return OR_CSA_GEOMETRY;
  }
  if (scale == 0.0f) scale = 1.0f / sqrtf((float)D);

  float* score = (float*)malloc(sizeof(float) * (size_t)cand);
  float* row = (float*)malloc(sizeof(float) * (size_t)D);
  if (!score || !row) {
    free(score);
    free(row);
    return (uint32_t)-1;
  }
  uint32_t flags = 0;
  for (int64_t b = 0; b < batch; b++) {
    for (int64_t s = 0; s < seq; s++) {
      const int64_t pos = start + s;
      const int64_t wstart = pos + 1 - OR_CSA_WINDOW > base ? pos + 1 - OR_CSA_WINDOW : base;
      const int32_t* sel = selected + ((b * index_heads + 0) * seq + s) * topk;
      for (int64_t h = 0; h < heads; h++) {
        const float* qrow = q + ((b * seq + s) * heads + h) * D;
        float* yrow = y + ((b * seq + s) * heads + h) * D;
        float m = -INFINITY;
        for (int64_t c = 0; c < cand; c++) score[c] = -INFINITY;
        /* the dense window */
        for (int64_t c = 0; c < dense; c++) {
          const int64_t p = wstart + c;
          if (p > pos) continue;
          const float* kv = ckv + (b * cur_len + (p - base)) * D;
          float acc = 0.0f;
          for (int64_t d = 0; d < D; d++) {
            float prod = qrow[d] * kv[d];
            acc = acc + prod;
          }
          score[c] = acc * scale;
        }
        /* the selected records */
        for (int64_t j = 0; j < topk; j++) {
          const int64_t r = sel[j];
          if (r < 0) continue;
          if (r >= valid_records) {
            flags |= OR_CSA_RANGE;
            continue;
          }
          if (oracle_fp8_decode_record(records + (b * record_cap + r) * rec_bytes, D, OR_CSA_ROPE, row) != 0) {
            /* a NaN scale byte or code: the score is NaN, as the device decode gives */
            score[dense + j] = NAN;
            continue;
          }
          float acc = 0.0f;
          for (int64_t d = 0; d < D; d++) {
            float prod = qrow[d] * row[d];
            acc = acc + prod;
          }
          score[dense + j] = acc * scale;
        }
        /* additive bias, broadcast over extents of 1 ([CPU] `AttentionBias::at`) */
        if (bias) {
          for (int64_t c = 0; c < cand; c++) {
            if (score[c] == -INFINITY) continue;
            const int64_t at[4] = {b, h, s, c};
            int64_t off = 0;
            for (int a = 0; a < 4; a++) off = off * bias_dims[a] + (bias_dims[a] == 1 ? 0 : at[a]);
            score[c] = score[c] + bias[off];
          }
        }
        for (int64_t c = 0; c < cand; c++) m = fmaxf(m, score[c]); /* NaN is passed over */
        for (int64_t d = 0; d < D; d++) yrow[d] = 0.0f;
        if (m == -INFINITY) continue;
        float den = 0.0f;
        for (int64_t c = 0; c < cand; c++) {
          if (score[c] == -INFINITY) continue;
          den = den + (float)exp((double)(score[c] - m));
        }
        den = den + (float)exp((double)(sink[h] - m));
        if (!(den > 0.0f) || isinf(den)) {
          flags |= OR_CSA_DENOM;
          continue;
        }
        for (int64_t c = 0; c < cand; c++) {
          if (score[c] == -INFINITY) continue;
          const float p = (float)exp((double)(score[c] - m)) / den;
          const float* v;
          if (c < dense) {
            v = ckv + (b * cur_len + (wstart + c - base)) * D;
          } else {
            const int64_t r = sel[c - dense];
            if (oracle_fp8_decode_record(records + (b * record_cap + r) * rec_bytes, D, OR_CSA_ROPE, row) != 0)
              for (int64_t d = 0; d < D; d++) row[d] = NAN;
            v = row;
          }
          for (int64_t d = 0; d < D; d++) {
            float prod = p * v[d];
            yrow[d] = yrow[d] + prod;
          }
        }
      }
    }
  }
  free(score);
  free(row);
  return flags;
}

/* ---- CSA ratio-4 selection producer (the indexer) -------------------------
 * [CPU] `select_ratio4_topk`, `finalize_index_query`, `apply_compressed_rope`,
 * `hadamard_bf16`, `fp4_roundtrip`; [CSA] `csa_ratio4_index_select` (record
 * layout of the FP4 index keys, the (-score, +record) order, -1 padding).
 *
 * FP4 E2M1 block-32: per 32 values an E8M0 scale byte and 16 bytes of codes,
 * element 2i in the low nibble, 2i+1 in the high one. An E2M1 code is 1 sign,
 * 2 exponent bits (bias 1) and 1 mantissa bit: 0, 0.5, 1, 1.5, 2, 3, 4, 6.
 * The quantizer's source is not on the pages; the reading taken (the OCP MX
 * rule, as for the fp8 blocks): scale byte = floor(log2(amax)) - 2 + 127
 * (127 for an all-zero block), codes = nearest E2M1 value of x / 2^(e - 127),
 * ties to the even code, saturating at 6, sign kept. */

double oracle_e2m1_value(uint8_t code) {
  static const double mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
  const double v = mag[code & 7];
  return (code & 8) ? -v : v;
}

/* nearest E2M1 magnitude code of a non-negative double, ties to even code */
static uint8_t or_e2m1_encode_mag(double v) {
  static const double mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
  if (v >= 6.0) return 7;
  for (int c = 0; c < 7; c++) {
    const double lo = mag[c], hi = mag[c + 1];
    if (v <= hi) {
      const double dl = v - lo, dh = hi - v;
      if (dl < dh) return (uint8_t)c;
      if (dh < dl) return (uint8_t)(c + 1);
      return (uint8_t)((c & 1) ? c + 1 : c); /* tie: the even code */
    }
  }
  return 7;
}

/* Quantize 32 values: returns 0, or -1 for a non-finite value. out[] gets the
 * dequantized values (code times scale). */
int oracle_fp4_quantize_block32(const float* x, uint8_t* scale_out, uint8_t* packed, float* out) {
  double amax = 0.0;
  for (int i = 0; i < 32; i++) {
    if (!isfinite(x[i])) return -1;
    const double a = fabs((double)x[i]);
    if (a > amax) amax = a;
  }
  int e = 127;
  if (amax > 0.0) {
    int ex;
    frexp(amax, &ex); /* amax = f * 2^ex, f in [0.5, 1): floor(log2 amax) = ex - 1 */
    e = (ex - 1) - 2 + 127;
    if (e < 0) e = 0;
    if (e > 254) e = 254;
  }
  const double s = ldexp(1.0, e - 127);
  for (int i = 0; i < 16; i++) packed[i] = 0;
  for (int i = 0; i < 32; i++) {
    const double v = (double)x[i] / s;
    uint8_t c = or_e2m1_encode_mag(fabs(v));
    if (signbit(v)) c |= 8;
    packed[i / 2] |= (uint8_t)(c << (4 * (i & 1)));
    out[i] = (float)(oracle_e2m1_value(c) * s);
  }
  *scale_out = (uint8_t)e;
  return 0;
}

/* Decode one FP4 index key of `dim` values (dim/32 blocks of 17 bytes). */
void oracle_fp4_decode_key(const uint8_t* key, int64_t dim, float* out) {
  for (int64_t b = 0; b < dim / 32; b++) {
    const double s = oracle_e8m0_value(key[17 * b]);
    for (int i = 0; i < 32; i++) {
      const uint8_t byte = key[17 * b + 1 + i / 2];
      const uint8_t c = (uint8_t)((byte >> (4 * (i & 1))) & 15);
      out[32 * b + i] = (float)(oracle_e2m1_value(c) * s);
    }
  }
}

static float or_bf16_round(float x) { return or_bf16_to_f32(oracle_bf16_from_f32(x)); }

/* [CPU] `apply_compressed_rope`: pairs (2p, 2p+1) of the tail rotated by
 * position * frequency(p), frequency blending base^(-2p/rope) with a sixteenth
 * of it over pairs 15..25; fp32 arithmetic, each result rounded to bf16.
 * Reading: the page calls fp32 pow, sin and cos; here each is the exactly
 * rounded fp32 value (evaluated in double, rounded once), which any
 * implementation can reproduce; an fp32 library's last-bit differences would
 * otherwise flip FP4 codes downstream (many FP4 roundings land on ties). */
void oracle_compressed_rope(float* tail, int64_t rope, int64_t position) {
  const float base = 160000.0f, factor = 16.0f, low = 15.0f, high = 25.0f;
  const float pos = (float)position;
  for (int64_t p = 0; p < rope / 2; p++) {
    float ramp = ((float)p - low) / (high - low);
    if (ramp < 0.0f) ramp = 0.0f;
    if (ramp > 1.0f) ramp = 1.0f;
    const float bf = (float)pow((double)base, (double)(-((float)(2 * p)) / (float)rope));
    const float a = bf * (1.0f - ramp);
    const float c = bf / factor * ramp;
    const float freq = a + c;
    const float ang = pos * freq;
    const float sn = (float)sin((double)ang), cs = (float)cos((double)ang);
    const float re = tail[2 * p], im = tail[2 * p + 1];
    const float r0 = re * cs, r1 = im * sn, i0 = re * sn, i1 = im * cs;
    tail[2 * p] = or_bf16_round(r0 - r1);
    tail[2 * p + 1] = or_bf16_round(i0 + i1);
  }
}

/* The fast Walsh-Hadamard butterflies in fp32 (no scaling), n a power of two. */
void oracle_hadamard_f32(float* v, int64_t n) {
  for (int64_t span = 1; span < n; span *= 2)
    for (int64_t start = 0; start < n; start += 2 * span)
      for (int64_t o = 0; o < span; o++) {
        const float a = v[start + o], b = v[start + o + span];
        v[start + o] = a + b;
        v[start + o + span] = a - b;
      }
}

/* [CPU] `finalize_index_query`: bf16 round, compressed RoPE on the last `rope`
 * dims at `position`, Hadamard then times 1/sqrtf(dim) rounded to bf16, FP4
 * round trip. Returns 0, or -1 on a non-finite value in the FP4 step. */
int oracle_finalize_index_query(const float* src, int64_t dim, int64_t rope, int64_t position, float* q) {
  for (int64_t d = 0; d < dim; d++) q[d] = or_bf16_round(src[d]);
  oracle_compressed_rope(q + dim - rope, rope, position);
  oracle_hadamard_f32(q, dim);
  const float scale = 1.0f / sqrtf((float)dim);
  for (int64_t d = 0; d < dim; d++) q[d] = or_bf16_round(q[d] * scale);
  for (int64_t b = 0; b < dim / 32; b++) {
    uint8_t sc, packed[16];
    float out[32];
    if (oracle_fp4_quantize_block32(q + 32 * b, &sc, packed, out) != 0) return -1;
    for (int i = 0; i < 32; i++) q[32 * b + i] = out[i];
  }
  return 0;
}

/* Rust `f32::total_cmp` key: a strictly monotone map of the bits to int32. */
static int32_t or_total_key(float x) {
  int32_t i;
  memcpy(&i, &x, 4);
  return i ^ (int32_t)(((uint32_t)(i >> 31)) >> 1);
}

#define OR_SEL_NONFINITE 1u /* a score is not finite (the CPU page raises)       */
#define OR_SEL_TIE 2u       /* two candidate scores are equal (the CPU page raises) */
#define OR_SEL_GEOMETRY 4u  /* total < S                                          */

/* Scores and selection for every (b, s).
 *   iq  [B, S, H, dim] fp32 index queries; iw [B, S, H] fp32 weights
 *   keys [B, Rcap, dim/32*17] FP4 index keys
 *   sel  [B, S, K] int32 out: records by (-score, +record), -1 padded
 *   scores (optional) [B, S, Rcap] fp32 out: the candidates' scores (others NaN)
 * Query s sits at position total - S + s and scores records
 * r < min((position + 1) / 4, Rcap). score = sum over heads in ascending order
 * of max(dot, 0) * w * ((1/sqrtf(dim)) / sqrtf(H)), dot the ascending fp32 dot
 * of the finalized query with the decoded key. */
uint32_t oracle_csa_index_select(const float* iq, const float* iw, const uint8_t* keys, int64_t batch,
                                 int64_t seq, int64_t heads, int64_t dim, int64_t rope, int64_t record_cap,
                                 int64_t total, int64_t topk, int32_t* sel, float* scores_out) {
  if (total < seq) return OR_SEL_GEOMETRY;
  const int64_t kb = dim / 32 * 17;
  float ws = 1.0f / sqrtf((float)dim);
  ws = ws / sqrtf((float)heads);
  float* tq = (float*)malloc(sizeof(float) * (size_t)(heads * dim));
  float* key = (float*)malloc(sizeof(float) * (size_t)dim);
  float* sc = (float*)malloc(sizeof(float) * (size_t)(record_cap > 0 ? record_cap : 1));
  unsigned char* taken = (unsigned char*)malloc((size_t)(record_cap > 0 ? record_cap : 1));
  if (!tq || !key || !sc || !taken) {
    free(tq);
    free(key);
    free(sc);
    free(taken);
    return (uint32_t)-1;
  }
  uint32_t flags = 0;
  for (int64_t b = 0; b < batch; b++) {
    for (int64_t s = 0; s < seq; s++) {
      const int64_t pos = total - seq + s;
      int64_t n = (pos + 1) / 4;
      if (n > record_cap) n = record_cap;
      if (n < 0) n = 0;
      for (int64_t h = 0; h < heads; h++)
        if (oracle_finalize_index_query(iq + ((b * seq + s) * heads + h) * dim, dim, rope, pos, tq + h * dim) != 0)
          flags |= OR_SEL_NONFINITE;
      const float* w = iw + (b * seq + s) * heads;
      for (int64_t r = 0; r < n; r++) {
        oracle_fp4_decode_key(keys + (b * record_cap + r) * kb, dim, key);
        float score = 0.0f;
        for (int64_t h = 0; h < heads; h++) {
          float acc = 0.0f;
          for (int64_t d = 0; d < dim; d++) {
            const float prod = tq[h * dim + d] * key[d];
            acc = acc + prod;
          }
          const float relu = acc > 0.0f ? acc : 0.0f;
          const float t0 = relu * w[h];
          const float t1 = t0 * ws;
          score = score + t1;
        }
        if (!isfinite(score)) flags |= OR_SEL_NONFINITE;
        sc[r] = score;
      }
      if (scores_out) {
        float* so = scores_out + (b * seq + s) * record_cap;
        for (int64_t r = 0; r < record_cap; r++) so[r] = r < n ? sc[r] : NAN;
      }
      /* exact ties (the CPU page rejects them) */
      for (int64_t i = 0; i < n; i++)
        for (int64_t j = i + 1; j < n; j++)
          if (sc[i] == sc[j]) flags |= OR_SEL_TIE;
      /* repeated selection of the first record in the (-score, +record) order */
      int32_t* out = sel + (b * seq + s) * topk;
      for (int64_t j = 0; j < topk; j++) out[j] = -1;
      memset(taken, 0, (size_t)n);
      for (int64_t j = 0; j < topk && j < n; j++) {
        int64_t best = -1;
        for (int64_t r = 0; r < n; r++) {
          if (taken[r]) continue;
          if (best < 0 || or_total_key(sc[r]) > or_total_key(sc[best])) best = r;
        }
        taken[best] = 1;
        out[j] = (int32_t)best;
      }
    }
  }
  free(tq);
  free(key);
  free(sc);
  free(taken);
  return flags;
}
