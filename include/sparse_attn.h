/*
 * sparse_attn.h -- C ABI of the MI355X (gfx950) selected-token sparse
 * attention library with KV-cache append.
 *
 * The operation is the one the IndexShare operator defines (docs.rs page
 * onnx-runtime-ep-cuda, src/kernels/index_share.rs): append the current K/V
 * rows to the past cache (past ++ current -> present), validate each row of
 * selected_indices, gather the selected keys, score them as
 * (Q*sqrt(scale)) . (K*sqrt(scale)), take a numerically stable fp32 softmax
 * over the selected keys and reduce probs . V. Two storage forms come from the
 * compressed-sparse-attention pages (onnx-runtime-ep-cpu/-cuda,
 * src/kernels/compressed_sparse_attention.rs): a single shared-latent cache
 * row that is both key and value, and fp8_e4m3_block64 records (`CacheFormat`).
 * The optional softcap is the standard Attention page's (onnx-runtime-ep-cuda,
 * src/kernels/standard_attention.rs, module doc "Semantics").
 *
 * Conventions for every entry point below:
 *  - Every tensor pointer is a HIP DEVICE pointer owned by the caller; the
 *    library never frees or retains it past the call. Tensors are dense and
 *    row-major in the shapes stated.
 *  - Calls are asynchronous on the context's stream. sparse_attn_kv_append,
 *    sparse_attn_validate_indices, sparse_attn_forward and
 *    sparse_attn_reset_error_async perform no allocation, no host
 *    synchronisation and no device-to-host copy, so they may be recorded into
 *    a HIP graph.
 *  - A bad argument, shape, dtype, capacity or unsupported combination is
 *    reported by the return status BEFORE anything is launched, and
 *    sparse_attn_last_error() then holds a message.
 *  - Conditions only the device can see (index-row violations, append lengths
 *    held in device arrays, non-finite values given to the fp8 quantizer) are
 *    OR-latched into the context's device error word; sparse_attn_read_error
 *    returns it. A caller discards the outputs of a call whose word is nonzero.
 */
#ifndef SPARSE_ATTN_H
#define SPARSE_ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct sparse_attn_ctx sparse_attn_ctx;

typedef enum {
  SA_OK = 0,
  SA_E_ARG = 1,          /* NULL pointer, non-positive size, bad enum value     */
  SA_E_SHAPE = 2,        /* sizes inconsistent with each other or the config    */
  SA_E_DTYPE = 3,        /* dtype / cache format combination not allowed        */
  SA_E_CAPACITY = 4,     /* past_len + cur_len does not fit the present capacity */
  SA_E_UNSUPPORTED = 5,  /* valid request outside what this build implements     */
  SA_E_HIP = 6,          /* a HIP runtime call failed                            */
  SA_E_STATE = 7,        /* NULL or destroyed context, or sizes beyond create's max */
  SA_E_INDEX = 8         /* sparse_attn_read_error: the error word is nonzero    */
} sa_status;

/* element dtype of query, Y and a dense cache (codes as the IndexShare
 * kernels' load_float/store_float: 0 f32, 1 f16, 2 bf16) */
enum { SA_F32 = 0, SA_F16 = 1, SA_BF16 = 2 };
/* cache storage: dense rows of the element dtype, or fp8_e4m3_block64 records
 * ((Dk - rope)/64 blocks of [1 E8M0 scale byte, 64 E4M3FN bytes], then `rope`
 * little-endian BF16 values; the CSA CPU page's `CacheFormat`) */
enum { SA_CACHE_DENSE = 0, SA_CACHE_FP8_E4M3_BLOCK64 = 1 };
/* SEPARATE: K and V caches, Dk == Dv (IndexShare). SHARED_LATENT: one cache
 * whose row is the key and whose first Dv dims are the value (the CSA pages'
 * records are both key and value). */
enum { SA_KV_SEPARATE = 0, SA_KV_SHARED_LATENT = 1 };
enum { SA_IDX_I32 = 0, SA_IDX_I64 = 1 };

/* Device error-word bits. The first six are index-row classes in the check
 * order of the IndexShare host `validate_indices`; 512 is IndexShare's
 * capture-error bit (INDEX_SHARE_CAPTURE_ERROR_INDEX), set with any of them. */
#define SA_ERR_SENTINEL 0x01u        /* an index below -1                        */
#define SA_ERR_AFTER_PAD 0x02u       /* a non-(-1) index after trailing padding  */
#define SA_ERR_RANGE 0x04u           /* an index >= the batch's cache length     */
#define SA_ERR_DUPLICATE 0x08u       /* an index equal to the previous one       */
#define SA_ERR_ORDER 0x10u           /* an index below the previous one          */
#define SA_ERR_ALL_PAD 0x20u         /* a row with no valid index                */
#define SA_ERR_APPEND_CAPACITY 0x40u /* device past_len[b] < 0, > past capacity, or
                                        past_len[b] + cur_len > present capacity;
                                        that batch's rows are not written         */
#define SA_ERR_QUANT_NONFINITE 0x80u /* fp8 quantize-on-append met a NaN/Inf     */
#define SA_ERR_CSA_GEOMETRY 0x100u   /* sparse_attn_csa_forward: total_len does not
                                        fit the sizes (see there); nothing written */
#define SA_ERR_INDEX_ANY 512u
#define SA_ERR_APPEND_ANY 1024u
#define SA_ERR_CSA_DENOM 0x800u      /* sparse_attn_csa_forward: a softmax
                                        denominator not finite and positive      */
#define SA_ERR_INDEX_NONFINITE 0x1000u /* sparse_attn_csa_index_select: a record's
                                          score is not finite                     */
#define SA_ERR_INDEX_TIE 0x2000u       /* sparse_attn_csa_index_select: two of a
                                          row's candidate scores are equal (the CSA
                                          CPU page's select_ratio4_topk rejects
                                          such a row)                             */

typedef struct {
  int32_t num_heads;      /* Hq > 0 (IndexShare attr num_heads)                         */
  int32_t kv_num_heads;   /* Hkv > 0, Hq % Hkv == 0 (attr kv_num_heads)                 */
  int32_t head_dim_qk;    /* Dk: query/key head dim                                     */
  int32_t head_dim_v;     /* Dv: value head dim; SEPARATE requires Dv == Dk, SHARED_LATENT Dv <= Dk */
  int32_t rope_dim;       /* fp8 records only: BF16 tail width; (Dk - rope) % 64 == 0   */
  int32_t dtype;          /* SA_F32 / SA_F16 / SA_BF16                                  */
  int32_t cache_format;   /* SA_CACHE_*; fp8 requires SHARED_LATENT and dtype bf16      */
  int32_t kv_layout;      /* SA_KV_*                                                    */
  int32_t index_dtype;    /* SA_IDX_*                                                   */
  float scale;            /* 0 -> 1/sqrtf(Dk); else finite and > 0 (attr scale)         */
  float softcap;          /* 0 -> off; else finite and > 0: s = softcap*tanh(s/softcap) */
  int64_t max_batch;      /* largest batch any call will pass                           */
  int64_t max_q_seq;      /* largest query length                                       */
  int64_t max_index_width;/* largest selected_indices row width                         */
  int64_t max_cache_len;  /* largest cache capacity (rows per (batch, kv head))         */
} sa_config;

/* Create a context: checks the config against the operator's attribute rules
 * (IndexShare page, kernel `create`: num_heads and kv_num_heads positive,
 * scale finite and > 0 when given; `launch_rows` takes an absent scale as
 * 1/sqrt(head size), here scale 0; head sizes as `validate_shapes` requires
 * them, with the shared-latent and fp8_e4m3_block64 forms of the CSA CPU
 * page's `CacheFormat`), then allocates the device error word and the split-K
 * partial buffers sized from the max_* fields (IndexShare `ensure_scratch`:
 * buffers sized once, at addresses that stay fixed so a captured graph can
 * keep them). hip_stream may be NULL (the null stream).
 * Returns SA_E_ARG / SA_E_DTYPE / SA_E_SHAPE / SA_E_UNSUPPORTED for a bad
 * config (nothing allocated), SA_E_HIP if an allocation fails (everything
 * already allocated is released). *out is NULL on failure. */
sa_status sparse_attn_create(const sa_config* cfg, void* hip_stream, sparse_attn_ctx** out);

/* Release the context's device buffers after draining its stream (IndexShare
 * page, the kernel's `drop`: its scratch lives exactly as long as the
 * operator instance). NULL is accepted and ignored; a
 * pointer that is not a live context returns SA_E_STATE and frees nothing. */
sa_status sparse_attn_destroy(sparse_attn_ctx* ctx);

/* Change the stream later calls are launched on. */
sa_status sparse_attn_set_stream(sparse_attn_ctx* ctx, void* hip_stream);

/*
 * A1/A2: KV append (IndexShare `build_present`, `build_present_capacity`).
 *   present[b,h,t] = past[b,h,t]                 for t < past_len[b]
 *                  = cur[b,h,t - past_len[b]]    for past_len[b] <= t < past_len[b] + cur_len
 * Rows at or beyond past_len[b] + cur_len are not touched.
 *   past_k/past_v       [B, Hkv, past_capacity, row]; may be NULL when past_capacity == 0
 *   past_len            device int32 [B], or NULL meaning every batch holds past_capacity rows
 *   cur_k/cur_v         [B, Hkv, cur_len, row]
 *   present_k/present_v [B, Hkv, present_capacity, row]
 * `row` is Dk (K) / Dv (V) elements of the config dtype, or one fp8 record.
 * present == past is the in-place capacity mode: only the cur_len new rows
 * are written, and past_capacity must equal present_capacity (one row stride;
 * SA_E_ARG otherwise). present != past is concat mode: past rows are copied too.
 * SHARED_LATENT: pass past_v, cur_v and present_v as NULL.
 * cur_is_unquantized_bf16 (fp8 caches only): cur_k is bf16 [B, Hkv, cur_len, Dk]
 * and each new row is quantized on the device into a record (block scale
 * floor(log2 amax) - 8 + 127, E4M3FN nearest-even saturating at 448; the CSA
 * CPU page's `finalize_attention_record` pack loop); otherwise cur_k holds
 * records and the append is a byte copy.
 * present_len: optional device int32 [B] output, past_len[b] + cur_len
 * (written for cur_len == 0 too).
 * Host errors: SA_E_CAPACITY when past_len is NULL and
 * past_capacity + cur_len > present_capacity. Device errors:
 * SA_ERR_APPEND_CAPACITY, SA_ERR_QUANT_NONFINITE.
 */
sa_status sparse_attn_kv_append(sparse_attn_ctx* ctx, int64_t batch, const void* past_k,
                                const void* past_v, int64_t past_capacity, const int32_t* past_len,
                                const void* cur_k, const void* cur_v, int64_t cur_len,
                                int32_t cur_is_unquantized_bf16, void* present_k, void* present_v,
                                int64_t present_capacity, int32_t* present_len);

/*
 * A3: validate selected_indices [B, Hi, Sq, W] (Hi is 1 or Hq), int32 or
 * int64 per the config. Per row, columns are checked left to right with the
 * IndexShare host `validate_indices` rules; the first failing column decides
 * the row's class (SA_ERR_* bit index + 1; 0 = valid). A row of only -1 is
 * ALL_PAD.
 *   valid_len   device int32 [B]: cache length of each batch (an index must be
 *               below it); NULL means every batch has cache_len.
 *   error_word  device uint32: OR of the invalid rows' class bits | 512;
 *               NULL means the context's word.
 *   row_class   optional device uint8 [B*Hi*Sq]: each row's class.
 *   first_bad   device uint64: smallest row*(W+1)+col over invalid rows
 *               (col == W for ALL_PAD). NULL means the context's slot, which
 *               keeps the FIRST failing call since the last reset (with the
 *               failing value, its left neighbour and the bound, for the
 *               message sparse_attn_read_error builds); a caller-owned slot
 *               takes the atomic minimum over calls.
 * The word and slot accumulate across calls until
 * sparse_attn_reset_error_async.
 */
sa_status sparse_attn_validate_indices(sparse_attn_ctx* ctx, const void* indices, int64_t batch,
                                       int64_t index_heads, int64_t q_seq, int64_t width,
                                       const int32_t* valid_len, int64_t cache_len,
                                       uint32_t* error_word, uint8_t* row_class,
                                       uint64_t* first_bad);

/*
 * A4-A10: the forward (IndexShare `index_share_row` semantics).
 *   q          [B, Hq, Sq, Dk] config dtype
 *   present_k  [B, Hkv, cache_capacity, Dk] dense, or records
 *   present_v  [B, Hkv, cache_capacity, Dv] (SEPARATE) or NULL (SHARED_LATENT)
 *   valid_len  device int32 [B] or NULL (= cache_capacity): gather bound
 *   indices    [B, Hi, Sq, W], rows of strictly increasing keys padded with -1
 *   y          [B, Hq, Sq, Dv] config dtype (bf16/f16 rounded to nearest even)
 * For each output row (b, h, q): kvh = h / (Hq/Hkv), index row ih = Hi==1 ? 0 : h,
 * n = entries before the first -1; y = softmax_s(softcap(scale * q.k_s)) . v_s
 * over the n selected keys, fp32 throughout. A key outside [0, bound) is read
 * as key 0 (IndexShare clamps so a bad row stays in bounds); its row is
 * reported by validation, not here. fused_validate != 0 also runs
 * sparse_attn_validate_indices into the context's word first, on the stream.
 */
sa_status sparse_attn_forward(sparse_attn_ctx* ctx, const void* q, int64_t batch, int64_t q_seq,
                              const void* present_k, const void* present_v,
                              int64_t cache_capacity, const int32_t* valid_len,
                              const void* indices, int64_t index_heads, int64_t width, void* y,
                              int32_t fused_validate);

/* The forward with IndexShare's optional 7th input, the additive
 * attention_bias (IndexShare page: `bias_at`, `index_share_row`,
 * `validate_bias_shape`; the CPU page's `AttentionBias`). Arguments as
 * sparse_attn_forward, plus
 *   bias        NULL (then exactly sparse_attn_forward), or a dense row-major
 *               tensor of the config dtype whose shape bias_shape[bias_rank]
 *               (host array, 0 <= rank <= 4) is right-aligned against
 *               [B, Hq, Sq, cache_capacity]; each extent is 1 (broadcast) or
 *               the target's.
 * For output row (b, h, q) and selected key k (its cache position, clamped as
 * in sparse_attn_forward) the score becomes softcap(scale * q.k) +
 * bias[b, h, q, k]; a row whose scores are all -inf gives zeros. A biased
 * call runs on the MFMA kernel of its layout (sparse_attn_query_plan path 4
 * grouped-query, 2 bf16 shared-latent, 3 fp8 shared-latent records; on path
 * 2 the general latent kernel with its split-K combine, not the decode
 * kernel) when the configuration takes one, else on the generic vector
 * kernel (path 0). Host errors: those of sparse_attn_forward, and
 * SA_E_SHAPE for a rank above 4 or an extent that does not broadcast.
 * Asynchronous and capturable. */
sa_status sparse_attn_forward_bias(sparse_attn_ctx* ctx, const void* q, int64_t batch, int64_t q_seq,
                                   const void* present_k, const void* present_v,
                                   int64_t cache_capacity, const int32_t* valid_len,
                                   const void* indices, int64_t index_heads, int64_t width,
                                   const void* bias, const int64_t* bias_shape, int32_t bias_rank,
                                   void* y, int32_t fused_validate);

/* Capacity-mode length recovery (IndexShare page, kernel `capacity_write_pos`
 * and the capacity branch of its launch sequence). When the present cache
 * aliases a fixed-capacity past, its shape no longer carries the live length;
 * the attention_bias's causal/padding frontier does. For each batch entry b:
 *   valid_len[b] = 1 + the largest k < cache_capacity with bias[b, h, q, k]
 *                  finite for some (h, q); 0 when there is none
 *   write_pos[b] = valid_len[b] - cur_len, or 0 when valid_len[b] < cur_len
 * write_pos is the past_len of the in-place sparse_attn_kv_append that places
 * this step's cur_len rows, valid_len the bound of sparse_attn_validate_indices
 * and sparse_attn_forward_bias.
 *   bias, bias_shape, bias_rank  as sparse_attn_forward_bias, against
 *               [B, Hq, Sq, cache_capacity]; required
 *   valid_len, write_pos         device int32 [B] outputs
 * Host errors: SA_E_ARG (NULL bias or outputs, q_seq or cache_capacity < 1,
 * cache_capacity >= 2^31, cur_len < 0), SA_E_STATE (batch outside
 * [1, max_batch]), SA_E_SHAPE (bias shape). Asynchronous and capturable. */
sa_status sparse_attn_capacity_lengths(sparse_attn_ctx* ctx, const void* bias, const int64_t* bias_shape,
                                       int32_t bias_rank, int64_t batch, int64_t q_seq,
                                       int64_t cache_capacity, int64_t cur_len, int32_t* valid_len,
                                       int32_t* write_pos);

/* One capacity-mode attention step over a cache kept in place (IndexShare's
 * capacity branch: `capacity_write_pos`, the `build_present_capacity`
 * launches and the rows; the branch does not depend on the layout), the
 * same as
 *   [sparse_attn_reset_error_async if reset_error]
 *   sparse_attn_capacity_lengths(bias, ..., cur_len, valid_len, write_pos)
 *   sparse_attn_kv_append(past = present = cache, past_len = write_pos, cur)
 *   sparse_attn_forward_bias(present = cache, valid_len, bias, fused_validate = 1)
 *   cache_k, cache_v [B, Hkv, cache_capacity, D] read and written; cur_k,
 *                    cur_v [B, Hkv, cur_len, D]; 1 <= cur_len <= cache_capacity.
 *                    A shared-latent cache passes cache_k (its bf16 rows or
 *                    fp8 records) and cur_k (rows in the cache's own format)
 *                    with cache_v = cur_v = NULL.
 *   valid_len, write_pos  device int32 [B] outputs
 * The reset, the lengths and the append are one launch when the cache is
 * dense, its rows a multiple of 16 bytes and the tensors 16-byte aligned
 * (Dk == Dv for separate caches). Host errors: those of the four calls, checked before
 * anything is launched; SA_E_ARG for a V tensor passed with a shared-latent
 * cache or missing with separate ones; SA_E_UNSUPPORTED for separate caches
 * that are not dense. Asynchronous and capturable. */
sa_status sparse_attn_capacity_step(sparse_attn_ctx* ctx, const void* q, int64_t batch, int64_t q_seq,
                                    void* cache_k, void* cache_v, int64_t cache_capacity, const void* cur_k,
                                    const void* cur_v, int64_t cur_len, const void* indices,
                                    int64_t index_heads, int64_t width, const void* bias,
                                    const int64_t* bias_shape, int32_t bias_rank, void* y,
                                    int32_t* valid_len, int32_t* write_pos, int32_t reset_error);

/* One attention step over a shared-latent cache kept in place (capacity
 * mode): the same as
 *   [sparse_attn_reset_error_async if reset_error]
 *   sparse_attn_kv_append(past = present = cache, cur,
 *                         cur_is_unquantized_bf16, present_len)
 *   sparse_attn_forward(present = cache, valid_len = present_len,
 *                       fused_validate = 1)
 * (IndexShare's capacity-mode present build followed by the operator; the
 * append and the attention row are the ones documented above).
 * cache [B, 1, cache_capacity, row] is read and written; cur [B, 1, cur_len,
 * .] holds rows in the cache's storage format (bf16 rows, or packed
 * fp8_e4m3_block64 records), or bf16 rows to quantize when
 * cur_is_unquantized_bf16 (fp8 caches only); past_len [B] is read and
 * present_len [B] written on the device.
 * On the shared-latent MFMA paths (query_plan path 2 or 3) with cur_len <= 8
 * this is ONE forward launch (plus the split-K combine): every workgroup
 * writes (or quantizes) its batch's current rows into the cache before it
 * gathers, and the launch's last workgroup merges (or, with reset_error,
 * replaces) the error word. In every other case the three calls above run in
 * sequence. Errors: host-side statuses of those calls; device-side bits as
 * they latch them (a capacity failure appends nothing and sets
 * SA_ERR_APPEND_CAPACITY | SA_ERR_APPEND_ANY; a non-finite bf16 row is left
 * unwritten and sets SA_ERR_QUANT_NONFINITE | SA_ERR_APPEND_ANY).
 * SA_E_UNSUPPORTED for separate K/V caches. Every host check of the three
 * calls (including the index geometry and the q / indices / y pointers) is
 * made before the reset or the append is launched, so a rejected step leaves
 * the cache, present_len and the error word as they were. Asynchronous and
 * capturable. */
sa_status sparse_attn_step(sparse_attn_ctx* ctx, const void* q, int64_t batch, int64_t q_seq, void* cache,
                           int64_t cache_capacity, const int32_t* past_len, const void* cur,
                           int64_t cur_len, int32_t cur_is_unquantized_bf16, int32_t* present_len,
                           const void* indices, int64_t index_heads, int64_t width, void* y,
                           int32_t reset_error);

/* The same step over separate K and V caches kept in place:
 *   [sparse_attn_reset_error_async if reset_error]
 *   sparse_attn_kv_append(past = present = (cache_k, cache_v), past_len, cur_k, cur_v, present_len)
 *   sparse_attn_forward(present = (cache_k, cache_v), valid_len = present_len, fused_validate = 1)
 * cache_k, cache_v [B, Hkv, cache_capacity, D] read and written; cur_k, cur_v
 * [B, Hkv, cur_len, D] (config dtype); past_len [B] read and present_len [B]
 * written on the device; 0 <= cur_len <= cache_capacity.
 * On the grouped-query MFMA path (sparse_attn_query_plan path 4), when a
 * workgroup's (query, head) rows fill at most half its waves (decode-like:
 * min(q_seq, 128 / group) * group <= 64) and the four tensors are 16-byte
 * aligned, this is ONE forward launch (plus the split-KV combine): every workgroup writes its (batch, kv head)'s current rows into
 * the caches before it gathers, checks its share of the index columns, and
 * the launch's last arrival merges (or, with reset_error, replaces) the error
 * word. In every other case the three calls above run in sequence. Errors:
 * host-side statuses of those calls (SA_E_UNSUPPORTED for a shared-latent
 * cache), all checked before anything is launched; device-side bits as they
 * latch them (a capacity failure appends nothing and sets
 * SA_ERR_APPEND_CAPACITY | SA_ERR_APPEND_ANY). Asynchronous and capturable. */
sa_status sparse_attn_step_kv(sparse_attn_ctx* ctx, const void* q, int64_t batch, int64_t q_seq, void* cache_k,
                              void* cache_v, int64_t cache_capacity, const int32_t* past_len, const void* cur_k,
                              const void* cur_v, int64_t cur_len, int32_t* present_len, const void* indices,
                              int64_t index_heads, int64_t width, void* y, int32_t reset_error);

/* CSA ratio-4 selection producer (the indexer): the index-selection stage of
 * the compressed-sparse-attention operator's ratio-4 path (onnx-runtime-ep-cpu,
 * src/kernels/compressed_sparse_attention.rs, `select_ratio4_topk` and
 * `finalize_index_query`; onnx-runtime-ep-cuda, same file, kernel
 * `csa_ratio4_index_select`). For batch b and query s at position
 * p = total - S + s:
 *   - each index head's query is finalized: rounded to bf16, the compressed
 *     RoPE applied to its last 64 dims at position p, Walsh-Hadamard
 *     transformed and scaled by 1/sqrt(128) (rounded to bf16), and rounded
 *     through FP4 E2M1 block-32 (E8M0 scale floor(log2 amax) - 2 + 127,
 *     nearest E2M1 value, ties to the even code);
 *   - every record r < min((p + 1) / 4, key_cap) is scored
 *     sum over heads h (ascending) of max(q_h . k_r, 0) * w_h * ((1/sqrt(128)) / sqrt(H)),
 *     in fp32;
 *   - the first K records in (-score, +record) order are written, then -1.
 *   index_query   [B, S, H, 128] fp32; H a multiple of 16, at most 64
 *   index_weight  [B, S, H] fp32
 *   index_keys    [B, key_cap, 68] bytes: 4 blocks of [E8M0 scale, 16 bytes of
 *                 E2M1 codes, element 2i in the low nibble]; key_cap <= 32768
 *   total_len     DEVICE pointer to one int64: total_sequence_length
 *   selected      [B, out_heads, S, K] int32 out; every index-head row gets the
 *                 same selection (as the pages replicate it); 1 <= K <= 2048
 *   workspace     device scratch of sparse_attn_csa_index_workspace_bytes(B, S, H,
 *                 key_cap) bytes, owned by the caller (the scores, the
 *                 finalized queries and their block scale exponents);
 *                 contents on return are unspecified
 * Each head dot equals the CPU page's ascending fp32 fold for any block
 * scales: the matrix-core dot is used where no partial sum can round, the
 * fold itself elsewhere. Exact score ties, which the CPU page rejects, are
 * ordered by ascending record and reported as SA_ERR_INDEX_TIE (float
 * equality of any two of a row's candidate scores; a NaN equals nothing).
 * Host errors: SA_E_ARG (NULL pointer, size < 1), SA_E_UNSUPPORTED
 * (H, K or key_cap out of range). Device: SA_ERR_CSA_GEOMETRY when total < S
 * (nothing written); SA_ERR_INDEX_NONFINITE when a score is not finite (it is
 * still ranked, by the fp32 total order). Asynchronous and capturable. */
sa_status sparse_attn_csa_index_select(sparse_attn_ctx* ctx, const float* index_query,
                                       const float* index_weight, const uint8_t* index_keys,
                                       int64_t batch, int64_t q_seq, int64_t heads, int64_t key_cap,
                                       const int64_t* total_len, int64_t topk, int64_t out_heads,
                                       int32_t* selected, void* workspace);

/* Bytes of scratch sparse_attn_csa_index_select needs for these sizes (0 on a
 * size < 1). */
size_t sparse_attn_csa_index_workspace_bytes(int64_t batch, int64_t q_seq, int64_t heads,
                                             int64_t key_cap);

/* CSA ratio-4 selected sink attention: the attention stage of the
 * compressed-sparse-attention operator's ratio-4 path (onnx-runtime-ep-cuda,
 * src/kernels/compressed_sparse_attention.rs, kernel
 * `csa_ratio4_sink_attention`; onnx-runtime-ep-cpu, same file,
 * `ratio4_attention`, the cursor checks of its driver, and `AttentionBias`).
 * For batch b, query s at position p = total - S + s and head h, the
 * candidates are
 *   - the dense causal window: current_kv rows at positions
 *     max(total - Tcur, p + 1 - 128) .. p, numbered c = 0, 1, ... from the
 *     window start, of which there are Cd = min(Tcur, 128) when total == S and
 *     Cd = 128 otherwise (a number above p is no candidate);
 *   - the K selected records, numbered Cd + j for slot j; a negative index is
 *     no candidate, an index >= total / 4 (not yet complete) is no candidate
 *     and sets SA_ERR_RANGE | SA_ERR_INDEX_ANY.
 * Score = (query . row) * scale (+ bias[b, h, s, c] broadcast over extents of
 * 1); m = max over the candidates; y = sum_c e^(score_c - m) row_c / (sum_c
 * e^(score_c - m) + e^(head_sink[h] - m)); a head with no candidate gives
 * zeros. Arithmetic: the products run on the matrix cores with every fp32
 * operand split into three bf16 pieces (exact for record rows), fp32
 * accumulation, fp32 softmax; within 1e-5 of the fp32 definition.
 *   query       [B, S, H, 512] fp32; H a multiple of 16
 *   current_kv  [B, Tcur, 512] fp32 (absolute positions total - Tcur .. total - 1)
 *   records     [B, record_cap, 583] bytes: fp8_e4m3_block64 records of 512
 *               dims (7 blocks of [E8M0 scale, 64 E4M3FN codes], then 64
 *               little-endian BF16 values); record_cap * 583 < 2^31
 *   selected    [B, index_heads, S, K] int32; the rows of index head 0 are
 *               read (the pages repeat one selection over the index heads);
 *               1 <= K <= 2048
 *   head_sink   [H] fp32
 *   bias        NULL, or fp32 with the right-aligned shape bias_dims[4]
 *               (host array; each 1 or the extent of [B, H, S, Cd + K]; the
 *               last extent is checked on the device, as Cd needs total)
 *   total_len   DEVICE pointer to one int64: total_sequence_length
 *   scale       0 -> 1/sqrt(512); else finite and > 0
 *   y           [B, S, H, 512] fp32
 * Host errors: SA_E_ARG (NULL pointer, size < 1, bad scale), SA_E_SHAPE
 * (bias extents), SA_E_UNSUPPORTED (H % 16, K > 2048, Tcur * 2048 or
 * record_cap * 583 >= 2^31). Device: SA_ERR_CSA_GEOMETRY when total < S,
 * total < Tcur, total - Tcur > max(0, total - S + 1 - 128), total / 4 >
 * record_cap or the bias's last extent is neither 1 nor Cd + K (then nothing
 * is written); SA_ERR_CSA_DENOM when a denominator is not finite and positive
 * (NaN or overflowing inputs). Uses the context's stream and error word only
 * (not its config). Asynchronous and capturable. */
sa_status sparse_attn_csa_forward(sparse_attn_ctx* ctx, const float* query, int64_t batch,
                                  int64_t q_seq, int64_t heads, const float* current_kv,
                                  int64_t cur_len, const uint8_t* records, int64_t record_cap,
                                  const int32_t* selected, int64_t index_heads, int64_t topk,
                                  const float* head_sink, const float* bias,
                                  const int64_t* bias_dims, const int64_t* total_len, float scale,
                                  float* y);

/* Zero the context's error word and set first_bad to UINT64_MAX, with a tiny
 * kernel on the stream (no memset node, so it is safe inside a graph). This is
 * the reset of IndexShare's capture-error word (page module doc on capture:
 * `validate_index_rows` latches INDEX_SHARE_CAPTURE_ERROR_INDEX into a
 * persistent word that the host reads outside the captured region).
 * SA_E_STATE for a dead context; otherwise only a launch failure (SA_E_HIP). */
sa_status sparse_attn_reset_error_async(sparse_attn_ctx* ctx);

/* Synchronise the stream and copy the context's error word and first_bad slot
 * to the host (either pointer may be NULL). NOT capturable. Returns
 * SA_E_INDEX when the word is nonzero and, for an index error, puts the
 * IndexShare wording of the first failing row into sparse_attn_last_error(). */
sa_status sparse_attn_read_error(sparse_attn_ctx* ctx, uint32_t* word, uint64_t* first_bad);

/* The last host-side message for this context ("" if none). With ctx NULL:
 * the message of this thread's last sparse_attn_forward_latent_static call. */
const char* sparse_attn_last_error(const sparse_attn_ctx* ctx);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture without a memory pool, tight serving loops, harnesses that forbid
 * hipMalloc): sparse_attn_forward with fused_validate = 0 on a context of
 * layout SHARED_LATENT, dense bf16 cache, 64 query heads, Dk 576, Dv 512 and
 * one index list per (batch, query), but without any context. No call
 * allocates: the split-K partials live in a static device array of
 * SA_STATIC_SCRATCH_BYTES, one per GPU the library runs on, reserved when the
 * library is loaded there and held until the process ends.
 *   q, cache, valid_len, indices, y   as sparse_attn_forward (cache is the
 *                  shared-latent present cache [B, 1, cache_capacity, 576]
 *                  bf16; indices [B, 1, Sq, W] of index_dtype)
 *   index_dtype    SA_IDX_I32 or SA_IDX_I64
 *   scale, softcap as sa_config (scale 0 -> 1/sqrt(576); softcap 0 -> off)
 *   hip_stream     the stream to launch on (NULL: the null stream)
 * Results equal sparse_attn_forward's on the same inputs (same kernels and
 * split count). Index rows are not validated. Errors, before any launch:
 * SA_E_ARG (NULL tensor, non-positive size, scale or softcap negative or not
 * finite), SA_E_DTYPE (index_dtype), SA_E_UNSUPPORTED (capacity beyond the
 * kernels' 32-bit offsets), SA_E_CAPACITY when batch * Sq rows at the planned
 * split count need more partials (rows * splits * 131,584 bytes) than the
 * scratch holds; SA_E_HIP for a failed launch. The message is
 * sparse_attn_last_error(NULL). Every call on one GPU shares that GPU's
 * scratch: calls that overlap on one GPU (different streams, host threads)
 * race and must be ordered by the caller. Asynchronous and capturable. */
#define SA_STATIC_SCRATCH_BYTES (48u << 20)
sa_status sparse_attn_forward_latent_static(const void* q, int64_t batch, int64_t q_seq, const void* cache,
                                            int64_t cache_capacity, const int32_t* valid_len,
                                            const void* indices, int32_t index_dtype, int64_t width,
                                            float scale, float softcap, void* y, void* hip_stream);

/* Report which forward path and split count a call with these sizes takes:
 * *path = 0 generic (VALU), 1 shared-latent MFMA over fp8_e4m3_block64
 * records (register-staged), 2 shared-latent MFMA over a bf16 cache,
 * 3 shared-latent MFMA over fp8_e4m3_block64 records with 64 RoPE dims
 * (wave-pair kernel), 4 grouped-query MFMA (bf16 separate K/V caches of
 * 128 dims, one index list per (batch, query)); *splits >= 1. */
sa_status sparse_attn_query_plan(const sparse_attn_ctx* ctx, int64_t batch, int64_t q_seq,
                                 int64_t index_heads, int64_t width, int32_t* path,
                                 int32_t* splits);

/* Optional kernel timing. With max_launches > 0, each later
 * sparse_attn_forward records a HIP event pair on the context stream right
 * before and after its main attention kernel (the per-split kernel when the
 * keys are split; not the validation or combine kernels), for up to
 * max_launches calls. The events are created here, not on the launch path.
 * max_launches == 0 turns it off and releases the events. */
sa_status sparse_attn_profile_enable(sparse_attn_ctx* ctx, int32_t max_launches);

/* Synchronise, then return the summed duration in milliseconds and the
 * number of timed launches since the last read, and start counting again. */
sa_status sparse_attn_profile_read(sparse_attn_ctx* ctx, double* total_ms, int64_t* launches);

/* Measurement aids (not part of the attention path): kernels that measure the
 * device's attainable peaks, against which the kernels' roofline fractions are
 * reported beside the vendor figures. Both launch asynchronously on the
 * context stream; the caller times them (e.g. with events on that stream).
 *
 * sparse_attn_measure_copy: copies `bytes` from src to dst (device buffers,
 * 16-byte aligned, not overlapping, bytes a positive multiple of 16) with
 * streaming loads and stores; HBM traffic = 2 * bytes.
 * sparse_attn_measure_read: reads `bytes` from src (16-byte aligned, bytes a
 * positive multiple of 16) with streaming loads; sink is device uint32
 * [SA_PEAK_READ_SINK_WORDS], of which the first
 * min(ceil(bytes / 16384), 1024) * 256 words are written (values meaningless).
 * sparse_attn_measure_mfma: `workgroups` workgroups of 4 waves, each wave
 * running iters x 8 independent bf16 16x16x32 matrix-core products, i.e.
 * workgroups * 4 * iters * 8 * 16384 flops; out is device float
 * [workgroups * 256] (written, values meaningless). workgroups in 1..65536,
 * iters in 1..2^20.
 * Host errors: SA_E_ARG for the conditions above. */
#define SA_PEAK_READ_SINK_WORDS (1024 * 256)
sa_status sparse_attn_measure_copy(sparse_attn_ctx* ctx, void* dst, const void* src, int64_t bytes);
sa_status sparse_attn_measure_read(sparse_attn_ctx* ctx, uint32_t* sink, const void* src, int64_t bytes);
sa_status sparse_attn_measure_mfma(sparse_attn_ctx* ctx, float* out, int64_t workgroups, int32_t iters);

/* Library version string. */
const char* sparse_attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_ATTN_H */
