/*
 * pkv -- paged KV attention, KV scatter and batched sampling for MI355X (gfx950).
 *
 * The C ABI of libpkv.so: the data-parallel hot path of one step of a
 * mini-SGLang-style engine's forward_batch, per layer:
 *
 *   1. pkv_store_kv                 scatter this step's K/V rows into the paged pool
 *      (pkv_qk_norm_rope_store_kv   the same store fused with Qwen3's per-head q/k
 *                                   RMSNorm and the rotary embedding);
 *      (pkv_embedding_gather        the embedding rows of the step's token ids,
 *                                   the first op of forward_batch)
 *   2. pkv_paged_attention_decode   GQA attention of one new token per request
 *      (pkv_paged_attention_decode_store   the same with step 1's store done by
 *                                   the attention call itself);
 *      pkv_paged_attention_extend   causal GQA attention of a chunk of new tokens
 *                                   over a cached prefix (prefill / extend);
 *   3. pkv_sample                   temperature -> top-k -> top-p (-> min_p) -> draw per row,
 *                                   or argmax when the whole batch is greedy.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers named "device" point to GPU memory; everything else is host memory.
 * - The caller allocates and owns every buffer (pools, tables, lengths, q, o,
 *   logits, uniforms, outputs, workspaces). The library allocates nothing and
 *   keeps no per-call state.
 * - Each compute call validates its arguments on the host, then only ENQUEUES
 *   kernels on `stream` (a hipStream_t; NULL = the null stream) and returns.
 *   There is no implicit synchronisation. Buffers must stay alive and unchanged
 *   until the stream has passed the call. Outputs must not alias inputs.
 * - Return value: PKV_OK (0) or a negative pkv_status. On a negative status
 *   nothing was enqueued (except PKV_ERR_HIP, which reports a failed launch)
 *   and pkv_last_error() describes the problem.
 * - Data-dependent checks happen on the device: an out-of-range slot, table
 *   row or length is never dereferenced; the affected row is skipped (its
 *   output is left unwritten or zero, as documented per call) and a bit is set
 *   in the device fault word, which pkv_read_faults() returns and clears.
 * - head_dim must be 128. num_q_heads must be a multiple of kv_heads.
 *
 * Sources, cited by page title and section:
 *   [ENG]  mini-sglang handbook, "Engine 与采样器": sections 显存规划,
 *          forward_batch, 采样器, 测试.
 *   [CORE] mini-sglang handbook, "核心数据结构：Req、Batch、Context": sections
 *          SamplingParams, Req：请求的三个长度, Batch, Context.
 *   [TINY] mini-sglang handbook, "第 0 步：一个能跑的最小推理引擎": the dense
 *          reference attention function (section 这份代码在做什么).
 *   [DISS] "Mini-SGLang 完整剖析": sections 4.4.3 (KV pool), 4.6.4-4.6.7
 *          (attention metadata, store_kv before attention), 4.8.4-4.8.6
 *          (greedy rule, sampler arguments), 4.9.4-4.9.5 (store kernel
 *          contract), 5.2 (page budget).
 *   [SRC4] "Mini-SGLang 源码解析（四）：GPU 计算引擎系统": sections 14.3-14.5.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PKV_OK = 0,
  PKV_ERR_NULL = -1,       /* a required pointer is NULL */
  PKV_ERR_DTYPE = -2,      /* unsupported or inconsistent dtype */
  PKV_ERR_SHAPE = -3,      /* unsupported head_dim / head counts / sizes / strides */
  PKV_ERR_LENGTHS = -4,    /* host-visible length bounds inconsistent */
  PKV_ERR_ALIGN = -5,      /* pointer or stride not 16-byte aligned */
  PKV_ERR_WORKSPACE = -6,  /* workspace NULL or smaller than required */
  PKV_ERR_HIP = -7,        /* a HIP runtime call failed */
  PKV_ERR_DEVICE = -8      /* the current device is not a supported gfx950 part */
} pkv_status;

typedef enum { PKV_F32 = 0, PKV_BF16 = 1 } pkv_dtype;
typedef enum { PKV_I32 = 0, PKV_I64 = 1 } pkv_itype;

/* Device fault bits (see pkv_read_faults). */
#define PKV_FAULT_STORE_SLOT   0x1u  /* store_kv: out_loc[i] outside [0, num_slots) */
#define PKV_FAULT_LENGTH       0x2u  /* attention: a request's lengths are invalid */
#define PKV_FAULT_TABLE_SLOT   0x4u  /* attention: a page-table entry outside [0, num_slots); its key reads as a zero K and V row */
#define PKV_FAULT_TABLE_ROW    0x8u  /* attention: table_idx[r] outside [0, pt_rows) */
#define PKV_FAULT_QROWS        0x10u /* extend: sum of extend lengths exceeds total_q or max_extend */
#define PKV_FAULT_OUT_LOC      0x20u /* decode_store: page_table[t_r, S_r - 1] != out_loc[r] */

/*
 * One layer of the paged KV pool, token-granular view ([DISS] 4.4.3: the pool
 * tensor (2, layers, num_pages, page_size, kv_heads, head_dim) viewed per
 * layer as [num_pages * page_size, kv_heads, head_dim]; [CORE] Context: the
 * page table stores one slot per token whatever the page size).
 *   k, v        device, [num_slots, kv_heads, head_dim], 16-byte aligned.
 *   num_slots   (num_pages + 1) * page_size; the extra page is the dummy page
 *               padded requests write to ([ENG] 初始化的顺序).
 *   row_stride  elements between consecutive slots (>= kv_heads * head_dim,
 *               row_stride * itemsize a multiple of 16).
 *   page_size   tokens per page; slot = page * page_size + offset ([DISS] 4.6.4).
 *               The kernels read slots from the token-granular table, so any
 *               page_size >= 1 works.
 *   dtype       PKV_F32 or PKV_BF16; q, k, v and o of a call share it.
 */
typedef struct {
  void* k;
  void* v;
  int64_t num_slots;
  int64_t row_stride;
  int32_t kv_heads;
  int32_t head_dim;
  int32_t page_size;
  int32_t dtype;
} pkv_pool;

/*
 * store_kv ([DISS] 4.4.3 and 4.9.4; [DISS] 4.6.7: it runs before the attention
 * kernel of the same layer): for i in [0, n): pool.k[out_loc[i]] = k[i] and
 * pool.v[out_loc[i]] = v[i], each row kv_heads * head_dim elements copied
 * bit-for-bit.
 *   out_loc   device, [n] of int32 (loc_type PKV_I32) or int64 (PKV_I64).
 *             Slots must be unique except for the dummy slot, whose content
 *             is then unspecified. Out-of-range slots are skipped and flagged
 *             (PKV_FAULT_STORE_SLOT).
 *   k, v      device, [n, kv_heads, head_dim] in pool.dtype, rows k_stride /
 *             v_stride elements apart (strides * itemsize multiples of 16).
 *   n         rows to write; n == 0 is a no-op.
 */
int pkv_store_kv(const pkv_pool* pool, const void* out_loc, int32_t loc_type, int64_t n,
                 const void* k, int64_t k_stride, const void* v, int64_t v_stride,
                 void* stream);

/*
 * Embedding row gather of the vocab-parallel embedding ([DISS] 4.9.2-4.9.3:
 * VocabParallelEmbedding's indexing(weights, ids, vocab_range), the first op
 * of forward_batch). For i in [0, n):
 *   out[i] = weight[ids[i] - vocab_start]  if vocab_start <= ids[i] < vocab_end,
 *   out[i] = 0 (every element)             otherwise,
 * rows copied bit for bit, so the outputs of shards that partition the
 * vocabulary add up to the whole table's gather (reading of vocab_range: the
 * pages name it without spelling it out).
 *   weight    device, [weight_rows, hidden] of dtype (PKV_BF16 or PKV_F32), rows
 *             weight_stride elements apart, 16-byte aligned (unused if weight_rows == 0).
 *   ids       device, int32 [n]; any value is allowed (out of range -> zero row).
 *   out       device, [n, hidden] of dtype, rows out_stride elements apart.
 *   hidden * itemsize a multiple of 16 bytes; 0 <= vocab_start <= vocab_end and
 *   vocab_end - vocab_start <= weight_rows (PKV_ERR_SHAPE otherwise).
 */
int pkv_embedding_gather(const void* weight, int32_t dtype, int64_t weight_rows, int64_t weight_stride,
                         int32_t hidden, const int32_t* ids, int64_t n, int64_t vocab_start, int64_t vocab_end,
                         void* out, int64_t out_stride, void* stream);

/*
 * q/k norm + rotary embedding + store_kv, fused ([TINY] its rmsnorm and rope
 * operators and the layer function: Qwen3 normalises each q and k head with
 * its own weight, then rotates it; [DISS] 4.6.7: the layer does both in
 * place before the attention backend stores k and v). For token i in [0, n)
 * at position p = positions[i], every head vector x of 128 dims is
 *   y = w * x / sqrt(mean(x^2) + eps)          (w = q_norm_weight or k_norm_weight)
 *   y'[j] = y[j] cos(a_j) - y[j+64] sin(a_j),  y'[j+64] = y[j] sin(a_j) + y[j+64] cos(a_j),
 *   a_j = fp32(p) * f_j (an fp32 product),     f_j = fp32(1 / fp32(rope_theta^(2j/128))), j < 64;
 * q_out[i] = y' of every query head, pool.k[out_loc[i]] = y' of every KV
 * head, pool.v[out_loc[i]] = v[i] bit-for-bit. Arithmetic in fp32; q_out and
 * the K rows are rounded to nearest even into pool.dtype.
 *   out_loc   device, [n] of int32 (PKV_I32) or int64 (PKV_I64) slots; an
 *             out-of-range slot skips that token's K/V store and is flagged
 *             (PKV_FAULT_STORE_SLOT); its q_out row is still written.
 *   q, q_out  device, [n, num_q_heads, 128] in pool.dtype, token rows
 *             q_stride / q_out_stride elements apart (0 = dense). q_out may
 *             be q (in place); otherwise they must not overlap. Both NULL:
 *             the k side only (q then goes through the attention call's own
 *             prologue, pkv_q_norm_rope); num_q_heads and q_norm_weight are
 *             then ignored.
 *   k, v      device, [n, kv_heads, 128] in pool.dtype, rows k_stride / v_stride apart.
 *   positions device, int32 [n], absolute token positions (cached_len + t for
 *             the t-th new token of a request).
 *   q_norm_weight, k_norm_weight  device, [128] in pool.dtype, 16-byte aligned.
 *   eps >= 0, rope_theta > 1 (taken as the fp32 value passed).
 * num_q_heads <= 32 and kv_heads <= 16 (PKV_ERR_SHAPE above).
 */
int pkv_qk_norm_rope_store_kv(const pkv_pool* pool, const void* out_loc, int32_t loc_type, int64_t n,
                              const void* q, int64_t q_stride, void* q_out, int64_t q_out_stride,
                              int32_t num_q_heads, const void* k, int64_t k_stride, const void* v,
                              int64_t v_stride, const int32_t* positions, const void* q_norm_weight,
                              const void* k_norm_weight, float eps, float rope_theta, void* stream);

/*
 * Decode attention ([TINY] attention with one query row; [DISS] 4.6.5 decode
 * metadata). For request r (page-table row t_r = table_idx ? table_idx[r] : r)
 * with S_r = device_len[r] keys -- the new token's row already stored -- and
 * every query head h (KV head g = h / (num_q_heads / kv_heads)):
 *   s_j = sm_scale * q[r,h,:] . K[slot(r,j), g, :],  slot(r,j) = page_table[t_r * pt_stride + j],
 *   o[r,h,:] = sum_{j < S_r} softmax(s)_j V[slot(r,j), g, :].
 * cached_len is accepted for symmetry with extend (a decode row has
 * cached_len = device_len - 1) and is not read.
 *   q         device, [bs, num_q_heads, 128], token rows q_stride elements
 *             apart (0 = num_q_heads * 128).
 *   o         device, [bs, num_q_heads, 128], rows o_stride apart (0 = dense);
 *             same dtype as the pool, rounded to nearest-even for bf16.
 *   page_table device int32, pt_rows rows of pt_stride entries.
 *   device_len device int32 [bs]; 1 <= S_r <= pt_stride, else the row is
 *             zero-filled and flagged.
 *   max_total_kv host upper bound of sum(S_r); sizes the split-K plan.
 *   sm_scale  0 => 1/sqrt(head_dim); any other value, negative ones
 *             included, scales the scores as given (also for extend).
 *   ws        device workspace of at least pkv_decode_workspace_size(...) bytes
 *             for split-K partial results (no initialisation needed).
 */
int pkv_paged_attention_decode(const pkv_pool* pool, const void* q, int64_t q_stride,
                               void* o, int64_t o_stride, int32_t bs, int32_t num_q_heads,
                               const int32_t* page_table, int32_t pt_rows, int64_t pt_stride,
                               const int32_t* table_idx, const int32_t* cached_len,
                               const int32_t* device_len, int64_t max_total_kv, float sm_scale,
                               void* ws, size_t ws_bytes, void* stream);

size_t pkv_decode_workspace_size(int32_t bs, int32_t num_q_heads, int64_t max_total_kv);

/*
 * store_kv fused into decode attention: the decode step's store, then
 * attention ([DISS] 4.6.7: the new rows are stored before the layer's
 * attention reads them; 4.9.4 for the store), in one call. For every request
 * r with valid lengths:
 *   pool.k[out_loc[r]] = k[r], pool.v[out_loc[r]] = v[r] (rows copied bit for
 *   bit, as pkv_store_kv), and
 *   o[r] = decode attention as pkv_paged_attention_decode, with key S_r - 1
 *   taken from the new row k[r] / v[r] and keys j < S_r - 1 from the pool.
 * This is pkv_store_kv followed by pkv_paged_attention_decode, bit for bit,
 * whenever page_table[t_r, S_r - 1] == out_loc[r] and no other key of the
 * batch reads an out_loc slot -- what an engine that takes out_loc from the
 * page table's new entries has. A request whose table entry S_r - 1 is not
 * out_loc[r] still attends to its new row as key S_r - 1 and sets
 * PKV_FAULT_OUT_LOC; an out_loc[r] outside [0, num_slots) is not written and
 * sets PKV_FAULT_STORE_SLOT; a request skipped for an invalid length or table
 * row (its output zero-filled, PKV_FAULT_LENGTH or PKV_FAULT_TABLE_ROW) stores
 * nothing.
 *   out_loc   device, [bs] of int32 (loc_type PKV_I32) or int64 (PKV_I64).
 *   k, v      device, [bs, kv_heads, 128] in pool.dtype, rows k_stride /
 *             v_stride elements apart (0 = dense; strides * itemsize multiples
 *             of 16).
 * The other arguments, the workspace and the errors are those of
 * pkv_paged_attention_decode (k and v checked as in pkv_store_kv).
 */
int pkv_paged_attention_decode_store(const pkv_pool* pool, const void* out_loc, int32_t loc_type,
                                     const void* k, int64_t k_stride, const void* v, int64_t v_stride,
                                     const void* q, int64_t q_stride, void* o, int64_t o_stride, int32_t bs,
                                     int32_t num_q_heads, const int32_t* page_table, int32_t pt_rows,
                                     int64_t pt_stride, const int32_t* table_idx, const int32_t* cached_len,
                                     const int32_t* device_len, int64_t max_total_kv, float sm_scale,
                                     void* ws, size_t ws_bytes, void* stream);

/*
 * Qwen3's q prologue folded into attention ([TINY] its rmsnorm and rope
 * operators and the layer function, which normalise each q head with q_norm
 * and rotate it right before attention; [DISS] 4.6.7). With it, the attention
 * entry points below take the raw projected q and compute, for each query
 * head vector x of a token at absolute position p,
 *   y = w * x / sqrt(mean(x^2) + eps),  then the rotation of
 *   pkv_qk_norm_rope_store_kv (pairs j, j + 64 turned by fp32(p) * f_j),
 * in fp32, rounded to the pool dtype, before the dot products. p is
 * device_len - 1 for a decode row and cached_len + t for extend row t. The k
 * side goes through pkv_qk_norm_rope_store_kv with q = q_out = NULL.
 *   q_norm_weight  device, [128] in the pool dtype, 16-byte aligned.
 *   eps >= 0, rope_theta > 1.
 */
typedef struct {
  const void* q_norm_weight;
  float eps;
  float rope_theta;
} pkv_q_norm_rope;

/* pkv_paged_attention_decode with the q prologue (qnr must not be NULL). */
int pkv_paged_attention_decode_qnr(const pkv_pool* pool, const void* q, int64_t q_stride,
                                   void* o, int64_t o_stride, int32_t bs, int32_t num_q_heads,
                                   const int32_t* page_table, int32_t pt_rows, int64_t pt_stride,
                                   const int32_t* table_idx, const int32_t* cached_len,
                                   const int32_t* device_len, int64_t max_total_kv, float sm_scale,
                                   const pkv_q_norm_rope* qnr, void* ws, size_t ws_bytes, void* stream);

/*
 * Decode attention that allocates nothing, for callers that cannot allocate
 * device memory or pass a workspace: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc. Same arguments, kernels and
 * results as pkv_paged_attention_decode, without ws / ws_bytes: the split-K
 * partials go to a scratch array inside the library, one per GPU, of
 * PKV_NOALLOC_SCRATCH_BYTES bytes, held from the library's first call on that
 * GPU until the process ends. A call whose pkv_decode_workspace_size(bs,
 * num_q_heads, max_total_kv) exceeds it returns PKV_ERR_WORKSPACE before
 * anything is enqueued (16 MiB covers bs <= 768 at 16 query heads with any
 * max_total_kv). The call itself allocates nothing and calls no allocating
 * routine. Every call on one GPU shares that GPU's scratch: calls that can
 * overlap in time on one GPU (different streams, or concurrent host threads
 * on different streams) race and give wrong results; calls ordered on one
 * stream are safe. The scratch needs no initialisation (every byte a call
 * reads was written earlier in the same call).
 */
#define PKV_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int pkv_paged_attention_decode_noalloc(const pkv_pool* pool, const void* q, int64_t q_stride,
                                       void* o, int64_t o_stride, int32_t bs, int32_t num_q_heads,
                                       const int32_t* page_table, int32_t pt_rows, int64_t pt_stride,
                                       const int32_t* table_idx, const int32_t* cached_len,
                                       const int32_t* device_len, int64_t max_total_kv, float sm_scale,
                                       void* stream);

/*
 * Extend (causal prefill over a cached prefix; [TINY] attention with its
 * absolute-position causal mask; [DISS] 4.6.5 cu_seqlens_q as the exclusive
 * prefix sum of extend_len). Request r has C_r = cached_len[r] cached tokens
 * and S_r = device_len[r] tokens after this step (E_r = S_r - C_r query rows;
 * all S_r K/V rows, prefix and new, are read from the pool, so store_kv for
 * this step must precede the call). Query row t of request r sits at absolute
 * position C_r + t and attends to keys j <= C_r + t.
 *   q, o      device, ragged [total_q, num_q_heads, 128]: request r owns rows
 *             [sum_{r'<r} E_r', sum_{r'<=r} E_r'). Rows beyond sum(E) are
 *             not touched.
 *   cached_len, device_len device int32 [bs]; need 0 <= C_r < S_r <= pt_stride,
 *             E_r <= max_extend and sum(E) <= total_q, else the request is
 *             skipped (its output rows are not written) and flagged.
 *   total_q, max_extend host bounds of sum(E_r) and max(E_r).
 *   ws        bf16 pools: unused (may be NULL, ws_bytes 0). fp32 pools: device
 *             workspace of pkv_extend_workspace_size(bs, num_q_heads, total_q,
 *             PKV_F32) bytes, 16-byte aligned (no initialisation needed).
 * bf16 pools run the MFMA kernel. fp32 pools (an fp32 engine's prefill) run
 * every query row as a decode row of C_r + t + 1 keys over the request's
 * table row, through the decode kernels (fp32 throughout); total_q is then
 * limited to 4096 rows (PKV_ERR_SHAPE above).
 */
int pkv_paged_attention_extend(const pkv_pool* pool, const void* q, int64_t q_stride,
                               void* o, int64_t o_stride, int32_t bs, int32_t num_q_heads,
                               const int32_t* page_table, int32_t pt_rows, int64_t pt_stride,
                               const int32_t* table_idx, const int32_t* cached_len,
                               const int32_t* device_len, int64_t total_q, int32_t max_extend,
                               float sm_scale, void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes of pkv_paged_attention_extend for a pool of `dtype`: 0 for
 * PKV_BF16; for PKV_F32 the rows' decode lengths and a decode workspace (0 if
 * total_q is outside [1, 4096]). */
size_t pkv_extend_workspace_size(int32_t bs, int32_t num_q_heads, int64_t total_q, int32_t dtype);

/* pkv_paged_attention_extend with the q prologue (qnr must not be NULL). */
int pkv_paged_attention_extend_qnr(const pkv_pool* pool, const void* q, int64_t q_stride,
                                   void* o, int64_t o_stride, int32_t bs, int32_t num_q_heads,
                                   const int32_t* page_table, int32_t pt_rows, int64_t pt_stride,
                                   const int32_t* table_idx, const int32_t* cached_len,
                                   const int32_t* device_len, int64_t total_q, int32_t max_extend,
                                   float sm_scale, const pkv_q_norm_rope* qnr, void* ws, size_t ws_bytes,
                                   void* stream);

/*
 * Batched sampler ([ENG] 采样器; [SRC4] 14.3-14.4; [DISS] 4.8.4-4.8.6).
 *   logits    device, [bs, vocab] of logits_dtype (PKV_BF16 or PKV_F32), rows
 *             row_stride elements apart, 16-byte aligned rows. Finite values.
 *   temperature device float [bs], or NULL: the whole batch is greedy and
 *             every row is argmax (ties -> lowest index).
 *   top_k     device int32 [bs] or NULL; top_k <= 0 or >= vocab: no top-k.
 *   top_p     device float [bs] or NULL; top_p >= 1: no top-p; else clamped
 *             to >= 1e-6.
 *   min_p     device float [bs] or NULL ([ENG] 练习 and its answer); min_p <= 0:
 *             no min_p; values above 1 act as 1.
 *   uniforms  device float [bs], u in [0, 1); may be NULL iff temperature is NULL.
 *   out_tokens device int32 [bs].
 * Row semantics when temperature is given: temperature <= 1e-6 -> argmax of
 * the logits (ties -> lowest index). Otherwise p ~ softmax(logits / T);
 * tokens ranked by logit (ties -> lower index first); top-k keeps ranks < k;
 * top-p keeps a ranked token iff the renormalised kept mass before it is
 * < top_p (the first token always survives); top-k is applied before top-p.
 * min_p keeps a token iff its probability is at least min_p times the
 * largest probability of the row (on the full tempered distribution, not the
 * renormalised top-k set); the kept set is the intersection of that set with
 * the top-k / top-p set (both are prefixes of the ranking, so the first
 * token always survives).
 * The draw scans the kept tokens in vocabulary order and returns the first
 * whose running kept mass exceeds u * (total kept mass) (the last kept token
 * if rounding finds none).
 *   ws        device workspace of pkv_sample_workspace_size(bs, vocab) bytes,
 *             16-byte aligned; required (per-slice records and masses, and
 *             the key histograms of bf16 rows or the candidate lists of fp32
 *             rows, written by the first of two kernels and read by the
 *             second; the size covers both dtypes). Its
 *             contents need no initialisation and are not kept between
 *             calls; calls that share a workspace must not overlap in time
 *             (different streams race). PKV_ERR_WORKSPACE if missing or
 *             short, PKV_ERR_ALIGN if misaligned. vocab is limited to 2^20
 *             tokens (PKV_ERR_SHAPE above).
 */
int pkv_sample(const void* logits, int32_t logits_dtype, int32_t bs, int32_t vocab,
               int64_t row_stride, const float* temperature, const int32_t* top_k,
               const float* top_p, const float* min_p, const float* uniforms,
               int32_t* out_tokens, void* ws, size_t ws_bytes, void* stream);

size_t pkv_sample_workspace_size(int32_t bs, int32_t vocab);

/* ------------------------------------------------------------------ host-only helpers */

/*
 * KV pool page count ([ENG] 显存规划; [DISS] 5.2): bytes per page =
 * 2 * head_dim * kv_heads_per_rank * page_size * itemsize * num_layers;
 * available = (int64)(memory_ratio * free_before) - model_bytes;
 * pages = available / bytes per page. kv_heads_per_rank = kv_heads / tp_size
 * (or 1 when tp_size > kv_heads, replicated). Returns the page count, or a
 * negative pkv_status: PKV_ERR_SHAPE for bad sizes, PKV_ERR_LENGTHS when
 * fewer than two pages fit ("Not enough memory for KV cache").
 */
int64_t pkv_num_pages(int32_t head_dim, int32_t kv_heads, int32_t tp_size, int32_t page_size,
                      int32_t itemsize, int32_t num_layers, int64_t free_before,
                      int64_t model_bytes, double memory_ratio);

/*
 * Batch sampling arguments from per-request parameters ([ENG] 采样器,
 * Sampler.prepare; [CORE] SamplingParams.is_greedy). Inputs: n requests'
 * temperature T[i], top_k K[i], top_p P[i] (host arrays). A request is greedy
 * iff (T <= 0 or K == 1) and P == 1. Outputs (host arrays of n):
 *   T_out = max(greedy ? 0 : T, 1e-6), K_out = K >= 1 ? K : vocab,
 *   P_out = min(max(P, 1e-6), 1).
 * *flags receives PKV_PREP_ALL_GREEDY (pass temperature = NULL to pkv_sample),
 * PKV_PREP_USE_TOP_K (some K_out != vocab) and PKV_PREP_USE_TOP_P (some
 * P_out < 1); arrays whose flag is clear may be passed as NULL.
 * Returns PKV_OK or PKV_ERR_NULL / PKV_ERR_SHAPE.
 */
#define PKV_PREP_ALL_GREEDY 0x1
#define PKV_PREP_USE_TOP_K 0x2
#define PKV_PREP_USE_TOP_P 0x4
int pkv_prepare_sampling(int32_t n, const float* T, const int32_t* K, const float* P,
                         int32_t vocab, float* T_out, int32_t* K_out, float* P_out,
                         int32_t* flags);

/*
 * Reads and clears the current device's fault word (PKV_FAULT_* bits set by
 * kernels that met out-of-range data). Synchronises `stream` first.
 */
int pkv_read_faults(void* stream, uint32_t* faults);

/* Message for the last non-zero status returned on this thread ("" if none). */
const char* pkv_last_error(void);

/* Library version string. */
const char* pkv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
