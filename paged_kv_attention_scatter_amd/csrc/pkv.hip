// libpkv: host side of the C ABI declared in include/pkv.h.
//
// Every entry point validates its arguments on the host (returning a
// negative pkv_status before anything is enqueued), then launches the gfx950
// kernels on the caller's stream. The library allocates no device memory;
// the only device state it owns is the 4-byte fault word below.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "pkv.h"
#include "common.hpp"
#include "store_kv.hpp"
#include "qk_rope.hpp"
#include "embed.hpp"
#include "decode.hpp"
#include "extend.hpp"
#include "sample.hpp"

// Kernels OR PKV_FAULT_* bits into this word when they meet out-of-range data.
__device__ uint32_t pkv_fault_word;

// Device scratch of the entry points that allocate nothing (the *_noalloc
// variants): one copy per GPU, held until the process ends. On the host this
// name is only a stand-in, not a device address: kernels get the per-device
// address that hipGetSymbolAddress returns (DeviceState::scratch) instead.
constexpr size_t kScratchBytes = PKV_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch regions are 256-byte aligned");
__device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return PKV_OK;
}

constexpr int kMaxDevices = 64;

struct DeviceState {
  bool init = false;
  int status = PKV_OK;
  uint32_t* faults = nullptr;  // device address of pkv_fault_word on this device
  void* scratch = nullptr;     // device address of `scratch` on this device
  int num_cus = 0;
};

std::mutex g_dev_mutex;
DeviceState g_dev[kMaxDevices];

// Per-device set-up: check the part is gfx950 and resolve the fault word's
// device address (the symbol's host-side name is not a device pointer).
int device_state(DeviceState** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(PKV_ERR_DEVICE, "device index %d unsupported", dev);
  std::lock_guard<std::mutex> lock(g_dev_mutex);
  DeviceState& s = g_dev[dev];
  if (!s.init) {
    s.init = true;
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) {
      s.status = PKV_ERR_HIP;
    } else if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) {
      s.status = PKV_ERR_DEVICE;
    } else {
      s.num_cus = prop.multiProcessorCount;
      void* p = nullptr;
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(pkv_fault_word));
      if (e != hipSuccess) s.status = PKV_ERR_HIP;
      else s.faults = static_cast<uint32_t*>(p);
      void* sp = nullptr;
      if (s.status == PKV_OK) {
        e = hipGetSymbolAddress(&sp, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !sp) s.status = PKV_ERR_HIP;
        else s.scratch = sp;
      }
    }
  }
  if (s.status != PKV_OK)
    return fail(s.status, "device %d unusable (needs gfx950; HIP set-up failed or wrong arch)", dev);
  *out = &s;
  return PKV_OK;
}

int check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "%s launch: %s", what, hipGetErrorString(e));
  return ok();
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int itemsize(int32_t dtype) { return dtype == PKV_BF16 ? 2 : (dtype == PKV_F32 ? 4 : 0); }

// Validates the pool descriptor; on success *isz is the element size.
int check_pool(const pkv_pool* pool, int* isz) {
  if (!pool) return fail(PKV_ERR_NULL, "pool is NULL");
  if (!pool->k || !pool->v) return fail(PKV_ERR_NULL, "pool.k / pool.v is NULL");
  *isz = itemsize(pool->dtype);
  if (!*isz) return fail(PKV_ERR_DTYPE, "pool.dtype %d is not PKV_F32 or PKV_BF16", pool->dtype);
  if (pool->head_dim != pkv::kHeadDim)
    return fail(PKV_ERR_SHAPE, "head_dim %d unsupported (must be 128)", pool->head_dim);
  if (pool->kv_heads < 1 || pool->kv_heads > 64)
    return fail(PKV_ERR_SHAPE, "kv_heads %d out of range", pool->kv_heads);
  if (pool->num_slots < 1) return fail(PKV_ERR_SHAPE, "num_slots %lld < 1", (long long)pool->num_slots);
  if (pool->page_size < 1) return fail(PKV_ERR_SHAPE, "page_size %d < 1", pool->page_size);
  const int64_t row = (int64_t)pool->kv_heads * pool->head_dim;
  if (pool->row_stride < row)
    return fail(PKV_ERR_SHAPE, "row_stride %lld < kv_heads * head_dim %lld",
                (long long)pool->row_stride, (long long)row);
  if (!aligned16(pool->k) || !aligned16(pool->v) || (pool->row_stride * *isz) % 16)
    return fail(PKV_ERR_ALIGN, "pool pointers and row_stride * itemsize must be 16-byte aligned");
  return PKV_OK;
}

int check_rows(const void* p, int64_t stride, int64_t min_stride, int isz, const char* name) {
  if (!p) return fail(PKV_ERR_NULL, "%s is NULL", name);
  if (stride < min_stride)
    return fail(PKV_ERR_SHAPE, "%s row stride %lld < %lld", name, (long long)stride, (long long)min_stride);
  if (!aligned16(p) || (stride * isz) % 16)
    return fail(PKV_ERR_ALIGN, "%s pointer and row stride * itemsize must be 16-byte aligned", name);
  return PKV_OK;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// 1 / theta^(2j/128) for j < 64: the power in fp64 rounded to fp32, then an
// fp32 division (kept per host thread for the last theta, a pure function of
// it), as the step-0 page's fp32 tensors compute it.
void rope_inv_freq(float rope_theta, float (&out)[pkv::kHeadDim / 2]) {
  thread_local float freq_theta = 0.f;
  thread_local float freq[pkv::kHeadDim / 2];
  if (freq_theta != rope_theta) {
    for (int j = 0; j < pkv::kHeadDim / 2; ++j) {
      const float p = (float)std::pow((double)rope_theta, (double)(2 * j) / (double)pkv::kHeadDim);
      freq[j] = 1.0f / p;
    }
    freq_theta = rope_theta;
  }
  std::memcpy(out, freq, sizeof freq);
}

// Validates the q prologue descriptor of the *_qnr entry points.
int check_qnr(const pkv_q_norm_rope* qnr) {
  if (!qnr || !qnr->q_norm_weight) return fail(PKV_ERR_NULL, "q prologue or its q_norm_weight is NULL");
  if (!aligned16(qnr->q_norm_weight)) return fail(PKV_ERR_ALIGN, "q_norm_weight must be 16-byte aligned");
  if (!(qnr->eps >= 0.f) || !(qnr->rope_theta > 1.f))
    return fail(PKV_ERR_SHAPE, "need eps >= 0 and rope_theta > 1 (eps %g, rope_theta %g)", qnr->eps,
                qnr->rope_theta);
  return PKV_OK;
}

}  // namespace

extern "C" {

const char* pkv_last_error(void) { return g_err.c_str(); }

const char* pkv_version(void) { return "pkv 0.1 (gfx950)"; }

int pkv_read_faults(void* stream, uint32_t* faults) {
  if (!faults) return fail(PKV_ERR_NULL, "faults is NULL");
  DeviceState* ds;
  int rc = device_state(&ds);
  if (rc) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint32_t v = 0;
  hipError_t e = hipMemcpyAsync(&v, ds->faults, sizeof v, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipMemsetAsync(ds->faults, 0, sizeof v, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "reading the fault word: %s", hipGetErrorString(e));
  *faults = v;
  return ok();
}

int pkv_store_kv(const pkv_pool* pool, const void* out_loc, int32_t loc_type, int64_t n,
                 const void* k, int64_t k_stride, const void* v, int64_t v_stride, void* stream) {
  int isz = 0;
  int rc = check_pool(pool, &isz);
  if (rc) return rc;
  if (n < 0) return fail(PKV_ERR_SHAPE, "n = %lld < 0", (long long)n);
  if (loc_type != PKV_I32 && loc_type != PKV_I64)
    return fail(PKV_ERR_DTYPE, "loc_type %d is not PKV_I32 or PKV_I64", loc_type);
  if (n == 0) return ok();
  if (!out_loc) return fail(PKV_ERR_NULL, "out_loc is NULL");
  const int64_t row = (int64_t)pool->kv_heads * pool->head_dim;
  if ((rc = check_rows(k, k_stride, row, isz, "k"))) return rc;
  if ((rc = check_rows(v, v_stride, row, isz, "v"))) return rc;
  DeviceState* ds;
  if ((rc = device_state(&ds))) return rc;
  constexpr int PK = 4;
  const int32_t packets = (int32_t)(row * isz / 16);
  const int64_t threads = n * (packets / PK);
  const int64_t blocks = (threads + 255) / 256;
  if (blocks > 0x7fffffffLL) return fail(PKV_ERR_SHAPE, "n = %lld too large", (long long)n);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t pool_pk = pool->row_stride * isz / 16, k_pk = k_stride * isz / 16, v_pk = v_stride * isz / 16;
  pkv::u32x4* kp = static_cast<pkv::u32x4*>(pool->k);
  pkv::u32x4* vp = static_cast<pkv::u32x4*>(pool->v);
  if (loc_type == PKV_I32)
    hipLaunchKernelGGL((pkv::store_kv_kernel<int32_t, PK>), dim3((uint32_t)blocks), dim3(256), 0, s, kp, vp,
                       pool_pk, pool->num_slots, static_cast<const int32_t*>(out_loc), n,
                       static_cast<const pkv::u32x4*>(k), k_pk, static_cast<const pkv::u32x4*>(v), v_pk, packets,
                       ds->faults);
  else
    hipLaunchKernelGGL((pkv::store_kv_kernel<int64_t, PK>), dim3((uint32_t)blocks), dim3(256), 0, s, kp, vp,
                       pool_pk, pool->num_slots, static_cast<const int64_t*>(out_loc), n,
                       static_cast<const pkv::u32x4*>(k), k_pk, static_cast<const pkv::u32x4*>(v), v_pk, packets,
                       ds->faults);
  return check_launch("store_kv");
}

int pkv_embedding_gather(const void* weight, int32_t dtype, int64_t weight_rows, int64_t weight_stride,
                         int32_t hidden, const int32_t* ids, int64_t n, int64_t vocab_start, int64_t vocab_end,
                         void* out, int64_t out_stride, void* stream) {
  const int isz = itemsize(dtype);
  if (!isz) return fail(PKV_ERR_DTYPE, "dtype %d is not PKV_F32 or PKV_BF16", dtype);
  if (n < 0 || hidden < 1 || weight_rows < 0)
    return fail(PKV_ERR_SHAPE, "need n >= 0, hidden >= 1, weight_rows >= 0 (%lld, %d, %lld)", (long long)n, hidden,
                (long long)weight_rows);
  if (((int64_t)hidden * isz) % 16)
    return fail(PKV_ERR_SHAPE, "hidden * itemsize = %lld is not a multiple of 16 bytes", (long long)hidden * isz);
  if (vocab_start < 0 || vocab_end < vocab_start || vocab_end - vocab_start > weight_rows)
    return fail(PKV_ERR_SHAPE, "vocab range [%lld, %lld) does not fit %lld weight rows", (long long)vocab_start,
                (long long)vocab_end, (long long)weight_rows);
  if (n == 0) return ok();
  if (!ids) return fail(PKV_ERR_NULL, "ids is NULL");
  int rc;
  if (weight_rows > 0 && (rc = check_rows(weight, weight_stride, hidden, isz, "weight"))) return rc;
  if ((rc = check_rows(out, out_stride, hidden, isz, "out"))) return rc;
  DeviceState* ds;
  if ((rc = device_state(&ds))) return rc;
  const int32_t packets = (int32_t)((int64_t)hidden * isz / 16);
  const int pk = packets % 4 == 0 ? 4 : (packets % 2 == 0 ? 2 : 1);
  const int64_t threads = n * (packets / pk);
  const int64_t blocks = (threads + 255) / 256;
  if (blocks > 0x7fffffffLL) return fail(PKV_ERR_SHAPE, "n = %lld too large", (long long)n);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const pkv::u32x4* w = static_cast<const pkv::u32x4*>(weight);
  pkv::u32x4* o = static_cast<pkv::u32x4*>(out);
  const int64_t w_pk = weight_stride * isz / 16, o_pk = out_stride * isz / 16;
  if (weight_rows == 0) vocab_end = vocab_start;  // every id is outside the shard
  if (pk == 4)
    hipLaunchKernelGGL(pkv::embed_gather_kernel<4>, dim3((uint32_t)blocks), dim3(256), 0, s, w, w_pk, ids, n,
                       vocab_start, vocab_end, o, o_pk, packets);
  else if (pk == 2)
    hipLaunchKernelGGL(pkv::embed_gather_kernel<2>, dim3((uint32_t)blocks), dim3(256), 0, s, w, w_pk, ids, n,
                       vocab_start, vocab_end, o, o_pk, packets);
  else
    hipLaunchKernelGGL(pkv::embed_gather_kernel<1>, dim3((uint32_t)blocks), dim3(256), 0, s, w, w_pk, ids, n,
                       vocab_start, vocab_end, o, o_pk, packets);
  (void)ds;
  return check_launch("embedding_gather");
}

int pkv_qk_norm_rope_store_kv(const pkv_pool* pool, const void* out_loc, int32_t loc_type, int64_t n,
                              const void* q, int64_t q_stride, void* q_out, int64_t q_out_stride,
                              int32_t num_q_heads, const void* k, int64_t k_stride, const void* v,
                              int64_t v_stride, const int32_t* positions, const void* q_norm_weight,
                              const void* k_norm_weight, float eps, float rope_theta, void* stream) {
  int isz = 0;
  int rc = check_pool(pool, &isz);
  if (rc) return rc;
  if (n < 0) return fail(PKV_ERR_SHAPE, "n = %lld < 0", (long long)n);
  if (loc_type != PKV_I32 && loc_type != PKV_I64)
    return fail(PKV_ERR_DTYPE, "loc_type %d is not PKV_I32 or PKV_I64", loc_type);
  const bool with_q = q != nullptr || q_out != nullptr;
  if (!with_q) num_q_heads = 0;  // k side only
  if (with_q && (num_q_heads < 1 || num_q_heads % pool->kv_heads))
    return fail(PKV_ERR_SHAPE, "num_q_heads %d is not a positive multiple of kv_heads %d", num_q_heads,
                pool->kv_heads);
  if (num_q_heads > 32 || pool->kv_heads > 16)
    return fail(PKV_ERR_SHAPE, "qk norm/rope supports up to 32 query and 16 KV heads (%d, %d)", num_q_heads,
                pool->kv_heads);
  if (!(eps >= 0.f) || !(rope_theta > 1.f))
    return fail(PKV_ERR_SHAPE, "need eps >= 0 and rope_theta > 1 (eps %g, rope_theta %g)", eps, rope_theta);
  if (n == 0) return ok();
  if (!out_loc || !positions) return fail(PKV_ERR_NULL, "out_loc / positions is NULL");
  if ((with_q && !q_norm_weight) || !k_norm_weight) return fail(PKV_ERR_NULL, "a norm weight is NULL");
  if ((with_q && !aligned16(q_norm_weight)) || !aligned16(k_norm_weight))
    return fail(PKV_ERR_ALIGN, "norm weights must be 16-byte aligned");
  const int64_t qrow = (int64_t)num_q_heads * pkv::kHeadDim, kvrow = (int64_t)pool->kv_heads * pkv::kHeadDim;
  if (with_q) {
    if (q_stride == 0) q_stride = qrow;
    if (q_out_stride == 0) q_out_stride = qrow;
    if ((rc = check_rows(q, q_stride, qrow, isz, "q"))) return rc;
    if ((rc = check_rows(q_out, q_out_stride, qrow, isz, "q_out"))) return rc;
  } else {
    q_norm_weight = k_norm_weight;  // never read (no query heads)
  }
  if ((rc = check_rows(k, k_stride, kvrow, isz, "k"))) return rc;
  if ((rc = check_rows(v, v_stride, kvrow, isz, "v"))) return rc;
  constexpr int TPB = pkv::kQkRopeThreads / pkv::kWave;  // tokens per workgroup
  const int64_t blocks = (n + TPB - 1) / TPB;
  if (blocks > 0x7fffffffLL) return fail(PKV_ERR_SHAPE, "n = %lld too large", (long long)n);
  DeviceState* ds;
  if ((rc = device_state(&ds))) return rc;
  pkv::QkRopeArgs a;
  a.k_pool = pool->k;
  a.v_pool = pool->v;
  a.pool_row = pool->row_stride;
  a.num_slots = pool->num_slots;
  a.out_loc = out_loc;
  a.n = n;
  a.q = q;
  a.q_stride = q_stride;
  a.q_out = q_out;
  a.q_out_stride = q_out_stride;
  a.k = k;
  a.k_stride = k_stride;
  a.v = v;
  a.v_stride = v_stride;
  a.positions = positions;
  a.q_w = q_norm_weight;
  a.k_w = k_norm_weight;
  a.hq = num_q_heads;
  a.hkv = pool->kv_heads;
  a.eps = eps;
  rope_inv_freq(rope_theta, a.inv_freq);
  a.faults = ds->faults;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int mq = std::max(1, (num_q_heads + 3) / 4), mk = (pool->kv_heads + 3) / 4;
  const bool i64 = loc_type == PKV_I64;
#define PKV_QKR_LAUNCH(T, MQ, MK)                                                                               \
  hipLaunchKernelGGL(i64 ? (pkv::qk_rope_store_kernel<T, int64_t, MQ, MK>) : (pkv::qk_rope_store_kernel<T, int32_t, MQ, MK>), \
                     dim3((uint32_t)blocks), dim3(pkv::kQkRopeThreads), 0, s, a)
#define PKV_QKR_MK(T, MQ)                  \
  if (mk <= 1) PKV_QKR_LAUNCH(T, MQ, 1);   \
  else if (mk <= 2) PKV_QKR_LAUNCH(T, MQ, 2); \
  else PKV_QKR_LAUNCH(T, MQ, 4);
#define PKV_QKR_MQ(T)                     \
  if (mq <= 1) { PKV_QKR_MK(T, 1) }       \
  else if (mq <= 2) { PKV_QKR_MK(T, 2) }  \
  else if (mq <= 4) { PKV_QKR_MK(T, 4) }  \
  else { PKV_QKR_MK(T, 8) }
  if (pool->dtype == PKV_BF16) {
    PKV_QKR_MQ(pkv::bf16_t)
  } else {
    PKV_QKR_MQ(float)
  }
#undef PKV_QKR_MQ
#undef PKV_QKR_MK
#undef PKV_QKR_LAUNCH
  return check_launch("qk_norm_rope_store_kv");
}

// ------------------------------------------------------------------ host-only helpers

int64_t pkv_num_pages(int32_t head_dim, int32_t kv_heads, int32_t tp_size, int32_t page_size,
                      int32_t itemsize, int32_t num_layers, int64_t free_before, int64_t model_bytes,
                      double memory_ratio) {
  if (head_dim < 1 || kv_heads < 1 || tp_size < 1 || page_size < 1 || itemsize < 1 || num_layers < 1)
    return fail(PKV_ERR_SHAPE, "sizes must be positive");
  int64_t heads;
  if (kv_heads >= tp_size) {
    if (kv_heads % tp_size) return fail(PKV_ERR_SHAPE, "kv_heads %d not divisible by tp %d", kv_heads, tp_size);
    heads = kv_heads / tp_size;
  } else {
    if (tp_size % kv_heads) return fail(PKV_ERR_SHAPE, "tp %d not a multiple of kv_heads %d", tp_size, kv_heads);
    heads = 1;
  }
  const int64_t per_page = 2LL * head_dim * heads * page_size * itemsize * num_layers;
  const int64_t available = (int64_t)(memory_ratio * (double)free_before) - model_bytes;
  const int64_t n = available >= 0 ? available / per_page : -1;
  if (n <= 1) return fail(PKV_ERR_LENGTHS, "Not enough memory for KV cache (%lld pages)", (long long)n);
  ok();
  return n;
}

int pkv_prepare_sampling(int32_t n, const float* T, const int32_t* K, const float* P, int32_t vocab,
                         float* T_out, int32_t* K_out, float* P_out, int32_t* flags) {
  if (n < 0 || vocab < 1) return fail(PKV_ERR_SHAPE, "n must be >= 0 and vocab >= 1");
  if (!flags || (n > 0 && (!T || !K || !P || !T_out || !K_out || !P_out)))
    return fail(PKV_ERR_NULL, "a required array is NULL");
  const float kMin = 1e-6f;
  bool all_greedy = true, use_k = false, use_p = false;
  for (int32_t i = 0; i < n; ++i) {
    const bool greedy = (T[i] <= 0.f || K[i] == 1) && P[i] == 1.f;
    all_greedy = all_greedy && greedy;
    T_out[i] = std::fmax(greedy ? 0.f : T[i], kMin);
    K_out[i] = K[i] >= 1 ? K[i] : vocab;
    P_out[i] = std::fmin(std::fmax(P[i], kMin), 1.f);
    use_k = use_k || K_out[i] != vocab;
    use_p = use_p || P_out[i] < 1.f;
  }
  *flags = (all_greedy ? PKV_PREP_ALL_GREEDY : 0) | (use_k ? PKV_PREP_USE_TOP_K : 0) |
           (use_p ? PKV_PREP_USE_TOP_P : 0);
  return ok();
}

}  // extern "C"

// Entry points whose host code lives next to their kernels.
#include "decode_host.inc"
#include "extend_host.inc"
#include "sample_host.inc"
