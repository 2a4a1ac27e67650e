// Paged GQA decode attention: split-K over a flattened key space.
//
// Definition ("第 0 步：一个能跑的最小推理引擎", the dense attention function,
// with one query row): query head h of request r reads KV head
// g = h / (HQ / HKV); s_j = scale * q . K[slot(r, j)] over the request's
// device_len keys; o = softmax(s) . V. The slots come from the request's row
// of the token-granular page table ("核心数据结构：Req、Batch、Context",
// section Context).
//
// Work split (an intra-GPU split-KV, not the pages' design, which calls
// FlashInfer's decode kernel): the keys of all requests are laid end to end
// (cu = exclusive prefix sum of device_len) and cut into P equal items, so the
// work per workgroup is the same whatever the length mix. Item i covers keys
// [i*T/P, (i+1)*T/P). A request cut by item boundaries yields one partial
// (running max m, sum l, unnormalised accumulator) per item it touches,
// stored at partial slot (item + request); a second kernel merges them. A
// request that lies inside one item is finished in place.
//
// Inside an item, each of the NWAVE waves takes a contiguous quarter of the
// segment's keys. One token row of the pool (all HKV heads x 128 dims, 2 KiB
// in bf16) is read by one wave: lane l covers KV head l / (64 / HKV) and
// DPL = 2 * HKV consecutive dims, so every load instruction moves one whole
// row, coalesced, whatever the slot. The q.K partial dot of a lane is
// reduced over the 64 / HKV lanes of its head with DPP. Each lane keeps the
// online-softmax state of its head's G query heads for its dims; the waves of
// the workgroup merge through LDS at the end of a segment. No LDS staging of
// K/V: every K/V element is used by exactly one wave.
#pragma once

#include "common.hpp"

namespace pkv {

typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));

struct DecodeArgs {
  const void* k_pool;
  const void* v_pool;
  int64_t pool_row;     // elements between slots
  int64_t num_slots;
  const void* q;
  int64_t q_stride;     // elements between query tokens
  void* o;
  int64_t o_stride;
  int32_t bs;
  int32_t num_items;    // workgroups launched: the plan's items for max_total_kv
  const int32_t* page_table;
  int32_t pt_rows;
  int64_t pt_stride;
  const int32_t* table_idx;
  const int32_t* device_len;
  float scale_log2;     // sm_scale * log2(e)
  float* part_ml;       // [P + bs][HQ][2]  (m in log2 units, l)
  float* part_acc;      // [P + bs][HQ][128]
  int32_t* cu_out;      // [bs + 1] prefix of valid lengths (written by block 0)
  uint32_t* faults;
  // q prologue (Qwen3's q_norm + rotary embedding), or q_w == nullptr
  const void* q_w;      // [128] norm weight, element type T
  float q_eps;
  float inv_freq[64];   // fp32 rotary frequencies 1 / theta^(2j / 128)
  // rows of device_len 0 are no rows at all (skipped without a fault, their
  // output untouched): the padding of the extend rows run as decode rows
  int32_t skip_empty;
  // store_kv fused in (k_new == nullptr: no store): key S - 1 of request r is
  // the new row k_new[r] / v_new[r], which the wave that reads it also writes
  // to pool slot out_loc[r]
  const void* k_new;
  const void* v_new;
  int64_t kn_stride;    // elements between new rows
  int64_t vn_stride;
  const void* out_loc;  // [bs] int32, or int64 when loc64
  int32_t loc64;
};

template <typename T>
struct ElemTraits;
template <>
struct ElemTraits<bf16_t> {
  static constexpr int kPerWord = 2;
};
template <>
struct ElemTraits<float> {
  static constexpr int kPerWord = 1;
};

// The split plan: 256-key items, at most kDecodeMaxItems; a batch too small
// to fill the chip that way gets up to kDecodeSmallItems smaller items of at
// least kDecodeMinKeysPerItem keys, so one long request spreads over many CUs. The host sizes
// the grid with it from its bound on the total; the kernels recompute it from
// the actual total (never more than the grid), so a loose bound -- a graph
// captured for the largest batch it replays -- still splits the real keys.
constexpr int kDecodeMaxItems = 1024;     // 256 CUs x 4 resident workgroups
constexpr int kDecodeKeysPerItem = 256;
constexpr int kDecodeSmallItems = 512;
constexpr int kDecodeMinKeysPerItem = 32;

__host__ __device__ inline int decode_num_items(int64_t total, int cap) {
  int64_t p = (total + kDecodeKeysPerItem - 1) / kDecodeKeysPerItem;
  int64_t small = (total + kDecodeMinKeysPerItem - 1) / kDecodeMinKeysPerItem;
  if (small > kDecodeSmallItems) small = kDecodeSmallItems;
  if (p < small) p = small;
  if (p > cap) p = cap;
  if (p < 1) p = 1;
  return (int)p;
}

// Item containing flattened key position p (largest i with floor(i*T/P) <= p).
__device__ __forceinline__ int item_of(int64_t p, int64_t T, int P) {
  return (int)(((p + 1) * (int64_t)P - 1) / T);
}
__device__ __forceinline__ int64_t item_begin(int i, int64_t T, int P) {
  return ((int64_t)i * T) / P;
}

template <typename T, int NWD>
__device__ __forceinline__ void load_lane_row(uint32_t (&w)[NWD], const T* base) {
  // NWD words = NWD * 4 bytes, 16-byte aligned (DPL * sizeof(T) >= 16 for the
  // supported shapes).
  // Plain loads: with the caches cold (each row read once per step), they
  // measured about 1% faster at bs 256 than non-temporal ones, and more on
  // small batches.
  const u32x4* p = reinterpret_cast<const u32x4*>(base);
#pragma unroll
  for (int i = 0; i < NWD / 4; ++i) {
    u32x4 x = p[i];
    w[4 * i + 0] = x.x;
    w[4 * i + 1] = x.y;
    w[4 * i + 2] = x.z;
    w[4 * i + 3] = x.w;
  }
}

template <int NWD>
__device__ __forceinline__ void store_lane_row(void* base, const uint32_t (&w)[NWD]) {
  u32x4* p = reinterpret_cast<u32x4*>(base);
#pragma unroll
  for (int i = 0; i < NWD / 4; ++i) p[i] = u32x4{w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]};
}

template <typename T, int NWD>
__device__ __forceinline__ float lane_dot(const uint32_t (&qw)[NWD], const uint32_t (&kw)[NWD]) {
  float s = 0.f;
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int i = 0; i < NWD; ++i)
      s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_v, qw[i]),
                                          __builtin_bit_cast(bf16x2_v, kw[i]), s, false);
  } else {
#pragma unroll
    for (int i = 0; i < NWD; ++i) s = fmaf(__uint_as_float(qw[i]), __uint_as_float(kw[i]), s);
  }
  return s;
}

template <typename T, int NWD>
__device__ __forceinline__ void lane_axpy(float (&acc)[NWD * ElemTraits<T>::kPerWord], float p,
                                          const uint32_t (&vw)[NWD]) {
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int i = 0; i < NWD; ++i) {
      acc[2 * i] = fmaf(p, bf16_lo(vw[i]), acc[2 * i]);
      acc[2 * i + 1] = fmaf(p, bf16_hi(vw[i]), acc[2 * i + 1]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < NWD; ++i) acc[i] = fmaf(p, __uint_as_float(vw[i]), acc[i]);
  }
}

template <typename T>
__device__ __forceinline__ void store_out(T* o, float x);
template <>
__device__ __forceinline__ void store_out<bf16_t>(bf16_t* o, float x) {
  *o = (bf16_t)f32_to_bf16_bits(x);
}
template <>
__device__ __forceinline__ void store_out<float>(float* o, float x) {
  *o = x;
}

// The q prologue of the fused path ("第 0 步：一个能跑的最小推理引擎": the
// layer's q_norm, then rope at the token's position; "Mini-SGLang 完整剖析"
// section 4.6.7): this lane's DPL dims of one query head, normalised over the
// head (a sum over its LPH lanes), times the norm weight, then rotated: dims
// j < 64 and j + 64 form a pair turned by pos * inv_freq[j], the other
// member held by the lane LPH / 2 away. Arithmetic in fp32, the result in T.
template <typename T, int LPH, int DPL, int NWD>
__device__ __forceinline__ void q_norm_rope(uint32_t (&qw)[NWD], const DecodeArgs& a, int dofs, float pos) {
  constexpr int EPW = ElemTraits<T>::kPerWord;
  float x[DPL], w[DPL];
#pragma unroll
  for (int i = 0; i < NWD; ++i) {
    if constexpr (EPW == 2) {
      x[2 * i] = bf16_lo(qw[i]);
      x[2 * i + 1] = bf16_hi(qw[i]);
    } else {
      x[i] = __uint_as_float(qw[i]);
    }
  }
  const T* wp = reinterpret_cast<const T*>(a.q_w) + dofs;
#pragma unroll
  for (int d = 0; d < DPL; ++d) {
    if constexpr (EPW == 2) w[d] = bf16_to_f32(wp[d]);
    else w[d] = reinterpret_cast<const float*>(wp)[d];
  }
  float ss = 0.f;
#pragma unroll
  for (int d = 0; d < DPL; ++d) ss = fmaf(x[d], x[d], ss);
  ss = group_sum<LPH>(ss);
  const float rn = 1.0f / sqrtf(fmaf(ss, 1.0f / (float)kHeadDim, a.q_eps));
  const bool first = dofs < kHeadDim / 2;
  float y[DPL];
#pragma unroll
  for (int d = 0; d < DPL; ++d) {
    const float u = x[d] * rn * w[d];
    const float up = __shfl_xor(u, LPH / 2, 64);  // the pair's other member
    float sn, cs;
    sincosf(pos * a.inv_freq[(dofs + d) & (kHeadDim / 2 - 1)], &sn, &cs);
    y[d] = first ? u * cs - up * sn : up * sn + u * cs;
  }
#pragma unroll
  for (int i = 0; i < NWD; ++i) {
    if constexpr (EPW == 2) qw[i] = pack_bf16x2(y[2 * i], y[2 * i + 1]);
    else qw[i] = __float_as_uint(y[i]);
  }
}

template <typename T, int HKV, int G, int NWAVE, int KB>
__global__ void __launch_bounds__(NWAVE * 64) decode_splitk_kernel(DecodeArgs a) {
  constexpr int HQ = HKV * G;
  constexpr int LPH = kWave / HKV;              // lanes per KV head
  constexpr int DPL = kHeadDim / LPH;           // dims per lane
  constexpr int EPW = ElemTraits<T>::kPerWord;
  constexpr int NWD = DPL / EPW;                // 32-bit words per lane per row
  constexpr int NT = NWAVE * kWave;
  static_assert(NWD % 4 == 0, "lane share of a row must be a multiple of 16 bytes");

  extern __shared__ int32_t cu[];               // [bs + 1]
  __shared__ float sm_m[NWAVE][HQ];
  __shared__ float sm_l[NWAVE][HQ];
  __shared__ float sm_acc[NWAVE][HQ][kHeadDim];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane / LPH;
  const int dofs = (lane % LPH) * DPL;
  const int bs = a.bs;

  const bool report = blockIdx.x == 0;
  block_exclusive_scan<NT>(cu, bs, [&](int r) -> int32_t {
    const int32_t s = a.device_len[r];
    const int32_t row = a.table_idx ? a.table_idx[r] : r;
    const bool row_ok = row >= 0 && row < a.pt_rows;
    if (a.skip_empty && s == 0) return 0;
    const bool len_ok = s >= 1 && (int64_t)s <= a.pt_stride;
    if (report && !row_ok) raise_fault(a.faults, 0x8u);
    if (report && !len_ok) raise_fault(a.faults, 0x2u);
    return (row_ok && len_ok) ? s : 0;
  });
  if (report)
    for (int i = threadIdx.x; i <= bs; i += NT) a.cu_out[i] = cu[i];

  const int64_t total = cu[bs];
  const int P = decode_num_items(total, a.num_items);
  const int item = blockIdx.x;
  if (total == 0 || item >= P) return;
  const int64_t b0 = item_begin(item, total, P), b1 = item_begin(item + 1, total, P);
  if (b0 >= b1) return;

  // First request whose key range contains b0: largest r with cu[r] <= b0.
  int lo = 0, hi = bs;  // invariant: cu[lo] <= b0 < cu[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu[mid] <= b0) lo = mid; else hi = mid;
  }
  int r = lo;

  const T* kpool = reinterpret_cast<const T*>(a.k_pool);
  const T* vpool = reinterpret_cast<const T*>(a.v_pool);
  const int64_t head_ofs = (int64_t)g * kHeadDim + dofs;

  int64_t pos = b0;
  while (pos < b1) {
    while (cu[r + 1] <= pos) ++r;  // skip empty requests
    const int64_t seg_end = min(b1, (int64_t)cu[r + 1]);
    const int32_t S = cu[r + 1] - cu[r];
    const int32_t j0 = (int32_t)(pos - cu[r]), j1 = (int32_t)(seg_end - cu[r]);
    const int32_t row = a.table_idx ? a.table_idx[r] : r;
    const int32_t* pt = a.page_table + (int64_t)row * a.pt_stride;

    // q of this lane's G heads.
    uint32_t qw[G][NWD];
    {
      const T* qb = reinterpret_cast<const T*>(a.q) + (int64_t)r * a.q_stride;
#pragma unroll
      for (int hh = 0; hh < G; ++hh)
        load_lane_row<T, NWD>(qw[hh], qb + (int64_t)(g * G + hh) * kHeadDim + dofs);
      if (a.q_w) {  // fused q prologue: the new token sits at position S - 1
#pragma unroll
        for (int hh = 0; hh < G; ++hh) q_norm_rope<T, LPH, DPL, NWD>(qw[hh], a, dofs, (float)(S - 1));
      }
    }

    float m[G], l[G], acc[G][DPL];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      m[hh] = -INFINITY;
      l[hh] = 0.f;
#pragma unroll
      for (int d = 0; d < DPL; ++d) acc[hh][d] = 0.f;
    }

    const int32_t len = j1 - j0;
    const int32_t per = (len + NWAVE - 1) / NWAVE;
    const int32_t wj0 = min(j1, j0 + wave * per);
    const int32_t wj1 = min(j1, wj0 + per);

    // Page-table entries one 64-key chunk ahead: the next chunk's slots are
    // in flight while this chunk's rows are read.
    int32_t next = lane < wj1 - wj0 ? pt[wj0 + lane] : -1;
    for (int32_t jb = wj0; jb < wj1; jb += kWave) {
      const int32_t nchunk = min(kWave, wj1 - jb);
      const int32_t s = next, pt_raw = next;
      next = lane < wj1 - (jb + kWave) ? pt[jb + kWave + lane] : -1;
      // -1: no key (past this wave's range); -2: an entry outside the pool,
      // whose key reads as a zero K and V row.
      int32_t myslot = -1;
      if (lane < nchunk) {
        if (s >= 0 && (int64_t)s < a.num_slots) {
          myslot = s;
        } else {
          myslot = -2;
          if (!(a.k_new && jb + lane == S - 1)) raise_fault(a.faults, 0x4u);  // the new key's entry: checked below
        }
      }
      for (int32_t kb = 0; kb < nchunk; kb += KB) {
        uint32_t kw[KB][NWD], vw[KB][NWD];
        int32_t sl[KB];
#pragma unroll
        for (int kk = 0; kk < KB; ++kk) {
          sl[kk] = (kb + kk < nchunk) ? __builtin_amdgcn_readlane(myslot, kb + kk) : -1;
          // the new row (wave-uniform; a block may run past this wave's keys,
          // whose key S - 1 is then another wave's): read from k_new / v_new
          if (a.k_new && kb + kk < nchunk && jb + kb + kk == S - 1) {
            const int32_t tslot = __builtin_amdgcn_readlane(pt_raw, kb + kk);
            load_lane_row<T, NWD>(kw[kk], reinterpret_cast<const T*>(a.k_new) + (int64_t)r * a.kn_stride + head_ofs);
            load_lane_row<T, NWD>(vw[kk], reinterpret_cast<const T*>(a.v_new) + (int64_t)r * a.vn_stride + head_ofs);
            const int64_t loc = a.loc64 ? reinterpret_cast<const int64_t*>(a.out_loc)[r]
                                        : (int64_t)reinterpret_cast<const int32_t*>(a.out_loc)[r];
            if (loc >= 0 && loc < a.num_slots) {
              store_lane_row<NWD>(const_cast<T*>(kpool) + loc * a.pool_row + head_ofs, kw[kk]);
              store_lane_row<NWD>(const_cast<T*>(vpool) + loc * a.pool_row + head_ofs, vw[kk]);
            } else if (lane == 0) {
              raise_fault(a.faults, 0x1u);
            }
            if (lane == 0 && (int64_t)tslot != loc) raise_fault(a.faults, 0x20u);
            sl[kk] = 0;  // a key (its slot is not read)
          } else if (sl[kk] >= 0) {
            load_lane_row<T, NWD>(kw[kk], kpool + (int64_t)sl[kk] * a.pool_row + head_ofs);
            load_lane_row<T, NWD>(vw[kk], vpool + (int64_t)sl[kk] * a.pool_row + head_ofs);
          } else {
#pragma unroll
            for (int i = 0; i < NWD; ++i) kw[kk][i] = vw[kk][i] = 0u;
          }
        }
        float sc[KB][G];
#pragma unroll
        for (int kk = 0; kk < KB; ++kk)
#pragma unroll
          for (int hh = 0; hh < G; ++hh) {
            const float d = group_sum<LPH>(lane_dot<T, NWD>(qw[hh], kw[kk]));
            sc[kk][hh] = sl[kk] != -1 ? d * a.scale_log2 : -INFINITY;
          }
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
          float mb = sc[0][hh];
#pragma unroll
          for (int kk = 1; kk < KB; ++kk) mb = fmaxf(mb, sc[kk][hh]);
          const float mn = fmaxf(m[hh], mb);
          if (mn == -INFINITY) continue;          // nothing valid yet for this head
          if (mn > m[hh]) {
            const float corr = fast_exp2(m[hh] - mn);
            l[hh] *= corr;
#pragma unroll
            for (int d = 0; d < DPL; ++d) acc[hh][d] *= corr;
            m[hh] = mn;
          }
#pragma unroll
          for (int kk = 0; kk < KB; ++kk) {
            const float p = fast_exp2(sc[kk][hh] - mn);
            l[hh] += p;
            lane_axpy<T, NWD>(acc[hh], p, vw[kk]);
          }
        }
      }
    }

    // Merge the waves of this workgroup.
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const int h = g * G + hh;
      if (lane % LPH == 0) {
        sm_m[wave][h] = m[hh];
        sm_l[wave][h] = l[hh];
      }
#pragma unroll
      for (int d = 0; d < DPL; ++d) sm_acc[wave][h][dofs + d] = acc[hh][d];
    }
    __syncthreads();
    const bool final_out = (j0 == 0 && j1 == S);
    const int slot = item + r;
    for (int idx = threadIdx.x; idx < HQ * kHeadDim; idx += NT) {
      const int h = idx / kHeadDim, d = idx % kHeadDim;
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < NWAVE; ++w) M = fmaxf(M, sm_m[w][h]);
      float L = 0.f, A = 0.f;
#pragma unroll
      for (int w = 0; w < NWAVE; ++w) {
        const float mw = sm_m[w][h];
        const float c = (mw == -INFINITY) ? 0.f : fast_exp2(mw - M);
        L += sm_l[w][h] * c;
        A += sm_acc[w][h][d] * c;
      }
      if (final_out) {
        T* ob = reinterpret_cast<T*>(a.o) + (int64_t)r * a.o_stride + (int64_t)h * kHeadDim + d;
        store_out<T>(ob, L > 0.f ? A / L : 0.f);
      } else {
        a.part_acc[((int64_t)slot * HQ + h) * kHeadDim + d] = A;
        if (d == 0) {
          a.part_ml[((int64_t)slot * HQ + h) * 2 + 0] = M;
          a.part_ml[((int64_t)slot * HQ + h) * 2 + 1] = L;
        }
      }
    }
    __syncthreads();
    pos = seg_end;
  }
}

// Merge the partials of every request that was cut by item boundaries; zero
// the output of requests whose lengths were invalid. One workgroup per
// (request, query head) of NT threads: thread t takes the request's items
// i0 + g, i0 + g + NT/16, ... (g = t / 16) for dims [8 (t % 16), 8 (t % 16) + 8)
// and merges them online (four items' loads in flight per step); the item
// groups then meet in LDS. A request cut into many items (small batches use
// small items) costs a few memory round trips, not one per item; a large
// batch, whose requests span a handful of items each, takes the narrow form
// so that idle groups cost no LDS round.
constexpr int kCombineThreads = 512;      // wide form: 32 item groups
constexpr int kCombineThreadsNarrow = 64;  // narrow form: 4 item groups

template <typename T, int HQ, int NT>
__global__ void __launch_bounds__(NT) decode_combine_kernel(DecodeArgs a) {
  constexpr int kGroups = NT / 16;  // item groups
  constexpr int kU = 4;             // items in flight per thread per step
  const int r = blockIdx.x, h = blockIdx.y;
  const int32_t* cu = a.cu_out;
  const int64_t total = cu[a.bs];
  const int32_t c0 = cu[r], c1 = cu[r + 1];
  T* ob = reinterpret_cast<T*>(a.o) + (int64_t)r * a.o_stride + (int64_t)h * kHeadDim;
  const int t = threadIdx.x, grp = t >> 4, d0 = (t & 15) * 8;
  if (c1 == c0) {  // invalid request: skipped by the main kernel
    if (!(a.skip_empty && a.device_len[r] == 0))
      for (int d = t; d < kHeadDim; d += NT) store_out<T>(ob + d, 0.f);
    return;
  }
  const int P = decode_num_items(total, a.num_items);
  const int i0 = item_of(c0, total, P), i1 = item_of(c1 - 1, total, P);
  if (i0 == i1) return;  // finished in place
  // An item that holds no key of the request wrote nothing: it is skipped.
  auto live = [&](int i) { return i <= i1 && item_begin(i, total, P) != item_begin(i + 1, total, P); };
  float m = -INFINITY, l = 0.f, A[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int i = i0 + grp; i <= i1; i += kGroups * kU) {
    float2 v[kU];
    u32x4 x[kU][2];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int it = i + u * kGroups;
      const bool ok = live(it);
      v[u] = ok ? reinterpret_cast<const float2*>(a.part_ml)[(int64_t)(it + r) * HQ + h] : make_float2(-INFINITY, 0.f);
      const u32x4* src = reinterpret_cast<const u32x4*>(a.part_acc + ((int64_t)(it + r) * HQ + h) * kHeadDim + d0);
      x[u][0] = ok ? src[0] : u32x4{0u, 0u, 0u, 0u};
      x[u][1] = ok ? src[1] : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (v[u].x == -INFINITY) continue;
      const float mn = fmaxf(m, v[u].x);
      const float co = fast_exp2(m - mn), cn = fast_exp2(v[u].x - mn);  // m = -inf gives co = 0
      l = l * co + v[u].y * cn;
#pragma unroll
      for (int e = 0; e < 8; ++e) A[e] = A[e] * co + __uint_as_float(x[u][e >> 2][e & 3]) * cn;
      m = mn;
    }
  }
  __shared__ float sm_m[kGroups], sm_l[kGroups];
  __shared__ float sm_a[kGroups][kHeadDim];
  if ((t & 15) == 0) {
    sm_m[grp] = m;
    sm_l[grp] = l;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) sm_a[grp][d0 + e] = A[e];
  __syncthreads();
  for (int d = t; d < kHeadDim; d += NT) {
    float M = -INFINITY;
#pragma unroll
    for (int g = 0; g < kGroups; ++g) M = fmaxf(M, sm_m[g]);
    float L = 0.f, Ad = 0.f;
#pragma unroll
    for (int g = 0; g < kGroups; ++g) {
      const float c = sm_m[g] == -INFINITY ? 0.f : fast_exp2(sm_m[g] - M);
      L += sm_l[g] * c;
      Ad += sm_a[g][d] * c;
    }
    store_out<T>(ob + d, L > 0.f ? Ad / L : 0.f);
  }
}

// Extend rows as decode rows (the fp32 extend path): query row t of request
// r attends to keys 0 .. C_r + t, exactly a decode row of C_r + t + 1 keys
// over the request's table row ("第 0 步" dense attention with its causal
// mask; "Mini-SGLang 完整剖析" section 4.6.5 for the ragged row order). For
// every ragged row v < total_q: vlen[v] = C_r + t + 1 and vrow[v] = the
// request's table row, or vlen[v] = 0 for rows past the batch's and for the
// rows of an invalid request. The ragged offsets, checks and fault bits are
// the extend kernel's: a request owns max(S - C, 0) rows whatever else is
// wrong with it. Each workgroup scans the requests' extend lengths itself.
constexpr int kExpandThreads = 256;

__global__ void __launch_bounds__(kExpandThreads) extend_rows_kernel(
    const int32_t* cached_len, const int32_t* device_len, const int32_t* table_idx, int32_t bs, int32_t pt_rows,
    int64_t pt_stride, int32_t max_extend, int64_t total_q, int32_t* vlen, int32_t* vrow, uint32_t* faults) {
  extern __shared__ int32_t cu[];  // [bs + 1]
  const bool report = blockIdx.x == 0;
  auto valid = [&](int r, int32_t* row) {
    const int32_t C = cached_len[r], S = device_len[r];
    *row = table_idx ? table_idx[r] : r;
    const bool len_ok = C >= 0 && C < S && (int64_t)S <= pt_stride && S - C <= max_extend;
    const bool row_ok = *row >= 0 && *row < pt_rows;
    return (len_ok ? 0u : 0x2u) | (row_ok ? 0u : 0x8u);
  };
  block_exclusive_scan<kExpandThreads>(cu, bs, [&](int r) -> int32_t {
    const int32_t C = cached_len[r], S = device_len[r];
    if (report) {
      int32_t row;
      const uint32_t bad = valid(r, &row);
      if (bad) raise_fault(faults, (bad & 0x8u) ? 0x8u : 0x2u);
    }
    return S > C ? S - C : 0;
  });
  const int64_t v = (int64_t)blockIdx.x * kExpandThreads + threadIdx.x;
  if (report && threadIdx.x == 0 && (int64_t)cu[bs] > total_q) raise_fault(faults, 0x10u);
  if (v >= total_q) return;
  int32_t len = 0, trow = 0;
  if (v < cu[bs]) {
    int lo = 0, hi = bs;  // cu[lo] <= v < cu[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (cu[mid] <= v) lo = mid; else hi = mid;
    }
    const int r = lo;
    int32_t row;
    if (!valid(r, &row) && (int64_t)cu[r + 1] <= total_q) {  // a request whose rows do not all fit is skipped
      len = cached_len[r] + (int32_t)(v - cu[r]) + 1;
      trow = row;
    }
  }
  vlen[v] = len;
  vrow[v] = trow;
}

}  // namespace pkv
