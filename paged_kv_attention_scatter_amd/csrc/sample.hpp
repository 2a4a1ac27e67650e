// Batched per-request sampler: argmax, or temperature -> top-k -> top-p -> draw.
//
// Semantics ("Engine 与采样器", section 采样器; "Mini-SGLang 源码解析（四）：GPU
// 计算引擎系统", sections 14.3-14.4): p = softmax(logits / T); top-k keeps the
// k most probable tokens; the kept mass is renormalised; top-p keeps a ranked
// token iff the kept mass ranked before it is < p; one token is drawn from
// the rest. Greedy rows (T <= 1e-6, or no temperature array) are argmax.
//
// The pages' GPU path calls FlashInfer's rejection-sampling kernels; this is
// a different, exact design for one workgroup per row:
//
// * The row is loaded once into registers: wave w owns a contiguous index
//   range, lane l reads 16-byte chunk (w * CPW + c * 64 + l) in round c, so
//   every load is coalesced and index order is (wave, round, lane, element).
// * Ranking uses order-preserving integer keys of the logits (-0 == +0), so
//   argmax and top-k are exact: ties go to the lower index.
// * Weights are w(l) = exp2((l - l_max) * log2(e) / T); equal logits get the
//   same weight, bit for bit. Mass sums are fp32 within one 16-byte chunk and
//   fp64 above.
// * Fast path for the cuts: a count histogram of d = key_max - key over the
//   256 largest key values. Because every element of a bin has the same key,
//   the mass of a bin is count * w(key) -- the top-k threshold, the top-k
//   kept mass and the top-p cut all come from 256 bins, not from V elements.
//   If a cut falls below the window, a generic radix descent over the full
//   key (8 bits per pass, fp64 mass histograms) finds it instead.
// * Ties at a cut are resolved by index: the first n equal-key tokens in
//   index order are kept.
// * The draw scans kept weights in index order (wave prefix, then round, then
//   lane, then element) for the first running mass > u * W.
#pragma once

#include "common.hpp"

namespace pkv {

struct SampleArgs {
  const void* logits;
  int64_t row_stride;   // elements
  int32_t bs;
  int32_t vocab;
  const float* temperature;  // NULL = all greedy
  const int32_t* top_k;
  const float* top_p;
  const float* uniforms;
  int32_t* out;
};

template <typename T>
struct SampleElem;

template <>
struct SampleElem<bf16_t> {
  static constexpr int kPerChunk = 8;
  static constexpr int kKeyBits = 16;
  __device__ static uint32_t raw(const u32x4& x, int e) {
    const uint32_t w = x[e >> 1];
    return (e & 1) ? (w >> 16) : (w & 0xffffu);
  }
  __device__ static uint32_t key(uint32_t b) {
    if (b == 0x8000u) b = 0;  // -0 ranks with +0
    return (b & 0x8000u) ? (~b & 0xffffu) : (b | 0x8000u);
  }
  __device__ static float key_value(uint32_t k) {
    const uint32_t b = (k & 0x8000u) ? (k & 0x7fffu) : (~k & 0xffffu);
    return __uint_as_float(b << 16);
  }
  __device__ static uint32_t raw_scalar(const void* p, int64_t i) {
    return static_cast<const uint16_t*>(p)[i];
  }
};

template <>
struct SampleElem<float> {
  static constexpr int kPerChunk = 4;
  static constexpr int kKeyBits = 32;
  __device__ static uint32_t raw(const u32x4& x, int e) { return x[e]; }
  __device__ static uint32_t key(uint32_t b) {
    if (b == 0x80000000u) b = 0;
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  }
  __device__ static float key_value(uint32_t k) {
    const uint32_t b = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
    return __uint_as_float(b);
  }
  __device__ static uint32_t raw_scalar(const void* p, int64_t i) {
    return static_cast<const uint32_t*>(p)[i];
  }
};

// ---------------------------------------------------------------- wave / block reductions

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o, 64));
  return v;
}
__device__ __forceinline__ int32_t wave_min_i32(int32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = min(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ int32_t wave_max_i32(int32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, __shfl_xor(v, o, 64));
  return v;
}
// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ double wave_incl_scan_f64(double v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  return v;
}

template <int NW>
struct BlockRed {
  double f[NW];
  int32_t i[NW];
  uint32_t u[NW];
};

template <int NW>
__device__ double block_sum_f64(double v, BlockRed<NW>& sh, int wave, int lane) {
  v = wave_sum_f64(v);
  __syncthreads();
  if (lane == 0) sh.f[wave] = v;
  __syncthreads();
  double t = 0.0;
#pragma unroll
  for (int w = 0; w < NW; ++w) t += sh.f[w];
  return t;
}
template <int NW>
__device__ uint32_t block_max_u32(uint32_t v, BlockRed<NW>& sh, int wave, int lane) {
  v = wave_max_u32(v);
  __syncthreads();
  if (lane == 0) sh.u[wave] = v;
  __syncthreads();
  uint32_t t = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) t = max(t, sh.u[w]);
  return t;
}
template <int NW>
__device__ int32_t block_min_i32(int32_t v, BlockRed<NW>& sh, int wave, int lane) {
  v = wave_min_i32(v);
  __syncthreads();
  if (lane == 0) sh.i[wave] = v;
  __syncthreads();
  int32_t t = 0x7fffffff;
#pragma unroll
  for (int w = 0; w < NW; ++w) t = min(t, sh.i[w]);
  return t;
}
template <int NW>
__device__ int32_t block_max_i32(int32_t v, BlockRed<NW>& sh, int wave, int lane) {
  v = wave_max_i32(v);
  __syncthreads();
  if (lane == 0) sh.i[wave] = v;
  __syncthreads();
  int32_t t = -1;
#pragma unroll
  for (int w = 0; w < NW; ++w) t = max(t, sh.i[w]);
  return t;
}

// ---------------------------------------------------------------- the row

// A row split over NT threads. REG: the chunks live in registers (MAXR
// rounds at most); otherwise every pass re-reads them from memory.
template <typename T, int NT, int MAXR, bool REG>
struct Row {
  using E = SampleElem<T>;
  static constexpr int EPC = E::kPerChunk;
  const T* base;
  int V, nchunks, cpw, rounds, wave, lane;
  u32x4 reg[REG ? MAXR : 1];

  __device__ int chunk_id(int c) const { return wave * cpw + c * kWave + lane; }
  __device__ bool chunk_ok(int c) const {
    return c * kWave + lane < cpw && chunk_id(c) < nchunks;
  }
  __device__ u32x4 fetch(int c) const {
    u32x4 x = {0u, 0u, 0u, 0u};
    if (!chunk_ok(c)) return x;
    const int64_t ch = chunk_id(c);
    if ((ch + 1) * EPC <= V) return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base) + ch);
    // the last, partial chunk of a row: element by element
    for (int e = 0; e < EPC; ++e) {
      const int64_t i = ch * EPC + e;
      if (i < V) {
        const uint32_t r = E::raw_scalar(base, i);
        if constexpr (EPC == 8) x[e >> 1] |= (e & 1) ? (r << 16) : r;
        else x[e] = r;
      }
    }
    return x;
  }
  __device__ void init(const T* b, int vocab, int nt_waves, int w, int l) {
    base = b;
    V = vocab;
    nchunks = (vocab + EPC - 1) / EPC;
    cpw = (nchunks + nt_waves - 1) / nt_waves;
    rounds = (cpw + kWave - 1) / kWave;
    wave = w;
    lane = l;
    if constexpr (REG) {
#pragma unroll
      for (int c = 0; c < MAXR; ++c)
        if (c < rounds) reg[c] = fetch(c);
    }
  }
  // f(index, key, raw bits, round) for every element of this thread, in index order.
  template <class F>
  __device__ __forceinline__ void visit(int c, const u32x4& x, F& f) const {
    const int base_idx = chunk_id(c) * EPC;
#pragma unroll
    for (int e = 0; e < EPC; ++e) {
      const int i = base_idx + e;
      if (i < V) {
        const uint32_t r = E::raw(x, e);
        f(i, E::key(r), r);
      }
    }
  }
  template <class F>
  __device__ __forceinline__ void for_each(F f) const {
    if constexpr (REG) {
#pragma unroll
      for (int c = 0; c < MAXR; ++c)
        if (c < rounds && chunk_ok(c)) visit(c, reg[c], f);
    } else {
      for (int c = 0; c < rounds; ++c)
        if (chunk_ok(c)) visit(c, fetch(c), f);
    }
  }
  // Elements of round c only (for the crossing searches).
  template <class F>
  __device__ __forceinline__ void for_round(int c, F f) const {
    if constexpr (REG) {
#pragma unroll
      for (int cc = 0; cc < MAXR; ++cc)
        if (cc == c && chunk_ok(cc)) visit(cc, reg[cc], f);
    } else {
      if (chunk_ok(c)) visit(c, fetch(c), f);
    }
  }
};

// Weight of logit l relative to the row maximum: exp2((l - l_max) * c2).
__device__ __forceinline__ float row_weight(float l, float lmax, float c2) {
  return fast_exp2((l - lmax) * c2);
}

// First element, in index order, at which the running sum of v(i) >= 0
// exceeds `target`; -1 if none. v(i, key, raw) -> float. Sums: fp32 within a
// 16-byte chunk, fp64 above.
template <typename RowT, int NW, class VF>
__device__ int32_t find_crossing(const RowT& row, VF v, double target, BlockRed<NW>& sh, double* wave_tot,
                                 int32_t* result) {
  const int wave = row.wave, lane = row.lane;
  double tsum = 0.0;
  row.for_each([&](int, uint32_t key, uint32_t raw) { tsum += (double)v(key, raw); });
  const double wsum = wave_sum_f64(tsum);
  __syncthreads();
  if (lane == 0) wave_tot[wave] = wsum;
  if (threadIdx.x == 0) *result = -1;
  __syncthreads();
  double pre = 0.0;
  int wstar = -1;
  for (int w = 0; w < NW; ++w) {
    if (target < pre + wave_tot[w]) { wstar = w; break; }
    pre += wave_tot[w];
  }
  if (wave == wstar) {
    double rem = target - pre;
    for (int c = 0; c < row.rounds; ++c) {
      float cs = 0.f;
      row.for_round(c, [&](int, uint32_t key, uint32_t raw) { cs += v(key, raw); });
      const double incl = wave_incl_scan_f64((double)cs, lane);
      const double tot = __shfl(incl, 63, 64);
      if (rem < tot) {
        const double excl = incl - (double)cs;
        const bool mine = excl <= rem && rem < incl;
        const uint64_t who = __ballot(mine);
        const int l0 = who ? __builtin_ctzll(who) : 63;
        if (lane == l0) {
          float run = 0.f;
          int32_t found = -1, last = -1;
          row.for_round(c, [&](int i, uint32_t key, uint32_t raw) {
            const float x = v(key, raw);
            if (x > 0.f) last = i;
            run += x;
            if (found < 0 && excl + (double)run > rem) found = i;
          });
          *result = found >= 0 ? found : last;
        }
        break;
      }
      rem -= tot;
    }
  }
  __syncthreads();
  return *result;
}

// Generic radix descent over the full key (8 bits per pass) among elements
// with pred(key, raw). By count (mass == false): finds the key of the element
// ranked `kth` (1-based, descending). By mass: finds the key group where the
// mass ranked before it is < target <= that plus the group's mass.
// Returns the key; *above = count (or mass) strictly above it, *eq = its count.
template <typename RowT, int NT, int NW, int KEYBITS, class PF, class WF>
__device__ uint32_t radix_descend(const RowT& row, PF pred, WF weight, bool by_mass, double goal,
                                  uint32_t* hcnt, double* hmass, BlockRed<NW>& sh, double* above_out,
                                  uint32_t* eq_out, uint32_t* sel) {
  uint32_t prefix = 0, mask = 0;
  double above = 0.0;
  uint32_t eq = 0;
  for (int shift = KEYBITS - 8; shift >= 0; shift -= 8) {
    for (int b = threadIdx.x; b < 256; b += NT) {
      hcnt[b] = 0;
      hmass[b] = 0.0;
    }
    __syncthreads();
    row.for_each([&](int, uint32_t key, uint32_t raw) {
      if ((key & mask) == prefix && pred(key, raw)) {
        const uint32_t dgt = (key >> shift) & 0xffu;
        atomicAdd(&hcnt[dgt], 1u);
        if (by_mass) atomicAdd(&hmass[dgt], (double)weight(key, raw));
      }
    });
    __syncthreads();
    if (threadIdx.x == 0) {
      // Scan digits from the top. (256 bins, once per pass: cheap next to the
      // element pass above.)
      double acc = above;
      uint32_t pick = 0, pick_eq = 0;
      double pick_above = acc;
      bool found = false;
      int last_nonzero = -1;
      for (int b = 255; b >= 0; --b) {
        if (hcnt[b] == 0) continue;
        last_nonzero = b;
        const double amount = by_mass ? hmass[b] : (double)hcnt[b];
        if (acc + amount >= goal) {
          pick = (uint32_t)b;
          pick_above = acc;
          pick_eq = hcnt[b];
          found = true;
          break;
        }
        acc += amount;
      }
      if (!found) {  // rounding: the goal lies beyond everything -> the lowest group
        pick = (uint32_t)(last_nonzero < 0 ? 0 : last_nonzero);
        pick_eq = last_nonzero < 0 ? 0 : hcnt[pick];
        pick_above = acc - (by_mass ? (last_nonzero < 0 ? 0.0 : hmass[pick]) : (double)pick_eq);
      }
      sel[0] = pick;
      sel[1] = pick_eq;
      reinterpret_cast<double*>(sel + 2)[0] = pick_above;
    }
    __syncthreads();
    prefix |= sel[0] << shift;
    mask |= 0xffu << shift;
    eq = sel[1];
    above = reinterpret_cast<const double*>(sel + 2)[0];
    __syncthreads();
  }
  *above_out = above;
  *eq_out = eq;
  return prefix;
}

constexpr int kSampleWindow = 256;  // key values below the row maximum held in the fast histogram

template <typename T, int NT, int MAXR, bool REG>
__global__ void __launch_bounds__(NT) sample_kernel(SampleArgs a) {
  using E = SampleElem<T>;
  constexpr int NW = NT / kWave;
  constexpr int kEPC = E::kPerChunk;
  const int row_id = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;

  __shared__ BlockRed<NW> sh;
  __shared__ uint32_t hist[kSampleWindow];
  __shared__ float wtab[kSampleWindow];
  __shared__ double wave_tot[NW];
  __shared__ int32_t result;
  __shared__ uint32_t rcnt[256];
  __shared__ double rmass[256];
  __shared__ uint32_t sel[4];

  Row<T, NT, MAXR, REG> row;
  row.init(reinterpret_cast<const T*>(a.logits) + (int64_t)row_id * a.row_stride, a.vocab, NW, wave, lane);
  const int V = a.vocab;

  // ---- pass 1: maximum key, then its lowest index (argmax)
  uint32_t kmax_t = 0;
  row.for_each([&](int, uint32_t key, uint32_t) { kmax_t = max(kmax_t, key); });
  const uint32_t kmax = block_max_u32<NW>(kmax_t, sh, wave, lane);
  int32_t first = 0x7fffffff;
  if (kmax_t == kmax)
    row.for_each([&](int i, uint32_t key, uint32_t) { if (key == kmax && i < first) first = i; });
  const int32_t argmax = block_min_i32<NW>(first, sh, wave, lane);

  const float temp = a.temperature ? a.temperature[row_id] : 0.f;
  if (!a.temperature || temp <= 1e-6f) {
    if (threadIdx.x == 0) a.out[row_id] = argmax;
    return;
  }
  int32_t k = a.top_k ? a.top_k[row_id] : 0;
  const bool use_k = k > 0 && k < V;
  if (!use_k) k = V;
  float p = a.top_p ? a.top_p[row_id] : 1.f;
  const bool use_p = p < 1.f;
  if (use_p) p = fmaxf(p, 1e-6f);
  const float u = a.uniforms[row_id];
  const float lmax = E::key_value(kmax);
  const float c2 = 1.4426950408889634f / temp;
  auto wkey = [&](uint32_t key) { return row_weight(E::key_value(key), lmax, c2); };

  // ---- pass 2: window histogram of d = kmax - key; full mass W when there is no top-k
  for (int b = threadIdx.x; b < kSampleWindow; b += NT) {
    hist[b] = 0;
    wtab[b] = (kmax >= (uint32_t)b) ? wkey(kmax - (uint32_t)b) : 0.f;
  }
  __syncthreads();
  double wsum_t = 0.0;
  {
    float chunk_acc = 0.f;
    int last_chunk = -1;
    row.for_each([&](int i, uint32_t key, uint32_t) {
      const uint32_t d = kmax - key;
      if (d < (uint32_t)kSampleWindow) atomicAdd(&hist[d], 1u);
      if (!use_k) {
        const int ch = i / kEPC;
        if (ch != last_chunk) {
          wsum_t += (double)chunk_acc;
          chunk_acc = 0.f;
          last_chunk = ch;
        }
        chunk_acc += row_weight(E::key_value(key), lmax, c2);
      }
    });
    wsum_t += (double)chunk_acc;
  }
  __syncthreads();

  // Top-k threshold: key K_k, count strictly above it, how many equal keys to keep.
  uint32_t kk_key = 0;      // smallest kept key under top-k (0 = keep all)
  uint32_t kk_take = 0;     // equal-key elements kept at kk_key
  uint32_t kk_eq = 0;       // equal-key elements present at kk_key
  bool k_in_window = false;
  if (use_k) {
    if (threadIdx.x == 0) {
      uint32_t acc = 0;
      int dk = -1;
      for (int d = 0; d < kSampleWindow; ++d) {
        if (acc + hist[d] >= (uint32_t)k) { dk = d; break; }
        acc += hist[d];
      }
      sel[0] = (uint32_t)dk;
      sel[1] = acc;
    }
    __syncthreads();
    const int dk = (int)sel[0];
    const uint32_t above = sel[1];
    __syncthreads();
    if (dk >= 0) {
      k_in_window = true;
      kk_key = kmax - (uint32_t)dk;
      kk_eq = hist[dk];
      kk_take = (uint32_t)k - above;
    } else {
      double ab;
      uint32_t eq;
      kk_key = radix_descend<decltype(row), NT, NW, E::kKeyBits>(
          row, [](uint32_t, uint32_t) { return true; }, [](uint32_t, uint32_t) { return 0.f; }, false,
          (double)k, rcnt, rmass, sh, &ab, &eq, sel);
      kk_eq = eq;
      kk_take = (uint32_t)k - (uint32_t)ab;
    }
  }
  // Index cutoff for ties at the top-k threshold: keep equal keys with index <= kk_last.
  int32_t kk_last = 0x7fffffff;
  if (use_k && kk_take < kk_eq) {
    kk_last = find_crossing<decltype(row), NW>(
        row, [&](uint32_t key, uint32_t) { return key == kk_key ? 1.f : 0.f; }, (double)kk_take - 0.5, sh,
        wave_tot, &result);
  }
  auto kept_k = [&](int i, uint32_t key) {
    return !use_k || key > kk_key || (key == kk_key && i <= kk_last);
  };

  // Kept mass after top-k.
  double Wk;
  if (!use_k) {
    Wk = block_sum_f64<NW>(wsum_t, sh, wave, lane);
  } else if (k_in_window) {
    // every kept element is inside the window: count * weight per bin
    if (threadIdx.x == 0) {
      double acc = 0.0;
      const int dk = (int)(kmax - kk_key);
      for (int d = 0; d < dk; ++d) acc += (double)hist[d] * (double)wtab[d];
      acc += (double)kk_take * (double)wtab[dk];
      wave_tot[0] = acc;
    }
    __syncthreads();
    Wk = wave_tot[0];
    __syncthreads();
  } else {
    double t = 0.0;
    float chunk_acc = 0.f;
    int last_chunk = -1;
    row.for_each([&](int i, uint32_t key, uint32_t) {
      if (!kept_k(i, key)) return;
      const int ch = i / kEPC;
      if (ch != last_chunk) {
        t += (double)chunk_acc;
        chunk_acc = 0.f;
        last_chunk = ch;
      }
      chunk_acc += wkey(key);
    });
    t += (double)chunk_acc;
    Wk = block_sum_f64<NW>(t, sh, wave, lane);
  }

  // ---- top-p cut: key kp_key, keep equal keys with index <= kp_last
  uint32_t kp_key = 0;
  int32_t kp_last = 0x7fffffff;
  bool p_in_window = false;
  if (use_p) {
    const double target = (double)p * Wk;
    const int dk_lim = use_k ? (k_in_window ? (int)(kmax - kk_key) : -2) : kSampleWindow - 1;
    // window path: valid when every kept element's bin is known (top-k inside
    // the window, or no top-k)
    if (dk_lim != -2) {
      if (threadIdx.x == 0) {
        double acc = 0.0;
        int dstar = -1;
        uint32_t n_at = 0;
        double above = 0.0;
        for (int d = 0; d <= dk_lim && d < kSampleWindow; ++d) {
          const uint32_t n = (use_k && d == dk_lim) ? kk_take : hist[d];
          if (n == 0) continue;
          const double m = (double)n * (double)wtab[d];
          if (acc + m >= target) { dstar = d; n_at = n; above = acc; break; }
          acc += m;
        }
        sel[0] = (uint32_t)dstar;
        sel[1] = n_at;
        reinterpret_cast<double*>(sel + 2)[0] = above;
      }
      __syncthreads();
      const int dstar = (int)sel[0];
      const uint32_t n_at = sel[1];
      const double above = reinterpret_cast<const double*>(sel + 2)[0];
      __syncthreads();
      if (dstar >= 0) {
        p_in_window = true;
        kp_key = kmax - (uint32_t)dstar;
        const double w = (double)wtab[dstar];
        double need = ceil((target - above) / w);
        if (need < 1.0) need = 1.0;
        const uint32_t take = need >= (double)n_at ? n_at : (uint32_t)need;
        const uint32_t eq_present = (use_k && kp_key == kk_key) ? kk_take : hist[dstar];
        if (take < eq_present) {
          kp_last = find_crossing<decltype(row), NW>(
              row, [&](uint32_t key, uint32_t) { return key == kp_key ? 1.f : 0.f; }, (double)take - 0.5, sh,
              wave_tot, &result);
          if (use_k && kp_key == kk_key) kp_last = min(kp_last, kk_last);
        } else if (use_k && kp_key == kk_key) {
          kp_last = kk_last;
        }
      }
    }
    if (!p_in_window) {
      double above;
      uint32_t eq;
      kp_key = radix_descend<decltype(row), NT, NW, E::kKeyBits>(
          row, [&](uint32_t key, uint32_t) { return key >= kk_key; },
          [&](uint32_t key, uint32_t) { return wkey(key); }, true, target, rcnt, rmass, sh, &above, &eq,
          sel);
      // equal keys kept under top-k at this key
      const uint32_t eq_present = (use_k && kp_key == kk_key) ? kk_take : eq;
      const double w = (double)wkey(kp_key);
      double need = ceil((target - above) / w);
      if (need < 1.0) need = 1.0;
      const uint32_t take = need >= (double)eq_present ? eq_present : (uint32_t)need;
      if (take < eq_present) {
        kp_last = find_crossing<decltype(row), NW>(
            row, [&](uint32_t key, uint32_t) { return key == kp_key ? 1.f : 0.f; }, (double)take - 0.5, sh,
            wave_tot, &result);
        if (use_k && kp_key == kk_key) kp_last = min(kp_last, kk_last);
      } else if (use_k && kp_key == kk_key) {
        kp_last = kk_last;
      }
    }
  }

  // ---- the draw: kept weights in index order, first running mass > u * W
  const bool top_only = use_p ? p_in_window : k_in_window;
  auto kept = [&](int i, uint32_t key) {
    if (!kept_k(i, key)) return false;
    if (use_p) return key > kp_key || (key == kp_key && i <= kp_last);
    return true;
  };
  // Weights of kept elements: from the window table when every kept element
  // is inside the window, else computed.
  int32_t idx = -1;
  {
    double tsum = 0.0;
    int32_t last_kept = -1;
    float chunk_acc = 0.f;
    int last_chunk = -1;
    row.for_each([&](int i, uint32_t key, uint32_t) {
      if (!kept(i, key)) return;
      const uint32_t d = kmax - key;
      const float w = (top_only && d < (uint32_t)kSampleWindow) ? wtab[d] : wkey(key);
      const int ch = i / kEPC;
      if (ch != last_chunk) {
        tsum += (double)chunk_acc;
        chunk_acc = 0.f;
        last_chunk = ch;
      }
      chunk_acc += w;
      last_kept = max(last_kept, i);
    });
    tsum += (double)chunk_acc;
    const double Wd = block_sum_f64<NW>(tsum, sh, wave, lane);
    const int32_t lastk = block_max_i32<NW>(last_kept, sh, wave, lane);
    const double target = (double)u * Wd;
    // crossing search with index-aware weights
    const double wsum = wave_sum_f64(tsum);
    __syncthreads();
    if (lane == 0) wave_tot[wave] = wsum;
    if (threadIdx.x == 0) result = -1;
    __syncthreads();
    double pre = 0.0;
    int wstar = -1;
    for (int w = 0; w < NW; ++w) {
      if (target < pre + wave_tot[w]) { wstar = w; break; }
      pre += wave_tot[w];
    }
    if (wave == wstar) {
      double rem = target - pre;
      for (int c = 0; c < row.rounds; ++c) {
        float cs = 0.f;
        row.for_round(c, [&](int i, uint32_t key, uint32_t) {
          if (!kept(i, key)) return;
          const uint32_t d = kmax - key;
          cs += (top_only && d < (uint32_t)kSampleWindow) ? wtab[d] : wkey(key);
        });
        const double incl = wave_incl_scan_f64((double)cs, lane);
        const double tot = __shfl(incl, 63, 64);
        if (rem < tot) {
          const double excl = incl - (double)cs;
          const bool mine = excl <= rem && rem < incl;
          const uint64_t who = __ballot(mine);
          const int l0 = who ? __builtin_ctzll(who) : 63;
          if (lane == l0) {
            float run = 0.f;
            int32_t found = -1, last = -1;
            row.for_round(c, [&](int i, uint32_t key, uint32_t) {
              if (!kept(i, key)) return;
              const uint32_t d = kmax - key;
              const float x = (top_only && d < (uint32_t)kSampleWindow) ? wtab[d] : wkey(key);
              if (x > 0.f) last = i;
              run += x;
              if (found < 0 && excl + (double)run > rem) found = i;
            });
            result = found >= 0 ? found : last;
          }
          break;
        }
        rem -= tot;
      }
    }
    __syncthreads();
    idx = result >= 0 ? result : lastk;
  }
  if (threadIdx.x == 0) a.out[row_id] = idx >= 0 ? idx : argmax;
}

}  // namespace pkv
