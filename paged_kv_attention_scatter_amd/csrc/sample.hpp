// Batched per-request sampler: argmax, or temperature -> top-k -> top-p -> draw.
//
// Semantics ("Engine 与采样器", section 采样器; "Mini-SGLang 源码解析（四）：GPU
// 计算引擎系统", sections 14.3-14.4): p = softmax(logits / T); top-k keeps the
// k most probable tokens; the kept mass is renormalised; top-p keeps a ranked
// token iff the kept mass ranked before it is < p; one token is drawn from
// the rest. Greedy rows (T <= 1e-6, or no temperature array) are argmax.
//
// The pages' GPU path calls FlashInfer's rejection-sampling kernels; this is
// a different, exact design with one workgroup per row:
//
// * The row is read from HBM once into registers: wave w owns a contiguous
//   range of 16-byte chunks and lane l holds chunk w * CPW + c * 64 + l in
//   round c, so every load is coalesced and index order is (wave, round,
//   lane, element). As chunks arrive each thread folds them into its maximum,
//   the first index of it and, for rows whose top-p runs over the whole row,
//   the mass relative to a running maximum.
// * Ranking uses order-preserving integer keys of the logits (-0 ranks with
//   +0), so argmax and top-k are exact; ties go to the lower index. Weights
//   are w(l) = exp2((l - l_max) * log2(e) / T), so equal logits weigh the same.
// * Fast path: per-wave count histograms of d = key_max - key over the 256
//   largest key values. All elements of a bin share one key and one weight,
//   so the top-k threshold, the kept mass and the top-p cut come from scans
//   over 256 bins. Every element at or above the final cut is then copied,
//   in index order, into an LDS list; the ties at the cut (the first n
//   equal-key tokens in index order are kept) and the draw (kept weights in
//   index order, first running mass > u * W) are resolved on that list.
// * Rows with neither top-k nor top-p draw over the whole row: per
//   (wave, round) group masses locate the group, one chunk round is scanned.
// * A cut below the window, or more candidates than the LDS list holds,
//   falls back to a generic path over the row in memory: a radix descent
//   over the full key (8 bits per pass, count and fp64 mass histograms) and
//   group-mass scans for ties and the draw.
// Mass sums are fp32 inside a 16-byte chunk and fp64 above (the in-wave tree
// of a group mass is fp32).
#pragma once

#include "common.hpp"

#define PKV_INLINE __device__ __attribute__((always_inline)) inline

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
  static PKV_INLINE float value(const u32x4& x, int e) {
    const uint32_t w = x[e >> 1];
    return (e & 1) ? __uint_as_float(w & 0xffff0000u) : __uint_as_float(w << 16);
  }
  static PKV_INLINE uint32_t key(float v) {
    uint32_t b = __float_as_uint(v) >> 16;
    if (b == 0x8000u) b = 0;  // -0 ranks with +0
    return (b & 0x8000u) ? (~b & 0xffffu) : (b | 0x8000u);
  }
  static PKV_INLINE float key_value(uint32_t k) {
    const uint32_t b = (k & 0x8000u) ? (k & 0x7fffu) : (~k & 0xffffu);
    return __uint_as_float(b << 16);
  }
  static PKV_INLINE void set_raw(u32x4& x, int e, const void* p, int64_t i) {
    const uint32_t r = static_cast<const uint16_t*>(p)[i];
    x[e >> 1] |= (e & 1) ? (r << 16) : r;
  }
};

template <>
struct SampleElem<float> {
  static constexpr int kPerChunk = 4;
  static constexpr int kKeyBits = 32;
  static PKV_INLINE float value(const u32x4& x, int e) { return __uint_as_float(x[e]); }
  static PKV_INLINE uint32_t key(float v) {
    uint32_t b = __float_as_uint(v);
    if (b == 0x80000000u) b = 0;
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  }
  static PKV_INLINE float key_value(uint32_t k) {
    const uint32_t b = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
    return __uint_as_float(b);
  }
  static PKV_INLINE void set_raw(u32x4& x, int e, const void* p, int64_t i) {
    x[e] = static_cast<const uint32_t*>(p)[i];
  }
};

constexpr int kSampleThreads = 512;
constexpr int kSampleWaves = kSampleThreads / kWave;
constexpr int kSampleWindow = 256;      // key values below the row maximum held in the fast histogram
constexpr int kSampleMaxRounds = 512;   // chunk rounds per wave with a group-mass slot (bounds the vocabulary)
constexpr int kSampleCap = 8192;        // candidates the LDS list holds

// ---------------------------------------------------------------- wave helpers

PKV_INLINE double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
PKV_INLINE float wave_max_f32(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
PKV_INLINE int32_t wave_min_i32(int32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = min(v, __shfl_xor(v, o, 64));
  return v;
}
PKV_INLINE int32_t wave_max_i32(int32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, __shfl_xor(v, o, 64));
  return v;
}
PKV_INLINE double wave_incl_scan_f64(double v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  return v;
}
// Inclusive scan and the exclusive value taken from the previous lane's
// inclusive one, so consecutive lanes' [excl, incl) intervals meet exactly.
PKV_INLINE double wave_scan_f64(double v, int lane, double* excl) {
  const double incl = wave_incl_scan_f64(v, lane);
  const double prev = __shfl_up(incl, 1, 64);
  *excl = lane > 0 ? prev : 0.0;
  return incl;
}
PKV_INLINE int32_t wave_incl_scan_i32(int32_t v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int32_t t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  return v;
}
// Sum over the wave, returned in every lane (fp32 tree).
PKV_INLINE float wave_total_f32(float v) {
  v = group_sum<16>(v);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0)) +
         __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16)) +
         __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32)) +
         __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
}

// Shared state of one row's workgroup.
struct SampleLds {
  uint32_t hw[kSampleWaves][kSampleWindow];     // per-wave window counts
  uint32_t hist[kSampleWindow];                 // window counts
  float wtab[kSampleWindow];                    // weight of the key at distance d below the maximum
  float gsum[kSampleWaves * kSampleMaxRounds];  // group masses, group = (wave, round)
  int32_t cidx[kSampleCap];                     // candidate list: index ...
  uint8_t cd[kSampleCap];                       // ... and its distance d
  uint32_t rcnt[256];                           // radix descent: digit counts
  double rmass[256];                            //                digit masses
  double wave_f[kSampleWaves];
  float wave_v[kSampleWaves];
  int32_t wave_i[kSampleWaves];
  int32_t wave_j[kSampleWaves];
  double scan_f[kSampleWaves];
  int32_t pick_bin;
  uint32_t pick_cnt;
  double pick_above;
  int32_t result;
};

// Block-wide sum, returned in every thread; starts and ends with a barrier.
PKV_INLINE double block_sum_f64(SampleLds& s, double v) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_sum_f64(v);
  __syncthreads();
  if (lane == 0) s.wave_f[wave] = v;
  __syncthreads();
  double t = 0.0;
  for (int w = 0; w < kSampleWaves; ++w) t += s.wave_f[w];
  __syncthreads();
  return t;
}
// Exclusive block scans in thread order; *total = the sum over the block.
PKV_INLINE int32_t block_excl_scan_i32(SampleLds& s, int32_t v, int32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int32_t incl = wave_incl_scan_i32(v, lane);
  __syncthreads();
  if (lane == 63) s.wave_j[wave] = incl;
  __syncthreads();
  int32_t off = 0, tot = 0;
  for (int w = 0; w < kSampleWaves; ++w) {
    if (w < wave) off += s.wave_j[w];
    tot += s.wave_j[w];
  }
  __syncthreads();
  *total = tot;
  return off + incl - v;
}
// Block scan in thread order: returns the exclusive prefix, *incl_out the
// inclusive one (equal to the next thread's exclusive prefix, bit for bit).
PKV_INLINE double block_scan_f64(SampleLds& s, double v, double* incl_out, double* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  double excl;
  const double incl = wave_scan_f64(v, lane, &excl);
  __syncthreads();
  if (lane == 63) s.scan_f[wave] = incl;
  __syncthreads();
  double off = 0.0, tot = 0.0;
  for (int w = 0; w < kSampleWaves; ++w) {
    if (w < wave) off += s.scan_f[w];
    tot += s.scan_f[w];
  }
  __syncthreads();
  *total = tot;
  *incl_out = off + incl;
  return off + excl;
}

// Scan over 256 bins in ascending order by the first four waves (one bin per
// thread): every thread gets the first bin whose inclusive running amount
// reaches `goal` (-1 if none), the amount strictly before it and count(bin).
template <class AF, class CF>
PKV_INLINE void window_select(SampleLds& s, AF amount, CF count, double goal, int* bin, double* before,
                              uint32_t* cnt) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __syncthreads();
  if (tid == 0) s.pick_bin = -1;
  double a = 0.0, incl = 0.0, excl = 0.0;
  if (wave < 4) {
    a = amount(tid);
    incl = wave_scan_f64(a, lane, &excl);
    if (lane == 63) s.scan_f[wave] = incl;
  }
  __syncthreads();
  if (wave < 4) {
    double off = 0.0;
    for (int w = 0; w < wave; ++w) off += s.scan_f[w];
    const double inc = off + incl, exc = off + excl;
    if (a > 0.0 && exc < goal && goal <= inc) {  // unique: the bins' intervals meet exactly
      s.pick_bin = tid;
      s.pick_above = exc;
      s.pick_cnt = count(tid);
    }
  }
  __syncthreads();
  *bin = s.pick_bin;
  *before = s.pick_above;
  *cnt = s.pick_cnt;
  __syncthreads();
}

// The row as 16-byte chunks. REG: MAXR rounds are loaded once into registers;
// otherwise every pass reads the chunks from memory.
template <typename T, int MAXR, bool REG>
struct SampleRow {
  using E = SampleElem<T>;
  static constexpr int EPC = E::kPerChunk;
  const T* base;
  int V, nchunks, cpw, rounds, wave, lane;
  u32x4 reg[REG ? MAXR : 1];

  PKV_INLINE int chunk_id(int c) const { return wave * cpw + c * kWave + lane; }
  PKV_INLINE bool chunk_ok(int c) const { return c * kWave + lane < cpw && chunk_id(c) < nchunks; }
  PKV_INLINE u32x4 fetch(int c) const {
    u32x4 x = {0u, 0u, 0u, 0u};
    if (!chunk_ok(c)) return x;
    const int64_t ch = chunk_id(c);
    if ((ch + 1) * EPC <= V) return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base) + ch);
#pragma unroll
    for (int e = 0; e < EPC; ++e)  // the last, partial chunk of a row
      if (ch * EPC + e < V) E::set_raw(x, e, base, ch * EPC + e);
    return x;
  }
  PKV_INLINE void init(const T* b, int vocab, int w, int l) {
    base = b;
    V = vocab;
    nchunks = (vocab + EPC - 1) / EPC;
    cpw = (nchunks + kSampleWaves - 1) / kSampleWaves;
    rounds = (cpw + kWave - 1) / kWave;
    wave = w;
    lane = l;
    if constexpr (REG) {
#pragma unroll
      for (int c = 0; c < MAXR; ++c)
        if (c < rounds) reg[c] = fetch(c);
    }
  }
  // f(c, x, ok) for every round c < rounds, in order; the loop is wave-uniform.
  template <class F>
  PKV_INLINE void for_rounds(F f) const {
    if constexpr (REG) {
#pragma unroll
      for (int c = 0; c < MAXR; ++c)
        if (c < rounds) f(c, reg[c], chunk_ok(c));
    } else {
      for (int c = 0; c < rounds; ++c) f(c, fetch(c), chunk_ok(c));
    }
  }
  // The chunk of round c, read again from memory: selecting one register
  // chunk by a run-time round would put the whole array in scratch.
  PKV_INLINE u32x4 chunk(int c) const { return fetch(c); }
  // f(i, l) for every element (index, logit) of chunk x of round c.
  template <class F>
  PKV_INLINE void elements(int c, const u32x4& x, bool ok, F f) const {
    if (!ok) return;
    const int i0 = chunk_id(c) * EPC;
#pragma unroll
    for (int e = 0; e < EPC; ++e)
      if (i0 + e < V) f(i0 + e, E::value(x, e));
  }
  template <class F>
  PKV_INLINE void for_each(F f) const {
    for_rounds([&](int c, const u32x4& x, bool ok) { elements(c, x, ok, f); });
  }
};

// w(l) = exp2((l - l_max) * c2)
PKV_INLINE float row_weight(float l, float lmax, float c2) { return fast_exp2((l - lmax) * c2); }

// Block sum of v(i, l) over the row.
template <class RowT, class VF>
PKV_INLINE double row_sum(const RowT& row, SampleLds& s, VF v) {
  double t = 0.0;
  row.for_rounds([&](int c, const u32x4& x, bool ok) {
    float cs = 0.f;
    row.elements(c, x, ok, [&](int i, float l) { cs += v(i, l); });
    t += (double)cs;
  });
  return block_sum_f64(s, t);
}

// First element, in index order, at which the running sum of v(i, l) >= 0
// exceeds target_of(total); if none, the last element with v > 0 (-1 if no
// element has v > 0). Group masses are stored per (wave, round); wave 0
// locates the group, the group's wave scans its one chunk round.
template <class RowT, class VF, class TF>
PKV_INLINE int32_t find_crossing(const RowT& row, SampleLds& s, VF v, TF target_of) {
  const int wave = row.wave, lane = row.lane, R = row.rounds;
  int32_t tlast = -1;
  __syncthreads();
  row.for_rounds([&](int c, const u32x4& x, bool ok) {
    float cs = 0.f;
    row.elements(c, x, ok, [&](int i, float l) {
      const float w = v(i, l);
      if (w > 0.f) tlast = i;
      cs += w;
    });
    const float g = wave_total_f32(cs);
    if (lane == 0) s.gsum[wave * R + c] = g;
  });
  const int32_t wlast = wave_max_i32(tlast);
  if (lane == 0) s.wave_i[wave] = wlast;
  if (threadIdx.x == 0) s.pick_bin = -1;
  __syncthreads();
  if (wave == 0) {
    // groups in index order: g = wave * R + round; each lane takes a contiguous run
    const int G = kSampleWaves * R, per = (G + kWave - 1) / kWave;
    const int g0 = min(G, lane * per), g1 = min(G, g0 + per);
    double own = 0.0;
    for (int g = g0; g < g1; ++g) own += (double)s.gsum[g];
    double run;
    const double incl = wave_scan_f64(own, lane, &run);
    const double total = __shfl(incl, 63, 64);
    const double target = target_of(total);
    if (own > 0.0 && run <= target && target < incl) {
      int gp = -1;
      double rp = 0.0;
      for (int g = g0; g < g1; ++g) {
        const double gs = (double)s.gsum[g];
        if (gs > 0.0) {
          gp = g;  // rounding left the target past the sequential sum: the last non-empty group
          rp = target - run;
          if (target < run + gs) break;
        }
        run += gs;
      }
      s.pick_bin = gp;
      s.pick_above = rp;
    }
  }
  __syncthreads();
  const int gstar = s.pick_bin;
  const double rem = s.pick_above;
  int32_t last = -1;
  for (int w = 0; w < kSampleWaves; ++w) last = max(last, s.wave_i[w]);
  if (gstar >= 0 && wave == gstar / R) {
    const int c = gstar % R;
    const u32x4 x = row.chunk(c);
    const bool ok = row.chunk_ok(c);
    float cs = 0.f;
    int32_t lastv = -1;
    row.elements(c, x, ok, [&](int i, float l) {
      const float w = v(i, l);
      if (w > 0.f) lastv = i;
      cs += w;
    });
    double excl;
    const double incl = wave_scan_f64((double)cs, lane, &excl);
    const uint64_t who = __ballot(cs > 0.f && excl <= rem && rem < incl);
    int32_t res = wave_max_i32(lastv);  // rounding pushed the target past the group: its last element
    if (who) {
      const int l0 = __ffsll((unsigned long long)who) - 1;
      int32_t found = -1;
      if (lane == l0) {
        float runf = 0.f;
        row.elements(c, x, ok, [&](int i, float l) {
          runf += v(i, l);
          if (found < 0 && excl + (double)runf > rem) found = i;
        });
        if (found < 0) found = lastv;
      }
      res = __shfl(found, l0, 64);
    }
    if (lane == 0) s.result = res;
  }
  __syncthreads();
  const int32_t r = gstar >= 0 ? s.result : last;
  __syncthreads();
  return r >= 0 ? r : last;
}

// Radix descent over the full key (8 bits per pass) among elements with
// pred(i, l). By count: the key of the element ranked `goal` (1-based,
// descending). By mass: the key group where the mass ranked before it is
// < goal <= that plus the group's mass (the lowest group if rounding never
// reaches goal). Returns the key; *above = count or mass strictly above it,
// *eq = the group's count.
template <class RowT, int KEYBITS, class PF, class WF>
PKV_INLINE uint32_t radix_descend(const RowT& row, SampleLds& s, PF pred, WF weight, bool by_mass, double goal,
                                  double* above_out, uint32_t* eq_out) {
  using E = typename RowT::E;
  uint32_t prefix = 0, mask = 0;
  double above = 0.0;
  uint32_t eq = 0;
  for (int shift = KEYBITS - 8; shift >= 0; shift -= 8) {
    __syncthreads();
    for (int b = threadIdx.x; b < 256; b += kSampleThreads) {
      s.rcnt[b] = 0;
      s.rmass[b] = 0.0;
    }
    __syncthreads();
    row.for_each([&](int i, float l) {
      const uint32_t key = E::key(l);
      if ((key & mask) == prefix && pred(i, l)) {
        const uint32_t dgt = (key >> shift) & 0xffu;
        atomicAdd(&s.rcnt[dgt], 1u);
        if (by_mass) atomicAdd(&s.rmass[dgt], (double)weight(l));
      }
    });
    // bin b of the scan is digit 255 - b (descending keys)
    int bin;
    double before;
    uint32_t cnt;
    window_select(
        s, [&](int b) { return by_mass ? s.rmass[255 - b] : (double)s.rcnt[255 - b]; },
        [&](int b) { return s.rcnt[255 - b]; }, goal - above, &bin, &before, &cnt);
    if (bin < 0) {  // rounding: goal beyond everything -> the lowest non-empty digit
      if (threadIdx.x == 0) {
        int lo = -1;
        double acc = 0.0, acc_lo = 0.0;
        for (int b = 255; b >= 0; --b)
          if (s.rcnt[b]) {
            acc_lo = acc;
            acc += by_mass ? s.rmass[b] : (double)s.rcnt[b];
            lo = b;
          }
        s.pick_bin = 255 - (lo < 0 ? 0 : lo);
        s.pick_cnt = lo < 0 ? 0 : s.rcnt[lo];
        s.pick_above = acc_lo;
      }
      __syncthreads();
      bin = s.pick_bin;
      cnt = s.pick_cnt;
      before = s.pick_above;
      __syncthreads();
    }
    prefix |= (uint32_t)(255 - bin) << shift;
    mask |= 0xffu << shift;
    above += before;
    eq = cnt;
  }
  *above_out = above;
  *eq_out = eq;
  return prefix;
}

// Row parameters and the results of the first passes, shared by both paths.
struct SampleRowState {
  float lmax, c2, u, p;
  uint32_t kmax;
  int32_t k, argmax;
  bool use_k, use_p;
  double wall;   // whole-row mass (rows with top-p and no top-k)
  int dk;        // window bin of the top-k threshold, -1 if below the window
  uint32_t kk_take, kk_eq;
};

// Generic cuts and draw over the row in memory (any cut depth, any number of
// kept tokens). The window histogram in s.hist / s.wtab is valid.
template <class RowT>
PKV_INLINE int32_t sample_generic(const RowT& row, SampleLds& s, const SampleRowState& st) {
  using E = typename RowT::E;
  const uint32_t kmax = st.kmax;
  const float lmax = st.lmax, c2 = st.c2;
  auto wt = [&](float l) { return row_weight(l, lmax, c2); };

  // top-k: threshold key kk_key; equal keys kept up to index kk_last
  uint32_t kk_key = 0, kk_take = st.kk_take, kk_eq = st.kk_eq;
  if (st.use_k) {
    if (st.dk >= 0) {
      kk_key = kmax - (uint32_t)st.dk;
    } else {
      double ab;
      kk_key = radix_descend<RowT, E::kKeyBits>(row, s, [](int, float) { return true; },
                                                [](float) { return 0.f; }, false, (double)st.k, &ab, &kk_eq);
      kk_take = (uint32_t)st.k - (uint32_t)ab;
    }
  }
  int32_t kk_last = 0x7fffffff;
  if (st.use_k && kk_take < kk_eq) {
    const double goal = (double)kk_take - 0.5;
    kk_last = find_crossing(
        row, s, [&](int, float l) { return E::key(l) == kk_key ? 1.f : 0.f; }, [&](double) { return goal; });
  }
  auto kept_k = [&](int i, float l) {
    if (!st.use_k) return true;
    const uint32_t key = E::key(l);
    return key > kk_key || (key == kk_key && i <= kk_last);
  };

  // kept mass after top-k
  double Wk = st.wall;
  if (st.use_k) Wk = row_sum(row, s, [&](int i, float l) { return kept_k(i, l) ? wt(l) : 0.f; });

  // top-p: cut key kp_key; equal keys kept up to index kp_last
  uint32_t kp_key = 0;
  int32_t kp_last = 0x7fffffff;
  if (st.use_p) {
    const double target = (double)st.p * Wk;
    int dstar = -1;
    double above = 0.0;
    uint32_t n_at = 0;
    if (!st.use_k || st.dk >= 0) {  // every kept element's bin is in the window
      const int dlim = st.use_k ? st.dk : kSampleWindow - 1;
      window_select(
          s,
          [&](int b) {
            const uint32_t n = b < dlim ? s.hist[b] : (b == dlim ? (st.use_k ? kk_take : s.hist[b]) : 0u);
            return (double)n * (double)s.wtab[b];
          },
          [&](int b) { return (st.use_k && b == st.dk) ? kk_take : s.hist[b]; }, target, &dstar, &above, &n_at);
    }
    if (dstar >= 0) {
      kp_key = kmax - (uint32_t)dstar;
    } else {
      kp_key = radix_descend<RowT, E::kKeyBits>(row, s, kept_k, wt, true, target, &above, &n_at);
    }
    // equal-key tokens at the cut: token j of the group (0-based) is kept iff above + j * w < target
    const double w = (double)wt(E::key_value(kp_key));
    double need = ceil((target - above) / w);
    if (!(need >= 1.0)) need = 1.0;
    const uint32_t take = need >= (double)n_at ? n_at : (uint32_t)need;
    if (take < n_at) {
      const double goal = (double)take - 0.5;
      kp_last = find_crossing(
          row, s, [&](int i, float l) { return (E::key(l) == kp_key && kept_k(i, l)) ? 1.f : 0.f; },
          [&](double) { return goal; });
    } else if (st.use_k && kp_key == kk_key) {
      kp_last = kk_last;
    }
  }

  // the draw: kept weights in index order, first running mass > u * W
  const float u = st.u;
  return find_crossing(
      row, s,
      [&](int i, float l) -> float {
        if (!kept_k(i, l)) return 0.f;
        const uint32_t key = E::key(l);
        if (st.use_p && !(key > kp_key || (key == kp_key && i <= kp_last))) return 0.f;
        return wt(l);
      },
      [&](double total) { return (double)u * total; });
}

template <typename T, int MAXR, bool REG>
__global__ void __launch_bounds__(kSampleThreads) sample_kernel(SampleArgs a) {
  using E = SampleElem<T>;
  using RowT = SampleRow<T, MAXR, REG>;
  constexpr int W = kSampleWindow;
  __shared__ SampleLds s;
  const int row_id = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int V = a.vocab;
  const T* row_ptr = reinterpret_cast<const T*>(a.logits) + (int64_t)row_id * a.row_stride;

  // Row parameters (uniform).
  SampleRowState st;
  const float temp = a.temperature ? a.temperature[row_id] : 0.f;
  const bool greedy = !a.temperature || temp <= 1e-6f;
  st.k = (!greedy && a.top_k) ? a.top_k[row_id] : 0;
  st.use_k = st.k > 0 && st.k < V;
  if (!st.use_k) st.k = V;
  st.p = (!greedy && a.top_p) ? a.top_p[row_id] : 1.f;
  st.use_p = st.p < 1.f;
  if (st.use_p) st.p = fmaxf(st.p, 1e-6f);
  st.c2 = greedy ? 0.f : 1.4426950408889634f / temp;
  st.u = greedy ? 0.f : a.uniforms[row_id];
  const bool full_mass = !greedy && st.use_p && !st.use_k;  // top-p over the whole row needs its mass
  const float c2 = st.c2;

  RowT row;
  row.init(row_ptr, V, wave, lane);

  // ---- pass 1: maximum, its first index, and (full_mass) the mass relative
  // to a running maximum
  float vmax = -INFINITY, mrun = -INFINITY;
  int32_t imax = 0x7fffffff;
  double wrun = 0.0;
  row.for_rounds([&](int c, const u32x4& x, bool ok) {
    float cmax = -INFINITY;
    int32_t carg = 0x7fffffff;
    row.elements(c, x, ok, [&](int i, float l) {
      if (l > cmax) {
        cmax = l;
        carg = i;
      }
    });
    if (cmax > vmax) {
      vmax = cmax;
      imax = carg;
    }
    if (full_mass && cmax > -INFINITY) {
      if (cmax > mrun) {
        wrun *= (double)fast_exp2((mrun - cmax) * c2);
        mrun = cmax;
      }
      float cs = 0.f;
      row.elements(c, x, ok, [&](int, float l) { cs += row_weight(l, mrun, c2); });
      wrun += (double)cs;
    }
  });
  float m = wave_max_f32(vmax);
  if (lane == 0) s.wave_v[wave] = m;
  __syncthreads();
  m = s.wave_v[0];
  for (int w = 1; w < kSampleWaves; ++w) m = fmaxf(m, s.wave_v[w]);
  st.lmax = m;
  const int32_t cand = wave_min_i32((vmax == m) ? imax : 0x7fffffff);
  if (lane == 0) s.wave_i[wave] = cand;
  __syncthreads();
  int32_t am = s.wave_i[0];
  for (int w = 1; w < kSampleWaves; ++w) am = min(am, s.wave_i[w]);
  st.argmax = am == 0x7fffffff ? 0 : am;
  if (greedy) {
    if (tid == 0) a.out[row_id] = st.argmax;
    return;
  }
  const float lmax = st.lmax;
  st.kmax = E::key(lmax);
  const uint32_t kmax = st.kmax;
  auto wt = [&](float l) { return row_weight(l, lmax, c2); };

  st.wall = 0.0;
  if (full_mass)
    st.wall = block_sum_f64(s, (mrun > -INFINITY) ? wrun * (double)fast_exp2((mrun - lmax) * c2) : 0.0);

  // ---- plain rows: the draw over the whole row
  if (!st.use_k && !st.use_p) {
    const float u = st.u;
    const int32_t idx = find_crossing(row, s, [&](int, float l) { return wt(l); },
                                      [&](double total) { return (double)u * total; });
    if (tid == 0) a.out[row_id] = idx >= 0 ? idx : st.argmax;
    return;
  }

  // ---- pass 2: per-wave window histograms of d = kmax - key
  __syncthreads();
  for (int b = tid; b < kSampleWaves * W; b += kSampleThreads) (&s.hw[0][0])[b] = 0;
  for (int b = tid; b < W; b += kSampleThreads)
    s.wtab[b] = kmax >= (uint32_t)b ? wt(E::key_value(kmax - (uint32_t)b)) : 0.f;
  __syncthreads();
  row.for_each([&](int, float l) {
    const uint32_t d = kmax - E::key(l);
    if (d < (uint32_t)W) atomicAdd(&s.hw[wave][d], 1u);
  });
  __syncthreads();
  for (int b = tid; b < W; b += kSampleThreads) {
    uint32_t n = 0;
    for (int w = 0; w < kSampleWaves; ++w) n += s.hw[w][b];
    s.hist[b] = n;
  }
  __syncthreads();

  // ---- top-k threshold from the window
  st.dk = -1;
  st.kk_take = 0;
  st.kk_eq = 0;
  bool fast = true;
  if (st.use_k) {
    double before;
    window_select(s, [&](int b) { return (double)s.hist[b]; }, [&](int b) { return s.hist[b]; }, (double)st.k,
                  &st.dk, &before, &st.kk_eq);
    if (st.dk >= 0)
      st.kk_take = (uint32_t)st.k - (uint32_t)before;
    else
      fast = false;
  }

  // ---- top-p cut from the window
  int dcut = st.dk;
  uint32_t take = st.kk_take;
  if (fast && st.use_p) {
    double Wk = st.wall;
    if (st.use_k) {
      double t = 0.0;
      if (tid < W) {
        const uint32_t n = tid < st.dk ? s.hist[tid] : (tid == st.dk ? st.kk_take : 0u);
        t = (double)n * (double)s.wtab[tid];
      }
      Wk = block_sum_f64(s, t);
    }
    const double target = (double)st.p * Wk;
    const int dlim = st.use_k ? st.dk : W - 1;
    int dstar;
    double above;
    uint32_t n_at;
    window_select(
        s,
        [&](int b) {
          const uint32_t n = b < dlim ? s.hist[b] : (b == dlim ? (st.use_k ? st.kk_take : s.hist[b]) : 0u);
          return (double)n * (double)s.wtab[b];
        },
        [&](int b) { return (st.use_k && b == st.dk) ? st.kk_take : s.hist[b]; }, target, &dstar, &above, &n_at);
    if (dstar < 0) {
      fast = false;
    } else {
      const double w = (double)s.wtab[dstar];
      double need = ceil((target - above) / w);
      if (!(need >= 1.0)) need = 1.0;
      dcut = dstar;
      take = need >= (double)n_at ? n_at : (uint32_t)need;
    }
  }

  // ---- candidates: every element with d <= dcut, copied in index order
  if (fast) {
    int32_t cw = 0;
    for (int b = lane; b <= dcut; b += kWave) cw += (int32_t)s.hw[wave][b];
    cw = __shfl(wave_incl_scan_i32(cw, lane), 63, 64);  // this wave's candidates
    int32_t ncand;
    const int32_t wbase = __shfl(block_excl_scan_i32(s, lane == 0 ? cw : 0, &ncand), 0, 64);
    if (ncand > kSampleCap) fast = false;

    if (fast) {
      int32_t run = wbase;
      row.for_rounds([&](int c, const u32x4& x, bool ok) {
        const int i0 = row.chunk_id(c) * E::kPerChunk;
        uint32_t flags = 0;
#pragma unroll
        for (int e = 0; e < E::kPerChunk; ++e) {
          const bool in = ok && i0 + e < V && (kmax - E::key(E::value(x, e))) <= (uint32_t)dcut;
          flags |= (uint32_t)in << e;
        }
        if (__ballot(flags != 0)) {
          const int32_t mine = __popc(flags);
          const int32_t incl = wave_incl_scan_i32(mine, lane);
          int32_t pos = run + incl - mine;
#pragma unroll
          for (int e = 0; e < E::kPerChunk; ++e) {
            if (flags & (1u << e)) {
              s.cidx[pos] = i0 + e;
              s.cd[pos] = (uint8_t)(kmax - E::key(E::value(x, e)));
              ++pos;
            }
          }
          run += __shfl(incl, 63, 64);
        }
      });
      __syncthreads();

      // ---- ties at the cut and the draw, on the list
      const int per = (ncand + kSampleThreads - 1) / kSampleThreads;
      const int j0 = min(ncand, tid * per), j1 = min(ncand, j0 + per);
      int32_t at = 0;
      for (int j = j0; j < j1; ++j) at += s.cd[j] == dcut;
      int32_t tot_at;
      const int32_t rank0 = block_excl_scan_i32(s, at, &tot_at);  // rank of this thread's first entry at the cut
      double own = 0.0;
      int32_t last_kept = -1;
      int32_t rank = rank0;
      for (int j = j0; j < j1; ++j) {
        const int d = s.cd[j];
        bool kept = d < dcut;
        if (d == dcut) kept = (uint32_t)(rank++) < take;
        if (kept) {
          own += (double)s.wtab[d];
          last_kept = j;
        }
      }
      double total, incl;
      const double excl = block_scan_f64(s, own, &incl, &total);
      const double target = (double)st.u * total;
      const int32_t lk = wave_max_i32(last_kept);
      if (lane == 0) s.wave_i[wave] = lk;
      if (tid == 0) s.result = -1;
      __syncthreads();
      if (own > 0.0 && excl <= target && target < incl) {
        rank = rank0;
        double runm = excl;
        int32_t found = last_kept;
        for (int j = j0; j < j1; ++j) {
          const int d = s.cd[j];
          bool kept = d < dcut;
          if (d == dcut) kept = (uint32_t)(rank++) < take;
          if (kept) {
            runm += (double)s.wtab[d];
            if (runm > target) {
              found = j;
              break;
            }
          }
        }
        s.result = found;
      }
      __syncthreads();
      int32_t j = s.result;
      if (j < 0)
        for (int w = 0; w < kSampleWaves; ++w) j = max(j, s.wave_i[w]);
      if (tid == 0) a.out[row_id] = j >= 0 ? s.cidx[j] : st.argmax;
      return;
    }
  }

  // ---- generic path over the row in memory
  SampleRow<T, 1, false> grow;
  grow.init(row_ptr, V, wave, lane);
  const int32_t idx = sample_generic(grow, s, st);
  if (tid == 0) a.out[row_id] = idx >= 0 ? idx : st.argmax;
}

}  // namespace pkv
