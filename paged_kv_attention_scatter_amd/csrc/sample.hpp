// Batched per-request sampler: argmax, or temperature -> top-k -> top-p -> draw.
//
// Semantics ("Engine 与采样器", section 采样器; "Mini-SGLang 源码解析（四）：GPU
// 计算引擎系统", sections 14.3-14.4): p = softmax(logits / T); top-k keeps the
// k most probable tokens; the kept mass is renormalised; top-p keeps a ranked
// token iff the kept mass ranked before it is < p; one token is drawn from
// the rest. Greedy rows (T <= 1e-6, or no temperature array) are argmax.
//
// The pages' GPU path calls FlashInfer's rejection-sampling kernels; this is
// a different, exact design with one workgroup per row. Ranking uses
// order-preserving integer keys of the logits (-0 ranks with +0), so argmax
// and top-k are exact and ties go to the lower index; weights are
// w(l) = exp2((l - l_max) * log2(e) / T), so equal logits weigh the same.
//
// bf16 rows (slice kernel + finish kernel):
// * Each row is cut into slices of 8192 tokens, one workgroup per slice
//   (about 19 per row on a 151936-token vocabulary, so the chip is full even
//   for small batches). A slice reads its tokens once, turns them into
//   order-preserving biased 16-bit keys with packed 16-bit integer ops (-0
//   and +0 share a key) and hands over its maximum, the first index of it,
//   its mass (rows whose draw or top-p runs over the whole row) and, in
//   index order, every token within 128 key values of its maximum.
// * The finish kernel (one workgroup per row) takes the row maximum, keeps
//   the handed-over tokens within 128 keys of it (a superset is handed over,
//   since no slice maximum exceeds the row's) in an LDS list in index order,
//   and finds the top-k threshold and the top-p cut from a count histogram of
//   the list: all tokens of a bin share one key and one weight. The ties at
//   the cut (the first n equal-key tokens in index order are kept) and the
//   draw (kept weights in index order, first running mass > u * W) run on
//   the list. Rows with neither top-k nor top-p locate their slice by the
//   slices' masses and scan it. Cuts below the window and lists that
//   overflow take the generic path below over the row in memory.
//
// fp32 rows (the memory kernel) and the generic path: every
// pass reads 16-byte chunks from memory (wave w owns a contiguous chunk range,
// lane l reads chunk w * CPW + 64c + l in round c). Cuts by radix descent over
// the full key (8 bits per pass, count and fp64 mass histograms); ties and the
// draw by per-(wave, round) group masses that locate one chunk round.
//
// Mass sums are fp32 over at most 8 tokens (a 16-byte chunk, or one round of
// a thread) or one wave's group, and fp64 above.
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
};

constexpr int kSampleThreads = 512;
constexpr int kSampleWaves = kSampleThreads / kWave;
constexpr int kSampleWindow = 128;      // bf16: key values at or below the maximum in the window list
constexpr int kSampleMaxRounds = 512;   // memory passes: chunk rounds per wave with a group-mass slot

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
PKV_INLINE int32_t wave_sum_i32(int32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
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
// Set bits of m below this lane.
PKV_INLINE int32_t lanes_below(uint64_t m) {
  return (int32_t)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// ---------------------------------------------------------------- packed bf16 keys

typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
typedef int16_t i16x2 __attribute__((ext_vector_type(2)));

PKV_INLINE u16x2 as_u16x2(uint32_t w) { return __builtin_bit_cast(u16x2, w); }
PKV_INLINE uint32_t as_u32(u16x2 v) { return __builtin_bit_cast(uint32_t, v); }

// Two bf16 values -> two biased 16-bit keys, order-preserving: a positive
// value b maps to 0x8000 + b, a negative one to 0x8000 - |b|, so -0 and +0
// share 0x8000 and -inf is 0x0080. Four packed/bitwise ops per pair.
PKV_INLINE uint32_t bf16x2_keys(uint32_t w) {
  const i16x2 sgn = __builtin_bit_cast(i16x2, w) >> (int16_t)15;  // 0xffff in negative halves
  const uint32_t sg = __builtin_bit_cast(uint32_t, sgn);
  const uint32_t x = w ^ (sg | 0x80008000u);     // positive: b | 0x8000; negative: 0x7fff - |b|
  return as_u32(as_u16x2(x) - as_u16x2(sg));      // negative halves + 1
}
// The bf16 value of a biased key.
PKV_INLINE float key16_value(uint32_t k) {
  const uint32_t b = k >= 0x8000u ? (k - 0x8000u) : (0x8000u | (0x8000u - k));
  return __uint_as_float(b << 16);
}

// ---------------------------------------------------------------- shared state

struct SampleLds {
  float gsum[kSampleWaves * kSampleMaxRounds];  // memory passes: group masses, group = (wave, round)
  uint32_t hist[256];    // window counts
  float wtab[256];       // weight of the key d below the maximum
  uint32_t rcnt[256];    // radix descent: digit counts
  double rmass[256];     //                digit masses
  int32_t seg_n[kSampleWaves];
  double wave_f[kSampleWaves];
  int32_t wave_i[kSampleWaves];
  int32_t wave_j[kSampleWaves];
  double scan_f[kSampleWaves];
  int32_t pick_bin;
  uint32_t pick_cnt;
  double pick_above;
  int32_t result;
};

// Block-wide reductions, returned in every thread; they start and end with a barrier.
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
PKV_INLINE int32_t block_reduce_i32(SampleLds& s, int32_t v, bool want_max) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = want_max ? wave_max_i32(v) : wave_min_i32(v);
  __syncthreads();
  if (lane == 0) s.wave_j[wave] = v;
  __syncthreads();
  int32_t t = s.wave_j[0];
  for (int w = 1; w < kSampleWaves; ++w) t = want_max ? max(t, s.wave_j[w]) : min(t, s.wave_j[w]);
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
// Returns the exclusive prefix; *incl_out = the inclusive one (equal to the
// next thread's exclusive prefix, bit for bit).
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

// ---------------------------------------------------------------- the row in memory

template <typename T>
struct SampleRow {
  using E = SampleElem<T>;
  static constexpr int EPC = E::kPerChunk;
  const T* base;
  int V, nchunks, cpw, rounds, wave, lane;

  PKV_INLINE void init(const T* b, int vocab, int w, int l) {
    base = b;
    V = vocab;
    nchunks = (vocab + EPC - 1) / EPC;
    cpw = (nchunks + kSampleWaves - 1) / kSampleWaves;
    rounds = (cpw + kWave - 1) / kWave;
    wave = w;
    lane = l;
  }
  PKV_INLINE int chunk_id(int c) const { return wave * cpw + c * kWave + lane; }
  PKV_INLINE bool chunk_ok(int c) const { return c * kWave + lane < cpw && chunk_id(c) < nchunks; }
  // The 16-byte block of chunk c, read whole: a row's last block may extend
  // past the vocabulary, but it is 16-byte aligned and starts inside the
  // row, so it never crosses a page; elements at or past V are never used.
  PKV_INLINE u32x4 fetch(int c) const {
    u32x4 x = {0u, 0u, 0u, 0u};
    if (chunk_ok(c)) x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base) + chunk_id(c));
    return x;
  }
  // f(c, x, ok) for every round c < rounds, in order (wave-uniform loop).
  template <class F>
  PKV_INLINE void for_rounds(F f) const {
    for (int c = 0; c < rounds; ++c) f(c, fetch(c), chunk_ok(c));
  }
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
    const u32x4 x = row.fetch(c);
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
template <class RowT, class PF, class WF>
PKV_INLINE uint32_t radix_descend(const RowT& row, SampleLds& s, PF pred, WF weight, bool by_mass, double goal,
                                  double* above_out, uint32_t* eq_out) {
  using E = typename RowT::E;
  uint32_t prefix = 0, mask = 0;
  double above = 0.0;
  uint32_t eq = 0;
  for (int shift = E::kKeyBits - 8; shift >= 0; shift -= 8) {
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

// Per-row parameters (wave-uniform).
struct SampleParams {
  float c2, u, p;
  int32_t k;
  bool greedy, use_k, use_p;

  PKV_INLINE void load(const SampleArgs& a, int row, int V) {
    const float temp = a.temperature ? a.temperature[row] : 0.f;
    greedy = !a.temperature || temp <= 1e-6f;
    k = (!greedy && a.top_k) ? a.top_k[row] : 0;
    use_k = k > 0 && k < V;
    if (!use_k) k = V;
    p = (!greedy && a.top_p) ? a.top_p[row] : 1.f;
    use_p = p < 1.f;
    if (use_p) p = fmaxf(p, 1e-6f);
    c2 = greedy ? 0.f : 1.4426950408889634f / temp;
    u = greedy ? 0.f : a.uniforms[row];
  }
};

// Cuts and draw over the row in memory (any cut depth, any number of kept
// tokens): radix descents for the top-k threshold and the top-p cut,
// group-mass scans for the ties at each cut and for the draw.
template <class RowT>
PKV_INLINE int32_t sample_generic(const RowT& row, SampleLds& s, const SampleParams& sp, float lmax) {
  using E = typename RowT::E;
  const float c2 = sp.c2;
  auto wt = [&](float l) { return row_weight(l, lmax, c2); };

  // top-k: threshold key kk_key; equal keys kept up to index kk_last
  uint32_t kk_key = 0, kk_eq = 0, kk_take = 0;
  int32_t kk_last = 0x7fffffff;
  if (sp.use_k) {
    double ab;
    kk_key = radix_descend(row, s, [](int, float) { return true; }, [](float) { return 0.f; }, false,
                           (double)sp.k, &ab, &kk_eq);
    kk_take = (uint32_t)sp.k - (uint32_t)ab;
    if (kk_take < kk_eq) {
      const double goal = (double)kk_take - 0.5;
      kk_last = find_crossing(
          row, s, [&](int, float l) { return E::key(l) == kk_key ? 1.f : 0.f; }, [&](double) { return goal; });
    }
  }
  auto kept_k = [&](int i, float l) {
    if (!sp.use_k) return true;
    const uint32_t key = E::key(l);
    return key > kk_key || (key == kk_key && i <= kk_last);
  };

  // top-p: cut key kp_key; equal keys kept up to index kp_last
  uint32_t kp_key = 0;
  int32_t kp_last = 0x7fffffff;
  if (sp.use_p) {
    const double Wk = row_sum(row, s, [&](int i, float l) { return kept_k(i, l) ? wt(l) : 0.f; });
    const double target = (double)sp.p * Wk;
    double above;
    uint32_t n_at;
    kp_key = radix_descend(row, s, kept_k, wt, true, target, &above, &n_at);
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
    } else if (sp.use_k && kp_key == kk_key) {
      kp_last = kk_last;
    }
  }

  // the draw: kept weights in index order, first running mass > u * W
  const float u = sp.u;
  return find_crossing(
      row, s,
      [&](int i, float l) -> float {
        if (!kept_k(i, l)) return 0.f;
        const uint32_t key = E::key(l);
        if (sp.use_p && !(key > kp_key || (key == kp_key && i <= kp_last))) return 0.f;
        return wt(l);
      },
      [&](double total) { return (double)u * total; });
}

// ---------------------------------------------------------------- memory kernel (fp32; long bf16 rows)

template <typename T>
__global__ void __launch_bounds__(kSampleThreads) sample_mem_kernel(SampleArgs a) {
  __shared__ SampleLds s;
  const int row_id = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  SampleParams sp;
  sp.load(a, row_id, a.vocab);
  SampleRow<T> row;
  row.init(reinterpret_cast<const T*>(a.logits) + (int64_t)row_id * a.row_stride, a.vocab, wave, lane);

  // maximum and the first index of it (-0 == +0 compare equal)
  float vmax = -INFINITY;
  int32_t imax = 0x7fffffff;
  row.for_each([&](int i, float l) {
    if (l > vmax) {
      vmax = l;
      imax = i;
    }
  });
  float m = wave_max_f32(vmax);
  __syncthreads();
  if (lane == 0) s.wave_f[wave] = m;
  __syncthreads();
  m = (float)s.wave_f[0];
  for (int w = 1; w < kSampleWaves; ++w) m = fmaxf(m, (float)s.wave_f[w]);
  const int32_t am = block_reduce_i32(s, vmax == m ? imax : 0x7fffffff, false);
  const int32_t argmax = am == 0x7fffffff ? 0 : am;
  int32_t idx;
  if (sp.greedy) {
    idx = argmax;
  } else if (!sp.use_k && !sp.use_p) {
    const float u = sp.u, c2 = sp.c2;
    idx = find_crossing(row, s, [&](int, float l) { return row_weight(l, m, c2); },
                        [&](double total) { return (double)u * total; });
  } else {
    idx = sample_generic(row, s, sp, m);
  }
  if (tid == 0) a.out[row_id] = idx >= 0 ? idx : argmax;
}

// ---------------------------------------------------------------- bf16: slice kernel + finish kernel

constexpr int kSliceThreads = 256;
constexpr int kSliceRounds = 4;                                 // 16-byte chunks per thread
constexpr int kSliceTokens = kSliceThreads * kSliceRounds * 8;  // 8192 tokens per slice
constexpr int kSliceCap = 1024;                                 // window tokens a slice can hand over
constexpr int kFinishCap = 8192;                                // window tokens a row can hold in LDS

// What a slice hands to the finish kernel.
struct SliceRec {
  int32_t kmax;     // largest biased key of the slice
  int32_t argmax;   // first row index holding it
  int32_t count;    // tokens within the window of the slice maximum (may exceed kSliceCap)
  int32_t pad;
  double mass;      // sum of exp2((l - l_slice_max) * c2) over the slice (rows that need it)
};

__host__ __device__ inline int sample_slices(int V) { return (V + kSliceTokens - 1) / kSliceTokens; }

// Slice kernel: workgroup b handles slice b % S of row b / S. It reads its
// 8192 tokens once (thread t holds chunks t, t + 256, t + 512, t + 768, so
// index order within the slice is (round, thread, token)), turns them into
// biased 16-bit keys, and writes its maximum, the first index of it, its
// mass (rows whose draw or top-p runs over the whole row) and, in index
// order, every token within kSampleWindow keys of its maximum as
// (row index, key). The window of the row maximum is inside the union of
// these windows, since no slice maximum exceeds the row maximum. A handed-over
// token is one word: (offset in the slice) << 16 | key; the list is built in
// LDS and written out with 16-byte stores.
__global__ void __launch_bounds__(kSliceThreads, 8) sample_slice_kernel(SampleArgs a, SliceRec* recs,
                                                                        uint32_t* ents) {
  constexpr int W = kSampleWindow;
  __shared__ uint32_t sh_u[kSliceThreads / kWave];
  __shared__ int32_t sh_i[kSliceThreads / kWave];
  __shared__ double sh_d[kSliceThreads / kWave];
  __shared__ uint32_t sh_sc[2][kSliceThreads / kWave];
  __shared__ __attribute__((aligned(16))) uint32_t sh_list[kSliceCap];
  const int V = a.vocab, S = sample_slices(V);
  const int row = blockIdx.x / S, slice = blockIdx.x % S;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  SampleParams sp;
  sp.load(a, row, V);
  const bool need_mass = !sp.greedy && !sp.use_k;            // plain rows and top-p over the whole row
  const bool need_list = !sp.greedy && (sp.use_k || sp.use_p);
  const int t0 = slice * kSliceTokens;
  const u32x4* crow = reinterpret_cast<const u32x4*>(reinterpret_cast<const bf16_t*>(a.logits) +
                                                     (int64_t)row * a.row_stride);
  const int last_chunk = (V - 1) / 8;

  // Load (indices clamped to the row's last chunk: every read stays inside
  // the row), then mask the tokens at or past V to -inf. Only the raw words
  // stay in registers; keys are recomputed where needed (three ops a pair).
  u32x4 raw[kSliceRounds];
#pragma unroll
  for (int i = 0; i < kSliceRounds; ++i) {
    const int ch = t0 / 8 + i * kSliceThreads + tid;
    raw[i] = __builtin_nontemporal_load(crow + min(ch, last_chunk));
  }
  u16x2 mx = {0, 0};
#pragma unroll
  for (int i = 0; i < kSliceRounds; ++i) {
    const int tok = t0 + 8 * (i * kSliceThreads + tid);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t w = raw[i][j];
      if (tok + 2 * j >= V) w = 0xff80ff80u;
      else if (tok + 2 * j + 1 >= V) w = (w & 0xffffu) | 0xff800000u;
      raw[i][j] = w;
      mx = __builtin_elementwise_max(mx, as_u16x2(bf16x2_keys(w)));
    }
  }
  const uint32_t tk = max((uint32_t)mx.x, (uint32_t)mx.y);
  // mass relative to this thread's maximum (rescaled to the slice maximum below)
  double mass = 0.0;
  if (need_mass) {
    const float c2 = sp.c2, off = -fmaxf(key16_value(tk), -1e30f) * c2;
#pragma unroll
    for (int i = 0; i < kSliceRounds; ++i) {
      float cs = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        cs += fast_exp2(fmaf(__uint_as_float(raw[i][j] << 16), c2, off));
        cs += fast_exp2(fmaf(__uint_as_float(raw[i][j] & 0xffff0000u), c2, off));
      }
      mass += (double)cs;
    }
  }
  // slice maximum
  const uint32_t wk = (uint32_t)wave_max_i32((int32_t)tk);
  if (lane == 0) sh_u[wave] = wk;
  __syncthreads();
  uint32_t kmax = sh_u[0];
#pragma unroll
  for (int w = 1; w < kSliceThreads / kWave; ++w) kmax = max(kmax, sh_u[w]);
  if (need_mass) {
    mass = wave_sum_f64(mass * (double)fast_exp2((fmaxf(key16_value(tk), -1e30f) -
                                                   fmaxf(key16_value(kmax), -1e30f)) * sp.c2));
    if (lane == 0) sh_d[wave] = mass;
  }
  // first index holding it
  int32_t found = 0x7fffffff;
  if (tk == kmax) {
#pragma unroll
    for (int i = kSliceRounds - 1; i >= 0; --i)
#pragma unroll
      for (int j = 3; j >= 0; --j) {
        const int tok = t0 + 8 * (i * kSliceThreads + tid) + 2 * j;
        const uint32_t k = bf16x2_keys(raw[i][j]);
        if ((k >> 16) == kmax) found = tok + 1;
        if ((k & 0xffffu) == kmax) found = tok;
      }
  }
  found = wave_min_i32(found);
  if (lane == 0) sh_i[wave] = found;
  // window tokens: key > th, i.e. the saturated key - th is nonzero
  int32_t count = 0;
  if (need_list) {
    const uint32_t th = kmax > (uint32_t)W ? kmax - (uint32_t)W : 0u;
    const u16x2 thpk = as_u16x2(th * 0x10001u);
    uint32_t n[kSliceRounds];
#pragma unroll
    for (int i = 0; i < kSliceRounds; ++i) {
      n[i] = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const u16x2 sv = __builtin_elementwise_sub_sat(as_u16x2(bf16x2_keys(raw[i][j])), thpk);
        n[i] += (sv.x != 0) + (sv.y != 0);
      }
    }
    // positions in (round, thread) order: two 16-bit-lane scans over the block
    const uint32_t p01 = n[0] | (n[1] << 16), p23 = n[2] | (n[3] << 16);
    const uint32_t i01 = (uint32_t)wave_incl_scan_i32((int32_t)p01, lane);
    const uint32_t i23 = (uint32_t)wave_incl_scan_i32((int32_t)p23, lane);
    if (lane == 63) {
      sh_sc[0][wave] = i01;
      sh_sc[1][wave] = i23;
    }
    __syncthreads();
    uint32_t o01 = 0, o23 = 0, t01 = 0, t23 = 0;
#pragma unroll
    for (int w = 0; w < kSliceThreads / kWave; ++w) {
      if (w < wave) {
        o01 += sh_sc[0][w];
        o23 += sh_sc[1][w];
      }
      t01 += sh_sc[0][w];
      t23 += sh_sc[1][w];
    }
    const uint32_t e01 = o01 + i01 - p01, e23 = o23 + i23 - p23;  // exclusive, per 16-bit lane
    const uint32_t tot[4] = {t01 & 0xffffu, t01 >> 16, t23 & 0xffffu, t23 >> 16};
    uint32_t pos[4] = {e01 & 0xffffu, (e01 >> 16) + tot[0], (e23 & 0xffffu) + tot[0] + tot[1],
                       (e23 >> 16) + tot[0] + tot[1] + tot[2]};
    count = (int32_t)(tot[0] + tot[1] + tot[2] + tot[3]);
#pragma unroll
    for (int i = 0; i < kSliceRounds; ++i) {
      if (n[i]) {
        const uint32_t off = 8 * (i * kSliceThreads + tid);  // token offset within the slice
        uint32_t p = pos[i];
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const uint32_t kw = bf16x2_keys(raw[i][j]);
            const uint32_t k = h ? (kw >> 16) : (kw & 0xffffu);
            if (k > th) {
              if (p < (uint32_t)kSliceCap) sh_list[p] = ((off + 2 * j + h) << 16) | k;
              ++p;
            }
          }
      }
    }
    __syncthreads();
    const int nw = (min(count, kSliceCap) + 3) / 4;  // 16-byte stores
    u32x4* out = reinterpret_cast<u32x4*>(ents + (int64_t)blockIdx.x * kSliceCap);
    for (int q = tid; q < nw; q += kSliceThreads) out[q] = reinterpret_cast<const u32x4*>(sh_list)[q];
  }
  __syncthreads();
  if (tid == 0) {
    SliceRec r;
    r.kmax = (int32_t)kmax;
    int32_t am = sh_i[0];
    for (int w = 1; w < kSliceThreads / kWave; ++w) am = min(am, sh_i[w]);
    r.argmax = am;
    r.count = count;
    r.pad = 0;
    double m = 0.0;
    if (need_mass)
      for (int w = 0; w < kSliceThreads / kWave; ++w) m += sh_d[w];
    r.mass = m;
    recs[blockIdx.x] = r;
  }
}

// Exclusive block scan of v (thread order) that also returns the block
// maximum of m, with the same three barriers; *incl_out equals the next
// thread's exclusive prefix bit for bit.
PKV_INLINE double block_scan_f64_max(SampleLds& s, double v, int32_t m, double* incl_out, double* total,
                                     int32_t* mmax) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  double excl;
  const double incl = wave_scan_f64(v, lane, &excl);
  m = wave_max_i32(m);
  __syncthreads();
  if (lane == 63) {
    s.scan_f[wave] = incl;
    s.wave_j[wave] = m;
  }
  __syncthreads();
  double off = 0.0, tot = 0.0;
  int32_t mx = s.wave_j[0];
  for (int w = 0; w < kSampleWaves; ++w) {
    if (w < wave) off += s.scan_f[w];
    tot += s.scan_f[w];
    mx = max(mx, s.wave_j[w]);
  }
  __syncthreads();
  *total = tot;
  *mmax = mx;
  *incl_out = off + incl;
  return off + excl;
}

// First of W <= 128 bins (ascending) whose running amount reaches goal, by
// one wave (two bins per lane): *bin = -1 if none, *before = the amount
// strictly before it, *cnt = count(bin). No barriers.
template <class AF, class CF>
PKV_INLINE void wave_select128(AF amount, CF count, double goal, int* bin, double* before, uint32_t* cnt) {
  const int lane = threadIdx.x & 63;
  const double a0 = amount(2 * lane), a1 = amount(2 * lane + 1);
  double excl;
  const double incl = wave_scan_f64(a0 + a1, lane, &excl);
  int b = -1;
  double bef = 0.0;
  if (a0 + a1 > 0.0 && excl < goal && goal <= incl) {  // at most one lane
    if (a0 > 0.0 && goal <= excl + a0) {
      b = 2 * lane;
      bef = excl;
    } else {
      b = 2 * lane + 1;
      bef = excl + a0;
    }
  }
  const uint64_t who = __ballot(b >= 0);
  if (!who) {
    *bin = -1;
    *before = 0.0;
    *cnt = 0;
    return;
  }
  const int l0 = __ffsll((unsigned long long)who) - 1;
  *bin = __shfl(b, l0, 64);
  *before = __shfl(bef, l0, 64);
  const uint32_t c = b >= 0 ? count(b) : 0u;
  *cnt = (uint32_t)__shfl((int32_t)c, l0, 64);
}

// Finish kernel: one workgroup per row merges the slices' results.
__global__ void __launch_bounds__(kSampleThreads) sample_finish_kernel(SampleArgs a, const SliceRec* recs,
                                                                       const uint32_t* ents) {
  constexpr int W = kSampleWindow;
  static_assert(W <= 128, "wave_select128 covers 128 bins");
  __shared__ SampleLds s;
  __shared__ int32_t f_idx[kFinishCap];
  __shared__ uint8_t f_d[kFinishCap];
  __shared__ int32_t f_cnt[256 + 1];
  __shared__ int32_t h_i[8];
  __shared__ double h_f[2];
  const int V = a.vocab, S = sample_slices(V);
  const int row = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  SampleParams sp;
  sp.load(a, row, V);
  const float c2 = sp.c2;
  const SliceRec* rr = recs + (int64_t)row * S;
  const bool plain = !sp.greedy && !sp.use_k && !sp.use_p;

  // ---- wave 0: everything about the slices (at most 256; lane l holds slices l, l + 64, ...)
  if (wave == 0) {
    SliceRec rec[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (u * kWave + lane < S) rec[u] = rr[u * kWave + lane];  // one round of loads
    int32_t mk = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (u * kWave + lane < S) mk = max(mk, rec[u].kmax);
    mk = wave_max_i32(mk);  // row maximum
    int32_t am = 0x7fffffff;
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (u * kWave + lane < S && rec[u].kmax == mk) am = min(am, rec[u].argmax);
    am = wave_min_i32(am);  // its first index: slices are in index order
    int32_t T = 0, ovf = 0, psl = -1;
    double wall = 0.0, rem = INFINITY;
    if (!sp.greedy) {
      const float lmax = key16_value((uint32_t)mk);
      double sm[4];  // slice masses in units of the row maximum
#pragma unroll
      for (int u = 0; u < 4; ++u)
        sm[u] = u * kWave + lane < S && !sp.use_k
                    ? rec[u].mass * (double)fast_exp2((fmaxf(key16_value((uint32_t)rec[u].kmax), -1e30f) - lmax) * c2)
                    : 0.0;
      if (!sp.use_k) wall = wave_sum_f64(sm[0] + sm[1] + sm[2] + sm[3]);
      if (plain) {  // the slice where the running mass passes u * W
        const double target = (double)sp.u * wall;
        double off = 0.0;
        int32_t last = -1;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (psl < 0 && u * kWave < S) {
            double ex;
            const double in = wave_scan_f64(sm[u], lane, &ex);
            const uint64_t who = __ballot(sm[u] > 0.0 && off + ex <= target && target < off + in);
            if (who) {
              const int l0 = __ffsll((unsigned long long)who) - 1;
              psl = u * kWave + l0;
              rem = target - (off + __shfl(ex, l0, 64));
            }
            last = max(last, wave_max_i32(sm[u] > 0.0 ? u * kWave + lane : -1));
            off += __shfl(in, 63, 64);
          }
        }
        if (psl < 0) psl = max(last, 0);  // rounding left the target past every slice: the last one with mass
      } else {  // flattened window tokens of the slices whose maximum reaches the threshold
        const uint32_t thr = (uint32_t)mk >= (uint32_t)(W - 1) ? (uint32_t)mk - (uint32_t)(W - 1) : 0u;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (u * kWave < S) {
            const int sl = u * kWave + lane;
            int32_t c = 0;
            if (sl < S && (uint32_t)rec[u].kmax >= thr) {
              c = min(rec[u].count, kSliceCap);
              ovf |= rec[u].count > kSliceCap;
            }
            const int32_t in = wave_incl_scan_i32(c, lane);
            if (sl < S) f_cnt[sl] = T + in - c;
            T += __shfl(in, 63, 64);
          }
        }
        ovf = wave_max_i32(ovf);
        if (lane == 0) f_cnt[S] = T;
      }
    }
    if (lane == 0) {
      h_i[0] = mk;
      h_i[1] = am;
      h_i[2] = T;
      h_i[3] = ovf;
      h_i[4] = psl;
      h_f[0] = wall;
      h_f[1] = rem;
    }
  }
  __syncthreads();
  const uint32_t kmax = (uint32_t)h_i[0];
  const int32_t argmax = h_i[1] == 0x7fffffff ? 0 : h_i[1];
  if (sp.greedy) {
    if (tid == 0) a.out[row] = argmax;
    return;
  }
  const float lmax = key16_value(kmax);
  const double wall = h_f[0];
  SampleRow<bf16_t> mrow;  // the row in memory, for the paths the window does not cover
  mrow.init(reinterpret_cast<const bf16_t*>(a.logits) + (int64_t)row * a.row_stride, V, wave, lane);

  if (plain) {
    // ---- plain rows: the token inside the chosen slice; thread t scans tokens [16t, 16t + 16)
    const int sl = h_i[4];
    const double rem = h_f[1];
    const bf16_t* tp = reinterpret_cast<const bf16_t*>(a.logits) + (int64_t)row * a.row_stride +
                       (int64_t)sl * kSliceTokens + 16 * tid;
    const int base = sl * kSliceTokens + 16 * tid;
    float w[16];
    double own = 0.0;
    int32_t lastp = -1;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (base + 8 * q < V) x = *reinterpret_cast<const u32x4*>(tp + 8 * q);
      float cs = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int i = base + 8 * q + e;
        w[8 * q + e] = i < V ? row_weight(SampleElem<bf16_t>::value(x, e), lmax, c2) : 0.f;
        if (w[8 * q + e] > 0.f) lastp = i;
        cs += w[8 * q + e];
      }
      own += (double)cs;
    }
    double in2, tot2;
    int32_t lk;
    const double ex2 = block_scan_f64_max(s, own, lastp, &in2, &tot2, &lk);
    if (tid == 0) s.result = -1;
    __syncthreads();
    if (own > 0.0 && ex2 <= rem && rem < in2) {
      double run = ex2;
      int32_t res = lastp;
      bool done = false;
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (!done && w[e] > 0.f) {
          run += (double)w[e];
          if (run > rem) {
            res = base + e;
            done = true;
          }
        }
      s.result = res;
    }
    __syncthreads();
    const int32_t r = s.result >= 0 ? s.result : lk;
    if (tid == 0) a.out[row] = r >= 0 ? r : argmax;
    return;
  }

  // ---- rows with top-k or top-p: the window of the row maximum (keys >= thr, d = kmax - key < W)
  const uint32_t thr = kmax >= (uint32_t)(W - 1) ? kmax - (uint32_t)(W - 1) : 0u;
  const int32_t T = h_i[2];
  // Thread t takes flattened positions [g0, g1) (slice by slice, index order).
  const int gper = (T + kSampleThreads - 1) / kSampleThreads;
  const int g0 = min(T, tid * gper), g1 = min(T, g0 + gper);
  int sl0 = 0;  // the slice holding g0: the last slice that starts at or before it
  for (int lo = 0, hi = S - 1; lo <= hi;) {
    const int mid = (lo + hi) >> 1;
    if (f_cnt[mid] <= g0) {
      sl0 = mid;
      lo = mid + 1;
    } else {
      hi = mid - 1;
    }
  }
  // Batches of kB positions; the first batch stays in registers for the
  // second pass (one batch covers rows of up to 512 * kB handed-over tokens).
  constexpr int kB = 16;
  auto load_batch = [&](int q0, int& sl, uint32_t* idx, uint32_t* key) {
#pragma unroll
    for (int u = 0; u < kB; ++u) {
      const int q = q0 + u;
      idx[u] = 0;
      key[u] = 0;
      if (q < g1) {
        while (f_cnt[sl + 1] <= q) ++sl;
        const uint32_t e = ents[((int64_t)row * S + sl) * kSliceCap + (q - f_cnt[sl])];
        idx[u] = (uint32_t)sl * kSliceTokens + (e >> 16);
        key[u] = e & 0xffffu;  // 0 (below every real key) past g1
      }
    }
  };
  uint32_t bidx[kB], bkey[kB];
  int sl_next = sl0;
  load_batch(g0, sl_next, bidx, bkey);
  int32_t npass = 0;
#pragma unroll
  for (int u = 0; u < kB; ++u) npass += bkey[u] >= thr && bkey[u] != 0;
  {
    int sl = sl_next;
    for (int q0 = g0 + kB; q0 < g1; q0 += kB) {
      uint32_t ti[kB], tk[kB];
      load_batch(q0, sl, ti, tk);
#pragma unroll
      for (int u = 0; u < kB; ++u) npass += tk[u] >= thr && tk[u] != 0;
    }
  }
  int32_t n;
  const int32_t pbase = block_excl_scan_i32(s, npass, &n);
  const bool ok = h_i[3] == 0 && n <= kFinishCap;
  if (ok) {
    int32_t p = pbase;
    auto put = [&](const uint32_t* ti, const uint32_t* tk) {
#pragma unroll
      for (int u = 0; u < kB; ++u)
        if (tk[u] >= thr && tk[u] != 0) {
          f_idx[p] = (int32_t)ti[u];
          f_d[p] = (uint8_t)(kmax - tk[u]);
          ++p;
        }
    };
    put(bidx, bkey);
    int sl = sl_next;
    for (int q0 = g0 + kB; q0 < g1; q0 += kB) {
      uint32_t ti[kB], tk[kB];
      load_batch(q0, sl, ti, tk);
      put(ti, tk);
    }
  }
  for (int b = tid; b < 256; b += kSampleThreads) {
    s.hist[b] = 0;
    s.wtab[b] = (b < W && (uint32_t)b <= kmax) ? row_weight(key16_value(kmax - (uint32_t)b), lmax, c2) : 0.f;
  }
  __syncthreads();
  if (ok)
    for (int q = tid; q < n; q += kSampleThreads) atomicAdd(&s.hist[f_d[q]], 1u);
  __syncthreads();

  // ---- cuts, by wave 0
  if (wave == 0) {
    int dcut = -1;
    uint32_t take = 0;
    if (ok) {
      auto hc = [&](int b) { return b < W ? s.hist[b] : 0u; };
      int dk = -1;
      uint32_t kk_take = 0, kk_eq = 0;
      if (sp.use_k) {
        double before;
        wave_select128([&](int b) { return (double)hc(b); }, hc, (double)sp.k, &dk, &before, &kk_eq);
        if (dk >= 0) kk_take = (uint32_t)sp.k - (uint32_t)before;
      }
      dcut = dk;
      take = kk_take;
      if (sp.use_p && (!sp.use_k || dk >= 0)) {
        const int dlim = sp.use_k ? dk : W - 1;
        auto nb = [&](int b) { return b < dlim ? hc(b) : (b == dlim ? (sp.use_k ? kk_take : hc(b)) : 0u); };
        double Wk = wall;
        if (sp.use_k) Wk = wave_sum_f64((double)nb(2 * lane) * (double)s.wtab[2 * lane] +
                                        (double)nb(2 * lane + 1) * (double)s.wtab[2 * lane + 1]);
        const double target = (double)sp.p * Wk;
        int dstar;
        double above;
        uint32_t n_at;
        wave_select128([&](int b) { return (double)nb(b) * (double)s.wtab[b]; }, nb, target, &dstar, &above,
                       &n_at);
        dcut = dstar;
        if (dstar >= 0) {
          // equal-key tokens at the cut: token j of the group (0-based) is kept iff above + j * w < target
          double need = ceil((target - above) / (double)s.wtab[dstar]);
          if (!(need >= 1.0)) need = 1.0;
          take = need >= (double)n_at ? n_at : (uint32_t)need;
        }
      }
    }
    if (lane == 0) {
      h_i[5] = dcut;
      h_i[6] = (int32_t)take;
    }
  }
  __syncthreads();
  const int dcut = h_i[5];
  const uint32_t take = (uint32_t)h_i[6];

  if (dcut >= 0) {
    // ---- ties at the cut and the draw, on the list: thread t takes [q0, q1)
    const int per = (n + kSampleThreads - 1) / kSampleThreads;
    const int q0 = min(n, tid * per), q1 = min(n, q0 + per);
    int32_t nat = 0;
    for (int q = q0; q < q1; ++q) nat += f_d[q] == dcut;
    int32_t tot_at;
    const int32_t rank0 = block_excl_scan_i32(s, nat, &tot_at);  // rank of this thread's first token at the cut
    double own = 0.0;
    int32_t last_kept = -1;
    {
      int32_t rank = rank0;
      for (int q = q0; q < q1; ++q) {
        const int d = f_d[q];
        const bool kept = d < dcut || (d == dcut && (uint32_t)(rank++) < take);
        if (kept) {
          own += (double)s.wtab[d];
          last_kept = f_idx[q];
        }
      }
    }
    double tot, incl;
    int32_t lk;  // list order is index order: the largest kept index is the last kept token
    const double excl = block_scan_f64_max(s, own, last_kept, &incl, &tot, &lk);
    const double target = (double)sp.u * tot;
    if (tid == 0) s.result = -1;
    __syncthreads();
    if (own > 0.0 && excl <= target && target < incl) {
      int32_t rank = rank0, res = last_kept;
      double run = excl;
      for (int q = q0; q < q1; ++q) {
        const int d = f_d[q];
        const bool kept = d < dcut || (d == dcut && (uint32_t)(rank++) < take);
        if (kept) {
          run += (double)s.wtab[d];
          if (run > target) {
            res = f_idx[q];
            break;
          }
        }
      }
      s.result = res;
    }
    __syncthreads();
    const int32_t res = s.result >= 0 ? s.result : lk;
    if (tid == 0) a.out[row] = res >= 0 ? res : argmax;
    return;
  }

  // ---- the cut lies below the window, or a list overflowed
  const int32_t idx = sample_generic(mrow, s, sp, lmax);
  if (tid == 0) a.out[row] = idx >= 0 ? idx : argmax;
}

}  // namespace pkv
