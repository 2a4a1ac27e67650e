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
// bf16 rows (the register kernel):
// * The row is read from HBM once into registers as 32-bit words (two
//   tokens). Wave w owns words [w * WPW, (w + 1) * WPW); in round c, slot j
//   lane l holds word w * WPW + (4c + j) * 64 + l, so every load is a
//   coalesced 256-byte read and index order is (wave, round, slot, lane,
//   half). Words past the row read a constant -inf pair instead, so no pass
//   needs a bounds mask.
// * As words arrive they are turned in place into pairs of biased 16-bit
//   keys with packed 16-bit integer ops, and folded into a running maximum;
//   rows whose top-p runs over the whole row also fold in their mass,
//   relative to a per-thread reference raised with the running maximum.
// * A second pass copies every token within 128 key values of the maximum
//   into a per-wave LDS list, in index order (one saturating packed
//   subtract, one ballot and one lane count per word slot). The top-k
//   threshold and the top-p cut come from a count histogram of the list: all
//   tokens of a bin share one key and one weight. The ties at the cut (the
//   first n equal-key tokens in index order are kept) and the draw (kept
//   weights in index order, first running mass > u * W) run on the list.
// * Rows with neither top-k nor top-p, cuts below the 128-key window and
//   lists that overflow take the paths below over the row in memory.
//
// fp32 rows, and bf16 rows too long for registers (the memory kernel): every
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
constexpr int kSampleWindow = 128;      // register kernel: key values at or below the maximum in the list
constexpr int kSampleSegment = 1024;    // register kernel: list entries per wave
constexpr int kSampleCap = kSampleSegment * kSampleWaves;
constexpr int kSampleMaxRounds = 512;   // memory passes: chunk rounds per wave with a group-mass slot
constexpr int kSampleWordsPerRound = 4 * kWave;  // register kernel: words a wave reads per round

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
  union {
    struct {
      uint32_t g[kSampleCap];    // register kernel list: slot code of the word within its wave ...
      uint32_t sv[kSampleCap];   // ... and its two saturated key offsets (0 = not in the window)
    } list;
    float gsum[kSampleWaves * kSampleMaxRounds];  // memory passes: group masses, group = (wave, round)
  } big;
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
    if (lane == 0) s.big.gsum[wave * R + c] = g;
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
    for (int g = g0; g < g1; ++g) own += (double)s.big.gsum[g];
    double run;
    const double incl = wave_scan_f64(own, lane, &run);
    const double total = __shfl(incl, 63, 64);
    const double target = target_of(total);
    if (own > 0.0 && run <= target && target < incl) {
      int gp = -1;
      double rp = 0.0;
      for (int g = g0; g < g1; ++g) {
        const double gs = (double)s.big.gsum[g];
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

// ---------------------------------------------------------------- bf16 register kernel

template <int MAXR>
__global__ void __launch_bounds__(kSampleThreads) sample_bf16_kernel(SampleArgs a) {
  constexpr int W = kSampleWindow;
  __shared__ SampleLds s;
  const int row_id = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int V = a.vocab;
  SampleParams sp;
  sp.load(a, row_id, V);
  const float c2 = sp.c2;
  const bool full_mass = !sp.greedy && sp.use_p && !sp.use_k;  // top-p over the whole row needs its mass

  // word (c, j) of this thread: g = gbase + (4c + j) * 64
  const uint32_t* wrow = reinterpret_cast<const uint32_t*>(a.logits) + (int64_t)row_id * (a.row_stride / 2);
  const int nw = (V + 1) / 2;   // words holding the row
  const int nfull = V / 2;      // words whose both halves lie in the row
  const int rounds = (nw + kSampleWaves * kSampleWordsPerRound - 1) / (kSampleWaves * kSampleWordsPerRound);
  const int wbase = wave * rounds * kSampleWordsPerRound;  // first word of this wave (uniform)
  const int gbase = wbase + lane;

  // Loads run kAhead rounds ahead of pass 1 (4 per round, 56 in flight per
  // wave: under the 63 the wait counter can track), so pass 1 overlaps them.
  // Every load reads a word of the row (indices are clamped): rounds past
  // `rounds` repeat the last round and are never used, words past the row
  // are overwritten with -inf before use.
  constexpr int kAhead = 14;
  uint32_t r[MAXR][4];
  auto issue = [&](int c) {
    const int cc = min(c, rounds - 1);
#pragma unroll
    for (int j = 0; j < 4; ++j) r[c][j] = __builtin_nontemporal_load(wrow + min(gbase + (4 * cc + j) * kWave, nw - 1));
    __builtin_amdgcn_sched_barrier(0);  // keep the loads in round order, so each round waits only for itself
  };
#pragma unroll
  for (int c = 0; c < kAhead && c < MAXR; ++c) issue(c);

  // ---- pass 1: keys in place, running maximum, and (full_mass) the mass
  // relative to a per-thread reference that follows the running maximum
  u16x2 mx = {0, 0};
  uint32_t refk = 0;          // key of the reference (0: none yet)
  float refv = -1e30f;        // its value, clamped so that -inf logits give weight 0, never NaN
  double wsum = 0.0;
#pragma unroll
  for (int c = 0; c < MAXR; ++c) {
    if (c + kAhead < MAXR) issue(c + kAhead);
    if (c < rounds) {
      if (wbase + (4 * c + 4) * kWave > nfull) {  // (uniform) this round reaches past the row
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int g = gbase + (4 * c + j) * kWave;
          if (g >= nfull) r[c][j] = (g == nfull && (V & 1)) ? ((r[c][j] & 0xffffu) | 0xff800000u) : 0xff80ff80u;
        }
      }
      uint32_t raw[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        raw[j] = r[c][j];
        r[c][j] = bf16x2_keys(raw[j]);
        mx = __builtin_elementwise_max(mx, as_u16x2(r[c][j]));
      }
      if (full_mass) {
        const uint32_t rk = max((uint32_t)mx.x, (uint32_t)mx.y);
        if (rk > refk) {
          const float nv = fmaxf(key16_value(rk), -1e30f);
          wsum *= (double)fast_exp2((refv - nv) * c2);
          refv = nv;
          refk = rk;
        }
        const float off = -refv * c2;
        float cs = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          cs += fast_exp2(fmaf(__uint_as_float(raw[j] << 16), c2, off));
          cs += fast_exp2(fmaf(__uint_as_float(raw[j] & 0xffff0000u), c2, off));
        }
        wsum += (double)cs;
      }
    }
  }
  const uint32_t tk = max((uint32_t)mx.x, (uint32_t)mx.y);
  const uint32_t kmax = (uint32_t)block_reduce_i32(s, (int32_t)tk, true);
  const float lmax = key16_value(kmax);

  // argmax: the first index holding kmax, searched only by threads that hold
  // it. Positions are kept as 2 * (slot code) + half, slot code =
  // (4c + j) * 64 + lane, and turned into an index once at the end, so that
  // no per-word index stays live from the loads.
  int32_t found = 0x7fffffff;
  if (tk == kmax) {
#pragma unroll
    for (int c = 0; c < MAXR; ++c) {
      if (c < rounds && found == 0x7fffffff) {
        const u16x2 m4 = __builtin_elementwise_max(__builtin_elementwise_max(as_u16x2(r[c][0]), as_u16x2(r[c][1])),
                                                   __builtin_elementwise_max(as_u16x2(r[c][2]), as_u16x2(r[c][3])));
        if (m4.x == kmax || m4.y == kmax) {
#pragma unroll
          for (int j = 3; j >= 0; --j) {  // the last assignment is the first position
            const int code = (4 * c + j) * kWave + lane;
            if ((r[c][j] >> 16) == kmax) found = 2 * code + 1;
            if ((r[c][j] & 0xffffu) == kmax) found = 2 * code;
          }
        }
      }
    }
    found += 2 * wave * rounds * kSampleWordsPerRound;
  }
  const int32_t am = block_reduce_i32(s, found, false);
  const int32_t argmax = am == 0x7fffffff ? 0 : am;
  if (sp.greedy) {
    if (tid == 0) a.out[row_id] = argmax;
    return;
  }

  SampleRow<bf16_t> mrow;  // the row in memory, for the paths the list does not cover
  mrow.init(reinterpret_cast<const bf16_t*>(a.logits) + (int64_t)row_id * a.row_stride, V, wave, lane);
  if (!sp.use_k && !sp.use_p) {
    const float u = sp.u;
    const int32_t idx = find_crossing(mrow, s, [&](int, float l) { return row_weight(l, lmax, c2); },
                                      [&](double total) { return (double)u * total; });
    if (tid == 0) a.out[row_id] = idx >= 0 ? idx : argmax;
    return;
  }
  const double wall = full_mass ? block_sum_f64(s, wsum * (double)fast_exp2((refv - lmax) * c2)) : 0.0;

  // ---- pass 2: every token within W keys of the maximum into the wave's
  // list segment, in index order. s_half = key - th (saturated) is > 0
  // exactly for those tokens, and d = kmax - key = d0 - s_half.
  const uint32_t th = kmax > (uint32_t)W ? kmax - (uint32_t)W : 0u;
  const uint32_t d0 = kmax - th;
  const u16x2 thpk = as_u16x2(th * 0x10001u);
  int32_t run = 0;
  const int seg = wave * kSampleSegment;
#pragma unroll
  for (int c = 0; c < MAXR; ++c) {
    if (c < rounds) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t sv = as_u32(__builtin_elementwise_sub_sat(as_u16x2(r[c][j]), thpk));
        const uint64_t m = __ballot(sv != 0u);
        if (m) {
          const int32_t pos = run + lanes_below(m);
          if (sv != 0u && pos < kSampleSegment) {
            s.big.list.g[seg + pos] = (uint32_t)((4 * c + j) * kWave + lane);  // slot code; word = wave base + code
            s.big.list.sv[seg + pos] = sv;
          }
          run += __popcll(m);
        }
      }
    }
  }
  if (lane == 0) s.seg_n[wave] = run;
  for (int b = tid; b < 256; b += kSampleThreads) {
    s.hist[b] = 0;
    s.wtab[b] = (b < W && (uint32_t)b <= kmax) ? row_weight(key16_value(kmax - (uint32_t)b), lmax, c2) : 0.f;
  }
  __syncthreads();
  int32_t segn[kSampleWaves], n = 0;
  bool fits = true;
#pragma unroll
  for (int w = 0; w < kSampleWaves; ++w) {
    segn[w] = s.seg_n[w];
    fits = fits && segn[w] <= kSampleSegment;
    n += segn[w];
  }

  // ---- histogram of the list, then the cuts
  int dcut = -1;
  uint32_t take = 0;
  if (fits) {
#pragma unroll
    for (int w = 0; w < kSampleWaves; ++w)
      for (int q = tid; q < segn[w]; q += kSampleThreads) {
        const uint32_t sv = s.big.list.sv[w * kSampleSegment + q];
        if (sv & 0xffffu) atomicAdd(&s.hist[d0 - (sv & 0xffffu)], 1u);
        if (sv >> 16) atomicAdd(&s.hist[d0 - (sv >> 16)], 1u);
      }
    __syncthreads();
    int dk = -1;
    uint32_t kk_take = 0, kk_eq = 0;
    if (sp.use_k) {
      double before;
      window_select(s, [&](int b) { return (double)s.hist[b]; }, [&](int b) { return s.hist[b]; }, (double)sp.k,
                    &dk, &before, &kk_eq);
      if (dk >= 0) kk_take = (uint32_t)sp.k - (uint32_t)before;
    }
    dcut = dk;
    take = kk_take;
    if (sp.use_p && (!sp.use_k || dk >= 0)) {
      double Wk = wall;
      if (sp.use_k) {
        double t = 0.0;
        if (tid < W) {
          const uint32_t nb = tid < dk ? s.hist[tid] : (tid == dk ? kk_take : 0u);
          t = (double)nb * (double)s.wtab[tid];
        }
        Wk = block_sum_f64(s, t);
      }
      const double target = (double)sp.p * Wk;
      const int dlim = sp.use_k ? dk : W - 1;
      int dstar;
      double above;
      uint32_t n_at;
      window_select(
          s,
          [&](int b) {
            const uint32_t nb = b < dlim ? s.hist[b] : (b == dlim ? (sp.use_k ? kk_take : s.hist[b]) : 0u);
            return (double)nb * (double)s.wtab[b];
          },
          [&](int b) { return (sp.use_k && b == dk) ? kk_take : s.hist[b]; }, target, &dstar, &above, &n_at);
      dcut = dstar;
      if (dstar >= 0) {
        // equal-key tokens at the cut: token j of the group (0-based) is kept iff above + j * w < target
        double need = ceil((target - above) / (double)s.wtab[dstar]);
        if (!(need >= 1.0)) need = 1.0;
        take = need >= (double)n_at ? n_at : (uint32_t)need;
      }
    }
  }

  if (dcut >= 0) {
    // ---- ties at the cut and the draw, on the list in index order. Thread
    // t takes list positions [q0, q1) of the concatenated segments.
    const int per = (n + kSampleThreads - 1) / kSampleThreads;
    const int q0 = min(n, tid * per), q1 = min(n, q0 + per);
    const int wwords = rounds * kSampleWordsPerRound;  // words per wave
    auto word_of = [&](int e) { return (e / kSampleSegment) * wwords + (int)s.big.list.g[e]; };
    auto slot_of = [&](int q) {  // list slot of position q (constant indices into segn)
      int w = 0, base = 0;
#pragma unroll
      for (int ww = 0; ww < kSampleWaves - 1; ++ww)
        if (w == ww && q - base >= segn[ww]) {
          base += segn[ww];
          w = ww + 1;
        }
      return w * kSampleSegment + (q - base);
    };
    int32_t nat = 0;
    for (int q = q0; q < q1; ++q) {
      const uint32_t sv = s.big.list.sv[slot_of(q)];
      nat += ((sv & 0xffffu) && d0 - (sv & 0xffffu) == (uint32_t)dcut) +
             ((sv >> 16) && d0 - (sv >> 16) == (uint32_t)dcut);
    }
    int32_t tot_at;
    const int32_t rank0 = block_excl_scan_i32(s, nat, &tot_at);  // rank of this thread's first token at the cut
    // weight of half h of a list entry, advancing the running rank at the cut
    auto kept_w = [&](uint32_t sv, int h, int32_t& rank) -> float {
      const uint32_t sh = h ? (sv >> 16) : (sv & 0xffffu);
      if (!sh) return 0.f;
      const uint32_t d = d0 - sh;
      if ((int)d > dcut) return 0.f;
      if ((int)d == dcut && (uint32_t)(rank++) >= take) return 0.f;
      return s.wtab[d];
    };
    double own = 0.0;
    int32_t last_kept = -1;
    {
      int32_t rank = rank0;
      for (int q = q0; q < q1; ++q) {
        const int e = slot_of(q);
        const uint32_t sv = s.big.list.sv[e];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const float w = kept_w(sv, h, rank);
          if (w > 0.f) {
            own += (double)w;
            last_kept = (int32_t)(2 * word_of(e) + h);
          }
        }
      }
    }
    double total, incl;
    const double excl = block_scan_f64(s, own, &incl, &total);
    const double target = (double)sp.u * total;
    const int32_t lk = block_reduce_i32(s, last_kept, true);  // list order is index order
    if (tid == 0) s.result = -1;
    __syncthreads();
    if (own > 0.0 && excl <= target && target < incl) {
      int32_t rank = rank0, res = last_kept;
      double runm = excl;
      bool done = false;
      for (int q = q0; q < q1 && !done; ++q) {
        const int e = slot_of(q);
        const uint32_t sv = s.big.list.sv[e];
        for (int h = 0; h < 2 && !done; ++h) {
          const float w = kept_w(sv, h, rank);
          if (w > 0.f) {
            runm += (double)w;
            if (runm > target) {
              res = (int32_t)(2 * word_of(e) + h);
              done = true;
            }
          }
        }
      }
      s.result = res;
    }
    __syncthreads();
    const int32_t res = s.result >= 0 ? s.result : lk;
    if (tid == 0) a.out[row_id] = res >= 0 ? res : argmax;
    return;
  }

  // ---- the cut lies below the window, or the list overflowed
  const int32_t idx = sample_generic(mrow, s, sp, lmax);
  if (tid == 0) a.out[row_id] = idx >= 0 ? idx : argmax;
}

}  // namespace pkv
