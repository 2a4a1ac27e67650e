// Batched per-request sampler: argmax, or temperature -> top-k -> top-p -> draw.
//
// Semantics ("Engine 与采样器", section 采样器; "Mini-SGLang 源码解析（四）：GPU
// 计算引擎系统", sections 14.3-14.4): p = softmax(logits / T); top-k keeps the
// k most probable tokens; the kept mass is renormalised; top-p keeps a ranked
// token iff the kept mass ranked before it is < p; one token is drawn from
// the rest. Greedy rows (T <= 1e-6, or no temperature array) are argmax.
// min_p ("Engine 与采样器", section 练习 and its answer) keeps a token iff its
// probability is at least min_p times the largest, on the full tempered
// distribution; that set is intersected with the top-k / top-p set.
//
// The pages' GPU path calls FlashInfer's rejection-sampling kernels; this is
// a different, exact design. Ranking uses
// order-preserving integer keys of the logits (-0 ranks with +0), so argmax
// and top-k are exact and ties go to the lower index; weights are
// w(l) = exp2((l - l_max) * log2(e) / T), so equal logits weigh the same.
//
// bf16 rows (slice kernel + finish kernel):
// * Each row is cut into slices of 8192 tokens, one workgroup per slice
//   (19 per row on a 151936-token vocabulary, so the chip is full even for
//   small batches). A slice reads its tokens once, turns them into
//   order-preserving biased 16-bit keys with packed 16-bit integer ops (-0
//   and +0 share a key) and hands over its maximum key and the first index
//   of it, its mass relative to its maximum (rows that draw from the whole
//   row or cut top-p over it) and a 256-bin count histogram of the keys
//   within 255 of its maximum (rows with top-k, top-p or min_p).
// * The finish kernel (one workgroup per row) takes the row maximum and
//   shifts every slice histogram by the slice's distance to it, so the bins
//   add into the row's window histogram. All tokens of a bin share one key
//   and one weight: the top-k threshold and the top-p cut come from counts
//   times weights, the ties at the cut keep the first n equal-key tokens in
//   index order, and every slice's kept mass follows from its histogram.
//   The min_p cut is the first bin whose weight is below min_p (a bin's
//   tokens share one weight, so it never splits a bin). The draw (kept
//   weights in index order, first running mass > u * W) picks one slice by
//   those masses and scans its 8192 tokens. Cuts below the window take the
//   generic path below over the row in memory.
//
// fp32 rows (slice kernel + finish kernel): the slices are the same 8192
// tokens with 32-bit keys. A slice hands over its maximum, its mass and, for
// rows with a cut, a candidate list: every token of the slice at or above a
// floor picked from a histogram of the keys' upper 16 bits (the bins of an
// fp32 row do not share one weight, so the cuts are not taken from counts).
// The finish kernel runs the generic cuts and draw over the lists, which
// hold exactly the row's tokens at or above the largest floor; when a cut
// lies below them, over the row in memory.
//
// The generic path: every pass reads 16-byte chunks (wave w owns a
// contiguous chunk range, lane l reads chunk w * CPW + 64c + l in round c).
// Cuts by radix descent over the full key (8 bits per pass, count and fp64
// mass histograms); ties and the draw by per-(wave, round) group masses that
// locate one chunk round.
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
  const float* min_p;        // NULL = no min_p
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

constexpr int kSampleMaxRounds = 256;   // memory passes: chunk rounds per wave with a group-mass slot

// ---------------------------------------------------------------- wave helpers

// Wave-wide reductions and scans on DPP row moves and readlane (no LDS
// round trips). Every lane of the wave must be active.

template <int CTRL>
PKV_INLINE double dpp_f64(double x) {
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  const uint32_t lo = (uint32_t)dpp_i32<CTRL>((int32_t)(uint32_t)u);
  const uint32_t hi = (uint32_t)dpp_i32<CTRL>((int32_t)(uint32_t)(u >> 32));
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
PKV_INLINE double lane_f64(double x, int l) {
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int32_t)(uint32_t)u, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int32_t)(uint32_t)(u >> 32), l);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
// Combine over the 16 lanes of each row (every lane ends with its row's
// value): lane ^ 1, lane ^ 2, the other quad, the other half.
template <class T, class Op>
PKV_INLINE T row_reduce(T v, Op op) {
  if constexpr (sizeof(T) == 8) {
    v = op(v, dpp_f64<0xB1>(v));
    v = op(v, dpp_f64<0x4E>(v));
    v = op(v, dpp_f64<0x141>(v));
    v = op(v, dpp_f64<0x140>(v));
  } else {
    v = op(v, (T)dpp_i32<0xB1>((int32_t)v));
    v = op(v, (T)dpp_i32<0x4E>((int32_t)v));
    v = op(v, (T)dpp_i32<0x141>((int32_t)v));
    v = op(v, (T)dpp_i32<0x140>((int32_t)v));
  }
  return v;
}
PKV_INLINE double wave_sum_f64(double v) {
  v = row_reduce(v, [](double x, double y) { return x + y; });
  return (lane_f64(v, 0) + lane_f64(v, 16)) + (lane_f64(v, 32) + lane_f64(v, 48));
}
PKV_INLINE float wave_max_f32(float v) {
  const int32_t r = row_reduce(__float_as_int(v), [](int32_t x, int32_t y) {
    return __float_as_int(fmaxf(__int_as_float(x), __int_as_float(y)));
  });
  return fmaxf(fmaxf(__int_as_float(lane_i32(r, 0)), __int_as_float(lane_i32(r, 16))),
               fmaxf(__int_as_float(lane_i32(r, 32)), __int_as_float(lane_i32(r, 48))));
}
PKV_INLINE int32_t wave_min_i32(int32_t v) {
  v = row_reduce(v, [](int32_t x, int32_t y) { return min(x, y); });
  return min(min(lane_i32(v, 0), lane_i32(v, 16)), min(lane_i32(v, 32), lane_i32(v, 48)));
}
PKV_INLINE int32_t wave_sum_i32(int32_t v) {
  v = row_reduce(v, [](int32_t x, int32_t y) { return x + y; });
  return (lane_i32(v, 0) + lane_i32(v, 16)) + (lane_i32(v, 32) + lane_i32(v, 48));
}
PKV_INLINE int32_t wave_max_i32(int32_t v) {
  v = row_reduce(v, [](int32_t x, int32_t y) { return max(x, y); });
  return max(max(lane_i32(v, 0), lane_i32(v, 16)), max(lane_i32(v, 32), lane_i32(v, 48)));
}
// Inclusive scans: Kogge-Stone inside each row (shifts 1, 2, 4, 8), then the
// totals of the rows before (o_k = o_{k-1} + t_{k-1}) added to every lane of
// row k. *row_off = o_k of this lane's row.
PKV_INLINE double wave_incl_scan_f64(double v, int lane, double* row_off = nullptr) {
  v += dpp_f64<0x111>(v);
  v += dpp_f64<0x112>(v);
  v += dpp_f64<0x114>(v);
  v += dpp_f64<0x118>(v);
  const double o1 = lane_f64(v, 15);
  const double o2 = o1 + lane_f64(v, 31);
  const double o3 = o2 + lane_f64(v, 47);
  const int row = lane >> 4;
  const double off = row == 0 ? 0.0 : (row == 1 ? o1 : (row == 2 ? o2 : o3));
  if (row_off) *row_off = off;
  return row == 0 ? v : v + off;
}
// Inclusive scan and the exclusive value taken from the previous lane's
// inclusive one, so consecutive lanes' [excl, incl) intervals meet exactly
// (the first lane of row k gets o_k, which equals lane 16k - 1's inclusive
// value t_{k-1} + o_{k-1} bit for bit).
PKV_INLINE double wave_scan_f64(double v, int lane, double* excl) {
  double off;
  const double incl = wave_incl_scan_f64(v, lane, &off);
  const double prev = dpp_f64<0x111>(incl);
  *excl = (lane & 15) ? prev : off;
  return incl;
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
// The inverse: two biased keys -> the two bf16 values (-0 comes back as +0).
PKV_INLINE uint32_t bf16x2_from_keys(uint32_t k) {
  const i16x2 sgn = __builtin_bit_cast(i16x2, k ^ 0x80008000u) >> (int16_t)15;  // 0xffff where key < 0x8000
  const uint32_t sg = __builtin_bit_cast(uint32_t, sgn);
  return as_u32(as_u16x2(k ^ (sg | 0x80008000u)) - as_u16x2(sg));
}
// The bf16 value of a biased key.
PKV_INLINE float key16_value(uint32_t k) {
  const uint32_t b = k >= 0x8000u ? (k - 0x8000u) : (0x8000u | (0x8000u - k));
  return __uint_as_float(b << 16);
}

// ---------------------------------------------------------------- shared state

template <int NW>
struct SampleLds {
  float gsum[NW * kSampleMaxRounds];  // memory passes: group masses, group = (wave, round)
  uint32_t hist[256];    // window counts
  float wtab[256];       // weight of the key d below the maximum
  uint32_t rcnt[256];    // radix descent: digit counts
  double rmass[256];     //                digit masses
  int32_t seg_n[NW];
  double wave_f[NW];
  int32_t wave_i[NW];
  int32_t wave_j[NW];
  double scan_f[NW];
  int32_t pick_bin;
  uint32_t pick_cnt;
  double pick_above;
  int32_t result;
};

// Block-wide reductions, returned in every thread; they start and end with a barrier.
template <int NW>
PKV_INLINE double block_sum_f64(SampleLds<NW>& s, double v) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_sum_f64(v);
  __syncthreads();
  if (lane == 0) s.wave_f[wave] = v;
  __syncthreads();
  double t = 0.0;
  for (int w = 0; w < NW; ++w) t += s.wave_f[w];
  __syncthreads();
  return t;
}
template <int NW>
PKV_INLINE int32_t block_reduce_i32(SampleLds<NW>& s, int32_t v, bool want_max) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = want_max ? wave_max_i32(v) : wave_min_i32(v);
  __syncthreads();
  if (lane == 0) s.wave_j[wave] = v;
  __syncthreads();
  int32_t t = s.wave_j[0];
  for (int w = 1; w < NW; ++w) t = want_max ? max(t, s.wave_j[w]) : min(t, s.wave_j[w]);
  __syncthreads();
  return t;
}
// Exclusive block scans in thread order; *total = the sum over the block.
template <int NW>
PKV_INLINE int32_t block_excl_scan_i32(SampleLds<NW>& s, int32_t v, int32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int32_t incl = wave_incl_scan_i32(v, lane);
  __syncthreads();
  if (lane == 63) s.wave_j[wave] = incl;
  __syncthreads();
  int32_t off = 0, tot = 0;
  for (int w = 0; w < NW; ++w) {
    if (w < wave) off += s.wave_j[w];
    tot += s.wave_j[w];
  }
  __syncthreads();
  *total = tot;
  return off + incl - v;
}
// Returns the exclusive prefix; *incl_out = the inclusive one (equal to the
// next thread's exclusive prefix, bit for bit).
template <int NW>
PKV_INLINE double block_scan_f64(SampleLds<NW>& s, double v, double* incl_out, double* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  double excl;
  const double incl = wave_scan_f64(v, lane, &excl);
  __syncthreads();
  if (lane == 63) s.scan_f[wave] = incl;
  __syncthreads();
  double off = 0.0, tot = 0.0;
  for (int w = 0; w < NW; ++w) {
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
template <int NW, class AF, class CF>
PKV_INLINE void window_select(SampleLds<NW>& s, AF amount, CF count, double goal, int* bin, double* before,
                              uint32_t* cnt, double* total = nullptr) {
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
  if (total) *total = (s.scan_f[0] + s.scan_f[1]) + (s.scan_f[2] + s.scan_f[3]);  // all 256 bins
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

template <typename T, int NW>
struct SampleRow {
  using E = SampleElem<T>;
  static constexpr int EPC = E::kPerChunk;
  static constexpr int kPerChunk = EPC;
  const T* base;
  int V, nchunks, cpw, rounds, wave, lane;

  PKV_INLINE void init(const T* b, int vocab, int w, int l) {
    base = b;
    V = vocab;
    nchunks = (vocab + EPC - 1) / EPC;
    cpw = (nchunks + NW - 1) / NW;
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
  // The loads of four rounds are issued before the first is used, so each
  // lane keeps four 16-byte reads in flight (one workgroup per row is
  // otherwise bound by the latency of one read at a time).
  template <class F>
  PKV_INLINE void for_rounds(F f) const {
    int c = 0;
    for (; c + 4 <= rounds; c += 4) {
      const u32x4 x0 = fetch(c), x1 = fetch(c + 1), x2 = fetch(c + 2), x3 = fetch(c + 3);
      f(c, x0, chunk_ok(c));
      f(c + 1, x1, chunk_ok(c + 1));
      f(c + 2, x2, chunk_ok(c + 2));
      f(c + 3, x3, chunk_ok(c + 3));
    }
    for (; c < rounds; ++c) f(c, fetch(c), chunk_ok(c));
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
  // g(e, valid, i, l) for every element slot e of chunk x of round c
  template <class G>
  PKV_INLINE void elements_all(int c, const u32x4& x, bool ok, G g) const {
    const int i0 = chunk_id(c) * EPC;
#pragma unroll
    for (int e = 0; e < EPC; ++e) g(e, ok && i0 + e < V, i0 + e, E::value(x, e));
  }
  template <class F>
  PKV_INLINE void for_each(F f) const {
    for_rounds([&](int c, const u32x4& x, bool ok) { elements(c, x, ok, f); });
  }
};

constexpr int kCandCap = 1024;  // fp32 rows: listed tokens per slice at most
constexpr int kMaxSlicesPow2 = 128;  // a power of two >= the slices of a row (binary search)

// fp32 rows: the slices' candidate lists read as one row. Entry j of slice
// s's list is (logit bits, vocabulary index) of the j-th token the slice
// listed, in index order, so the lists one after another are in index order
// too. The lists are packed: chunk q (two entries, 16 bytes) is chunk
// q - beg[s] of slice s, the last slice with beg[s] <= q (beg = exclusive
// prefix of the slices' chunk counts, found by a binary search). An entry
// past its list's end reads as the NaN pattern 0xffffffff, whose key is 0;
// every token whose key is below `floor` (>= 1) is absent, so what remains
// is exactly the row's tokens with key >= floor (each slice lists all of its
// tokens at or above its own floor, and floor is the largest of those).
template <int NW>
struct CandRow {
  using E = SampleElem<float>;
  static constexpr int kPerChunk = 2;
  const uint2* lists;
  const int32_t* beg;  // [slices] first packed chunk of each list
  const int32_t* cnt;  // [slices] list lengths
  int slices;
  uint32_t floor;
  int nchunks, cpw, rounds, wave, lane;

  PKV_INLINE void init(const uint2* l, const int32_t* b, const int32_t* n, int S, int chunks, uint32_t floor_key,
                       int w, int ln) {
    lists = l;
    beg = b;
    cnt = n;
    slices = S;
    floor = floor_key;
    nchunks = chunks;
    cpw = (nchunks + NW - 1) / NW;
    rounds = (cpw + kWave - 1) / kWave;
    wave = w;
    lane = ln;
  }
  PKV_INLINE int chunk_id(int c) const { return wave * cpw + c * kWave + lane; }
  PKV_INLINE bool chunk_ok(int c) const { return c * kWave + lane < cpw && chunk_id(c) < nchunks; }
  // the slice holding chunk q: the last with beg <= q
  PKV_INLINE int locate(int q) const {
    int sl = 0;
#pragma unroll
    for (int step = kMaxSlicesPow2 / 2; step > 0; step >>= 1)
      if (sl + step < slices && beg[sl + step] <= q) sl += step;
    return sl;
  }
  // chunk c, its slice sl found from a slice at or before it
  PKV_INLINE u32x4 fetch_from(int c, int& sl) const {
    u32x4 x = {0xffffffffu, 0xffffffffu, 0xffffffffu, 0xffffffffu};
    if (chunk_ok(c)) {
      const int q = chunk_id(c);
      while (sl + 1 < slices && beg[sl + 1] <= q) ++sl;
      const int j = kPerChunk * (q - beg[sl]);
      x = *reinterpret_cast<const u32x4*>(lists + (int64_t)sl * kCandCap + j);
      if (j + 1 >= cnt[sl]) x[2] = 0xffffffffu;
    }
    return x;
  }
  PKV_INLINE u32x4 fetch(int c) const {
    int sl = chunk_ok(c) ? locate(chunk_id(c)) : 0;
    return fetch_from(c, sl);
  }
  // a lane's chunks rise with the round, so its slice is carried forward
  // (one binary search per pass, then a step or two per round)
  template <class F>
  PKV_INLINE void for_rounds(F f) const {
    int sl = chunk_ok(0) ? locate(chunk_id(0)) : 0;
    int c = 0;
    for (; c + 4 <= rounds; c += 4) {
      const u32x4 x0 = fetch_from(c, sl), x1 = fetch_from(c + 1, sl), x2 = fetch_from(c + 2, sl),
                  x3 = fetch_from(c + 3, sl);
      f(c, x0, chunk_ok(c));
      f(c + 1, x1, chunk_ok(c + 1));
      f(c + 2, x2, chunk_ok(c + 2));
      f(c + 3, x3, chunk_ok(c + 3));
    }
    for (; c < rounds; ++c) f(c, fetch_from(c, sl), chunk_ok(c));
  }
  template <class F>
  PKV_INLINE void elements(int c, const u32x4& x, bool ok, F f) const {
    if (!ok) return;
#pragma unroll
    for (int e = 0; e < kPerChunk; ++e) {
      const float l = __uint_as_float(x[2 * e]);
      if (E::key(l) >= floor) f((int)x[2 * e + 1], l);
    }
  }
  template <class G>
  PKV_INLINE void elements_all(int c, const u32x4& x, bool ok, G g) const {
#pragma unroll
    for (int e = 0; e < kPerChunk; ++e) {
      const float l = __uint_as_float(x[2 * e]);
      g(e, ok && E::key(l) >= floor, (int)x[2 * e + 1], l);
    }
  }
  template <class F>
  PKV_INLINE void for_each(F f) const {
    for_rounds([&](int c, const u32x4& x, bool ok) { elements(c, x, ok, f); });
  }
};

// fp32 rows: candidates packed in LDS (logit bits, vocabulary index), in
// index order; two entries per 16-byte chunk.
constexpr int kLdsCands = 4096;
template <int NW>
struct LdsRow {
  using E = SampleElem<float>;
  static constexpr int kPerChunk = 2;
  const uint2* ents;
  int n, nchunks, cpw, rounds, wave, lane;

  PKV_INLINE void init(const uint2* e, int count, int w, int l) {
    ents = e;
    n = count;
    nchunks = (count + kPerChunk - 1) / kPerChunk;
    cpw = (nchunks + NW - 1) / NW;
    rounds = (cpw + kWave - 1) / kWave;
    wave = w;
    lane = l;
  }
  PKV_INLINE int chunk_id(int c) const { return wave * cpw + c * kWave + lane; }
  PKV_INLINE bool chunk_ok(int c) const { return c * kWave + lane < cpw && chunk_id(c) < nchunks; }
  PKV_INLINE u32x4 fetch(int c) const {
    u32x4 x = {0u, 0u, 0u, 0u};
    if (chunk_ok(c)) x = *reinterpret_cast<const u32x4*>(ents + kPerChunk * chunk_id(c));
    return x;
  }
  template <class F>
  PKV_INLINE void for_rounds(F f) const {
    for (int c = 0; c < rounds; ++c) f(c, fetch(c), chunk_ok(c));
  }
  template <class F>
  PKV_INLINE void elements(int c, const u32x4& x, bool ok, F f) const {
    if (!ok) return;
    const int j = kPerChunk * chunk_id(c);
#pragma unroll
    for (int e = 0; e < kPerChunk; ++e)
      if (j + e < n) f((int)x[2 * e + 1], __uint_as_float(x[2 * e]));
  }
  template <class G>
  PKV_INLINE void elements_all(int c, const u32x4& x, bool ok, G g) const {
    const int j = kPerChunk * chunk_id(c);
#pragma unroll
    for (int e = 0; e < kPerChunk; ++e) g(e, ok && j + e < n, (int)x[2 * e + 1], __uint_as_float(x[2 * e]));
  }
  template <class F>
  PKV_INLINE void for_each(F f) const {
    for_rounds([&](int c, const u32x4& x, bool ok) { elements(c, x, ok, f); });
  }
};

// w(l) = exp2((l - l_max) * c2)
PKV_INLINE float row_weight(float l, float lmax, float c2) { return fast_exp2((l - lmax) * c2); }

// Block sum of v(i, l) over the row.
template <class RowT, int NW, class VF>
PKV_INLINE double row_sum(const RowT& row, SampleLds<NW>& s, VF v) {
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
template <class RowT, int NW, class VF, class TF>
PKV_INLINE int32_t find_crossing(const RowT& row, SampleLds<NW>& s, VF v, TF target_of) {
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
    const int G = NW * R, per = (G + kWave - 1) / kWave;
    const int g0 = min(G, lane * per), g1 = min(G, g0 + per);
    double own = 0.0;
    for (int g = g0; g < g1; ++g) own += (double)s.gsum[g];
    double run;
    const double incl = wave_scan_f64(own, lane, &run);
    const double total = lane_f64(incl, 63);
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
  for (int w = 0; w < NW; ++w) last = max(last, s.wave_i[w]);
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
      res = lane_i32(found, l0);
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
template <class RowT, int NW, class PF, class WF>
PKV_INLINE uint32_t radix_descend(const RowT& row, SampleLds<NW>& s, PF pred, WF weight, bool by_mass, double goal,
                                  double* above_out, uint32_t* eq_out, double* total_out = nullptr) {
  using E = typename RowT::E;
  uint32_t prefix = 0, mask = 0;
  double above = 0.0;
  uint32_t eq = 0;
  for (int shift = E::kKeyBits - 8; shift >= 0; shift -= 8) {
    __syncthreads();
    for (int b = threadIdx.x; b < 256; b += NW * kWave) {
      s.rcnt[b] = 0;
      s.rmass[b] = 0.0;
    }
    __syncthreads();
    // Near the top of a ranking most tokens share the leading digits, and
    // LDS atomics on one address serialise: a wave first adds each digit
    // that at least 8 of its lanes hold as one combined update (up to two
    // such digits per element slot), then the rest one by one.
    row.for_rounds([&](int c, const u32x4& x, bool ok) {
      constexpr int EPC = RowT::kPerChunk;
      bool act[EPC];
      uint32_t dg[EPC];
      double wv[EPC];
      row.elements_all(c, x, ok, [&](int e, bool valid, int i, float l) {
        const uint32_t key = E::key(l);
        act[e] = valid && (key & mask) == prefix && pred(i, l);
        dg[e] = (key >> shift) & 0xffu;
        wv[e] = (by_mass && act[e]) ? (double)weight(l) : 0.0;
      });
      const int lane = threadIdx.x & 63;
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
#pragma unroll
        for (int it = 0; it < 2; ++it) {
          const uint64_t pend = __ballot(act[e]);
          if (!pend) break;  // uniform
          const int leader = __ffsll((unsigned long long)pend) - 1;
          const uint32_t ld = (uint32_t)lane_i32((int32_t)dg[e], leader);
          const bool mine = act[e] && dg[e] == ld;
          const uint64_t m = __ballot(mine);
          if (__popcll(m) < 8) break;  // uniform: few lanes share it
          const double ms = by_mass ? wave_sum_f64(mine ? wv[e] : 0.0) : 0.0;
          if (lane == leader) {
            atomicAdd(&s.rcnt[ld], (uint32_t)__popcll(m));
            if (by_mass) atomicAdd(&s.rmass[ld], ms);
          }
          act[e] = act[e] && !mine;
        }
        if (act[e]) {
          atomicAdd(&s.rcnt[dg[e]], 1u);
          if (by_mass) atomicAdd(&s.rmass[dg[e]], wv[e]);
        }
      }
    });
    // bin b of the scan is digit 255 - b (descending keys)
    int bin;
    double before;
    uint32_t cnt;
    window_select(
        s, [&](int b) { return by_mass ? s.rmass[255 - b] : (double)s.rcnt[255 - b]; },
        [&](int b) { return s.rcnt[255 - b]; }, goal - above, &bin, &before, &cnt,
        shift == E::kKeyBits - 8 ? total_out : nullptr);  // the first digit's bins hold everything
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
  float c2, u, p, mp;
  int32_t k;
  bool greedy, use_k, use_p, use_mp;

  PKV_INLINE void load(const SampleArgs& a, int row, int V) {
    const float temp = a.temperature ? a.temperature[row] : 0.f;
    greedy = !a.temperature || temp <= 1e-6f;
    k = (!greedy && a.top_k) ? a.top_k[row] : 0;
    use_k = k > 0 && k < V;
    if (!use_k) k = V;
    p = (!greedy && a.top_p) ? a.top_p[row] : 1.f;
    use_p = p < 1.f;
    if (use_p) p = fmaxf(p, 1e-6f);
    mp = (!greedy && a.min_p) ? fminf(a.min_p[row], 1.f) : 0.f;  // above 1 acts as 1
    use_mp = mp > 0.f;
    c2 = greedy ? 0.f : 1.4426950408889634f / temp;
    u = greedy ? 0.f : a.uniforms[row];
  }
  // every token kept: the draw runs over the whole row's mass
  PKV_INLINE bool plain() const { return !greedy && !use_k && !use_p && !use_mp; }
  // the whole row's mass is needed: plain rows, and top-p over the whole row
  PKV_INLINE bool need_mass() const { return !greedy && !use_k && (use_p || !use_mp); }
  // a cut is needed
  PKV_INLINE bool need_cut() const { return !greedy && (use_k || use_p || use_mp); }
};

// Copies the elements of `row` into out[] in index order when there are at
// most cap of them; returns their count, or -1 (nothing written) if more.
// Group counts per (wave, round) go through s.gsum (exact in fp32), an
// exclusive scan over the groups in order gives each group's start, and a
// second pass writes. Block-uniform; all threads call it.
template <class RowT, int NW>
PKV_INLINE int compact_row(const RowT& row, SampleLds<NW>& s, uint2* out, int cap) {
  const int wave = row.wave, lane = row.lane, R = row.rounds;
  __syncthreads();
  row.for_rounds([&](int c, const u32x4& x, bool ok) {
    int m = 0;
    row.elements(c, x, ok, [&](int, float) { ++m; });
    const int t = wave_sum_i32(m);
    if (lane == 0) s.gsum[wave * R + c] = (float)t;
  });
  __syncthreads();
  if (wave == 0) {  // exclusive prefix over the groups in index order; each lane a contiguous run
    const int G = NW * R, per = (G + kWave - 1) / kWave;
    const int g0 = min(G, lane * per), g1 = min(G, g0 + per);
    int own = 0;
    for (int g = g0; g < g1; ++g) own += (int)s.gsum[g];
    const int incl = wave_incl_scan_i32(own, lane);
    int run = incl - own;
    for (int g = g0; g < g1; ++g) {
      const int v = (int)s.gsum[g];
      s.gsum[g] = (float)run;
      run += v;
    }
    if (lane == 63) s.pick_cnt = (uint32_t)incl;
  }
  __syncthreads();
  const int total = (int)s.pick_cnt;
  if (total > cap) return -1;
  row.for_rounds([&](int c, const u32x4& x, bool ok) {
    int m = 0;
    row.elements(c, x, ok, [&](int, float) { ++m; });
    int pos = (int)s.gsum[wave * R + c] + wave_incl_scan_i32(m, lane) - m;
    row.elements(c, x, ok, [&](int i, float l) { out[pos++] = make_uint2(__float_as_uint(l), (uint32_t)i); });
  });
  __syncthreads();
  return total;
}

// Cuts and draw over the row in memory (any cut depth, any number of kept
// tokens): radix descents for the top-k threshold and the top-p cut,
// group-mass scans for the ties at each cut and for the draw.
//
// Over a part of the row that holds every token at or above some key (the
// candidate lists), `covered` is given: the result is the whole row's iff
// every cut falls inside that part, which holds when it has at least k
// tokens (top-k), when its mass reaches the top-p target (top-p without
// top-k, whose target is p times the whole row's mass w_row), and, for
// min_p alone, when every token outside it (logits <= below_max) or one of
// its own falls below min_p; *covered is false (and the result
// meaningless) otherwise. Block-uniform.
template <class RowT, int NW>
PKV_INLINE int32_t sample_generic(const RowT& row, SampleLds<NW>& s, const SampleParams& sp, float lmax,
                                  const double* w_row = nullptr, bool* covered = nullptr,
                                  float below_max = INFINITY) {
  using E = typename RowT::E;
  const float c2 = sp.c2;
  auto wt = [&](float l) { return row_weight(l, lmax, c2); };
  if (covered) {
    *covered = true;
    // min_p alone: covered when every token below the part weighs below
    // min_p (below_max: the largest logit below it), or one of its own does
    if (sp.use_mp && !sp.use_k && !sp.use_p && !(wt(below_max) < sp.mp) &&
        row_sum(row, s, [&](int, float l) { return wt(l) < sp.mp ? 1.f : 0.f; }) == 0.0) {
      *covered = false;
      return -1;
    }
  }

  // top-k: threshold key kk_key; equal keys kept up to index kk_last
  uint32_t kk_key = 0, kk_eq = 0, kk_take = 0;
  int32_t kk_last = 0x7fffffff;
  if (sp.use_k) {
    double ab, n_all;
    kk_key = radix_descend(row, s, [](int, float) { return true; }, [](float) { return 0.f; }, false,
                           (double)sp.k, &ab, &kk_eq, &n_all);
    if (covered && n_all < (double)sp.k) {  // fewer than k tokens: the threshold lies below them
      *covered = false;
      return -1;
    }
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
    // top-p over the whole row (a part of it given): the whole row's mass
    const bool whole = covered && !sp.use_k;
    const double Wk = whole ? *w_row : row_sum(row, s, [&](int i, float l) { return kept_k(i, l) ? wt(l) : 0.f; });
    const double target = (double)sp.p * Wk;
    double above, m_all;
    uint32_t n_at;
    kp_key = radix_descend(row, s, kept_k, wt, true, target, &above, &n_at, &m_all);
    if (whole && m_all < target) {  // the part's mass falls short: the cut lies below it
      *covered = false;
      return -1;
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
        const float w = wt(l);
        if (sp.use_mp && w < sp.mp) return 0.f;  // min_p: a whole key group at a time (one key, one weight)
        return w;
      },
      [&](double total) { return (double)u * total; });
}

// ---------------------------------------------------------------- bf16: slice kernel + finish kernel

constexpr int kSliceThreads = 256;                                // 4 waves: many workgroups per CU
constexpr int kSliceWaves = kSliceThreads / kWave;
constexpr int kSliceRounds = 4;                                   // 16-byte chunks per thread
constexpr int kSliceTokens = kSliceThreads * kSliceRounds * 8;    // 8192 tokens per slice
constexpr int kHistBins = 256;      // window: keys within 255 of a maximum
constexpr int kHistWords = kHistBins / 2;                         // 16-bit counts, two per word
constexpr int kHistUnits = kHistBins / 8;                         // 16-byte units of a histogram
constexpr int kMaxSlices = 128;     // slices per row (2^20 tokens)
constexpr int kFinishThreads = 1024;
constexpr int kFinishWaves = kFinishThreads / kWave;
constexpr int kDrawChunks = kSliceTokens / (8 * kFinishThreads);  // 1: 8 tokens per finishing thread

__host__ __device__ inline int sample_slices(int V) { return (V + kSliceTokens - 1) / kSliceTokens; }
static_assert((int64_t)kMaxSlices * kSliceTokens <= (int64_t)kSampleMaxRounds * kWave * kFinishWaves * 4,
              "the generic path covers every row the slices cover (fp32: four tokens per chunk)");
static_assert((int64_t)kMaxSlices * kCandCap / 2 <= (int64_t)kSampleMaxRounds * kWave * kFinishWaves &&
                  kLdsCands / 2 <= kSampleMaxRounds * kWave * kFinishWaves,
              "candidate passes fit the group table (two entries per chunk)");
static_assert(kMaxSlices <= kFinishThreads, "one slice per finishing thread");
static_assert(kMaxSlices <= kMaxSlicesPow2 && kMaxSlices <= 2 * kWave, "slices of a row: two per lane, binary search");

// What the slices leave for the finish kernel.
struct SampleWs {
  uint64_t* recs;      // [bs * S]: slice maximum key | first index of it << 32
  double* masses;      // [bs * S]: slice mass relative to the slice maximum
  uint32_t* hists;     // bf16: [bs * S * kHistWords]: slice window histograms (16-bit counts)
  uint2* cands;        // fp32: [bs * S * kCandCap]: candidate lists (logit bits, index)
  uint2* meta;         // fp32: [bs * S]: (list floor key, list length)
};


// First of NB bins (ascending) whose running amount reaches goal, by one
// wave (NB / 64 consecutive bins per lane): *bin = -1 if none, *before = the
// amount strictly before it, *cnt = count(bin). No barriers.
template <int NB, class AF, class CF>
PKV_INLINE void wave_select_bins(AF amount, CF count, double goal, int* bin, double* before, uint32_t* cnt) {
  constexpr int P = NB / kWave;
  const int lane = threadIdx.x & 63;
  double a[P], sum = 0.0;
#pragma unroll
  for (int e = 0; e < P; ++e) {
    a[e] = amount(P * lane + e);
    sum += a[e];
  }
  double excl;
  const double incl = wave_scan_f64(sum, lane, &excl);
  int b = -1;
  double bef = 0.0;
  if (sum > 0.0 && excl < goal && goal <= incl) {  // at most one lane: the lanes' intervals meet exactly
    double run = excl, lastbef = 0.0;
    int lastb = -1;
#pragma unroll
    for (int e = 0; e < P; ++e)
      if (a[e] > 0.0) {
        if (b < 0 && goal <= run + a[e]) {
          b = P * lane + e;
          bef = run;
        }
        lastb = P * lane + e;
        lastbef = run;
        run += a[e];
      }
    if (b < 0) {  // rounding inside the lane: its last non-empty bin
      b = lastb;
      bef = lastbef;
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
  *bin = lane_i32(b, l0);
  *before = lane_f64(bef, l0);
  const uint32_t c = b >= 0 ? count(b) : 0u;
  *cnt = (uint32_t)lane_i32((int32_t)c, l0);
}

struct SliceLds {
  uint32_t hist[kHistBins + kWave];  // + one discard bin per lane
  double wmass[kSliceWaves];
  uint32_t wave_k[kSliceWaves];
  int32_t wave_i[kSliceWaves];
};

// Slice kernel: workgroup b reads slice b / bs of row b % bs (rows vary
// fastest, so greedy and sampled rows share every CU). Thread t holds
// chunks t, t + 256, t + 512, t + 768 of the slice. The tokens become biased
// 16-bit keys; the slice writes its maximum and the first index of it, its
// mass relative to its maximum (SampleParams::need_mass) and a count
// histogram of the keys within 255 of its maximum (bin d = kmax - key;
// SampleParams::need_cut).
PKV_INLINE void slice_phase(const SampleArgs& a, const SampleWs& ws, int row, int slice, SliceLds& L) {
  uint32_t* hist = L.hist;
  double* wmass = L.wmass;
  uint32_t* wave_k = L.wave_k;
  int32_t* wave_i = L.wave_i;
  const int V = a.vocab, S = sample_slices(V);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  SampleParams sp;
  sp.load(a, row, V);
  const bool need_mass = sp.need_mass();
  const bool need_hist = sp.need_cut();
  const bool tail = slice == S - 1;  // the only slice with tokens at or past V
  const u32x4* crow = reinterpret_cast<const u32x4*>(reinterpret_cast<const bf16_t*>(a.logits) +
                                                     (int64_t)row * a.row_stride);
  const int last_chunk = (V - 1) / 8;
  const int t0s = slice * kSliceTokens;
  u32x4 raw[kSliceRounds], key[kSliceRounds];
#pragma unroll
  for (int i = 0; i < kSliceRounds; ++i)  // indices clamped to the row's last chunk: reads stay in the row
    raw[i] = __builtin_nontemporal_load(crow + min(t0s / 8 + i * kSliceThreads + tid, last_chunk));
  if (need_hist)  // ordered before the atomics by the barrier of the block maximum
    for (int b = tid; b < kHistBins + kWave; b += kSliceThreads) hist[b] = 0;
  // Biased keys; a token at or past V gets key 0, below every real key, so
  // it never wins the maximum and never enters a window.
  // (The checks against V run in the tail slice only: a uniform branch.)
  if (tail) {
#pragma unroll
    for (int i = 0; i < kSliceRounds; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t k = bf16x2_keys(raw[i][j]);
        const int tok = t0s + 8 * (i * kSliceThreads + tid) + 2 * j;
        if (tok >= V) k = 0u;
        else if (tok + 1 >= V) k &= 0xffffu;
        key[i][j] = k;
      }
  } else {
#pragma unroll
    for (int i = 0; i < kSliceRounds; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) key[i][j] = bf16x2_keys(raw[i][j]);
  }
  u16x2 mx = {0, 0};
#pragma unroll
  for (int i = 0; i < kSliceRounds; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) mx = __builtin_elementwise_max(mx, as_u16x2(key[i][j]));
  const uint32_t tk = max((uint32_t)mx.x, (uint32_t)mx.y);
  // mass relative to this thread's maximum (rescaled below), from the raw
  // bf16 values (the keys only mark the tail's missing tokens): fp32 within
  // a chunk, fp64 above
  double mass = 0.0;
  if (need_mass) {
    // weights exp2((l - t_max) * c2): the difference first (exact for two
    // bf16 values), then one rounding of the product, so the thread's
    // reference carries no rounding of its own
    const float c2 = sp.c2, tmaxv = fmaxf(key16_value(tk), -1e30f);
    auto chunk_mass = [&](const u32x4& x, const u32x4& k, bool masked) {
      float cs = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t w = x[j];
        float w0 = fast_exp2((__uint_as_float(w << 16) - tmaxv) * c2);
        float w1 = fast_exp2((__uint_as_float(w & 0xffff0000u) - tmaxv) * c2);
        if (masked) {  // key 0: no token
          if ((k[j] & 0xffffu) == 0u) w0 = 0.f;
          if ((k[j] >> 16) == 0u) w1 = 0.f;
        }
        cs += w0;
        cs += w1;
      }
      return cs;
    };
    if (tail) {
#pragma unroll
      for (int i = 0; i < kSliceRounds; ++i) mass += (double)chunk_mass(raw[i], key[i], true);
    } else {
#pragma unroll
      for (int i = 0; i < kSliceRounds; ++i) mass += (double)chunk_mass(raw[i], key[i], false);
    }
  }
  const uint32_t wk = (uint32_t)wave_max_i32((int32_t)tk);
  if (lane == 0) wave_k[wave] = wk;
  __syncthreads();
  uint32_t kmax = wave_k[0];
#pragma unroll
  for (int w = 1; w < kSliceWaves; ++w) kmax = max(kmax, wave_k[w]);
  if (need_mass) {
    const double sc = (double)fast_exp2((fmaxf(key16_value(tk), -1e30f) - fmaxf(key16_value(kmax), -1e30f)) * sp.c2);
    const double m = wave_sum_f64(mass * sc);
    if (lane == 0) wmass[wave] = m;
  }
  // first index holding the maximum
  int32_t found = 0x7fffffff;
  if (tk == kmax) {
#pragma unroll
    for (int i = kSliceRounds - 1; i >= 0; --i)
#pragma unroll
      for (int j = 3; j >= 0; --j) {
        const int tok = t0s + 8 * (i * kSliceThreads + tid) + 2 * j;
        if ((key[i][j] >> 16) == kmax) found = tok + 1;
        if ((key[i][j] & 0xffffu) == kmax) found = tok;
      }
  }
  found = wave_min_i32(found);
  if (lane == 0) wave_i[wave] = found;
  // window histogram (keys > th, bin d = kmax - key); a token outside the
  // window goes to a discard bin, so no lane ever branches. Outside the tail
  // every key is in [1, kmax]: d = kmax - key for two tokens at once, and
  // min(d, 256 + lane) sends a token outside the window to a discard bin
  // (this lane's, or for d in [256, 256 + lane) another lane's).
  if (need_hist) {
    if (tail) {
      const uint32_t th = kmax > (uint32_t)kHistBins ? kmax - (uint32_t)kHistBins : 0u;
      const uint32_t discard = kHistBins + lane;
#pragma unroll
      for (int i = 0; i < kSliceRounds; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t lo = key[i][j] & 0xffffu, hi = key[i][j] >> 16;
          atomicAdd(&hist[lo > th ? kmax - lo : discard], 1u);
          atomicAdd(&hist[hi > th ? kmax - hi : discard], 1u);
        }
    } else {
      const u16x2 km2 = as_u16x2(kmax * 0x10001u), disc2 = as_u16x2((uint32_t)(kHistBins + lane) * 0x10001u);
#pragma unroll
      for (int i = 0; i < kSliceRounds; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t d = as_u32(__builtin_elementwise_min(km2 - as_u16x2(key[i][j]), disc2));
          atomicAdd(&hist[d & 0xffffu], 1u);
          atomicAdd(&hist[d >> 16], 1u);
        }
    }
  }
  __syncthreads();
  const int64_t slot = (int64_t)row * S + slice;  // the row's slices in index order
  if (need_hist && tid < kHistWords)  // counts <= 8192 fit 16 bits
    ws.hists[slot * kHistWords + tid] = hist[2 * tid] | (hist[2 * tid + 1] << 16);
  if (tid == 0) {
    int32_t am = wave_i[0];
    double m = 0.0;
    for (int w = 0; w < kSliceWaves; ++w) {
      am = min(am, wave_i[w]);
      if (need_mass) m += wmass[w];
    }
    ws.recs[slot] = (uint64_t)kmax | ((uint64_t)(uint32_t)am << 32);
    if (need_mass) ws.masses[slot] = m;
  }
}

__global__ void __launch_bounds__(kSliceThreads) sample_slice_kernel(SampleArgs a, SampleWs ws) {
  __shared__ SliceLds L;
  slice_phase(a, ws, blockIdx.x % a.bs, blockIdx.x / a.bs, L);
}

template <int NW, int MS>
struct FinishLds {
  u32x4 units[MS * kHistUnits];    // the slices' histograms (16-byte units)
  float uprefix[MS * kHistUnits];  // each unit's slice mass before it (row window weights)
  double w_above[NW];   // draw: mass of each wave's tokens above the cut
  int32_t w_ties[NW];   // draw: each wave's tokens in the cut bin
  double sel_rem;       // wave 0's results: the draw target in its slice,
  int32_t sel_dcut, sel_take, sel_psl, sel_tie;  // the cut, its ties, the slice, ties before it
};

// Finish kernel: one workgroup per row. The row maximum is the largest
// slice maximum, so every slice histogram is the row histogram's bins
// d >= kmax_row - kmax_slice. All tokens of a bin share one key and one
// weight, so the top-k threshold and the top-p cut come from counts times
// weights; the ties at the cut keep the first n equal-key tokens in index
// order, which fixes every slice's kept mass without reading a token. The
// draw (kept weights in index order, first running mass > u * W) picks one
// slice by those masses, then one wave of it by the waves' kept masses, then
// one thread of that wave and one of its 8 tokens. Cuts below the window
// take the generic path over the row in memory.
//
// Every wave reads the slice records and works out the row maximum itself
// (the same data, the same operations, so the same results in every wave).
// While the row histogram is built, every 16-byte unit of a slice histogram
// is staged in LDS with its slice's mass before it, so wave 0 alone takes the
// cuts, every slice's kept mass (a prefix and at most seven bins) and the
// draw's slice in one go. The workgroup meets at four barriers (the zeroed
// histogram, the row histogram, wave 0's choice, the waves' draw masses);
// plain rows pick the slice in every wave and meet once.
template <int NT, int MS>
PKV_INLINE void finish_row(const SampleArgs& a, const SampleWs& ws, int row, SampleLds<NT / kWave>& s,
                           FinishLds<NT / kWave, MS>& f) {
  constexpr int NW = NT / kWave;
  constexpr int DC = kSliceTokens / (8 * NT);  // draw: 16-byte chunks per thread
  static_assert(DC >= 1 && MS <= NT && MS <= 2 * kWave && NW <= kWave,
                "a slice per thread; two slices per lane; one wave per lane");
  const int V = a.vocab, S = sample_slices(V);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const u32x4* crow = reinterpret_cast<const u32x4*>(reinterpret_cast<const bf16_t*>(a.logits) +
                                                     (int64_t)row * a.row_stride);
  const int last_chunk = (V - 1) / 8;
  const int64_t slot0 = (int64_t)row * S;

  // The slices' histograms as 16-byte units, loaded first (their addresses
  // need nothing else): unit q holds bins [8u, 8u + 8) (u = q % 32) of slice
  // q / 32; thread t takes units t + NT e.
  const u32x4* hrow = reinterpret_cast<const u32x4*>(ws.hists + slot0 * kHistWords);
  const int NU = S * kHistUnits;
  constexpr int kU = MS * kHistUnits / NT;  // 4 units per thread at most
  // (issued before the row's parameters arrive; a greedy or plain row's
  // workspace holds stale histograms and masses, read but never used)
  u32x4 v[kU];
#pragma unroll
  for (int e = 0; e < kU; ++e) {
    const int q = e * NT + tid;
    v[e] = q < NU ? hrow[q] : u32x4{0u, 0u, 0u, 0u};
  }
  // slice records (every wave; lane l holds slices l and l + 64) and masses
  const bool in0 = lane < S, in1 = lane + 64 < S;
  const uint64_t r0 = in0 ? ws.recs[slot0 + lane] : 0ull;
  const uint64_t r1 = in1 ? ws.recs[slot0 + lane + 64] : 0ull;
  const double mr0 = in0 ? ws.masses[slot0 + lane] : 0.0;  // relative to the slice maxima
  const double mr1 = in1 ? ws.masses[slot0 + lane + 64] : 0.0;
  SampleParams sp;
  sp.load(a, row, V);
  const bool need_mass = sp.need_mass();
  const bool plain = sp.plain();
  const float c2 = sp.c2;
  if (sp.greedy) {
    if (wave == 0) {
      const int32_t k0 = (int32_t)(uint32_t)r0, k1 = (int32_t)(uint32_t)r1;
      const int32_t mk = wave_max_i32(max(k0, k1));
      const int32_t am = wave_min_i32(min((in0 && k0 == mk) ? (int32_t)(r0 >> 32) : 0x7fffffff,
                                          (in1 && k1 == mk) ? (int32_t)(r1 >> 32) : 0x7fffffff));
      if (lane == 0) a.out[row] = am == 0x7fffffff ? 0 : am;  // slices are in index order
    }
    return;
  }
  if (!plain) {
    for (int b = tid; b < kHistBins; b += NT) s.hist[b] = 0;
    __syncthreads();  // A: the row histogram starts at zero (the loads above are still in flight)
  }

  // ---- row maximum, its first index, slice distances below it, slice
  // masses in units of the row maximum
  const int32_t k0 = (int32_t)(uint32_t)r0, k1 = (int32_t)(uint32_t)r1;
  const int32_t mk = wave_max_i32(max(k0, k1));
  const int32_t am = wave_min_i32(min((in0 && k0 == mk) ? (int32_t)(r0 >> 32) : 0x7fffffff,
                                      (in1 && k1 == mk) ? (int32_t)(r1 >> 32) : 0x7fffffff));
  const int32_t argmax = am == 0x7fffffff ? 0 : am;
  const uint32_t rkmax = (uint32_t)mk;
  const float lmax = key16_value(rkmax);
  const int32_t dl0 = mk - k0, dl1 = mk - k1;
  double m0 = 0.0, m1 = 0.0, wall = 0.0;  // wall: mass of the whole row (plain rows, top-p without top-k)
  if (need_mass) {
    if (in0) m0 = mr0 * (double)fast_exp2((fmaxf(key16_value((uint32_t)k0), -1e30f) - lmax) * c2);
    if (in1) m1 = mr1 * (double)fast_exp2((fmaxf(key16_value((uint32_t)k1), -1e30f) - lmax) * c2);
    wall = wave_sum_f64(m0 + m1);
  }

  int dcut = -1;      // cut bin (rows with a cut); tokens with d < dcut are kept
  uint32_t take = 0;  // tokens of bin dcut kept: the first ones in index order
  double wcut = 0.0;  // their weight
  int psl = 0;        // the slice holding the draw
  double rem = 0.0;   // the draw target within it
  int32_t tie_base = 0;  // cut-bin tokens of the row before it

  // The slice holding the draw, from the kept mass of slices lane and lane +
  // 64 (cut bin excluded) and their cut-bin tokens; one wave.
  auto select_slice = [&](double ms0, double ms1, int32_t cc0, int32_t cc1) {
    // cut-bin tokens of the slices before each slice
    const int32_t i0 = wave_incl_scan_i32(cc0, lane);
    const int32_t i1 = lane_i32(i0, 63) + wave_incl_scan_i32(cc1, lane);
    const int32_t cb0 = i0 - cc0, cb1 = i1 - cc1;
    if (!plain) {
      ms0 += (double)min(max((int32_t)take - cb0, 0), cc0) * wcut;
      ms1 += (double)min(max((int32_t)take - cb1, 0), cc1) * wcut;
    }
    // running kept mass over the slices in index order; consecutive slices'
    // [excl, incl) intervals meet exactly
    double ex0, ex1;
    const double in_0 = wave_scan_f64(ms0, lane, &ex0);
    const double t0 = lane_f64(in_0, 63);
    const double in_1 = wave_scan_f64(ms1, lane, &ex1) + t0;
    ex1 += t0;
    const double target = (double)sp.u * lane_f64(in_1, 63);
    const uint64_t b0 = __ballot(ms0 > 0.0 && ex0 <= target && target < in_0);
    const uint64_t b1 = __ballot(ms1 > 0.0 && ex1 <= target && target < in_1);
    if (b0) {
      const int l = __ffsll((unsigned long long)b0) - 1;
      psl = l;
      rem = target - lane_f64(ex0, l);
      tie_base = lane_i32(cb0, l);
    } else if (b1) {
      const int l = __ffsll((unsigned long long)b1) - 1;
      psl = 64 + l;
      rem = target - lane_f64(ex1, l);
      tie_base = lane_i32(cb1, l);
    } else {  // rounding left the target past every slice: the last slice with mass
      psl = max(wave_max_i32(max(ms0 > 0.0 ? lane : -1, ms1 > 0.0 ? lane + 64 : -1)), 0);
      rem = INFINITY;
      tie_base = psl < 64 ? lane_i32(cb0, psl) : lane_i32(cb1, psl - 64);
    }
  };

  if (plain) {
    select_slice(m0, m1, 0, 0);  // every wave: the same data, the same result
  } else {
    // distance of each unit's slice below the row maximum (from the lane
    // that holds the slice)
    int32_t ud[kU];
#pragma unroll
    for (int e = 0; e < kU; ++e) {
      ud[e] = 0;
      if (e * NT + wave * kWave < NU) {  // wave-uniform: waves past the units skip
        const int sl = min((e * NT + tid) / kHistUnits, MS - 1);
        const int32_t a0 = __shfl(dl0, sl & 63), a1 = __shfl(dl1, sl & 63);
        ud[e] = sl < 64 ? a0 : a1;
      }
    }
    // ---- the row histogram; every unit staged in LDS with its slice's mass
    // before it (exact counts times the window weights, fp32: the unit's eight
    // bins, then an exclusive scan over the slice's 32 units, one half-wave);
    // wave 0 writes the window weights
#pragma unroll
    for (int e = 0; e < kU; ++e) {
      if (e * NT + wave * kWave < NU) {  // wave-uniform
        const int q = e * NT + tid;
        const bool in = q < NU;
        const int b0 = 8 * (q % kHistUnits) + ud[e];
        float um = 0.f;
        if (in) {
          f.units[q] = v[e];
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            const uint32_t n = (v[e][c >> 1] >> (16 * (c & 1))) & 0xffffu;
            const int b = b0 + c;
            if (n && b < kHistBins) {
              atomicAdd(&s.hist[b], n);
              um = fmaf((float)n, (uint32_t)b <= rkmax ? row_weight(key16_value(rkmax - (uint32_t)b), lmax, c2) : 0.f,
                        um);
            }
          }
        }
        // exclusive prefix over the 32 units of the slice (lanes 32h .. 32h +
        // 31): Kogge-Stone inside each 16-lane row (row_shr 1, 2, 4, 8), the
        // half's first row total added to its second row, then the previous
        // lane's inclusive value
        float inc = um;
        inc += dpp<0x111>(inc);
        inc += dpp<0x112>(inc);
        inc += dpp<0x114>(inc);
        inc += dpp<0x118>(inc);
        const float row_tot = __shfl(inc, (lane & 32) + 15, 64);
        if (lane & 16) inc += row_tot;
        const float prev = __shfl(inc, (lane + 63) & 63, 64);
        if (in) f.uprefix[q] = (lane & 31) ? prev : 0.f;
      }
    }
    if (wave == 0)
#pragma unroll
      for (int e = 0; e < kHistBins / kWave; ++e) {
        const int b = e * kWave + lane;
        s.wtab[b] = (uint32_t)b <= rkmax ? row_weight(key16_value(rkmax - (uint32_t)b), lmax, c2) : 0.f;
      }
    __syncthreads();  // B

    // ---- cuts, every slice's kept mass and the draw's slice (wave 0)
    if (wave == 0) {
      auto hc = [&](int b) { return s.hist[b]; };
      int dk = -1;
      uint32_t kk_take = 0, kk_eq = 0;
      if (sp.use_k) {
        double before;
        wave_select_bins<kHistBins>([&](int b) { return (double)hc(b); }, hc, (double)sp.k, &dk, &before, &kk_eq);
        if (dk >= 0) kk_take = (uint32_t)sp.k - (uint32_t)before;
      }
      int dc = dk;
      uint32_t tk2 = kk_take;
      if (sp.use_p && (!sp.use_k || dk >= 0)) {
        const int dlim = sp.use_k ? dk : kHistBins - 1;
        auto nb = [&](int b) { return b < dlim ? hc(b) : (b == dlim ? (sp.use_k ? kk_take : hc(b)) : 0u); };
        double Wk = wall;
        if (sp.use_k) {
          double part = 0.0;
#pragma unroll
          for (int e = 0; e < kHistBins / kWave; ++e) {
            const int b = (kHistBins / kWave) * lane + e;
            part += (double)nb(b) * (double)s.wtab[b];
          }
          Wk = wave_sum_f64(part);
        }
        const double target = (double)sp.p * Wk;
        int dstar;
        double above;
        uint32_t n_at;
        wave_select_bins<kHistBins>([&](int b) { return (double)nb(b) * (double)s.wtab[b]; }, nb, target, &dstar,
                                    &above, &n_at);
        dc = dstar;
        if (dstar >= 0) {
          // equal-key tokens at the cut: token j of the group (0-based) is kept iff above + j * w < target
          double need = ceil((target - above) / (double)s.wtab[dstar]);
          if (!(need >= 1.0)) need = 1.0;
          tk2 = need >= (double)n_at ? n_at : (uint32_t)need;
        }
      }
      if (sp.use_mp) {
        // min_p keeps the bins whose weight (probability over the largest)
        // is at least mp: bins d < dm, dm the first bin below it (-1 when
        // every bin of the window is kept, i.e. its cut lies below the
        // window). Both sets are prefixes of the ranking, so their
        // intersection is the shorter one; bin dm keeps no token.
        int dm = -1;
#pragma unroll
        for (int e = kHistBins / kWave - 1; e >= 0; --e) {
          const uint64_t bl = __ballot(s.wtab[e * kWave + lane] < sp.mp);
          if (bl) dm = e * kWave + __ffsll((unsigned long long)bl) - 1;
        }
        if (!sp.use_k && !sp.use_p) {
          dc = dm;
          tk2 = 0;
        } else if (dc >= 0 && dm >= 0 && dm <= dc) {
          dc = dm;
          tk2 = 0;
        }
      }
      if (dc >= 0) {
        dcut = dc;
        take = tk2;
        wcut = (double)s.wtab[dc];
        // slice s's kept mass: its bins above the cut (slice bins below
        // j = dcut - distance), the units before j's unit from the staged
        // prefix, the rest of j's unit bin by bin; its cut-bin tokens: bin j
        auto slice_cut = [&](int sl, int32_t dist, double* msl, int32_t* cc) {
          *msl = 0.0;
          *cc = 0;
          if (sl >= S) return;
          const int j = dc - dist;
          if (j < 0) return;  // the whole slice lies below the cut
          const int u = j >> 3;
          const u32x4 x = f.units[sl * kHistUnits + u];
          float m = f.uprefix[sl * kHistUnits + u];
#pragma unroll
          for (int c = 0; c < 7; ++c)
            if (c < (j & 7)) m = fmaf((float)((x[c >> 1] >> (16 * (c & 1))) & 0xffffu), s.wtab[8 * u + c + dist], m);
          *msl = (double)m;
          *cc = (int32_t)((x[(j & 7) >> 1] >> (16 * (j & 1))) & 0xffffu);
        };
        double ms0, ms1;
        int32_t c0, c1;
        slice_cut(lane, dl0, &ms0, &c0);
        slice_cut(lane + 64, dl1, &ms1, &c1);
        select_slice(ms0, ms1, c0, c1);
      }
      if (lane == 0) {
        f.sel_dcut = dc;
        f.sel_take = (int32_t)tk2;
        f.sel_psl = psl;
        f.sel_tie = tie_base;
        f.sel_rem = rem;
      }
    }
    __syncthreads();  // C
    dcut = f.sel_dcut;
    if (dcut < 0) {  // the cut lies below the window
      SampleRow<bf16_t, NW> mrow;
      mrow.init(reinterpret_cast<const bf16_t*>(a.logits) + (int64_t)row * a.row_stride, V, wave, lane);
      const int32_t idx = sample_generic(mrow, s, sp, lmax);
      if (tid == 0) a.out[row] = idx >= 0 ? idx : argmax;
      return;
    }
    take = (uint32_t)f.sel_take;
    psl = f.sel_psl;
    tie_base = f.sel_tie;
    rem = f.sel_rem;
    wcut = (double)s.wtab[dcut];
  }

  // ---- the draw inside slice psl: thread t holds tokens [8t, 8t + 8) of it
  const int tok0 = psl * kSliceTokens + 8 * DC * tid;
  // Kept: keys above lo_key (plain rows: every real token, key 0 marks the
  // tokens at or past V); ties: keys equal to tie_key (none in plain rows).
  const uint32_t cut_key = rkmax - (uint32_t)max(dcut, 0);
  const uint32_t lo_key = plain ? 0u : cut_key, tie_key = plain ? 0xffffffffu : cut_key;
  const float wcut_f = (float)wcut;
  u32x4 x[DC], kx[DC];  // the tokens (bf16 pairs) and their biased keys
#pragma unroll
  for (int i = 0; i < DC; ++i) x[i] = crow[min(tok0 / 8 + i, last_chunk)];  // clamped: stays in the row
#pragma unroll
  for (int i = 0; i < DC; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) kx[i][j] = bf16x2_keys(x[i][j]);
  if (psl == S - 1)  // the tail slice (uniform): key 0, below every real key, at or past V
#pragma unroll
    for (int i = 0; i < DC; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int tok = tok0 + 8 * i + 2 * j;
        if (tok >= V) kx[i][j] = 0u;
        else if (tok + 1 >= V) kx[i][j] &= 0xffffu;
      }
  auto key_of = [&](int i, int e) -> uint32_t {
    const uint32_t kw = kx[i][e >> 1];
    return (e & 1) ? (kw >> 16) : (kw & 0xffffu);
  };
  // weight of token e of chunk i if it lies above the cut (0 otherwise)
  auto above_w = [&](int i, int e) -> float {
    const uint32_t w = x[i][e >> 1];
    const float wt = row_weight(__uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16)), lmax, c2);
    return key_of(i, e) > lo_key ? wt : 0.f;
  };
  // this thread's mass above the cut (fp32 over its tokens) and its cut-bin
  // tokens; the weights stay in registers for the replay
  float above = 0.f, wt[DC][8];
  int32_t nt = 0;
#pragma unroll
  for (int i = 0; i < DC; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      wt[i][e] = above_w(i, e);
      above += wt[i][e];
      nt += key_of(i, e) == tie_key ? 1 : 0;
    }
  double exA;
  const double inA = wave_scan_f64((double)above, lane, &exA);
  const int32_t inN = wave_incl_scan_i32(nt, lane), exN = inN - nt;
  if (lane == 63) {
    f.w_above[wave] = inA;
    f.w_ties[wave] = inN;
  }
  __syncthreads();  // E

  // ---- the wave holding the draw: lane w < NW takes wave w's kept mass
  // M_w = A_w + wcut * (its kept cut-bin tokens); a scan over the lanes gives
  // the waves' [R_w, R_{w+1}) in wave order
  const double Aw = lane < NW ? f.w_above[lane] : 0.0;
  const int32_t Nw = lane < NW ? f.w_ties[lane] : 0;
  const int32_t TBw = tie_base + wave_incl_scan_i32(Nw, lane) - Nw;  // cut-bin tokens of the row before wave `lane`
  const int32_t Kw = max((int32_t)take - TBw, 0);                    // of them, still to keep
  const double Mw = Aw + wcut * (double)min(Kw, Nw);
  double Rx;
  const double Ri = wave_scan_f64(Mw, lane, &Rx);
  const uint64_t whit = __ballot(Mw > 0.0 && Rx <= rem && rem < Ri);
  const bool past = !whit;  // rounding left the target past every wave: the last kept token
  const int wsel = whit ? __ffsll((unsigned long long)whit) - 1
                        : wave_max_i32(Mw > 0.0 ? lane : -1);
  if (wsel < 0) {  // nothing kept in the slice (every weight underflowed): the argmax
    if (tid == 0) a.out[row] = argmax;
    return;
  }
  const double Rsel = lane_f64(Rx, wsel);
  if (wave != wsel) return;
  // Lane intervals [excl, incl) of the chosen wave: consecutive lanes meet
  // exactly (the scans hand the previous lane's inclusive values on); the
  // last lane ends at R_wsel + M_wsel, within rounding of R_{wsel+1} (a
  // target in between takes the wave's last kept token).
  const int32_t K = lane_i32(Kw, wsel);
  const double excl = Rsel + (exA + wcut * (double)min(K, exN));
  const double incl = Rsel + (inA + wcut * (double)min(K, inN));
  // replay: kept weights in index order (the cut-bin tokens of rank < take)
  int32_t rank = lane_i32(TBw, wsel) + exN;
  double run = excl;
  int32_t res = -1, lastk = -1;
#pragma unroll
  for (int i = 0; i < DC; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float w = wt[i][e];
      if (key_of(i, e) == tie_key && (uint32_t)(rank++) < take) w = wcut_f;
      if (w > 0.f) {
        const int idx = tok0 + 8 * i + e;
        if (res < 0 && run + (double)w > rem) res = idx;
        lastk = idx;
        run += (double)w;
      }
    }
  const uint64_t hit = __ballot(!past && excl <= rem && rem < incl);
  int32_t r;
  if (hit) {
    const int l = __ffsll((unsigned long long)hit) - 1;
    r = lane_i32(res >= 0 ? res : lastk, l);  // rounding ran past the lane's tokens: its last kept one
  } else {
    r = wave_max_i32(lastk);  // the wave's last kept token
  }
  if (lane == 0) a.out[row] = r >= 0 ? r : argmax;
}

__global__ void __launch_bounds__(kFinishThreads) sample_finish_kernel(SampleArgs a, SampleWs ws) {
  __shared__ SampleLds<kFinishWaves> s;
  __shared__ FinishLds<kFinishWaves, kMaxSlices> f;
  finish_row<kFinishThreads, kMaxSlices>(a, ws, blockIdx.x, s, f);
}

// ---------------------------------------------------------------- fp32: slice kernel + finish kernel

constexpr int kSlice32Rounds = kSliceTokens / (4 * kSliceThreads);  // 8 chunks of 4 floats per thread

// fp32 slice kernel: workgroup b reads slice b / bs of row b % bs (thread t:
// chunks t + 256i, i < 8). It writes the slice maximum (32-bit key) and the
// first index of it, the mass relative to it (SampleParams::need_mass) and,
// for rows with a cut, a candidate list: every token of the slice whose key
// is at or above a floor, in index order. The floor comes from a count
// histogram of the keys' upper 16 bits within 255 of the slice maximum's:
// the deepest bin whose running count stays within kCandCap (for top-k, the
// first bin where it reaches k, if that fits: no deeper token of this slice
// can be among the row's k largest; for min_p alone, no deeper than the
// first bin that weighs below min_p).
__global__ void __launch_bounds__(kSliceThreads) sample_slice32_kernel(SampleArgs a, SampleWs ws) {
  using E = SampleElem<float>;
  constexpr int R = kSlice32Rounds;
  __shared__ uint32_t hist[kHistBins];
  __shared__ double wmass[kSliceWaves];
  __shared__ uint32_t wave_k[kSliceWaves];
  __shared__ int32_t wave_i[kSliceWaves];
  __shared__ int32_t rtot[R][kSliceWaves];
  __shared__ uint32_t floor_sh;
  const int V = a.vocab, S = sample_slices(V);
  const int row = blockIdx.x % a.bs, slice = blockIdx.x / a.bs;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  SampleParams sp;
  sp.load(a, row, V);
  const bool need_mass = sp.need_mass();
  const bool need_list = sp.need_cut();
  const bool tail = slice == S - 1;  // the only slice with tokens at or past V
  const u32x4* crow = reinterpret_cast<const u32x4*>(reinterpret_cast<const float*>(a.logits) +
                                                     (int64_t)row * a.row_stride);
  const int last_chunk = (V - 1) / 4;
  const int t0s = slice * kSliceTokens;
  u32x4 raw[R];
#pragma unroll
  for (int i = 0; i < R; ++i)  // indices clamped to the row's last chunk: reads stay in the row
    raw[i] = __builtin_nontemporal_load(crow + min(t0s / 4 + i * kSliceThreads + tid, last_chunk));
  if (need_list)  // ordered before the atomics by the barrier of the block maximum
    for (int b = tid; b < kHistBins; b += kSliceThreads) hist[b] = 0;
  // the tokens become their keys in place (0, below every real key, at or
  // past V); a key gives its logit back (-0 as +0, which weighs the same)
  if (tail) {
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t k = E::key(__uint_as_float(raw[i][e]));
        raw[i][e] = t0s + 4 * (i * kSliceThreads + tid) + e >= V ? 0u : k;
      }
  } else {
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) raw[i][e] = E::key(__uint_as_float(raw[i][e]));
  }
  auto key = [&](int i, int e) -> uint32_t { return raw[i][e]; };
  uint32_t tk = 0;
#pragma unroll
  for (int i = 0; i < R; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) tk = max(tk, key(i, e));
  double mass = 0.0;  // relative to this thread's maximum: fp32 within a chunk, fp64 above
  if (need_mass) {
    // weights exp2((l - t_max) * c2), the difference taken first (see the
    // bf16 slice kernel)
    const float c2 = sp.c2, tmaxv = fmaxf(E::key_value(tk), -1e30f);
#pragma unroll
    for (int i = 0; i < R; ++i) {
      float cs = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float w = fast_exp2((E::key_value(key(i, e)) - tmaxv) * c2);
        cs += key(i, e) ? w : 0.f;
      }
      mass += (double)cs;
    }
  }
  // unsigned maximum through the signed one: flipping the top bit keeps the order
  const uint32_t wk = (uint32_t)wave_max_i32((int32_t)(tk ^ 0x80000000u)) ^ 0x80000000u;
  if (lane == 0) wave_k[wave] = wk;
  __syncthreads();
  uint32_t kmax = wave_k[0];
#pragma unroll
  for (int w = 1; w < kSliceWaves; ++w) kmax = max(kmax, wave_k[w]);
  if (need_mass) {
    const double sc =
        (double)fast_exp2((fmaxf(E::key_value(tk), -1e30f) - fmaxf(E::key_value(kmax), -1e30f)) * sp.c2);
    const double m = wave_sum_f64(mass * sc);
    if (lane == 0) wmass[wave] = m;
  }
  int32_t found = 0x7fffffff;  // first index holding the maximum
  if (tk == kmax) {
#pragma unroll
    for (int i = R - 1; i >= 0; --i)
#pragma unroll
      for (int e = 3; e >= 0; --e)
        if (key(i, e) == kmax) found = t0s + 4 * (i * kSliceThreads + tid) + e;
  }
  found = wave_min_i32(found);
  if (lane == 0) wave_i[wave] = found;
  const uint32_t cmax = kmax >> 16;
  if (need_list) {  // bin d = cmax - (key >> 16); most tokens lie below the window and add nothing
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t k = key(i, e), d = cmax - (k >> 16);
        if (k != 0u && d < (uint32_t)kHistBins) atomicAdd(&hist[d], 1u);
      }
  }
  __syncthreads();
  if (need_list) {
    if (wave == 0) {  // the list's floor: lane l holds bins 4l .. 4l + 3
      uint32_t c[4], run = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        c[e] = hist[4 * lane + e];
        run += c[e];
      }
      const int32_t incl = wave_incl_scan_i32((int32_t)run, lane);
      int32_t cum = incl - (int32_t)run, d_cap = -1, d_k = 0x7fffffff;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        cum += (int32_t)c[e];
        if (cum <= kCandCap) d_cap = 4 * lane + e;
        if (cum >= sp.k && d_k == 0x7fffffff) d_k = 4 * lane + e;
      }
      d_cap = wave_max_i32(d_cap);
      d_k = wave_min_i32(d_k);
      // use_k: a bin whose running count reaches k and fits is deep enough
      int d = (sp.use_k && d_k <= d_cap) ? d_k : d_cap;
      if (sp.use_mp && !sp.use_k && !sp.use_p) {
        // min_p alone: a bin whose largest logit weighs below min_p against
        // this slice's maximum weighs below it against the row's too: it and
        // every deeper bin are never kept (the finish kernel checks that the
        // lists' floor lies below the cut)
        const float ls = E::key_value(kmax);
        int d_mp = 0x7fffffff;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int b = 4 * lane + e;
          if (b >= 1 && (uint32_t)b <= cmax &&
              row_weight(E::key_value(((cmax - (uint32_t)b) << 16) | 0xffffu), ls, sp.c2) < sp.mp)
            d_mp = min(d_mp, b);
        }
        d_mp = wave_min_i32(d_mp);
        if (d_mp != 0x7fffffff) d = min(d, d_mp - 1);
      }
      if (lane == 0) floor_sh = d < 0 ? 0xffffffffu : ((uint32_t)d >= cmax ? 1u : (cmax - (uint32_t)d) << 16);
    }
    __syncthreads();
  }
  const int64_t slot = (int64_t)row * S + slice;  // the row's slices in index order
  if (need_list) {
    // listed tokens (key >= floor) in index order: round-major, then thread, then element
    const uint32_t fl = floor_sh;
    int32_t n[R], incl[R];
#pragma unroll
    for (int i = 0; i < R; ++i) {
      n[i] = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) n[i] += key(i, e) >= fl ? 1 : 0;
      incl[i] = wave_incl_scan_i32(n[i], lane);
      if (lane == 63) rtot[i][wave] = incl[i];
    }
    __syncthreads();
    int32_t run = 0, off[R];
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
      for (int w = 0; w < kSliceWaves; ++w) {
        if (w == wave) off[i] = run + incl[i] - n[i];
        run += rtot[i][w];
      }
    uint2* list = ws.cands + slot * kCandCap;
#pragma unroll
    for (int i = 0; i < R; ++i) {
      int32_t pos = off[i];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (key(i, e) >= fl) {
          if (pos < kCandCap)
            list[pos] = make_uint2(__float_as_uint(E::key_value(key(i, e))),
                                   (uint32_t)(t0s + 4 * (i * kSliceThreads + tid) + e));
          ++pos;
        }
    }
    if (tid == 0) ws.meta[slot] = make_uint2(fl, (uint32_t)min(run, kCandCap));
  }
  if (tid == 0) {
    int32_t am = wave_i[0];
    double m = 0.0;
    for (int w = 0; w < kSliceWaves; ++w) {
      am = min(am, wave_i[w]);
      if (need_mass) m += wmass[w];
    }
    ws.recs[slot] = (uint64_t)kmax | ((uint64_t)(uint32_t)am << 32);
    if (need_mass) ws.masses[slot] = m;
  }
}

// fp32 finish kernel: one workgroup per row. Greedy rows take the argmax
// from the slice records. Rows without a cut pick the slice holding the draw
// by the slice masses and scan that slice in memory. Rows with a cut run the
// generic cuts and draw over the candidate lists (tokens at or above the
// largest list floor); when a cut falls outside them, over the row in memory.
__global__ void __launch_bounds__(kFinishThreads) sample_finish32_kernel(SampleArgs a, SampleWs ws) {
  using E = SampleElem<float>;
  __shared__ SampleLds<kFinishWaves> s;
  __shared__ __align__(16) uint2 lcands[kLdsCands];
  __shared__ int32_t sl_cnt[kMaxSlices];
  __shared__ int32_t sl_beg[kMaxSlices];
  __shared__ double sl_mass[kMaxSlices];
  __shared__ uint32_t h_u[5];
  __shared__ double h_f[2];
  const int V = a.vocab, S = sample_slices(V);
  const int row = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  SampleParams sp;
  sp.load(a, row, V);
  const bool plain = sp.plain();
  const float c2 = sp.c2;
  const float* lrow = reinterpret_cast<const float*>(a.logits) + (int64_t)row * a.row_stride;
  const int64_t slot0 = (int64_t)row * S;

  if (wave == 0) {  // slice records: lane l holds slices l and l + 64
    const bool in0 = lane < S, in1 = lane + 64 < S;
    const uint64_t r0 = in0 ? ws.recs[slot0 + lane] : 0ull, r1 = in1 ? ws.recs[slot0 + lane + 64] : 0ull;
    const uint32_t k0 = (uint32_t)r0, k1 = (uint32_t)r1;  // 0 for no slice: below every real key
    const uint32_t mk = (uint32_t)wave_max_i32((int32_t)(max(k0, k1) ^ 0x80000000u)) ^ 0x80000000u;
    const int32_t am = wave_min_i32(min((in0 && k0 == mk) ? (int32_t)(r0 >> 32) : 0x7fffffff,
                                        (in1 && k1 == mk) ? (int32_t)(r1 >> 32) : 0x7fffffff));
    const int32_t argmax = am == 0x7fffffff ? 0 : am;  // slices are in index order
    if (sp.greedy) {
      if (lane == 0) a.out[row] = argmax;
    } else {
      const float lmax = E::key_value(mk);
      double m0 = 0.0, m1 = 0.0, wall = 0.0;
      if (sp.need_mass()) {
        if (in0) m0 = ws.masses[slot0 + lane] * (double)fast_exp2((fmaxf(E::key_value(k0), -1e30f) - lmax) * c2);
        if (in1) m1 = ws.masses[slot0 + lane + 64] * (double)fast_exp2((fmaxf(E::key_value(k1), -1e30f) - lmax) * c2);
        wall = wave_sum_f64(m0 + m1);
      }
      uint32_t fl = 0;
      if (plain) {
        sl_mass[lane] = m0;
        sl_mass[lane + 64] = m1;
      } else {
        const uint2 me0 = in0 ? ws.meta[slot0 + lane] : make_uint2(0u, 0u);
        const uint2 me1 = in1 ? ws.meta[slot0 + lane + 64] : make_uint2(0u, 0u);
        fl = (uint32_t)wave_max_i32((int32_t)(max(me0.x, me1.x) ^ 0x80000000u)) ^ 0x80000000u;
        sl_cnt[lane] = (int32_t)me0.y;
        sl_cnt[lane + 64] = (int32_t)me1.y;
        // packed chunks: exclusive prefix of the lists' chunk counts, slices in order
        const int32_t c0 = ((int32_t)me0.y + 1) / 2, c1 = ((int32_t)me1.y + 1) / 2;
        const int32_t i0 = wave_incl_scan_i32(c0, lane);
        const int32_t i1 = lane_i32(i0, 63) + wave_incl_scan_i32(c1, lane);
        sl_beg[lane] = i0 - c0;
        sl_beg[lane + 64] = i1 - c1;
        if (lane == 0) h_u[4] = (uint32_t)lane_i32(i1, 63);
      }
      if (lane == 0) {
        h_u[0] = mk;
        h_u[1] = (uint32_t)argmax;
        h_u[2] = fl;
        h_f[0] = wall;
      }
    }
  }
  if (sp.greedy) return;
  __syncthreads();
  const float lmax = E::key_value(h_u[0]);
  const int32_t argmax = (int32_t)h_u[1];
  int32_t idx;
  if (plain) {
    if (wave == 0) {  // the slice holding the draw: running mass over the slices in index order
      const double ms0 = lane < S ? sl_mass[lane] : 0.0, ms1 = lane + 64 < S ? sl_mass[lane + 64] : 0.0;
      double ex0, ex1;
      const double in_0 = wave_scan_f64(ms0, lane, &ex0);
      const double t0 = lane_f64(in_0, 63);
      const double in_1 = wave_scan_f64(ms1, lane, &ex1) + t0;
      ex1 += t0;
      const double target = (double)sp.u * lane_f64(in_1, 63);
      const uint64_t b0 = __ballot(ms0 > 0.0 && ex0 <= target && target < in_0);
      const uint64_t b1 = __ballot(ms1 > 0.0 && ex1 <= target && target < in_1);
      int32_t psl;
      double rem;
      if (b0) {
        const int l = __ffsll((unsigned long long)b0) - 1;
        psl = l;
        rem = target - lane_f64(ex0, l);
      } else if (b1) {
        const int l = __ffsll((unsigned long long)b1) - 1;
        psl = 64 + l;
        rem = target - lane_f64(ex1, l);
      } else {  // rounding left the target past every slice: the last slice with mass
        psl = max(wave_max_i32(max(ms0 > 0.0 ? lane : -1, ms1 > 0.0 ? lane + 64 : -1)), 0);
        rem = INFINITY;
      }
      if (lane == 0) {
        h_u[3] = (uint32_t)psl;
        h_f[1] = rem;
      }
    }
    __syncthreads();
    const int psl = (int)h_u[3];
    const double rem = h_f[1];
    SampleRow<float, kFinishWaves> srow;
    srow.init(lrow + (int64_t)psl * kSliceTokens, min(kSliceTokens, V - psl * kSliceTokens), wave, lane);
    idx = find_crossing(srow, s, [&](int, float l) { return row_weight(l, lmax, c2); },
                        [&](double) { return rem; });
    if (idx >= 0) idx += psl * kSliceTokens;
  } else {
    const double wall = h_f[0];
    CandRow<kFinishWaves> crow;
    crow.init(ws.cands + slot0 * kCandCap, sl_beg, sl_cnt, S, (int)h_u[4], h_u[2], wave, lane);
    bool covered;
    const uint32_t fl = h_u[2];  // the largest logit below the lists' floor (none: -inf)
    const float below = fl > 1u ? E::key_value(fl - 1u) : -INFINITY;
    // the candidates into LDS when they fit (every later pass then reads
    // LDS); not tried when the lists are far longer than LDS holds (full
    // lists, as for top-p over the whole row, keep nearly every entry)
    const int nl = 2 * (int)h_u[4] <= 4 * kLdsCands ? compact_row(crow, s, lcands, kLdsCands) : -1;
    if (nl >= 0) {
      LdsRow<kFinishWaves> lrow;
      lrow.init(lcands, nl, wave, lane);
      idx = sample_generic(lrow, s, sp, lmax, &wall, &covered, below);
    } else {
      idx = sample_generic(crow, s, sp, lmax, &wall, &covered, below);
    }
    if (!covered) {
      SampleRow<float, kFinishWaves> frow;
      frow.init(lrow, V, wave, lane);
      idx = sample_generic(frow, s, sp, lmax);
    }
  }
  if (tid == 0) a.out[row] = idx >= 0 ? idx : argmax;
}

}  // namespace pkv
