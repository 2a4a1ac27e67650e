// Shared device helpers for the gfx950 kernels of libpkv.
//
// Wave64 throughout. Nothing here writes through the scalar data cache:
// every global store and atomic is a vector (global_*) operation.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

constexpr int kWave = 64;
constexpr int kHeadDim = 128;

typedef uint16_t bf16_t;  // bf16 bit pattern
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // one 16-byte packet

// ---------------------------------------------------------------- bf16 <-> f32

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(bf16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Round to nearest even (inputs finite).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// ---------------------------------------------------------------- cross-lane sums
// All-reduce a float over aligned groups of N lanes (N in 1,2,4,8,16,32,64).
// N <= 16 stays inside a DPP row; larger groups use cross-row shuffles.

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, true));
}

template <int N>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (N >= 2) x += dpp<0xB1>(x);    // quad_perm [1,0,3,2]: lane ^ 1
  if constexpr (N >= 4) x += dpp<0x4E>(x);    // quad_perm [2,3,0,1]: lane ^ 2
  if constexpr (N >= 8) x += dpp<0x141>(x);   // row_half_mirror: other quad of the 8-group
  if constexpr (N >= 16) x += dpp<0x140>(x);  // row_mirror: other half of the 16-row
  if constexpr (N >= 32) x += __shfl_xor(x, 16, 64);
  if constexpr (N >= 64) x += __shfl_xor(x, 32, 64);
  return x;
}

template <int N>
__device__ __forceinline__ float group_max(float x) {
  if constexpr (N >= 2) x = fmaxf(x, dpp<0xB1>(x));
  if constexpr (N >= 4) x = fmaxf(x, dpp<0x4E>(x));
  if constexpr (N >= 8) x = fmaxf(x, dpp<0x141>(x));
  if constexpr (N >= 16) x = fmaxf(x, dpp<0x140>(x));
  if constexpr (N >= 32) x = fmaxf(x, __shfl_xor(x, 16, 64));
  if constexpr (N >= 64) x = fmaxf(x, __shfl_xor(x, 32, 64));
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------- faults

__device__ __forceinline__ void raise_fault(uint32_t* faults, uint32_t bit) {
  if (faults) atomicOr(faults, bit);
}

// 32-bit DPP move; a lane without a source in its row reads 0.
template <int CTRL>
__device__ __forceinline__ int32_t dpp_i32(int32_t x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xf, 0xf, false);
}
__device__ __forceinline__ int32_t lane_i32(int32_t x, int l) { return __builtin_amdgcn_readlane(x, l); }

// Inclusive scan over the 64 lanes of a wave: Kogge-Stone inside each 16-lane
// row (row_shr 1, 2, 4, 8), then the totals of the rows before added to
// every lane of a row. Every lane of the wave must be active.
__device__ __forceinline__ int32_t wave_incl_scan_i32(int32_t v, int lane) {
  v += dpp_i32<0x111>(v);
  v += dpp_i32<0x112>(v);
  v += dpp_i32<0x114>(v);
  v += dpp_i32<0x118>(v);
  const int32_t o1 = lane_i32(v, 15);
  const int32_t o2 = o1 + lane_i32(v, 31);
  const int32_t o3 = o2 + lane_i32(v, 47);
  const int row = lane >> 4;
  return v + (row == 0 ? 0 : (row == 1 ? o1 : (row == 2 ? o2 : o3)));
}

// Exclusive prefix sums of per-request values, computed by a whole
// workgroup into LDS: on return cu[0] = 0 and cu[i + 1] = cu[i] + val(i)
// for i < n. `val` is evaluated once per element by the thread that owns it.
// Each thread owns a contiguous run of ceil(n / NT) elements; the threads'
// sums are scanned by wave DPP scans and one exchange of wave totals.
template <int NT, typename F>
__device__ void block_exclusive_scan(int32_t* cu, int n, F val) {
  static_assert(NT % kWave == 0 && NT <= 1024, "whole waves");
  constexpr int NW = NT / kWave;
  const int t = threadIdx.x, lane = t & (kWave - 1), wave = t / kWave;
  const int per = (n + NT - 1) / NT;
  const int b = min(n, t * per), e = min(n, b + per);
  int32_t s = 0;
  for (int i = b; i < e; ++i) {
    const int32_t v = val(i);
    cu[i + 1] = v;
    s += v;
  }
  __shared__ int32_t wave_tot[NW];
  const int32_t incl = wave_incl_scan_i32(s, lane);
  if (lane == kWave - 1) wave_tot[wave] = incl;
  __syncthreads();
  int32_t acc = incl - s;
  for (int w = 0; w < wave; ++w) acc += wave_tot[w];
  for (int i = b; i < e; ++i) {
    acc += cu[i + 1];
    cu[i + 1] = acc;
  }
  if (t == 0) cu[0] = 0;
  __syncthreads();
}

}  // namespace pkv
