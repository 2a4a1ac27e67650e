// q/k RMSNorm + rotary embedding + store_kv, fused: the step right before
// the attention kernel of every layer.
//
// "第 0 步：一个能跑的最小推理引擎" (its rmsnorm and rope operators and the
// layer function): each q and k head is normalised over its 128 dims,
// w * x / sqrt(mean(x^2) + eps) with the tensor's own norm weight (Qwen3's
// q_norm / k_norm), then rotated at the token's absolute position, dims j and
// j + 64 forming one pair turned by pos * inv_freq[j]. "Mini-SGLang 完整剖析"
// section 4.6.7: the layer normalises and rotates q and k in place, and the
// attention backend first stores k and v through out_loc.
//
// One wave per token, a 16-lane row per head vector: lane c of a row holds
// dims [4c, 4c + 4) and [64 + 4c, 64 + 4c + 4), so both members of each
// rotated pair sit in the same lane and the row's DPP sum gives the norm.
// Row r takes q heads r, r + 4, ..., k and v heads r, r + 4, ...; all of a
// lane's loads are issued before any arithmetic. The rotation of the lane's
// four pairs is computed once per token: the angle is the fp32 product of
// the position and the host-made fp32 frequency, as the step-0 page computes
// it, and sin/cos are taken of that fp32 angle.
#pragma once

#include "common.hpp"

namespace pkv {

struct QkRopeArgs {
  void* k_pool;
  void* v_pool;
  int64_t pool_row;      // elements between slots
  int64_t num_slots;
  const void* out_loc;
  int64_t n;             // tokens
  const void* q;
  int64_t q_stride;      // elements between token rows
  void* q_out;
  int64_t q_out_stride;
  const void* k;
  int64_t k_stride;
  const void* v;
  int64_t v_stride;
  const int32_t* positions;
  const void* q_w;       // [128] q norm weight
  const void* k_w;       // [128] k norm weight
  int32_t hq, hkv;
  float eps;
  float inv_freq[64];    // 1 / theta^(2j / 128), fp32
  uint32_t* faults;
};

constexpr int kQkRopeThreads = 256;  // 4 tokens per workgroup

// Four consecutive elements <-> four floats.
template <typename T>
struct Quad;
template <>
struct Quad<bf16_t> {
  typedef uint2 raw;
  static __device__ __forceinline__ raw load(const bf16_t* p) { return *reinterpret_cast<const uint2*>(p); }
  static __device__ __forceinline__ void store(bf16_t* p, raw x) { *reinterpret_cast<uint2*>(p) = x; }
  static __device__ __forceinline__ void unpack(raw x, float (&f)[4]) {
    f[0] = bf16_lo(x.x);
    f[1] = bf16_hi(x.x);
    f[2] = bf16_lo(x.y);
    f[3] = bf16_hi(x.y);
  }
  static __device__ __forceinline__ raw pack(const float (&f)[4]) {  // round to nearest even
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    const b2 lo = {(__bf16)f[0], (__bf16)f[1]}, hi = {(__bf16)f[2], (__bf16)f[3]};
    return make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
  }
};
template <>
struct Quad<float> {
  typedef float4 raw;
  static __device__ __forceinline__ raw load(const float* p) { return *reinterpret_cast<const float4*>(p); }
  static __device__ __forceinline__ void store(float* p, raw x) { *reinterpret_cast<float4*>(p) = x; }
  static __device__ __forceinline__ void unpack(raw x, float (&f)[4]) {
    f[0] = x.x;
    f[1] = x.y;
    f[2] = x.z;
    f[3] = x.w;
  }
  static __device__ __forceinline__ raw pack(const float (&f)[4]) { return make_float4(f[0], f[1], f[2], f[3]); }
};

// MQ / MK: q / kv heads per 16-lane row (heads r + 4i, i < MQ, below hq).
template <typename T, typename IdxT, int MQ, int MK>
__global__ void __launch_bounds__(kQkRopeThreads) qk_rope_store_kernel(QkRopeArgs a) {
  using Q = Quad<T>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t t = (int64_t)blockIdx.x * (kQkRopeThreads / kWave) + wave;
  if (t >= a.n) return;  // wave-uniform
  const int r = lane >> 4, c = lane & 15;
  const int d0 = 4 * c, d1 = kHeadDim / 2 + 4 * c;

  const T* qrow = reinterpret_cast<const T*>(a.q) + t * a.q_stride;
  const T* krow = reinterpret_cast<const T*>(a.k) + t * a.k_stride;
  const T* vrow = reinterpret_cast<const T*>(a.v) + t * a.v_stride;
  typename Q::raw qx[MQ][2], kx[MK][2], vx[MK][2];
#pragma unroll
  for (int i = 0; i < MQ; ++i) {
    const int h = r + 4 * i;
    if (h < a.hq) {
      qx[i][0] = Q::load(qrow + h * kHeadDim + d0);
      qx[i][1] = Q::load(qrow + h * kHeadDim + d1);
    }
  }
#pragma unroll
  for (int i = 0; i < MK; ++i) {
    const int h = r + 4 * i;
    if (h < a.hkv) {
      kx[i][0] = Q::load(krow + h * kHeadDim + d0);
      kx[i][1] = Q::load(krow + h * kHeadDim + d1);
      vx[i][0] = Q::load(vrow + h * kHeadDim + d0);
      vx[i][1] = Q::load(vrow + h * kHeadDim + d1);
    }
  }
  const int64_t slot = (int64_t)reinterpret_cast<const IdxT*>(a.out_loc)[t];
  float qw[2][4], kw[2][4];
  Q::unpack(Q::load(reinterpret_cast<const T*>(a.q_w) + d0), qw[0]);
  Q::unpack(Q::load(reinterpret_cast<const T*>(a.q_w) + d1), qw[1]);
  Q::unpack(Q::load(reinterpret_cast<const T*>(a.k_w) + d0), kw[0]);
  Q::unpack(Q::load(reinterpret_cast<const T*>(a.k_w) + d1), kw[1]);

  // rotation of pairs 4c + e (dims 4c + e and 64 + 4c + e)
  const float pos = (float)a.positions[t];
  float cs[4], sn[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float ang = pos * a.inv_freq[d0 + e];
    sincosf(ang, &sn[e], &cs[e]);
  }
  const float inv_d = 1.0f / (float)kHeadDim;
  // normalise one head vector (this lane's 8 of its 128 dims), rotate, pack
  auto norm_rope = [&](const typename Q::raw (&x)[2], const float (&w)[2][4], typename Q::raw (&y)[2]) {
    float a0[4], a1[4];
    Q::unpack(x[0], a0);
    Q::unpack(x[1], a1);
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) ss = fmaf(a0[e], a0[e], fmaf(a1[e], a1[e], ss));
    ss = group_sum<16>(ss);
    const float rn = 1.0f / sqrtf(fmaf(ss, inv_d, a.eps));
    float o0[4], o1[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float u = a0[e] * rn * w[0][e], v = a1[e] * rn * w[1][e];
      o0[e] = u * cs[e] - v * sn[e];
      o1[e] = u * sn[e] + v * cs[e];
    }
    y[0] = Q::pack(o0);
    y[1] = Q::pack(o1);
  };

  T* qo = reinterpret_cast<T*>(a.q_out) + t * a.q_out_stride;
#pragma unroll
  for (int i = 0; i < MQ; ++i) {
    const int h = r + 4 * i;
    if (h < a.hq) {  // uniform in the row, so the row's DPP sum sees 16 active lanes
      typename Q::raw y[2];
      norm_rope(qx[i], qw, y);
      Q::store(qo + h * kHeadDim + d0, y[0]);
      Q::store(qo + h * kHeadDim + d1, y[1]);
    }
  }
  if (slot < 0 || slot >= a.num_slots) {  // wave-uniform: the token's K/V are not stored
    if (lane == 0) raise_fault(a.faults, 0x1u);
    return;
  }
  T* kp = reinterpret_cast<T*>(a.k_pool) + slot * a.pool_row;
  T* vp = reinterpret_cast<T*>(a.v_pool) + slot * a.pool_row;
#pragma unroll
  for (int i = 0; i < MK; ++i) {
    const int h = r + 4 * i;
    if (h < a.hkv) {
      typename Q::raw y[2];
      norm_rope(kx[i], kw, y);
      Q::store(kp + h * kHeadDim + d0, y[0]);
      Q::store(kp + h * kHeadDim + d1, y[1]);
      Q::store(vp + h * kHeadDim + d0, vx[i][0]);
      Q::store(vp + h * kHeadDim + d1, vx[i][1]);
    }
  }
}

}  // namespace pkv
