// Paged causal extend (prefill over a cached prefix) on bf16 MFMA tiles.
//
// Definition ("第 0 步：一个能跑的最小推理引擎", the dense attention function;
// "Mini-SGLang 完整剖析" section 4.6.5 for the ragged query layout): request r
// has C = cached_len and S = device_len tokens; its E = S - C query rows are
// the new tokens at absolute positions C .. S-1, stored contiguously from row
// sum_{r' < r} E_r' of q. Query t sees keys j <= C + t, all read from the pool
// through the token-granular page table. GQA: query head h uses KV head
// h / (HQ / HKV). Scale sm_scale, fp32 online softmax.
//
// Work: one workgroup (8 waves) per (request, KV head, pair of query heads
// sharing it, block of 128 query positions); wave w owns positions
// [16w, 16w + 16) of the block for both query heads. Key blocks of 64 are
// gathered row by row (256 B per head per token) into LDS, so every K/V
// element fetched serves 128 positions x 2 heads (256 FLOP per byte).
// The grid is one-dimensional: the KV head is the fastest index (so with 8
// KV heads each XCD serves one head), then the query blocks of one request
// from the longest down, then the requests from the most work down -- so the
// workgroups that run at the same time on an XCD share one request's K/V
// rows in its L2, and the longest requests do not start last.
//
// MFMA layout (v_mfma_f32_16x16x32_bf16): the kernel computes S^T = K . Q^T,
// so each lane's four accumulators belong to ONE query (lane % 16) and four
// keys -- the softmax row statistics stay lane-local up to a 4-lane
// reduction -- and O^T = V^T . P^T, whose accumulators again belong to the
// lane's query, so rescaling is lane-local too. P^T is fed straight from the
// S^T accumulators as the B operand; that fixes the order in which keys enter
// the contraction.
//
// LDS: the K tile is row-major [64 keys][128 dims] with the 16-byte unit u
// of key row k stored at unit u ^ (k & 15), so tile stores (16 bytes of one
// key row per lane) and K fragment reads (16 bytes) are free of bank
// conflicts. The V tile is stored transposed, [128 dims][64 keys], two dims
// to a 256-byte pair row, with the keys of a row in the order the PV operand
// consumes them (key 32b + 16h + 4g + i at position 32b + 8g + 4h + i) and
// the 16 units of a pair row XOR-swizzled by a function of the pair-row
// index: every V fragment is one conflict-free 16-byte read, and the
// transposing stores (one 4-byte key pair per lane) are conflict-free too.
// (The LDS transpose read would serve the same operand from a row-major
// tile, but on gfx950 it moves a quarter of the bytes per cycle of a 16-byte
// read, which makes it the limit of this kernel.)
#pragma once

#include <type_traits>

#include "common.hpp"

namespace pkv {

typedef __bf16 bf16x8_v __attribute__((ext_vector_type(8)));
typedef float f32x4_v __attribute__((ext_vector_type(4)));

struct ExtendArgs {
  const void* k_pool;
  const void* v_pool;
  uint32_t row_bytes;    // bytes between slots
  uint32_t slot_limit;   // slots are valid below this (num_slots, capped at 2^31)
  const void* q;
  int64_t q_stride;      // elements between query rows
  void* o;
  int64_t o_stride;
  int32_t bs;
  int32_t kv_heads;
  int32_t group;         // query heads per KV head
  int32_t head_pairs;    // workgroups per KV head along the query heads
  const int32_t* page_table;
  int32_t pt_rows;
  int64_t pt_stride;
  const int32_t* table_idx;
  const int32_t* cached_len;
  const int32_t* device_len;
  int64_t total_q;
  int32_t max_extend;
  float scale_log2;      // |sm_scale| * log2(e)
  int32_t q_negate;      // sm_scale < 0: scores are taken with q negated
  uint32_t* faults;
  // q prologue (Qwen3's q_norm + rotary embedding), or q_w == nullptr
  const void* q_w;       // [128] bf16 norm weight
  float q_eps;
  float inv_freq[64];    // fp32 rotary frequencies 1 / theta^(2j / 128)
};

constexpr int kExtBlockQ = 128;  // query positions per workgroup
constexpr int kExtThreads = 512; // 8 waves
constexpr int kExtBlockK = 64;   // keys per LDS tile
constexpr int kExtReadAhead = 6; // LDS operand reads in flight ahead of the MFMAs

// Issue order for a loop of 16 LDS operand reads, each feeding `nh` MFMAs:
// the reads run kExtReadAhead ahead of the products that use them, so the
// LDS latency is hidden behind MFMAs rather than waited out before each one
// (left to itself the scheduler keeps only one or two reads in flight).
template <int nh>
__device__ __forceinline__ void lds_read_ahead_order() {
  __builtin_amdgcn_sched_group_barrier(0x100, kExtReadAhead, 0); // DS reads
#pragma unroll
  for (int i = 0; i < 16 - kExtReadAhead; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, nh, 0); // MFMAs
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, nh * kExtReadAhead, 0);
}
constexpr int kTileElems = kExtBlockK * kHeadDim;
// The running maximum is only moved when a score exceeds it by more than
// 2^kRescaleLog2 in weight: every weight then stays <= 2^kRescaleLog2, and
// the accumulators are rescaled only on those (rare) tiles.
constexpr float kRescaleLog2 = 8.0f;

// Element offset of dims [8u, 8u + 8) of key row k inside a tile.
__device__ __forceinline__ int tile_off(int k, int u) { return k * kHeadDim + ((u ^ (k & 15)) << 3); }

// V^T tile addressing (element offsets). Pair row rp holds dims 2rp and
// 2rp + 1; unit (p * 8 + pos / 8) of it moves to that index ^ vt_swz(rp).
__device__ __forceinline__ int vt_swz(int rp) { return ((rp ^ (rp >> 3)) & 7) | (((rp >> 2) & 1) << 3); }
__device__ __forceinline__ int vt_off(int dim, int pos) {
  const int rp = dim >> 1;
  return rp * 128 + (((((dim & 1) << 3) | (pos >> 3)) ^ vt_swz(rp)) << 3) + (pos & 7);
}
// Position of key k (0..63) inside a V^T row.
__device__ __forceinline__ int vt_pos(int k) { return (k & 32) | ((k & 12) << 1) | ((k & 16) >> 2) | (k & 3); }

template <int NH>
__global__ void __launch_bounds__(kExtThreads, 1) extend_kernel(ExtendArgs a) {
  // Two tile buffers: tile kb is computed from buffer kb & 1 while tile kb + 1
  // is written to the other one (one barrier per tile).
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][kTileElems];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2][kTileElems];
  __shared__ int32_t sh_qstart;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int lq = lane & 15, lg = lane >> 4;   // MFMA row-in-tile and k-group of this lane

  const int nqb = (a.max_extend + kExtBlockQ - 1) / kExtBlockQ;
  const int id = blockIdx.x;
  const int g = id % a.kv_heads;
  const int rest = id / a.kv_heads;
  const int qb = nqb - 1 - rest % nqb;         // longest blocks of a request first
  const int hp = (rest / nqb) % a.head_pairs;
  // Requests in order of their work, the largest first (each request's
  // blocks stay together, so they share its K/V rows in L2): grid position
  // rk is the request of rank rk by causal pairs E (2C + E + 1), ties by
  // index; batches above one request per thread keep the index order.
  const int rk = rest / (nqb * a.head_pairs);
  int r = rk;
  if (a.bs <= kExtThreads) {  // uniform
    __shared__ int64_t req_cost[kExtThreads];
    __shared__ int32_t sh_req;
    if (tid < a.bs) {
      const int64_t ci = a.cached_len[tid], si = a.device_len[tid];
      req_cost[tid] = si > ci ? (si - ci) * (2 * ci + (si - ci) + 1) : 0;
    }
    __syncthreads();
    if (tid < a.bs) {
      const int64_t mine = req_cost[tid];
      int rank = 0;
      for (int j = 0; j < a.bs; ++j) rank += (req_cost[j] > mine) || (req_cost[j] == mine && j < tid);
      if (rank == rk) sh_req = tid;
    }
    __syncthreads();
    r = sh_req;
  }

  const int32_t C = a.cached_len[r], S = a.device_len[r];
  const int32_t row = a.table_idx ? a.table_idx[r] : r;
  const bool len_ok = C >= 0 && C < S && (int64_t)S <= a.pt_stride && S - C <= a.max_extend;
  const bool row_ok = row >= 0 && row < a.pt_rows;
  if (!len_ok || !row_ok) {
    if (tid == 0 && qb == 0 && g == 0 && hp == 0) raise_fault(a.faults, !row_ok ? 0x8u : 0x2u);
    return;
  }
  const int32_t E = S - C;
  if (qb * kExtBlockQ >= E) return;

  // Query row offset of this request: sum of the earlier requests' extend lengths.
  {
    int64_t part = 0;
    for (int i = tid; i < r; i += kExtThreads) {
      const int32_t ci = a.cached_len[i], si = a.device_len[i];
      part += (si > ci) ? (si - ci) : 0;
    }
    __shared__ int64_t red[kExtThreads / kWave];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) part += __shfl_xor(part, o, 64);
    if (lane == 0) red[wave] = part;
    __syncthreads();
    if (tid == 0) {
      int64_t qs = 0;
      for (int w = 0; w < kExtThreads / kWave; ++w) qs += red[w];
      sh_qstart = (qs + E <= a.total_q) ? (int32_t)qs : -1;
    }
    __syncthreads();
  }
  const int32_t qstart = sh_qstart;
  if (qstart < 0) {
    if (tid == 0 && qb == 0 && g == 0 && hp == 0) raise_fault(a.faults, 0x10u);
    return;
  }

  const bf16_t* qg = reinterpret_cast<const bf16_t*>(a.q);
  const bf16_t* kpool = reinterpret_cast<const bf16_t*>(a.k_pool);
  const bf16_t* vpool = reinterpret_cast<const bf16_t*>(a.v_pool);
  const int32_t* pt = a.page_table + (int64_t)row * a.pt_stride;

  // This lane's query (MFMA column) and its validity.
  const int t = qb * kExtBlockQ + wave * 16 + lq;
  const bool t_ok = t < E;
  const int t_eff = t_ok ? t : E - 1;          // invalid rows mask like the last valid one
  const int h0 = g * a.group + hp * NH;

  // Q^T as B operands: 4 k-steps of 32 dims, 8 dims per lane.
  bf16x8_v qreg[NH][4];
#pragma unroll
  for (int hh = 0; hh < NH; ++hh) {
    const bf16_t* qrow = qg + (int64_t)(qstart + t_eff) * a.q_stride + (int64_t)(h0 + hh) * kHeadDim;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      u32x4 w = {0u, 0u, 0u, 0u};
      if (t_ok) w = *reinterpret_cast<const u32x4*>(qrow + ks * 32 + lg * 8);
      qreg[hh][ks] = __builtin_bit_cast(bf16x8_v, w);
    }
  }
  if (a.q_w) {
    // Fused q prologue ("第 0 步" layer function: q_norm, then rope at the
    // query's absolute position C + t; "Mini-SGLang 完整剖析" section 4.6.7).
    // The lane holds dims 32 ks + 8 lg + i of its query: the row's norm is a
    // sum over the four lanes lq + 16 lg, and dims j and j + 64 of a rotated
    // pair sit in k-steps ks and ks + 2 of the same lane. fp32, then bf16.
    const float pos = (float)(C + t_eff);
    float w[4][8], cs[2][8], sn[2][8];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const u32x4 wr = *reinterpret_cast<const u32x4*>(reinterpret_cast<const bf16_t*>(a.q_w) + ks * 32 + lg * 8);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        w[ks][2 * i] = bf16_lo(wr[i]);
        w[ks][2 * i + 1] = bf16_hi(wr[i]);
      }
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int i = 0; i < 8; ++i) sincosf(pos * a.inv_freq[ks * 32 + lg * 8 + i], &sn[ks][i], &cs[ks][i]);
#pragma unroll
    for (int hh = 0; hh < NH; ++hh) {
      float x[4][8];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const u32x4 raw = __builtin_bit_cast(u32x4, qreg[hh][ks]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[ks][2 * i] = bf16_lo(raw[i]);
          x[ks][2 * i + 1] = bf16_hi(raw[i]);
        }
      }
      float ss = 0.f;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int i = 0; i < 8; ++i) ss = fmaf(x[ks][i], x[ks][i], ss);
      ss += __shfl_xor(ss, 16, 64);
      ss += __shfl_xor(ss, 32, 64);
      const float rn = t_ok ? 1.0f / sqrtf(fmaf(ss, 1.0f / (float)kHeadDim, a.q_eps)) : 0.f;
      float y[4][8];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float u = x[ks][i] * rn * w[ks][i], v = x[ks + 2][i] * rn * w[ks + 2][i];
          y[ks][i] = u * cs[ks][i] - v * sn[ks][i];
          y[ks + 2][i] = u * sn[ks][i] + v * cs[ks][i];
        }
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const u32x4 packed = {pack_bf16x2(y[ks][0], y[ks][1]), pack_bf16x2(y[ks][2], y[ks][3]),
                              pack_bf16x2(y[ks][4], y[ks][5]), pack_bf16x2(y[ks][6], y[ks][7])};
        qreg[hh][ks] = __builtin_bit_cast(bf16x8_v, packed);
      }
    }
  }

  if (a.q_negate) {
    // The running maximum below is taken over raw scores scaled afterwards,
    // which needs a positive scale: a negative sm_scale is applied as its
    // magnitude to the scores of -q (a sign flip, exact in bf16).
#pragma unroll
    for (int hh = 0; hh < NH; ++hh)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        qreg[hh][ks] = __builtin_bit_cast(bf16x8_v, __builtin_bit_cast(u32x4, qreg[hh][ks]) ^ 0x80008000u);
  }

  f32x4_v oacc[NH][8];
#pragma unroll
  for (int hh = 0; hh < NH; ++hh)
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) oacc[hh][dt] = (f32x4_v){0.f, 0.f, 0.f, 0.f};
  // Running maximum m (score units), the score above which it moves (m +
  // kRescaleLog2 / sc) and the exponent offset -m * sc, the last two kept so
  // that a tile without a move costs one compare per head.
  float m[NH], mth[NH], moff[NH];
  f32x4_v lacc[NH];  // row sums (every element of a lane's vector holds its query's)
#pragma unroll
  for (int hh = 0; hh < NH; ++hh) {
    m[hh] = -INFINITY;
    mth[hh] = -INFINITY;
    moff[hh] = 0.f;
    lacc[hh] = (f32x4_v){0.f, 0.f, 0.f, 0.f};
  }

  // Keys this workgroup needs: j <= C + (last valid position of the block).
  const int t_last = min(E, (qb + 1) * kExtBlockQ) - 1;
  const int n_keys = C + t_last + 1;
  const int nkb = (n_keys + kExtBlockK - 1) / kExtBlockK;

  // Tile loader: thread -> 2 consecutive keys (kq*2 ..) x 8 dims (dg*8 ..).
  // Page-table entries are fetched two tiles ahead of the K/V rows they
  // address, and K/V rows one tile ahead of their use, so neither latency
  // sits between two tiles of MFMA work. Keys past the block's last key and
  // slots outside the pool load slot 0's row and are zeroed before they reach
  // LDS (an out-of-pool slot also raises the fault bit once, after the loop).
  // A wave loads four key rows, chosen (key pairs kq, kq + 1, kq + 8, kq + 9
  // of the 32) so that its transposed V stores cover all 64 LDS banks.
  const int kq = ((tid >> 4) & 1) | (((tid >> 6) & 3) << 1) | (((tid >> 5) & 1) << 3) | ((tid >> 8) << 4);
  const int dg = tid & 15;
  constexpr int KPT = kExtBlockK * 16 / kExtThreads;  // keys per thread
  const char* kbase = reinterpret_cast<const char*>(a.k_pool) + g * (kHeadDim * 2) + dg * 16;
  const char* vbase = reinterpret_cast<const char*>(a.v_pool) + g * (kHeadDim * 2) + dg * 16;
  int32_t slot_raw[KPT];   // page-table entries of the next tile to load
  bool key_ok[KPT];        // whether those keys exist (j < n_keys)
  auto load_slots = [&](int kb) {
#pragma unroll
    for (int e = 0; e < KPT; ++e) {
      const int j = kb * kExtBlockK + kq * KPT + e;
      key_ok[e] = j < n_keys;
      slot_raw[e] = pt[key_ok[e] ? j : 0];
    }
  };
  // Page-table entries of later tiles: wave 0 reads a tile's 64 entries (one
  // per lane) and puts them in LDS, where every thread finds its two.
  __shared__ __attribute__((aligned(8))) int32_t pt_ring[2][kExtBlockK];
  auto pt_entry = [&](int kb) {  // wave 0: this lane's entry of tile kb
    const int j = kb * kExtBlockK + lane;
    return j < n_keys ? pt[j] : 0;
  };
  auto slots_from_ring = [&](int kb, auto rbufc) {
    constexpr int rb = decltype(rbufc)::value;
    const int2 v = *reinterpret_cast<const int2*>(&pt_ring[rb][kq * KPT]);
    slot_raw[0] = v.x;
    slot_raw[1] = v.y;
#pragma unroll
    for (int e = 0; e < KPT; ++e) key_ok[e] = kb * kExtBlockK + kq * KPT + e < n_keys;
  };
  int32_t pt_next = 0;  // wave 0: the entry of the tile after the one in the ring
  u32x4 kreg[KPT], vreg[KPT];
  uint32_t zero_bits = 0;  // keys of the loaded tile to store as zeros
  bool bad_slot = false;
  auto load_tile = [&]() {
    zero_bits = 0;
#pragma unroll
    for (int e = 0; e < KPT; ++e) {
      const int32_t slot = key_ok[e] ? slot_raw[e] : -1;
      const bool ok = (uint32_t)slot < a.slot_limit;
      bad_slot |= !ok && slot != -1;
      zero_bits |= ok ? 0u : (1u << e);
      const uint64_t off = (uint64_t)(ok ? (uint32_t)slot : 0u) * a.row_bytes;
      // Plain loads: the request's other query blocks read the same rows,
      // and they find them in L2.
      kreg[e] = *reinterpret_cast<const u32x4*>(kbase + off);
      vreg[e] = *reinterpret_cast<const u32x4*>(vbase + off);
    }
  };
  auto store_tile = [&](auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    if (__any(zero_bits != 0)) {
#pragma unroll
      for (int e = 0; e < KPT; ++e)
        if (zero_bits & (1u << e)) {
          kreg[e] = (u32x4){0u, 0u, 0u, 0u};
          vreg[e] = (u32x4){0u, 0u, 0u, 0u};
        }
    }
#pragma unroll
    for (int e = 0; e < KPT; ++e) {
      const int k = kq * KPT + e;
      *reinterpret_cast<u32x4*>(&Ks[buf][tile_off(k, dg)]) = kreg[e];
    }
    // V^T: dim 8*dg + d of keys 2kq and 2kq + 1 as one 4-byte pair.
    static_assert(KPT == 2, "the V^T store packs two keys per lane");
    const int pos0 = vt_pos(kq * KPT);
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      const uint32_t pair = __builtin_amdgcn_perm(vreg[1][d >> 1], vreg[0][d >> 1], (d & 1) ? 0x07060302u : 0x05040100u);
      *reinterpret_cast<uint32_t*>(&Vs[buf][vt_off(8 * dg + d, pos0)]) = pair;
    }
  };

  const float sc = a.scale_log2;
  const float thr = kRescaleLog2 / sc;
  const int t_min_wave = qb * kExtBlockQ + wave * 16;
  typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
  bf16x8_v ones8;
#pragma unroll
  for (int j = 0; j < 8; ++j) ones8[j] = (__bf16)1.0f;

  // One key tile from LDS buffer `buf` (a compile-time constant, so every
  // LDS address below is a loop-invariant register plus an immediate).
  auto step = [&](int kb, auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    // S^T = K . Q^T for 4 key tiles of 16.
    f32x4_v s[NH][4];
#pragma unroll
    for (int hh = 0; hh < NH; ++hh)
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) s[hh][kt] = (f32x4_v){0.f, 0.f, 0.f, 0.f};
    // Each SIMD runs two waves of this workgroup in step; the one issuing
    // MFMAs is given priority over the one doing softmax arithmetic.
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8_v ka =
            __builtin_bit_cast(bf16x8_v, *reinterpret_cast<const u32x4*>(&Ks[buf][tile_off(kt * 16 + lq, ks * 4 + lg)]));
#pragma unroll
        for (int hh = 0; hh < NH; ++hh)
          s[hh][kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qreg[hh][ks], s[hh][kt], 0, 0, 0);
      }
    lds_read_ahead_order<NH>();

    // Tile kb + 1 (loaded during the previous tile) into the other buffer,
    // which no wave reads after the previous tile's barrier; rows of tile
    // kb + 2 and the slots of tile kb + 3 go out. Done here, the LDS stores
    // complete and the loads travel while the softmax arithmetic runs; the
    // wave keeps its raised priority until they are issued.
    if (kb + 1 < nkb) {
      store_tile(std::integral_constant<int, buf ^ 1>{});
      slots_from_ring(kb + 2, bufc);
      load_tile();
      if (wave == 0) {
        pt_ring[buf ^ 1][lane] = pt_next;  // tile kb + 3
        pt_next = pt_entry(kb + 4);
      }
    }
    __builtin_amdgcn_s_setprio(0);
    // Online softmax for this lane's query, on raw scores: weights are
    // exp2(s * sc - m * sc) against the running maximum m (score units). The
    // key of s[kt][i] is kb*64 + kt*16 + 4*lg + i; only the tiles that cross
    // this wave's diagonal are masked (a wave-uniform branch). m moves only
    // when some lane of the wave sees a score more than kRescaleLog2 above
    // it (wave-uniform too): then the exact maximum over the query's four
    // lanes is taken and the accumulators are rescaled.
    const bool need_mask = kb * kExtBlockK + kExtBlockK - 1 > C + t_min_wave;
    const int lim = C + t_eff - kb * kExtBlockK - 4 * lg;  // s[kt][i] is visible iff kt*16 + i <= lim
    bf16x8_v pb[NH][2];
#pragma unroll
    for (int hh = 0; hh < NH; ++hh) {
      float v[16];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) v[kt * 4 + i] = s[hh][kt][i];
      if (need_mask) {
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (kt * 16 + i > lim) v[kt * 4 + i] = -INFINITY;
      }
      // IEEE maximum (NaN-propagating) needs no quieting of its inputs and
      // maps to the three-input v_maximum3_f32.
      // A tree of three-input maxima over the 16 scores.
      auto max3 = [](float x, float y, float z) {
        return __builtin_elementwise_maximum(x, __builtin_elementwise_maximum(y, z));
      };
      const float a0 = max3(v[0], v[1], v[2]), a1 = max3(v[3], v[4], v[5]), a2 = max3(v[6], v[7], v[8]);
      const float a3 = max3(v[9], v[10], v[11]), a4 = max3(v[12], v[13], v[14]);
      const float mloc = __builtin_elementwise_maximum(max3(a0, a1, a2), max3(a3, a4, v[15]));
      // m = -inf (first tile) always moves; a lane whose keys are all masked
      // (mloc = -inf) never asks for a move.
      if (__any(mloc > mth[hh])) {
        float mb = fmaxf(mloc, __shfl_xor(mloc, 16, 64));
        mb = fmaxf(mb, __shfl_xor(mb, 32, 64));
        const float mn = fmaxf(m[hh], mb);
        const float corr = fast_exp2((m[hh] - mn) * sc);  // m = -inf: corr = 0
        m[hh] = mn;
        mth[hh] = mn + thr;
        moff[hh] = -mn * sc;
        lacc[hh] *= corr;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) oacc[hh][dt] *= corr;
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = fast_exp2(fmaf(v[i], sc, moff[hh]));
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        bf16x8_v bq;
#pragma unroll
        for (int j = 0; j < 8; ++j) bq[j] = (__bf16)v[(2 * k2 + (j >> 2)) * 4 + (j & 3)];
        pb[hh][k2] = bq;
      }
    }

    __builtin_amdgcn_s_setprio(1);
    // O^T += V^T . P^T: 8 tiles of 16 dims, 2 k-steps of 32 keys. Element j
    // of this lane's operand is dim 16*dt + lq, key 32*k2 + 16*(j / 4) +
    // 4*lg + j % 4: eight consecutive positions of that dim's V^T row.
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        const bf16x8_v va = __builtin_bit_cast(
            bf16x8_v, *reinterpret_cast<const u32x4*>(&Vs[buf][vt_off(16 * dt + lq, 32 * k2 + 8 * lg)]));
#pragma unroll
        for (int hh = 0; hh < NH; ++hh)
          oacc[hh][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[hh][k2], oacc[hh][dt], 0, 0, 0);
      }
    lds_read_ahead_order<NH>();
    __builtin_amdgcn_sched_barrier(0);
    // Row sums of the rounded weights (the ones the PV product uses) on the
    // MFMA unit: an all-ones V^T tile turns every output row into the sum.
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
      for (int hh = 0; hh < NH; ++hh)
        lacc[hh] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones8, pb[hh][k2], lacc[hh], 0, 0, 0);

    __builtin_amdgcn_s_setprio(0);
    __syncthreads();
  };

  load_slots(0);
  load_tile();        // tile 0
  load_slots(1);
  store_tile(std::integral_constant<int, 0>{});
  load_tile();        // tile 1
  if (wave == 0) {
    pt_ring[0][lane] = pt_entry(2);
    pt_next = pt_entry(3);
  }
  __syncthreads();
  for (int kb = 0; kb < nkb; kb += 2) {
    step(kb, std::integral_constant<int, 0>{});
    if (kb + 1 < nkb) step(kb + 1, std::integral_constant<int, 1>{});
  }
  if (bad_slot) raise_fault(a.faults, 0x4u);

  // Normalise and write: lane holds dims dt*16 + 4*lg + i of query t.
#pragma unroll
  for (int hh = 0; hh < NH; ++hh) {
    const float lt = lacc[hh][0];
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    if (t_ok) {
      bf16_t* orow = reinterpret_cast<bf16_t*>(a.o) + (int64_t)(qstart + t) * a.o_stride +
                     (int64_t)(h0 + hh) * kHeadDim;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        uint2 w;
        w.x = pack_bf16x2(oacc[hh][dt][0] * inv, oacc[hh][dt][1] * inv);
        w.y = pack_bf16x2(oacc[hh][dt][2] * inv, oacc[hh][dt][3] * inv);
        *reinterpret_cast<uint2*>(orow + dt * 16 + lg * 4) = w;
      }
    }
  }
}

}  // namespace pkv
