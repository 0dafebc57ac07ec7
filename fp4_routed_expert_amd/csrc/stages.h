// Device bodies of the front stages (top-k routing, stable expert sort,
// MXFP8 activation quantisation), shared by their stand-alone kernels and by
// the fused small-batch front kernel.
#pragma once

#include "common.h"

namespace moe {

constexpr int kMaxE = 1024;  // experts covered by the routing and sort kernels

// ----------------------------------------------------------------- routing
// Monotone map of an fp32 to uint32 (-0 first folded into +0 so they tie).
__device__ __forceinline__ uint32_t ordered_bits(float v) {
  uint32_t u = __float_as_uint(v + 0.0f);  // -0 + +0 = +0 under round-to-nearest
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float from_ordered_bits(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

// Wave-wide unsigned max by DPP: shifts inside each row of 16 lanes, then the
// two row broadcasts; lane 63 ends with the maximum, read back as a uniform.
// Lanes shifted in from outside a row read 0, the identity of unsigned max.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  uint32_t t;
  t = __builtin_amdgcn_update_dpp(0u, v, 0x111, 0xF, 0xF, false);  // row_shr:1
  v = v > t ? v : t;
  t = __builtin_amdgcn_update_dpp(0u, v, 0x112, 0xF, 0xF, false);  // row_shr:2
  v = v > t ? v : t;
  t = __builtin_amdgcn_update_dpp(0u, v, 0x114, 0xF, 0xF, false);  // row_shr:4
  v = v > t ? v : t;
  t = __builtin_amdgcn_update_dpp(0u, v, 0x118, 0xF, 0xF, false);  // row_shr:8
  v = v > t ? v : t;
  t = __builtin_amdgcn_update_dpp(0u, v, 0x142, 0xA, 0xF, false);  // row_bcast:15
  v = v > t ? v : t;
  t = __builtin_amdgcn_update_dpp(0u, v, 0x143, 0xC, 0xF, false);  // row_bcast:31
  v = v > t ? v : t;
  return __builtin_amdgcn_readlane(v, 63);
}

// Where a routing kernel reads its logits: S fp32 planes S_stride floats
// apart whose element-wise sum, taken in plane order, is the logit (S = 1:
// the logits themselves; S > 1: the K-slice partial sums of the router GEMM).
struct LogitSrc {
  const float* p;
  long sstride;
  int S;
};

// (((p[0] + p[1]) + p[2]) + ...) over the S planes at element i, loads issued
// eight at a time.
__device__ __forceinline__ float slice_sum(const float* __restrict__ p, long sstride, int S,
                                           long i) {
  float a = p[i];
  for (int s0 = 1; s0 < S; s0 += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = (s0 + u < S) ? p[(size_t)(s0 + u) * sstride + i] : 0.0f;
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (s0 + u < S) a += v[u];
  }
  return a;
}

__device__ __forceinline__ float load_logit(const LogitSrc& L, long i) {
  return L.S == 1 ? L.p[i] : slice_sum(L.p, L.sstride, L.S, i);
}

// Logits of one token held by one wave as 64-bit keys: high word the ordered
// score, low word E-1-e, so that the unsigned order is (score descending,
// expert index ascending) and every key is distinct.  Absent experts hold 0,
// below every real key.  NK = keys per lane, NK * 64 >= E.
template <int NK>
struct RouteKeys {
  uint64_t key[NK];
};

template <int NK>
__device__ __forceinline__ void load_route_keys(RouteKeys<NK>& r, const LogitSrc& L, long row0,
                                                int E, int lane) {
  float raw[NK];
#pragma unroll
  for (int i = 0; i < NK; ++i) {
    const int e = lane + 64 * i;
    raw[i] = (e < E) ? load_logit(L, row0 + e) : 0.0f;
  }
#pragma unroll
  for (int i = 0; i < NK; ++i) {
    const int e = lane + 64 * i;
    r.key[i] = (e < E) ? (((uint64_t)ordered_bits(raw[i]) << 32) | (uint32_t)(E - 1 - e)) : 0ull;
  }
}

// Slot j of a token's k + ns slots: lanes j < k take the routed top-k (from
// route_topk_token), lanes k <= j < k + ns the shared experts E + (j - k),
// always selected, with weight 1.  Returns false on lanes past the last slot.
__device__ __forceinline__ bool shared_slot(int E, int k, int ns, int lane, int* id, float* gate) {
  if (lane < k || lane >= k + ns) return false;
  *id = E + (lane - k);
  *gate = 1.0f;
  return true;
}

// Top-k of one token (pwwt.cn review, section 4.1 table row "MoE routing
// top-k": fp32 scores, ties to the lowest expert index; gates are the softmax
// over the k selected logits).  k rounds each take the wave-wide largest key
// (score word first, then the index word among the lanes holding that score)
// and remove it.  Lane j < k returns slot j's expert and gate; the softmax is
// taken relative to the largest logit and its denominator summed in slot
// order.  Returns false on lanes >= k.
template <int NK>
__device__ __forceinline__ bool route_topk_token(RouteKeys<NK>& r, int E, int k, int lane,
                                                 int* id_out, float* gate_out) {
  float l0 = 0.0f, den = 0.0f, my_ex = 0.0f;
  int my_id = 0;
  for (int j = 0; j < k; ++j) {
    uint64_t best = 0;
#pragma unroll
    for (int i = 0; i < NK; ++i) best = r.key[i] > best ? r.key[i] : best;
    const uint32_t hi = wave_max_u32((uint32_t)(best >> 32));
    const uint32_t lo = wave_max_u32(((uint32_t)(best >> 32) == hi) ? (uint32_t)best : 0u);
    const uint64_t sel = ((uint64_t)hi << 32) | lo;
    const float le = from_ordered_bits(hi);  // the selected logit itself, no reload
    if (j == 0) l0 = le;
    const float ex = expf(le - l0);          // uniform across the wave
    den += ex;
    if (lane == j) {
      my_id = E - 1 - (int)lo;
      my_ex = ex;
    }
#pragma unroll
    for (int i = 0; i < NK; ++i)
      if (r.key[i] == sel) r.key[i] = 0;
  }
  *id_out = my_id;
  *gate_out = my_ex / den;
  return lane < k;
}

// -------------------------------------------------------------------- sort
// Stable scatter of pairs [p0, p1) by a block of NT threads, given base[e] =
// the first free sorted position of expert e for this range.  A pair's rank
// among the earlier pairs of its expert comes from wavefront ballots (lanes
// with equal ids: intersect the 11 bit-planes of the ids) and a per-wave
// table in LDS; no position comes from an atomic, so the order inside each
// expert is ascending pair index (pwwt.cn review, section 4.2).  table is
// [NT/64][E] of zeros on entry and on exit.
template <int NT>
__device__ void stable_scatter(const int32_t* ids, int p0, int p1, int E, int* base, int* table,
                               int32_t* __restrict__ sorted_pair, int32_t* __restrict__ pair_pos) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int c = p0; c < p1; c += NT) {
    const int p = c + tid;
    const bool valid = p < p1;
    const int id = valid ? ids[p] : kMaxE;  // sentinel outside [0, E)
    uint64_t same = ~0ull;
#pragma unroll
    for (int b = 0; b < 11; ++b) {
      const uint64_t ones = __ballot((id >> b) & 1);
      same &= ((id >> b) & 1) ? ones : ~ones;
    }
    const int rank = __popcll(same & lt_mask);
    const int cnt = __popcll(same);
    const bool leader = valid && rank == 0;
    if (leader) table[w * E + id] = cnt;
    __syncthreads();
    if (valid) {
      int pre = 0;
      for (int i = 0; i < w; ++i) pre += table[i * E + id];
      const int pos = base[id] + pre + rank;
      sorted_pair[pos] = p;
      pair_pos[p] = pos;
    }
    __syncthreads();
    if (leader) {
      atomicAdd(&base[id], cnt);  // integer: order-free
      table[w * E + id] = 0;
    }
    __syncthreads();
  }
}

// Whole sort of P pairs by one 256-thread block: LDS-atomic histogram (integer
// counts are order-free), exclusive scan into offsets, stable scatter.  ids
// may live in global memory or in LDS.
struct SortSmallLds {
  int hist[kMaxE];
  int table[4 * kMaxE];
  int wave_tot[4];
};

__device__ void sort_small_body(const int32_t* ids, int P, int E, SortSmallLds& sm,
                                int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                int32_t* __restrict__ sorted_pair, int32_t* __restrict__ pair_pos) {
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += 256) sm.hist[e] = 0;
  for (int i = tid; i < 4 * E; i += 256) sm.table[i] = 0;
  __syncthreads();
  for (int p = tid; p < P; p += 256) atomicAdd(&sm.hist[ids[p]], 1);
  __syncthreads();
  for (int e = tid; e < E; e += 256) counts[e] = sm.hist[e];
  __syncthreads();
  const int total = block_exclusive_scan256(sm.hist, E, sm.wave_tot);
  for (int e = tid; e < E; e += 256) offsets[e] = sm.hist[e];
  if (tid == 0) offsets[E] = total;
  __syncthreads();
  stable_scatter<256>(ids, 0, P, E, sm.hist, sm.table, sorted_pair, pair_pos);
}

// ------------------------------------------------------------------- MXFP8
// One lane's share of the MXFP8 quantisation of bf16 data: the 8-element
// group i (one 128-bit load); four consecutive lanes hold one 32-element block
// and reduce its maximum with two DPP quad swaps, so all 64 lanes of the wave
// must call this together.  Writes 8 codes as one 64-bit store and, on the
// block's first lane, the E8M0 scale.
__device__ __forceinline__ void quant_group8(const uint4* __restrict__ x, long i, long n8,
                                             uint2* __restrict__ q, uint8_t* __restrict__ sc) {
  const bool live = i < n8;
  const uint4 raw = live ? x[i] : make_uint4(0, 0, 0, 0);
  float v[8];
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    v[2 * h] = __uint_as_float(w[h] << 16);  // bf16 -> fp32 is exact
    v[2 * h + 1] = __uint_as_float(w[h] & 0xFFFF0000u);
  }
  float amax = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[e]));
  amax = quad_max(amax);
  float mul;
  const uint32_t scode = mx_scale_from_amax(amax, &mul);
  const uint32_t lo = f32x4_to_e4m3(v[0] * mul, v[1] * mul, v[2] * mul, v[3] * mul);
  const uint32_t hi = f32x4_to_e4m3(v[4] * mul, v[5] * mul, v[6] * mul, v[7] * mul);
  if (live) {
    q[i] = make_uint2(lo, hi);
    if ((i & 3) == 0) sc[i >> 2] = (uint8_t)scode;
  }
}

}  // namespace moe
