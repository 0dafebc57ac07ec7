// Fused front of the layer for small token counts: top-k routing, the stable
// expert sort and the MXFP8 quantisation of x in one launch.
//
// For a decode batch each front stage is a few microseconds of pure latency,
// so they share one grid: block 0 routes every token (one wave per token, the
// next token's logits loaded while the current one is ranked), keeps the
// expert ids in LDS and sorts them there (the same histogram / scan / stable
// scatter as the stand-alone sort); blocks 1.. quantise x, 2048 elements each,
// while block 0 works.  Outputs are identical to the three stand-alone
// kernels'.
//
// Larger batches: routing and quantisation share one launch, the sort follows.
// The routing workgroups (4 tokens each, a chain of k dependent wave-wide
// reductions per token: latency) are spread evenly among the quantisation
// workgroups (2048 elements each: HBM bandwidth), so they run under the
// bandwidth-bound work instead of before it.
#include "stages.h"

namespace moe {
namespace {

constexpr int kFrontThreads = 256;
constexpr int kFrontWaves = kFrontThreads / 64;
constexpr int kFrontMaxP = kFrontMaxT * 32;  // k <= 32

// Routing over E experts with k + ns slots per token (ns shared experts with
// ids E .. E + ns - 1 after the routed slots); the sort covers E + ns experts.
template <int NK>
__global__ __launch_bounds__(kFrontThreads) void front_small_kernel(
    LogitSrc L, const uint4* __restrict__ x, int T, int E, int k, int ns, long n8,
    int32_t* __restrict__ ids, float* __restrict__ gates, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_pair,
    int32_t* __restrict__ pair_pos, uint2* __restrict__ xq, uint8_t* __restrict__ xs) {
  if (blockIdx.x > 0) {
    quant_group8(x, (long)(blockIdx.x - 1) * kFrontThreads + threadIdx.x, n8, xq, xs);
    return;
  }
  __shared__ SortSmallLds sm;
  __shared__ int sids[kFrontMaxP];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ld = k + ns;
  float raw[NK];
  auto fetch = [&](int t) {
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      const int e = lane + 64 * i;
      raw[i] = (e < E) ? load_logit(L, (long)t * E + e) : 0.0f;
    }
  };
  if (wave < T) fetch(wave);
  for (int t = wave; t < T; t += kFrontWaves) {
    RouteKeys<NK> r;
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      const int e = lane + 64 * i;
      r.key[i] = (e < E) ? (((uint64_t)ordered_bits(raw[i]) << 32) | (uint32_t)(E - 1 - e)) : 0ull;
    }
    if (t + kFrontWaves < T) fetch(t + kFrontWaves);
    int id;
    float g;
    if (route_topk_token<NK>(r, E, k, lane, &id, &g) || shared_slot(E, k, ns, lane, &id, &g)) {
      ids[(size_t)t * ld + lane] = id;
      gates[(size_t)t * ld + lane] = g;
      sids[t * ld + lane] = id;
    }
  }
  __syncthreads();
  sort_small_body(sids, T * ld, E + ns, sm, counts, offsets, sorted_pair, pair_pos);
}

// Workgroup b of the routing + quantisation grid: with Br routing groups and
// Bq quantisation groups, q = Bq / Br, the first Br (q + 1) workgroups come in
// runs of q quantisation groups followed by one routing group, and the
// remaining Bq - q Br quantisation groups follow.  Returns the routing group
// (>= 0) or -1 - the quantisation group.
__device__ __forceinline__ long front_role(long b, long Br, long q) {
  const long G = q + 1;
  if (b < Br * G) {
    const long g = b / G, o = b - g * G;
    return o == q ? g : -1 - (g * q + o);
  }
  return -1 - (Br * q + (b - Br * G));
}

template <int NK>
__global__ __launch_bounds__(kFrontThreads) void front_route_quant_kernel(
    LogitSrc L, const uint4* __restrict__ x, int T, int E, int k, int ns, long n8, long Br,
    long q, int32_t* __restrict__ ids, float* __restrict__ gates, uint2* __restrict__ xq,
    uint8_t* __restrict__ xs) {
  const long role = front_role(blockIdx.x, Br, q);
  if (role < 0) {
    quant_group8(x, (-1 - role) * kFrontThreads + threadIdx.x, n8, xq, xs);
    return;
  }
  const int lane = threadIdx.x & 63;
  const long t = role * kFrontWaves + (threadIdx.x >> 6);
  if (t >= T) return;
  const int ld = k + ns;
  RouteKeys<NK> r;
  load_route_keys<NK>(r, L, t * E, E, lane);
  int id;
  float g;
  if (route_topk_token<NK>(r, E, k, lane, &id, &g) || shared_slot(E, k, ns, lane, &id, &g)) {
    ids[t * ld + lane] = id;
    gates[t * ld + lane] = g;
  }
}

}  // namespace

hipError_t launch_front_route_quant(const float* logits, int S, const uint16_t* x, int T, int H,
                                    int E, int k, int ns, int32_t* ids, float* gates, uint8_t* xq,
                                    uint8_t* xs, hipStream_t s) {
  if (T < 1 || k + ns > 32 || E > kMaxE) return hipErrorInvalidValue;
  const LogitSrc L{logits, (long)T * E, S};
  const long n8 = (long)T * H / 8;  // H % 32 == 0: a block never straddles rows
  const long Br = (T + kFrontWaves - 1) / kFrontWaves;
  const long Bq = (n8 + kFrontThreads - 1) / kFrontThreads;
  const long q = Bq / Br;
  if (Br + Bq > 0x7fffffffL) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)(Br + Bq)), block(kFrontThreads);
  const uint4* xv = reinterpret_cast<const uint4*>(x);
  uint2* qv = reinterpret_cast<uint2*>(xq);
#define MOE_FRONT(nk)                                                                            \
  hipLaunchKernelGGL(front_route_quant_kernel<nk>, grid, block, 0, s, L, xv, T, E, k, ns, n8, Br, \
                     q, ids, gates, qv, xs)
  switch (route_keys_per_lane(E)) {
    case 1: MOE_FRONT(1); break;
    case 2: MOE_FRONT(2); break;
    case 4: MOE_FRONT(4); break;
    case 8: MOE_FRONT(8); break;
    default: MOE_FRONT(16); break;
  }
#undef MOE_FRONT
  return hipGetLastError();
}

hipError_t launch_front_small(const float* logits, int S, const uint16_t* x, int T, int H, int E,
                              int k, int ns, int32_t* ids, float* gates, int32_t* counts,
                              int32_t* offsets, int32_t* sorted_pair, int32_t* pair_pos,
                              uint8_t* xq, uint8_t* xs, hipStream_t s) {
  if (T < 1 || T > kFrontMaxT || k + ns > 32 || E + ns > kMaxE) return hipErrorInvalidValue;
  const LogitSrc L{logits, (long)T * E, S};
  const long n8 = (long)T * H / 8;
  const dim3 grid((unsigned)(1 + (n8 + kFrontThreads - 1) / kFrontThreads)), block(kFrontThreads);
  const uint4* xv = reinterpret_cast<const uint4*>(x);
  uint2* qv = reinterpret_cast<uint2*>(xq);
#define MOE_FRONT(nk)                                                                             \
  hipLaunchKernelGGL(front_small_kernel<nk>, grid, block, 0, s, L, xv, T, E, k, ns, n8, ids,     \
                     gates, counts, offsets, sorted_pair, pair_pos, qv, xs)
  switch (route_keys_per_lane(E)) {
    case 1: MOE_FRONT(1); break;
    case 2: MOE_FRONT(2); break;
    case 4: MOE_FRONT(4); break;
    case 8: MOE_FRONT(8); break;
    default: MOE_FRONT(16); break;
  }
#undef MOE_FRONT
  return hipGetLastError();
}

}  // namespace moe
