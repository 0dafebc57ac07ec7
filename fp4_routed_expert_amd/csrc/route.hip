// Top-k routing: one wavefront per token.
//
// Each lane keeps its share of the token's logits in registers as 64-bit keys
// whose unsigned order is (logit descending, expert index ascending); k rounds
// of a wave-wide max (xor butterfly over the 64 lanes) pick the slots in order.
// Scores are compared in fp32 with a fixed tie-break by expert id (pwwt.cn
// review, section 4.1 table row "MoE routing top-k" and section 4.2).
#include "common.h"

namespace moe {
namespace {

constexpr int kMaxPerLane = 16;  // E <= 1024

// Monotone map of an fp32 to uint32 (-0 first folded into +0 so they tie).
__device__ __forceinline__ uint32_t ordered_bits(float v) {
  uint32_t u = __float_as_uint(v + 0.0f);  // -0 + +0 = +0 under round-to-nearest
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float from_ordered_bits(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t x) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)x, m, 64);
    const uint32_t hi = __shfl_xor((uint32_t)(x >> 32), m, 64);
    const uint64_t y = ((uint64_t)hi << 32) | lo;
    x = y > x ? y : x;
  }
  return x;
}

__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits, int T,
                                                         int E, int k, int32_t* __restrict__ ids,
                                                         float* __restrict__ gates) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* row = logits + (size_t)t * E;
  uint64_t key[kMaxPerLane];
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) {
    const int e = lane + 64 * i;
    // index part: E-1-e so that a larger key means a lower expert index
    key[i] = (e < E) ? (((uint64_t)ordered_bits(row[e]) << 32) | (uint32_t)(E - 1 - e)) : 0ull;
  }
  // lane j keeps slot j; every lane sees the selected logit of each round
  float l0 = 0.0f, my_logit = 0.0f;
  int my_id = 0;
  for (int j = 0; j < k; ++j) {
    uint64_t best = 0;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) best = key[i] > best ? key[i] : best;
    best = wave_max_u64(best);
    const int e = E - 1 - (int)(uint32_t)best;
    const float le = from_ordered_bits((uint32_t)(best >> 32));  // the logit itself, no reload
    if (j == 0) l0 = le;
    if (lane == j) {
      my_id = e;
      my_logit = le;
    }
    // the owner lane removes the selected key (keys are unique: the index part differs)
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i)
      if (key[i] == best) key[i] = 0;
  }
  // softmax over the selected logits, relative to the largest (slot 0);
  // the denominator is a fixed-order butterfly sum
  const float ex = (lane < k) ? expf(my_logit - l0) : 0.0f;
  float den = ex;
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) den += __shfl_xor(den, m, 64);
  if (lane < k) {
    ids[(size_t)t * k + lane] = my_id;
    gates[(size_t)t * k + lane] = ex / den;
  }
}

}  // namespace

hipError_t launch_route_topk(const float* logits, int T, int E, int k, int32_t* ids,
                             float* gates, hipStream_t s) {
  const int waves_per_block = 4;
  const int grid = (T + waves_per_block - 1) / waves_per_block;
  hipLaunchKernelGGL(route_topk_kernel, dim3(grid), dim3(64 * waves_per_block), 0, s, logits, T,
                     E, k, ids, gates);
  return hipGetLastError();
}

}  // namespace moe
