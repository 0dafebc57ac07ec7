// Top-k routing: one wavefront per token.
//
// Each lane keeps its share of the token's logits in registers as 64-bit keys
// whose unsigned order is (logit descending, expert index ascending); k rounds
// of a wave-wide DPP max pick the slots in order.  Scores are compared in fp32
// with a fixed tie-break by expert id (pwwt.cn review, section 4.1 table row
// "MoE routing top-k" and section 4.2).
#include "stages.h"

namespace moe {
namespace {

template <int NK>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits, int T,
                                                         int E, int k, int32_t* __restrict__ ids,
                                                         float* __restrict__ gates) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (t >= T) return;
  RouteKeys<NK> r;
  load_route_keys<NK>(r, logits + (size_t)t * E, E, lane);
  int id;
  float g;
  if (route_topk_token<NK>(r, E, k, lane, &id, &g)) {
    ids[(size_t)t * k + lane] = id;
    gates[(size_t)t * k + lane] = g;
  }
}

}  // namespace

int route_keys_per_lane(int E) {
  return E <= 64 ? 1 : E <= 128 ? 2 : E <= 256 ? 4 : E <= 512 ? 8 : 16;
}

hipError_t launch_route_topk(const float* logits, int T, int E, int k, int32_t* ids,
                             float* gates, hipStream_t s) {
  const int waves_per_block = 4;
  const dim3 grid((T + waves_per_block - 1) / waves_per_block), block(64 * waves_per_block);
  switch (route_keys_per_lane(E)) {
    case 1: hipLaunchKernelGGL(route_topk_kernel<1>, grid, block, 0, s, logits, T, E, k, ids, gates); break;
    case 2: hipLaunchKernelGGL(route_topk_kernel<2>, grid, block, 0, s, logits, T, E, k, ids, gates); break;
    case 4: hipLaunchKernelGGL(route_topk_kernel<4>, grid, block, 0, s, logits, T, E, k, ids, gates); break;
    case 8: hipLaunchKernelGGL(route_topk_kernel<8>, grid, block, 0, s, logits, T, E, k, ids, gates); break;
    default: hipLaunchKernelGGL(route_topk_kernel<16>, grid, block, 0, s, logits, T, E, k, ids, gates); break;
  }
  return hipGetLastError();
}

}  // namespace moe
