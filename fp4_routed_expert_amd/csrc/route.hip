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

// ids/gates rows hold k + ns slots: the routed top-k of E, then ns shared experts
template <int NK>
__global__ __launch_bounds__(256) void route_topk_kernel(LogitSrc L, int T, int E, int k, int ns,
                                                         int32_t* __restrict__ ids,
                                                         float* __restrict__ gates) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (t >= T) return;
  const int ld = k + ns;
  RouteKeys<NK> r;
  load_route_keys<NK>(r, L, (long)t * E, E, lane);
  int id;
  float g;
  if (route_topk_token<NK>(r, E, k, lane, &id, &g) || shared_slot(E, k, ns, lane, &id, &g)) {
    ids[(size_t)t * ld + lane] = id;
    gates[(size_t)t * ld + lane] = g;
  }
}

}  // namespace

int route_keys_per_lane(int E) {
  return E <= 64 ? 1 : E <= 128 ? 2 : E <= 256 ? 4 : E <= 512 ? 8 : 16;
}

hipError_t launch_route_topk(const float* logits, int S, int T, int E, int k, int ns,
                             int32_t* ids, float* gates, hipStream_t s) {
  const int waves_per_block = 4;
  const dim3 grid((T + waves_per_block - 1) / waves_per_block), block(64 * waves_per_block);
  const LogitSrc L{logits, (long)T * E, S};
#define MOE_ROUTE(nk) \
  hipLaunchKernelGGL(route_topk_kernel<nk>, grid, block, 0, s, L, T, E, k, ns, ids, gates)
  switch (route_keys_per_lane(E)) {
    case 1: MOE_ROUTE(1); break;
    case 2: MOE_ROUTE(2); break;
    case 4: MOE_ROUTE(4); break;
    case 8: MOE_ROUTE(8); break;
    default: MOE_ROUTE(16); break;
  }
#undef MOE_ROUTE
  return hipGetLastError();
}

}  // namespace moe
