// Gate-weighted combine back to token order: y[t] = sum_j g[t,j] * O[pair_pos[t*k+j]],
// accumulated in slot order j = 0..k-1 in fp32 with no atomics (a fixed
// reduction order, pwwt.cn review section 4.2).  Each thread produces four
// consecutive outputs with 128-bit loads and stores; bandwidth bound.
#include "common.h"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void combine_kernel(const float4* __restrict__ O,
                                                      const float* __restrict__ gates,
                                                      const int32_t* __restrict__ pair_pos,
                                                      int k, int H4, float4* __restrict__ y) {
  const int t = blockIdx.x;
  const int c = blockIdx.y * blockDim.x + threadIdx.x;
  if (c >= H4) return;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < k; ++j) {
    const float g = gates[(size_t)t * k + j];
    const float4 o = O[(size_t)pair_pos[(size_t)t * k + j] * H4 + c];
    acc.x = fmaf(g, o.x, acc.x);
    acc.y = fmaf(g, o.y, acc.y);
    acc.z = fmaf(g, o.z, acc.z);
    acc.w = fmaf(g, o.w, acc.w);
  }
  y[(size_t)t * H4 + c] = acc;
}

}  // namespace

hipError_t launch_combine(const float* O, const float* gates, const int32_t* pair_pos, int T,
                          int k, int H, float* y, hipStream_t s) {
  const int H4 = H / 4;
  dim3 grid((unsigned)T, (unsigned)((H4 + 255) / 256));
  hipLaunchKernelGGL(combine_kernel, grid, dim3(256), 0, s, reinterpret_cast<const float4*>(O),
                     gates, pair_pos, k, H4, reinterpret_cast<float4*>(y));
  return hipGetLastError();
}

}  // namespace moe
