// Gate-weighted combine back to token order: y[t] = sum_j g[t,j] * O[pair_pos[t*k+j]],
// accumulated in slot order j = 0..k-1 in fp32 with no atomics (a fixed
// reduction order, pwwt.cn review section 4.2).  O holds the expert outputs
// as bf16 (a matrix-multiply output kept at low precision, its sum in fp32:
// the same review, section 4.1).  Each thread produces four consecutive
// outputs from 64-bit loads of O and one 128-bit store; bandwidth bound.
#include "common.h"

namespace moe {
namespace {

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__global__ __launch_bounds__(256) void combine_kernel(const uint2* __restrict__ O,
                                                      const float* __restrict__ gates,
                                                      const int32_t* __restrict__ pair_pos,
                                                      int k, int H4, float4* __restrict__ y) {
  const int t = blockIdx.x;
  const int c = blockIdx.y * blockDim.x + threadIdx.x;
  if (c >= H4) return;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < k; ++j) {
    const float g = gates[(size_t)t * k + j];
    const uint2 o = O[(size_t)pair_pos[(size_t)t * k + j] * H4 + c];
    acc.x = fmaf(g, bf16_lo(o.x), acc.x);
    acc.y = fmaf(g, bf16_hi(o.x), acc.y);
    acc.z = fmaf(g, bf16_lo(o.y), acc.z);
    acc.w = fmaf(g, bf16_hi(o.y), acc.w);
  }
  y[(size_t)t * H4 + c] = acc;
}

}  // namespace

hipError_t launch_combine(const uint16_t* O, const float* gates, const int32_t* pair_pos, int T,
                          int k, int H, float* y, hipStream_t s) {
  const int H4 = H / 4;
  dim3 grid((unsigned)T, (unsigned)((H4 + 255) / 256));
  hipLaunchKernelGGL(combine_kernel, grid, dim3(256), 0, s, reinterpret_cast<const uint2*>(O),
                     gates, pair_pos, k, H4, reinterpret_cast<float4*>(y));
  return hipGetLastError();
}

}  // namespace moe
