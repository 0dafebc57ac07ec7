// MXFP8 (OCP e4m3fn, one E8M0 scale per 32 elements) quantisation of bf16
// activations.  Four lanes share one 32-element block: each loads 8 bf16 with
// one 128-bit load, the block maximum is reduced over the four lanes with two
// xor shuffles, and each lane writes its 8 codes as one 64-bit store.  Purely
// bandwidth bound: 2 bytes in, 1 + 1/32 bytes out per element.
#include "common.h"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void quant_mxfp8_kernel(const uint4* __restrict__ x, long n8,
                                                          uint2* __restrict__ q,
                                                          uint8_t* __restrict__ sc) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;  // index of an 8-element group
  const bool live = i < n8;
  uint4 raw = live ? x[i] : make_uint4(0, 0, 0, 0);
  float v[8];
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    v[2 * h] = __uint_as_float(w[h] << 16);              // bf16 -> fp32 is exact
    v[2 * h + 1] = __uint_as_float(w[h] & 0xFFFF0000u);
  }
  float amax = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[e]));
  amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
  float mul;
  const uint32_t scode = mx_scale_from_amax(amax, &mul);
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) lo |= f32_to_e4m3(v[e] * mul) << (8 * e);
#pragma unroll
  for (int e = 0; e < 4; ++e) hi |= f32_to_e4m3(v[4 + e] * mul) << (8 * e);
  if (live) {
    q[i] = make_uint2(lo, hi);
    if ((i & 3) == 0) sc[i >> 2] = (uint8_t)scode;
  }
}

}  // namespace

hipError_t launch_quant_mxfp8(const uint16_t* x, long M, int K, uint8_t* q, uint8_t* sc,
                              hipStream_t s) {
  const long n8 = M * (long)K / 8;  // K % 32 == 0: a block never straddles rows
  const long grid = (n8 + 255) / 256;
  hipLaunchKernelGGL(quant_mxfp8_kernel, dim3((unsigned)grid), dim3(256), 0, s,
                     reinterpret_cast<const uint4*>(x), n8, reinterpret_cast<uint2*>(q), sc);
  return hipGetLastError();
}

}  // namespace moe
