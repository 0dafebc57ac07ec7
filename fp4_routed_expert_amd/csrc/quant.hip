// MXFP8 (OCP e4m3fn, one E8M0 scale per 32 elements) quantisation of bf16
// activations.  Four lanes share one 32-element block: each loads 8 bf16 with
// one 128-bit load, the block maximum is reduced over the four lanes with two
// xor shuffles, and each lane writes its 8 codes as one 64-bit store.  Purely
// bandwidth bound: 2 bytes in, 1 + 1/32 bytes out per element.
#include "stages.h"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void quant_mxfp8_kernel(const uint4* __restrict__ x, long n8,
                                                          uint2* __restrict__ q,
                                                          uint8_t* __restrict__ sc) {
  quant_group8(x, (long)blockIdx.x * blockDim.x + threadIdx.x, n8, q, sc);
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
