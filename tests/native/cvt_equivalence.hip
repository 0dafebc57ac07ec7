// Checks the gfx950 conversion instructions the kernels use against the
// library's rounding rules, over every input the kernels can give them:
//  - e4m3: f32x2_to_e4m3 / f32x4_to_e4m3 (v_cvt_pk_fp8_f32 after a clamp to
//    +-448) against f32_to_e4m3 (round to nearest even, saturating at 448,
//    sign kept) for every fp32 value with |a| < 512;
//  - bf16: f32_to_bf16 / f32x2_to_bf16 (v_cvt_pk_bf16_f32) against rounding
//    the bit pattern to nearest even, for every finite fp32 value that rounds
//    to a finite bf16.
// Prints one line per check, "<name> inputs <n> mismatches <m>", then the
// first few mismatching inputs; exits 0 when it ran (the caller reads m).
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>

#include "common.h"

using namespace moe;

namespace {

__device__ uint32_t bf16_rne_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ void report(unsigned long long* cnt, uint32_t* ex, int which, uint32_t x, uint32_t got, uint32_t want) {
  const unsigned long long slot = atomicAdd(&cnt[which], 1ull);
  if (slot < 8) {
    ex[(which * 8 + slot) * 3 + 0] = x;
    ex[(which * 8 + slot) * 3 + 1] = got;
    ex[(which * 8 + slot) * 3 + 2] = want;
  }
}

// magnitudes 0 .. hi (exclusive) as bit patterns, both signs
__global__ void check_e4m3(uint32_t hi, unsigned long long* cnt, uint32_t* ex) {
  for (uint32_t u = blockIdx.x * blockDim.x + threadIdx.x; u < hi; u += gridDim.x * blockDim.x) {
    const float p = __uint_as_float(u), n = -p;
    const uint32_t pair = f32x2_to_e4m3(p, n);
    const uint32_t quad = f32x4_to_e4m3(n, p, p, n);
    const uint32_t wp = f32_to_e4m3(p), wn = f32_to_e4m3(n);
    if (pair != (wp | (wn << 8))) report(cnt, ex, 0, u, pair, wp | (wn << 8));
    if (quad != (wn | (wp << 8) | (wp << 16) | (wn << 24))) report(cnt, ex, 0, u, quad, wn | (wp << 8) | (wp << 16) | (wn << 24));
  }
}

__global__ void check_bf16(uint32_t hi, unsigned long long* cnt, uint32_t* ex) {
  for (uint32_t u = blockIdx.x * blockDim.x + threadIdx.x; u < hi; u += gridDim.x * blockDim.x) {
    const float p = __uint_as_float(u), n = -p;
    const uint32_t one = f32_to_bf16(p);
    const uint32_t pair = f32x2_to_bf16(p, n);
    const uint32_t wp = bf16_rne_bits(p), wn = bf16_rne_bits(n);
    if (one != wp) report(cnt, ex, 1, u, one, wp);
    if (pair != (wp | (wn << 16))) report(cnt, ex, 1, u, pair, wp | (wn << 16));
  }
}

bool ok(hipError_t e, const char* what) {
  if (e != hipSuccess) std::printf("error %s: %s\n", what, hipGetErrorString(e));
  return e == hipSuccess;
}

}  // namespace

int main() {
  unsigned long long* cnt = nullptr;
  uint32_t* ex = nullptr;
  if (!ok(hipMalloc(&cnt, 2 * sizeof(unsigned long long)), "hipMalloc") ||
      !ok(hipMalloc(&ex, 2 * 8 * 3 * sizeof(uint32_t)), "hipMalloc") ||
      !ok(hipMemset(cnt, 0, 2 * sizeof(unsigned long long)), "hipMemset") ||
      !ok(hipMemset(ex, 0, 2 * 8 * 3 * sizeof(uint32_t)), "hipMemset"))
    return 1;
  const uint32_t e4m3_hi = 0x44000000u;  // 512.0
  const uint32_t bf16_hi = 0x7F7F8000u;  // the first value that rounds to bf16 infinity
  hipLaunchKernelGGL(check_e4m3, dim3(4096), dim3(256), 0, 0, e4m3_hi, cnt, ex);
  hipLaunchKernelGGL(check_bf16, dim3(4096), dim3(256), 0, 0, bf16_hi, cnt, ex);
  if (!ok(hipGetLastError(), "launch") || !ok(hipDeviceSynchronize(), "kernels")) return 1;
  unsigned long long h[2];
  uint32_t e[2 * 8 * 3];
  if (!ok(hipMemcpy(h, cnt, sizeof h, hipMemcpyDeviceToHost), "copy") ||
      !ok(hipMemcpy(e, ex, sizeof e, hipMemcpyDeviceToHost), "copy"))
    return 1;
  const char* names[2] = {"e4m3", "bf16"};
  const unsigned long long inputs[2] = {2ull * e4m3_hi, 2ull * bf16_hi};
  for (int w = 0; w < 2; ++w) {
    std::printf("%s inputs %llu mismatches %llu\n", names[w], inputs[w], h[w]);
    for (unsigned long long i = 0; i < h[w] && i < 8; ++i)
      std::printf("  x=%08x got=%08x want=%08x\n", e[(w * 8 + i) * 3], e[(w * 8 + i) * 3 + 1], e[(w * 8 + i) * 3 + 2]);
  }
  return 0;
}
