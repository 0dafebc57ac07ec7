// Issue rate of the gfx950 scaled MFMA v_mfma_scale_f32_16x16x128_f8f6f4 with
// one FP8 and one FP4 operand (the expert GEMMs' product), FP8 as A and FP4 as
// B or the other way round, with one or two waves per SIMD and NACC
// independent accumulators per wave.  One workgroup per CU; each lane stores
// one sum at the end.  Prints "<waves/SIMD>, <operand order>: <ms> <TFLOP/s>"
// (dense FLOP: 2 x 16 x 16 x 128 per instruction); the second of two passes is
// the one to read.  Measurement only: checks nothing.
#include <hip/hip_runtime.h>

#include <cstdio>

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

template <int NACC, int TH, bool kFp4A>
__global__ __launch_bounds__(TH) void rate(float* out, int iters) {
  v8i a = {(int)threadIdx.x, 1, 2, 3, 4, 5, 6, 7};
  const v4i bb = {(int)threadIdx.x * 3, 7, 6, 5};
  const v8i b = __builtin_shufflevector(bb, bb, 0, 1, 2, 3, -1, -1, -1, -1);
  v4f c[NACC];
#pragma unroll
  for (int i = 0; i < NACC; ++i) c[i] = v4f{0, 0, 0, 0};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < NACC; ++i) {
      if (kFp4A)
        c[i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b, a, c[i], 4, 0, 0, 127, 0, 127);
      else
        c[i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c[i], 0, 4, 0, 127, 0, 127);
    }
  }
  v4f s = c[0];
#pragma unroll
  for (int i = 1; i < NACC; ++i) s += c[i];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s.x + s.y + s.z + s.w;
}

bool ok(hipError_t e, const char* what) {
  if (e != hipSuccess) std::printf("error %s: %s\n", what, hipGetErrorString(e));
  return e == hipSuccess;
}

}  // namespace

int main() {
  int ncu = 0;
  float* out = nullptr;
  hipEvent_t e0, e1;
  if (!ok(hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, 0), "attribute") ||
      !ok(hipMalloc(&out, (size_t)ncu * 512 * sizeof(float)), "hipMalloc") ||
      !ok(hipEventCreate(&e0), "event") || !ok(hipEventCreate(&e1), "event"))
    return 1;
  const int iters = 2000;
  auto run = [&](auto kern, int threads, int nacc, const char* name) {
    hipLaunchKernelGGL(kern, dim3(ncu), dim3(threads), 0, 0, out, 10);
    float ms = 0.0f;
    if (!ok(hipGetLastError(), "launch") || !ok(hipDeviceSynchronize(), "warmup") ||
        !ok(hipEventRecord(e0), "record"))
      return false;
    hipLaunchKernelGGL(kern, dim3(ncu), dim3(threads), 0, 0, out, iters);
    if (!ok(hipGetLastError(), "launch") || !ok(hipEventRecord(e1), "record") ||
        !ok(hipEventSynchronize(e1), "sync") || !ok(hipEventElapsedTime(&ms, e0, e1), "elapsed"))
      return false;
    const double flop = (double)ncu * (threads / 64) * iters * nacc * 2.0 * 16 * 16 * 128;
    std::printf("%s: %.3f ms %.1f TFLOP/s\n", name, ms, flop / ms / 1e9);
    return true;
  };
  for (int rep = 0; rep < 2; ++rep) {
    if (!run(rate<24, 512, false>, 512, 24, "2 waves/SIMD, A fp8 B fp4") ||
        !run(rate<24, 512, true>, 512, 24, "2 waves/SIMD, A fp4 B fp8") ||
        !run(rate<48, 256, false>, 256, 48, "1 wave/SIMD, A fp8 B fp4") ||
        !run(rate<48, 256, true>, 256, 48, "1 wave/SIMD, A fp4 B fp8"))
      return 1;
  }
  return 0;
}
