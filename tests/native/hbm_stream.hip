// Streaming-read rate of HBM on one MI355X: every byte of a 4 GiB buffer
// (16x the 256 MiB last-level cache, so the reads reach HBM) read once per
// pass with 16-byte vector loads, as plain loads and as non-temporal loads
// (the decode kernels' weight loads), for a few grid sizes.  Prints
// "<form> grid <g> waves/CU <w>: <us> us <GB/s>"; the best pass of five per
// line.  Measurement only: checks nothing.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Each thread loads 4 x 16 bytes per iteration (4 loads in flight), the
// wave's loads covering 4 consecutive KiB; the grid strides over the buffer.
template <bool kNT>
__global__ __launch_bounds__(256) void stream(const u32x4* __restrict__ p, size_t n16, uint32_t* out) {
  const size_t lane = threadIdx.x & 63, wave = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const size_t nwaves = (size_t)gridDim.x * 4;
  uint32_t acc = 0;
  for (size_t base = wave * 256; base + 256 <= n16; base += nwaves * 256) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = kNT ? __builtin_nontemporal_load(p + base + 64 * u + lane) : p[base + 64 * u + lane];
#pragma unroll
    for (int u = 0; u < 4; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == 0x9E3779B9u) out[0] = acc;  // keeps the loads; never true for the buffer's bytes
}

bool ok(hipError_t e, const char* what) {
  if (e != hipSuccess) std::printf("error %s: %s\n", what, hipGetErrorString(e));
  return e == hipSuccess;
}

}  // namespace

int main() {
  const size_t bytes = (size_t)4 << 30;
  void* buf = nullptr;
  uint32_t* out = nullptr;
  if (!ok(hipMalloc(&buf, bytes), "hipMalloc") || !ok(hipMalloc(&out, 4), "hipMalloc") ||
      !ok(hipMemset(buf, 1, bytes), "hipMemset") || !ok(hipDeviceSynchronize(), "memset"))
    return 1;
  int ncu = 0;
  if (!ok(hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, 0), "attribute")) return 1;
  hipEvent_t e0, e1;
  if (!ok(hipEventCreate(&e0), "event") || !ok(hipEventCreate(&e1), "event")) return 1;
  const size_t n16 = bytes / 16;
  for (int nt = 0; nt < 2; ++nt) {
    for (int per_cu : {2, 4, 8}) {  // workgroups of 4 waves per CU
      const int grid = ncu * per_cu;
      float best = 1e30f;
      for (int rep = 0; rep < 6; ++rep) {
        if (!ok(hipEventRecord(e0), "record")) return 1;
        if (nt)
          hipLaunchKernelGGL(stream<true>, dim3(grid), dim3(256), 0, 0, (const u32x4*)buf, n16, out);
        else
          hipLaunchKernelGGL(stream<false>, dim3(grid), dim3(256), 0, 0, (const u32x4*)buf, n16, out);
        if (!ok(hipGetLastError(), "launch") || !ok(hipEventRecord(e1), "record") ||
            !ok(hipEventSynchronize(e1), "sync"))
          return 1;
        float ms = 0.0f;
        if (!ok(hipEventElapsedTime(&ms, e0, e1), "elapsed")) return 1;
        if (rep > 0 && ms < best) best = ms;  // the first pass warms up
      }
      std::printf("%s grid %d waves/CU %d: %.1f us %.0f GB/s\n", nt ? "non-temporal" : "plain", grid,
                  4 * per_cu, best * 1e3, (double)bytes / (best * 1e-3) / 1e9);
    }
  }
  return 0;
}
