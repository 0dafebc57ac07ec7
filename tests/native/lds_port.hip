// LDS traffic on one MI355X compute unit: LDS-DMA writes (global_load_lds
// _dwordx4, the prefill GEMMs' and the router's staging), 128-bit fragment
// reads (ds_read_b128), and both at once, with one workgroup of 8 waves per
// compute unit and a three-slot LDS ring of 48 KiB stages -- the shape of
// those kernels' K loops without their MFMAs.  Per iteration a workgroup
// DMAs one 48 KiB stage (six 1 KiB loads per wave, two stages in flight)
// from an L2-resident 2 MiB window and/or reads 128 KiB (sixteen 1 KiB reads
// per wave) from the stage written two iterations earlier; one barrier per
// iteration.  Also: the raw read rate (batches of sixteen 128-bit reads per
// wave with no barrier, alone and beside 8 or 16 KiB of DMA per batch), the
// same DMA from a 1.4 GiB buffer read as rows 14 KiB apart (an HBM stream, 8
// rows of 128 bytes per load, like the x rows of a K-step), and the time an
// LDS read issued right after the same wave's LDS-DMA load takes to return.
// Prints one line per case; the best of five launches.  Measurement only:
// checks nothing.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdio>

#include "lds_dma.h"

using namespace moe;

namespace {

constexpr int kStage = 49152;
constexpr int kRowB = 14336;  // row pitch of the strided case (a 7168-element bf16 row)

// MODE 0: DMA only; 1: reads only; 2: both; 3: DMA of row-strided HBM rows.
template <int MODE>
__global__ __launch_bounds__(512) void lds_traffic(const uint8_t* __restrict__ src, int iters,
                                                   uint32_t* __restrict__ sink) {
  __shared__ __align__(16) uint8_t lds[3 * kStage];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t ring = (uint32_t)(uintptr_t)(lds_u8*)lds;
  const uint8_t* win = src + (size_t)(blockIdx.x & 7) * (2u << 20);  // one window per XCD
  for (int i = tid; i < 3 * kStage / 16; i += 512) reinterpret_cast<uint4*>(lds)[i] = make_uint4(i, 1, 2, 3);
  __syncthreads();
  uint32_t acc = 0;
  for (int it = 0; it < iters; ++it) {
    const uint32_t slot = wave_u32(ring + (uint32_t)(it % 3) * kStage);
    if (MODE == 3) {
      // this workgroup's 384 rows, K bytes [128 it, 128 it + 128)
      const uint8_t* rb = wave_ptr(src + (size_t)blockIdx.x * 384 * kRowB + (size_t)it * 128);
#pragma unroll
      for (int u = 0; u < 6; ++u) {
        const int rg = wave * 6 + u;
        dma_x4(rb, (uint32_t)((rg * 8 + (lane >> 3)) * kRowB + (lane & 7) * 16), slot + (uint32_t)(rg * 1024));
      }
    } else if (MODE != 1) {
      const uint8_t* tb = wave_ptr(win + (size_t)(((blockIdx.x >> 3) + it) % 40) * kStage);
#pragma unroll
      for (int u = 0; u < 6; ++u)
        dma_x4(tb, (uint32_t)((wave * 6 + u) * 1024 + lane * 16), slot + (uint32_t)((wave * 6 + u) * 1024));
    }
    if (MODE == 1 || MODE == 2) {
      asm volatile("" ::: "memory");  // the reads are redone every iteration, never hoisted
      const uint8_t* rs = lds + ((it + 1) % 3) * kStage;  // the stage written two iterations ago
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const uint4 v = *reinterpret_cast<const uint4*>(rs + ((wave * 16 + u) * 1024 + lane * 16) % kStage);
        acc += (v.x ^ v.y) + (v.z ^ v.w);
      }
    }
    if (MODE != 1) wait_vmcnt<6>();  // this iteration's stage may stay in flight
    __syncthreads();
  }
  wait_vmcnt<0>();
  if (acc == 0x9E3779B9u) sink[tid] = acc;  // keeps the reads
}

// Raw read rate: per batch each wave issues 16 reads of 1 KiB with no
// barrier; NDMA (0, 1, 2) 1 KiB DMA loads per wave per batch go to a third
// slot that is never read, at most 8 in flight.
template <int NDMA>
__global__ __launch_bounds__(512) void lds_raw(const uint8_t* __restrict__ src, int iters,
                                               uint32_t* __restrict__ sink) {
  __shared__ __align__(16) uint8_t lds[3 * kStage];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  for (int i = tid; i < 3 * kStage / 16; i += 512) reinterpret_cast<uint4*>(lds)[i] = make_uint4(i, 1, 2, 3);
  __syncthreads();
  const uint32_t ring = (uint32_t)(uintptr_t)(lds_u8*)lds;
  const uint8_t* win = src + (size_t)(blockIdx.x & 7) * (2u << 20);
  uint4 a = make_uint4(0, 0, 0, 0);
  for (int it = 0; it < iters; ++it) {
    if (NDMA > 0) {
      const uint8_t* tb = wave_ptr(win + (size_t)(((blockIdx.x >> 3) + it) % 1000) * 2048);
      dma_x4(tb, (uint32_t)(lane * 16), wave_u32(ring + 2u * kStage + (uint32_t)((wave * 6 + (it % 6)) * 1024)));
      if (NDMA > 1)
        dma_x4(tb, (uint32_t)(1024 + lane * 16),
               wave_u32(ring + 2u * kStage + (uint32_t)((wave * 6 + ((it + 3) % 6)) * 1024)));
      wait_vmcnt<8>();
    }
    asm volatile("" ::: "memory");  // the reads are redone every batch
    const uint8_t* rs = lds + (it & 1) * kStage;
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const uint4 v = *reinterpret_cast<const uint4*>(rs + ((wave * 16 + u) * 1024 + lane * 16) % kStage);
      a.x ^= v.x;
      a.y ^= v.y;
      a.z ^= v.z;
      a.w ^= v.w;
    }
  }
  wait_vmcnt<0>();
  if ((a.x ^ a.y ^ a.z ^ a.w) == 0x9E3779B9u) sink[tid] = a.x;
}

// One wave per workgroup: an LDS-DMA load of a cold 4 KiB slice, then a
// 128-bit LDS read of other LDS bytes; clocks until the read's data is back
// (lgkmcnt 0) and until the DMA is complete (vmcnt 0).  kDma false: the read
// alone.
template <bool kDma>
__global__ __launch_bounds__(64) void read_after_dma(const uint8_t* __restrict__ src,
                                                     unsigned long long* __restrict__ out, int iters) {
  __shared__ __align__(16) uint8_t lds[2048];
  const int lane = threadIdx.x;
  const uint32_t l0 = (uint32_t)(uintptr_t)(lds_u8*)lds;
  reinterpret_cast<uint4*>(lds)[64 + lane] = make_uint4(lane, 1, 2, 3);
  __syncthreads();
  const uint32_t raddr = l0 + 1024 + lane * 16;
  unsigned long long s1 = 0, s2 = 0;
  uint32_t acc = 0;
  for (int it = 0; it < iters; ++it) {
    const uint8_t* base = src + ((size_t)blockIdx.x * iters + it) * 4096;
    const uint32_t off = lane * 16;
    unsigned long long t0, t1, t2;
    uint4 v;
    uint32_t saved;
    if (kDma) {
      asm volatile(
          "s_waitcnt vmcnt(0) lgkmcnt(0)\n\t"
          "s_memtime %0\n\t"
          "s_waitcnt lgkmcnt(0)\n\t"
          "s_mov_b32 %4, m0\n\t"
          "s_mov_b32 m0, %7\n\t"
          "s_nop 0\n\t"
          "global_load_lds_dwordx4 %5, %6\n\t"
          "s_mov_b32 m0, %4\n\t"
          "ds_read_b128 %3, %8\n\t"
          "s_waitcnt lgkmcnt(0)\n\t"
          "s_memtime %1\n\t"
          "s_waitcnt lgkmcnt(0)\n\t"
          "s_waitcnt vmcnt(0)\n\t"
          "s_memtime %2\n\t"
          "s_waitcnt lgkmcnt(0)\n\t"
          : "=&s"(t0), "=&s"(t1), "=&s"(t2), "=&v"(v), "=&s"(saved)
          : "v"(off), "s"(base), "s"(l0), "v"(raddr)
          : "memory");
    } else {
      asm volatile(
          "s_waitcnt vmcnt(0) lgkmcnt(0)\n\t"
          "s_memtime %0\n\t"
          "s_waitcnt lgkmcnt(0)\n\t"
          "ds_read_b128 %3, %4\n\t"
          "s_waitcnt lgkmcnt(0)\n\t"
          "s_memtime %1\n\t"
          "s_waitcnt lgkmcnt(0)\n\t"
          "s_memtime %2\n\t"
          "s_waitcnt lgkmcnt(0)\n\t"
          : "=&s"(t0), "=&s"(t1), "=&s"(t2), "=&v"(v)
          : "v"(raddr)
          : "memory");
    }
    acc += v.x;
    s1 += t1 - t0;
    s2 += t2 - t0;
  }
  if (lane == 0) {
    out[2 * blockIdx.x] = s1;
    out[2 * blockIdx.x + 1] = s2;
  }
  if (acc == 0x9E3779B9u) out[0] = 0;
}

bool ok(hipError_t e, const char* what) {
  if (e != hipSuccess) std::printf("error %s: %s\n", what, hipGetErrorString(e));
  return e == hipSuccess;
}

template <int M>
bool traffic(const char* name, const uint8_t* src, uint32_t* sink, int ncu, double kb_per_iter) {
  const int iters = M == 3 ? 112 : 2000;
  hipEvent_t a, b;
  if (!ok(hipEventCreate(&a), "event") || !ok(hipEventCreate(&b), "event")) return false;
  hipLaunchKernelGGL(lds_traffic<M>, dim3(ncu), dim3(512), 0, 0, src, 50, sink);
  if (!ok(hipDeviceSynchronize(), "warm-up")) return false;
  float best = 1e30f;
  for (int rep = 0; rep < 5; ++rep) {
    hipEventRecord(a);
    hipLaunchKernelGGL(lds_traffic<M>, dim3(ncu), dim3(512), 0, 0, src, iters, sink);
    hipEventRecord(b);
    if (!ok(hipEventSynchronize(b), name)) return false;
    float ms = 0;
    hipEventElapsedTime(&ms, a, b);
    best = std::min(best, ms);
  }
  const double us_iter = best * 1e3 / iters;
  std::printf("%-46s %8.3f us/iteration  %7.1f GB/s of LDS traffic per CU  (%.2f TB/s chip)\n", name,
              us_iter, kb_per_iter * 1024.0 / us_iter / 1e3, kb_per_iter * 1024.0 * ncu / us_iter / 1e6);
  hipEventDestroy(a);
  hipEventDestroy(b);
  return true;
}

template <int NDMA>
bool raw(const char* name, const uint8_t* src, uint32_t* sink, int ncu) {
  const int iters = 4000;
  hipEvent_t a, b;
  if (!ok(hipEventCreate(&a), "event") || !ok(hipEventCreate(&b), "event")) return false;
  hipLaunchKernelGGL(lds_raw<NDMA>, dim3(ncu), dim3(512), 0, 0, src, 100, sink);
  if (!ok(hipDeviceSynchronize(), "warm-up")) return false;
  float best = 1e30f;
  for (int rep = 0; rep < 5; ++rep) {
    hipEventRecord(a);
    hipLaunchKernelGGL(lds_raw<NDMA>, dim3(ncu), dim3(512), 0, 0, src, iters, sink);
    hipEventRecord(b);
    if (!ok(hipEventSynchronize(b), name)) return false;
    float ms = 0;
    hipEventElapsedTime(&ms, a, b);
    best = std::min(best, ms);
  }
  const double us = best * 1e3 / iters;
  std::printf("%-46s %8.4f us/batch  reads %6.1f GB/s per CU, DMA %5.1f GB/s per CU\n", name, us,
              128.0 * 1024 / us / 1e3, 8.0 * NDMA * 1024 / us / 1e3);
  hipEventDestroy(a);
  hipEventDestroy(b);
  return true;
}

template <bool kDma>
bool order(const char* name, const uint8_t* src, unsigned long long* d_out, unsigned long long* h) {
  const int nblk = 256, iters = 64;
  hipLaunchKernelGGL(read_after_dma<kDma>, dim3(nblk), dim3(64), 0, 0, src, d_out, iters);
  if (!ok(hipDeviceSynchronize(), name)) return false;
  if (!ok(hipMemcpy(h, d_out, 2 * nblk * sizeof(unsigned long long), hipMemcpyDeviceToHost), "copy")) return false;
  double a[256], b[256];
  for (int i = 0; i < nblk; ++i) {
    a[i] = (double)h[2 * i] / iters;
    b[i] = (double)h[2 * i + 1] / iters;
  }
  std::sort(a, a + nblk);
  std::sort(b, b + nblk);
  std::printf("%-46s LDS read back after %6.1f clocks, DMA complete after %6.1f clocks (medians)\n", name,
              a[nblk / 2], b[nblk / 2]);
  return true;
}

}  // namespace

int main() {
  int ncu = 0;
  if (!ok(hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, 0), "attribute")) return 1;
  const size_t bytes = (size_t)ncu * 384 * kRowB + (16u << 20);
  uint8_t* src = nullptr;
  uint32_t* sink = nullptr;
  unsigned long long* d_out = nullptr;
  static unsigned long long h[512];
  if (!ok(hipMalloc(&src, bytes), "malloc") || !ok(hipMemset(src, 3, bytes), "memset") ||
      !ok(hipMalloc(&sink, 512 * 4), "malloc") || !ok(hipMalloc(&d_out, sizeof(h)), "malloc"))
    return 1;
  std::printf("compute units %d, one workgroup of 8 waves each\n", ncu);
  if (!traffic<0>("DMA 48 KiB/iteration (L2)", src, sink, ncu, 48) ||
      !traffic<1>("ds_read_b128 128 KiB/iteration", src, sink, ncu, 128) ||
      !traffic<2>("both: DMA 48 KiB + reads 128 KiB", src, sink, ncu, 176) ||
      !traffic<3>("DMA 48 KiB/iteration, row-strided HBM stream", src, sink, ncu, 48))
    return 1;
  if (!raw<0>("raw reads, 128 KiB per batch, no barrier", src, sink, ncu) ||
      !raw<1>("raw reads + 8 KiB DMA per batch", src, sink, ncu) ||
      !raw<2>("raw reads + 16 KiB DMA per batch", src, sink, ncu))
    return 1;
  if (!order<false>("LDS read alone", src, d_out, h) || !order<true>("LDS read right after an LDS-DMA load", src, d_out, h))
    return 1;
  return 0;
}
