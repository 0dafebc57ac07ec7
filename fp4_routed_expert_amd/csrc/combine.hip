// Gate-weighted combine back to token order: y[t] = sum_j g[t,j] * O[pair_pos[t*k+j]]
// (+ the shared expert's row, when there is one), accumulated in slot order
// j = 0..k-1 (then the shared row) in fp32 with no atomics (a fixed
// reduction order, pwwt.cn review section 4.2).  O holds the expert outputs
// as bf16 (a matrix-multiply output kept at low precision, its sum in fp32:
// the same review, section 4.1).  Each thread produces four consecutive
// outputs from 64-bit loads of O and one 128-bit store; bandwidth bound at
// prefill sizes, latency bound at decode sizes (hence the batched loads).
// A workgroup of 128 threads covers 512 columns of one token; the grid is
// flat with the column chunk innermost, so the chunks of a token's k O rows
// are read by neighbouring workgroups at about the same time and each row
// streams whole (c4: 417 -> 377 us against a token-major 2-D grid of
// 256-thread groups).
#include "common.h"

namespace moe {
namespace {

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

typedef unsigned v2u __attribute__((ext_vector_type(2)));

constexpr int kCombineThreads = 128;

__global__ __launch_bounds__(kCombineThreads) void combine_kernel(const uint2* __restrict__ O,
                                                      const float* __restrict__ gates,
                                                      const int32_t* __restrict__ pair_pos,
                                                      const uint2* __restrict__ Os, int k, int H4,
                                                      float4* __restrict__ y) {
  const int nch = (H4 + kCombineThreads - 1) / kCombineThreads;
  const int t = (int)blockIdx.x / nch;
  const int c = ((int)blockIdx.x - t * nch) * kCombineThreads + (int)threadIdx.x;
  if (c >= H4) return;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  // slots in batches of 8: all their row indices and gates, then all their O
  // loads, are in flight together (a short last batch repeats its last slot's
  // loads and skips their sums); the sum still runs in slot order
  for (int j0 = 0; j0 < k; j0 += 8) {
    const int n = min(8, k - j0);
    int row[8];
    float g[8];
    uint2 o[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const size_t idx = (size_t)t * k + j0 + min(u, n - 1);
      row[u] = pair_pos[idx];
      g[u] = gates[idx];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const v2u w = __builtin_nontemporal_load(reinterpret_cast<const v2u*>(O + (size_t)row[u] * H4 + c));
      o[u] = make_uint2(w.x, w.y);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float4 a = make_float4(fmaf(g[u], bf16_lo(o[u].x), acc.x), fmaf(g[u], bf16_hi(o[u].x), acc.y),
                                   fmaf(g[u], bf16_lo(o[u].y), acc.z), fmaf(g[u], bf16_hi(o[u].y), acc.w));
      if (u < n) acc = a;
    }
  }
  if (Os) {  // the shared expert, weight 1, after the routed slots
    const uint2 o = Os[(size_t)t * H4 + c];
    acc.x += bf16_lo(o.x);
    acc.y += bf16_hi(o.x);
    acc.z += bf16_lo(o.y);
    acc.w += bf16_hi(o.y);
  }
  // O is read once and y written once per layer: non-temporal accesses
  __builtin_nontemporal_store(v4f{acc.x, acc.y, acc.z, acc.w}, reinterpret_cast<v4f*>(y + (size_t)t * H4 + c));
}

}  // namespace

hipError_t launch_combine(const uint16_t* O, const float* gates, const int32_t* pair_pos,
                          const uint16_t* O_shared, int T, int k, int H, float* y, hipStream_t s) {
  const int H4 = H / 4;
  const long blocks = (long)T * ((H4 + kCombineThreads - 1) / kCombineThreads);
  if (blocks > 0x7fffffffL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)blocks), dim3(kCombineThreads), 0, s, reinterpret_cast<const uint2*>(O),
                     gates, pair_pos, reinterpret_cast<const uint2*>(O_shared), k, H4,
                     reinterpret_cast<float4*>(y));
  return hipGetLastError();
}

}  // namespace moe
