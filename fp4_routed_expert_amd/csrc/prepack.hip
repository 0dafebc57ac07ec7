// Load-time prepack of the canonical expert weights into the MFMA tile order
// described in common.h (PackedLayout).  The W2 (down) layout is fixed here,
// once: the paper's first fast path produced an output permutation from a
// mismatched routed-expert W2 layout and the cure was to repair the layout at
// load time ("DeepSeek-V4-Flash on AMD gfx90a: Correctness Recovery and
// Inference Performance Engineering", abstract).  Pure byte moves: every
// output 16-byte chunk (or scale dword) is gathered from one canonical place.
#include "common.h"

namespace moe {
namespace {

__global__ void pack_up_weights(const uint4* __restrict__ w1, const uint4* __restrict__ w3,
                                PackedLayout L, uint4* __restrict__ out) {
  const int QT = L.I / 32;
  const long n = (long)L.E * QT * L.J * 256;
  const long rowc = L.H / 32;  // 16-byte chunks per canonical row (H/2 bytes)
  for (long c = (long)blockIdx.x * blockDim.x + threadIdx.x; c < n;
       c += (long)gridDim.x * blockDim.x) {
    const long blk = c >> 8;
    const int t = (int)((c >> 6) & 3), l = (int)(c & 63);
    const int j = (int)(blk % L.J);
    const long eq = blk / L.J;
    const int q = (int)(eq % QT);
    const long e = eq / QT;
    const long row = (long)q * 32 + (t & 1) * 16 + (l & 15);
    const uint4* src = (t < 2) ? w1 : w3;
    out[(L.upw_off >> 4) + c] = src[(e * L.I + row) * rowc + j * 4 + (l >> 4)];
  }
}

__global__ void pack_up_scales(const uint8_t* __restrict__ s1, const uint8_t* __restrict__ s3,
                               PackedLayout L, uint32_t* __restrict__ out) {
  const int QT = L.I / 32;
  const long n = (long)L.E * QT * L.J * 64;  // one dword per (e, q, j, lane)
  for (long d = (long)blockIdx.x * blockDim.x + threadIdx.x; d < n;
       d += (long)gridDim.x * blockDim.x) {
    const int l = (int)(d & 63);
    const long blk = d >> 6;
    const int j = (int)(blk % L.J);
    const long eq = blk / L.J;
    const int q = (int)(eq % QT);
    const long e = eq / QT;
    const long blkcol = (long)j * 4 + (l >> 4);  // 32-element block along H
    uint32_t v = 0;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const long row = (long)q * 32 + (t & 1) * 16 + (l & 15);
      const uint8_t* src = (t < 2) ? s1 : s3;
      v |= (uint32_t)src[(e * L.I + row) * (L.H / 32) + blkcol] << (8 * t);
    }
    out[(L.ups_off >> 2) + d] = v;
  }
}

__global__ void pack_down_weights(const uint4* __restrict__ w2, PackedLayout L,
                                  uint4* __restrict__ out) {
  const int QT2 = L.H / 32;
  const long n = (long)L.E * QT2 * L.J2 * 128;
  const long rowc = L.I / 32;
  for (long c = (long)blockIdx.x * blockDim.x + threadIdx.x; c < n;
       c += (long)gridDim.x * blockDim.x) {
    const long blk = c >> 7;
    const int t = (int)((c >> 6) & 1), l = (int)(c & 63);
    const int j2 = (int)(blk % L.J2);
    const long eq = blk / L.J2;
    const int q2 = (int)(eq % QT2);
    const long e = eq / QT2;
    const long row = (long)q2 * 32 + t * 16 + (l & 15);
    out[(L.dnw_off >> 4) + c] = w2[(e * L.H + row) * rowc + j2 * 4 + (l >> 4)];
  }
}

__global__ void pack_down_scales(const uint8_t* __restrict__ s2, PackedLayout L,
                                 uint16_t* __restrict__ out) {
  const int QT2 = L.H / 32;
  const long n = (long)L.E * QT2 * L.J2 * 64;  // one 16-bit pair per (e, q2, j2, lane)
  for (long d = (long)blockIdx.x * blockDim.x + threadIdx.x; d < n;
       d += (long)gridDim.x * blockDim.x) {
    const int l = (int)(d & 63);
    const long blk = d >> 6;
    const int j2 = (int)(blk % L.J2);
    const long eq = blk / L.J2;
    const int q2 = (int)(eq % QT2);
    const long e = eq / QT2;
    const long blkcol = (long)j2 * 4 + (l >> 4);
    uint32_t v = 0;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const long row = (long)q2 * 32 + t * 16 + (l & 15);
      v |= (uint32_t)s2[(e * L.H + row) * (L.I / 32) + blkcol] << (8 * t);
    }
    out[(L.dns_off >> 1) + d] = (uint16_t)v;
  }
}

unsigned grid_for(long n) {
  long g = (n + 255) / 256;
  return (unsigned)(g < 65536 * 16 ? g : 65536 * 16);
}

}  // namespace

hipError_t launch_prepack(const uint8_t* w1, const uint8_t* s1, const uint8_t* w3,
                          const uint8_t* s3, const uint8_t* w2, const uint8_t* s2,
                          const PackedLayout& L, uint8_t* packed, hipStream_t s) {
  const long QT = L.I / 32, QT2 = L.H / 32;
  hipLaunchKernelGGL(pack_up_weights, dim3(grid_for(L.E * QT * L.J * 256)), dim3(256), 0, s,
                     reinterpret_cast<const uint4*>(w1), reinterpret_cast<const uint4*>(w3), L,
                     reinterpret_cast<uint4*>(packed));
  hipLaunchKernelGGL(pack_up_scales, dim3(grid_for(L.E * QT * L.J * 64)), dim3(256), 0, s, s1, s3,
                     L, reinterpret_cast<uint32_t*>(packed));
  hipLaunchKernelGGL(pack_down_weights, dim3(grid_for(L.E * QT2 * L.J2 * 128)), dim3(256), 0, s,
                     reinterpret_cast<const uint4*>(w2), L, reinterpret_cast<uint4*>(packed));
  hipLaunchKernelGGL(pack_down_scales, dim3(grid_for(L.E * QT2 * L.J2 * 64)), dim3(256), 0, s, s2,
                     L, reinterpret_cast<uint16_t*>(packed));
  return hipGetLastError();
}

}  // namespace moe
