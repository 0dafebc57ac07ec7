// Router logits ahead of the top-k: logits[t, e] = sum_h x[t, h] * Wg[e, h],
// x and Wg as bf16, accumulated in fp32 by the bf16 matrix cores.  The
// review's precision policy lets the first layers of the MoE gate network run
// at low precision while the top-k compare stays fp32 (pwwt.cn review,
// section 4.1, the operator classes and the row "MoE routing top-k").
//
// v_mfma_f32_16x16x16bf16_1k: lane l supplies 4 bf16 of row l%16 (A) or
// column l%16 (B) for K slots 4*(l/16) .. +3.  The dot product does not care
// which K element sits in which slot as long as A and B agree, so each lane
// loads 8 consecutive bf16 (16 bytes) at K offset k0 + 8*(l/16) of its row and
// feeds the low 4 to one MFMA and the high 4 to a second: two MFMAs cover 32 K.
//
// A wave owns 16 tokens x 64 experts (4 output tiles, 16 fp32 per lane).  With
// more than 16 tokens the 4 waves of a workgroup take 4 token tiles of one
// 64-expert tile; with at most 16 tokens (decode) they split K instead and add
// their partial sums through LDS in wave order, so the result does not depend
// on timing.  Workgroups are laid out XCD by XCD: the expert tiles of one token
// tile run on one XCD and share its L2 copy of the x rows.
#include "common.h"

namespace moe {
namespace {

typedef short v4s __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v4s lo4(uint4 v) {
  return v4s{(short)(v.x & 0xFFFF), (short)(v.x >> 16), (short)(v.y & 0xFFFF), (short)(v.y >> 16)};
}
__device__ __forceinline__ v4s hi4(uint4 v) {
  return v4s{(short)(v.z & 0xFFFF), (short)(v.z >> 16), (short)(v.w & 0xFFFF), (short)(v.w >> 16)};
}

// One 32-K chunk of a wave: A (16 token rows) and B (4 x 16 expert rows).
struct Chunk {
  uint4 a;
  uint4 b[4];
};

__device__ __forceinline__ void load_chunk(Chunk& c, const uint16_t* __restrict__ xrow,
                                           const uint16_t* const (&wrow)[4], int k) {
  c.a = *reinterpret_cast<const uint4*>(xrow + k);
#pragma unroll
  for (int n = 0; n < 4; ++n) c.b[n] = *reinterpret_cast<const uint4*>(wrow[n] + k);
}

__device__ __forceinline__ void mma_chunk(const Chunk& c, v4f (&acc)[4]) {
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    acc[n] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(lo4(c.a), lo4(c.b[n]), acc[n], 0, 0, 0);
    acc[n] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(hi4(c.a), hi4(c.b[n]), acc[n], 0, 0, 0);
  }
}

// KW waves split K (KW = 4: one token tile per workgroup; KW = 1: 4 token tiles).
template <int KW>
__global__ __launch_bounds__(256) void router_kernel(const uint16_t* __restrict__ x,
                                                     const uint16_t* __restrict__ wg, int T, int H,
                                                     int E, float* __restrict__ logits) {
  constexpr int kMW = 4 / KW;  // token tiles per workgroup
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int NT = (T + 16 * kMW - 1) / (16 * kMW), NE = (E + 63) / 64;
  const int W = NT * NE;
  // XCD-major item order: workgroup b runs on XCD b % 8
  const int per = (W + 7) >> 3;
  const int item = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
  if ((blockIdx.x >> 3) >= (unsigned)per || item >= W) return;
  const int tt = item / NE, et = item % NE;
  const int t0 = 16 * (kMW * tt + (KW == 1 ? wave : 0));
  const int e0 = 64 * et;
  const int g = lane >> 4, r = lane & 15;
  // this lane's token row and expert rows (clamped: rows past T or E are
  // computed from the last valid row and never stored)
  const uint16_t* xrow = x + (size_t)min(t0 + r, T - 1) * H + 8 * g;
  const uint16_t* wrow[4];
#pragma unroll
  for (int n = 0; n < 4; ++n) wrow[n] = wg + (size_t)min(e0 + 16 * n + r, E - 1) * H + 8 * g;

  const int nchunk = H / 32;
  const int c0 = (KW == 1) ? 0 : (wave * nchunk) / KW;
  const int c1 = (KW == 1) ? nchunk : ((wave + 1) * nchunk) / KW;
  v4f acc[4];
#pragma unroll
  for (int n = 0; n < 4; ++n) acc[n] = v4f{0.f, 0.f, 0.f, 0.f};
  // two chunks in flight: the next chunk loads while this one multiplies
  Chunk cur, nxt;
  if (c0 < c1) load_chunk(cur, xrow, wrow, 32 * c0);
  for (int c = c0; c < c1; ++c) {
    if (c + 1 < c1) load_chunk(nxt, xrow, wrow, 32 * (c + 1));
    mma_chunk(cur, acc);
    cur = nxt;
  }

  if (KW > 1) {
    __shared__ v4f red[KW][4][64];
#pragma unroll
    for (int n = 0; n < 4; ++n) red[wave][n][lane] = acc[n];
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      v4f s = red[0][n][lane];
#pragma unroll
      for (int w = 1; w < KW; ++w) s += red[w][n][lane];
      acc[n] = s;
    }
  }
  // lane holds rows 4*(lane>>4)+v of the token tile, column lane&15 of each expert tile
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int e = e0 + 16 * n + r;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int t = t0 + 4 * g + v;
      if (t < T && e < E) logits[(size_t)t * E + e] = acc[n][v];
    }
  }
}

// The trivial routing of an always-selected expert: pair p = token p (k = 1),
// sorted order = token order, offsets {0, T}.
__global__ __launch_bounds__(256) void identity_route_kernel(int T, int32_t* __restrict__ sorted_pair,
                                                             int32_t* __restrict__ offsets) {
  const int p = blockIdx.x * 256 + threadIdx.x;
  if (p < T) sorted_pair[p] = p;
  if (p == 0) {
    offsets[0] = 0;
    offsets[1] = T;
  }
}

}  // namespace

hipError_t launch_identity_route(int T, int32_t* sorted_pair, int32_t* offsets, hipStream_t s) {
  hipLaunchKernelGGL(identity_route_kernel, dim3((unsigned)((T + 255) / 256)), dim3(256), 0, s, T,
                     sorted_pair, offsets);
  return hipGetLastError();
}

hipError_t launch_router(const uint16_t* x, const uint16_t* wg, int T, int H, int E,
                         float* logits, hipStream_t s) {
  const int kw = T <= 16 ? 4 : 1;
  const int mw = 4 / kw;
  const long W = (long)((T + 16 * mw - 1) / (16 * mw)) * ((E + 63) / 64);
  const unsigned nb = (unsigned)((W + 7) / 8 * 8);
  if (kw == 4)
    hipLaunchKernelGGL(router_kernel<4>, dim3(nb), dim3(256), 0, s, x, wg, T, H, E, logits);
  else
    hipLaunchKernelGGL(router_kernel<1>, dim3(nb), dim3(256), 0, s, x, wg, T, H, E, logits);
  return hipGetLastError();
}

}  // namespace moe
