// Decode path of the expert GEMMs: weight streaming for small token counts.
//
// With a handful of tokens per expert the layer is bound by reading the packed
// FP4 weights from HBM once.  One workgroup owns one expert and 32 output rows
// and streams those rows' packed tiles over the whole K range, its four waves
// splitting K; each wave issues 128-bit loads of whole 1 KiB tiles (a tile is
// contiguous in the packed layout, so a wave's load is one 1 KiB run) plus one
// dword per lane per K-step holding the four tiles' E8M0 scales.  Each wave
// issues the loads of kBatch K-steps back to back before using them, so that
// enough bytes are in flight per CU to cover HBM latency.  The dot products run on
// the gfx950 scaled MFMA (v_mfma_scale_f32_16x16x128_f8f6f4, MXFP8 activations
// as A, FP4 weights as B, one E8M0 scale per lane and operand), which applies
// the block scales in hardware: the token rows are padded to 16, compute is far
// below the roofline here.  The four waves' partial sums are added in a fixed
// order through LDS (no atomics: pwwt.cn review, section 4.2), then wave 0
// runs the epilogue -- SwiGLU and MXFP8 requantisation of h for the gate/up
// kernel, the fp32 store of O for the down kernel.
#include "common.h"

namespace moe {
namespace {

constexpr int kNW = 4;     // waves per workgroup, splitting K
constexpr int kBatch = 4;  // K-steps whose loads a wave issues together

// A operand (fp8) of the 16x16x128 scaled MFMA: lane l holds row l%16 and, for
// g = l/16, K elements [16g, 16g+16) in bytes 0-15 and [64+16g, 64+16g+16) in
// bytes 16-31 (measured on gfx950 with single-hot operands).  The A scale of
// (row m, 32-block b) is taken from lane 16b + m, i.e. lane l supplies the
// scale of block l/16 of its row.  `p` points at row + 16*(l/16).
__device__ __forceinline__ v8i load_a_fp8(const uint8_t* p) {
  const uint4 a0 = *reinterpret_cast<const uint4*>(p);
  const uint4 a1 = *reinterpret_cast<const uint4*>(p + 64);
  v8i r;
  r[0] = (int)a0.x; r[1] = (int)a0.y; r[2] = (int)a0.z; r[3] = (int)a0.w;
  r[4] = (int)a1.x; r[5] = (int)a1.y; r[6] = (int)a1.z; r[7] = (int)a1.w;
  return r;
}

__device__ __forceinline__ v8i widen_fp4(uint4 b) {
  v8i r;
  r[0] = (int)b.x; r[1] = (int)b.y; r[2] = (int)b.z; r[3] = (int)b.w;
  r[4] = 0; r[5] = 0; r[6] = 0; r[7] = 0;
  return r;
}

__device__ __forceinline__ v4f mfma_fp8_fp4(v8i a, v8i b, v4f c, int sa, int sb) {
  // cbsz = 0: A is fp8 e4m3; blgp = 4: B is fp4 e2m1; scales taken from byte 0
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 4, 0, sa, 0, sb);
}

__global__ __launch_bounds__(kNW * 64) void up_decode_kernel(
    const uint8_t* __restrict__ packed, PackedLayout L, const uint8_t* __restrict__ xq,
    const uint8_t* __restrict__ xs, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ sorted_pair, int k, uint8_t* __restrict__ hq,
    uint8_t* __restrict__ hs) {
  const int QT = L.I / 32;
  const int e = blockIdx.x / QT, q = blockIdx.x % QT;
  const int seg0 = offsets[e], seg1 = offsets[e + 1];
  if (seg0 >= seg1) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int H = L.H, I = L.I, J = L.J;
  const int j0 = (wave * J) / kNW, j1 = ((wave + 1) * J) / kNW;
  const uint8_t* wblk = packed + L.upw_block(e, q, 0) + lane * 16;
  const uint32_t* sblk = reinterpret_cast<const uint32_t*>(packed + L.ups_block(e, q, 0)) + lane;
  __shared__ v4f red[kNW][4][64];

  for (int m0 = seg0; m0 < seg1; m0 += 16) {
    const int row = m0 + (lane & 15);
    const bool valid = row < seg1;
    const int tok = valid ? sorted_pair[row] / k : 0;
    const uint8_t* arow = xq + (size_t)tok * H + (lane >> 4) * 16;
    const uint8_t* srow = xs + (size_t)tok * (H / 32) + (lane >> 4);
    v4f acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};
    for (int j = j0; j < j1; j += kBatch) {
      uint4 b[kBatch][4];
      uint32_t sw[kBatch];
      v8i a[kBatch];
      int sa[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        if (j + u < j1) {
          const uint8_t* wj = wblk + (size_t)(j + u) * 4096;
#pragma unroll
          for (int t = 0; t < 4; ++t) b[u][t] = *reinterpret_cast<const uint4*>(wj + t * 1024);
          sw[u] = sblk[(size_t)(j + u) * 64];
        }
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        if (j + u < j1) {
          a[u] = valid ? load_a_fp8(arow + (size_t)(j + u) * 128) : v8i{0, 0, 0, 0, 0, 0, 0, 0};
          sa[u] = valid ? (int)srow[(j + u) * 4] : 127;
        }
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        if (j + u < j1) {
#pragma unroll
          for (int t = 0; t < 4; ++t)
            acc[t] = mfma_fp8_fp4(a[u], widen_fp4(b[u][t]), acc[t], sa[u],
                                  (int)((sw[u] >> (8 * t)) & 0xFFu));
        }
      }
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) red[wave][t][lane] = acc[t];
    __syncthreads();
    if (wave == 0) {
      v4f s[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        s[t] = red[0][t][lane];
#pragma unroll
        for (int w = 1; w < kNW; ++w) s[t] += red[w][t][lane];
      }
      // lane holds rows 4*(lane>>4)+v of the tile, column lane&15 of each
      // 16-row group: tiles 0/1 are G for i = 32q + c and 32q + 16 + c,
      // tiles 2/3 the matching U.
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float h0 = silu_mul(s[0][v], s[2][v]);
        const float h1 = silu_mul(s[1][v], s[3][v]);
        float am = fmaxf(fabsf(h0), fabsf(h1));
#pragma unroll
        for (int m = 1; m < 16; m <<= 1) am = fmaxf(am, __shfl_xor(am, m, 64));
        float mul;
        const uint32_t sc = mx_scale_from_amax(am, &mul);
        const int r = m0 + 4 * (lane >> 4) + v;
        if (r < seg1) {
          uint8_t* hrow = hq + (size_t)r * I + q * 32 + (lane & 15);
          hrow[0] = (uint8_t)f32_to_e4m3(h0 * mul);
          hrow[16] = (uint8_t)f32_to_e4m3(h1 * mul);
          if ((lane & 15) == 0) hs[(size_t)r * (I / 32) + q] = (uint8_t)sc;
        }
      }
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(kNW * 64) void down_decode_kernel(
    const uint8_t* __restrict__ packed, PackedLayout L, const uint8_t* __restrict__ hq,
    const uint8_t* __restrict__ hs, const int32_t* __restrict__ offsets, float* __restrict__ O) {
  const int QT2 = L.H / 32;
  const int e = blockIdx.x / QT2, q2 = blockIdx.x % QT2;
  const int seg0 = offsets[e], seg1 = offsets[e + 1];
  if (seg0 >= seg1) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int H = L.H, I = L.I, J2 = L.J2;
  const int j0 = (wave * J2) / kNW, j1 = ((wave + 1) * J2) / kNW;
  const uint8_t* wblk = packed + L.dnw_block(e, q2, 0) + lane * 16;
  const uint16_t* sblk = reinterpret_cast<const uint16_t*>(packed + L.dns_block(e, q2, 0)) + lane;
  __shared__ v4f red[kNW][2][64];

  for (int m0 = seg0; m0 < seg1; m0 += 16) {
    const int row = m0 + (lane & 15);
    const bool valid = row < seg1;
    const uint8_t* arow = hq + (size_t)(valid ? row : 0) * I + (lane >> 4) * 16;
    const uint8_t* srow = hs + (size_t)(valid ? row : 0) * (I / 32) + (lane >> 4);
    v4f acc[2] = {v4f{0.f, 0.f, 0.f, 0.f}, v4f{0.f, 0.f, 0.f, 0.f}};
    for (int j = j0; j < j1; j += kBatch) {
      uint4 b[kBatch][2];
      uint32_t sw[kBatch];
      v8i a[kBatch];
      int sa[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        if (j + u < j1) {
          const uint8_t* wj = wblk + (size_t)(j + u) * 2048;
#pragma unroll
          for (int t = 0; t < 2; ++t) b[u][t] = *reinterpret_cast<const uint4*>(wj + t * 1024);
          sw[u] = sblk[(size_t)(j + u) * 64];
        }
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        if (j + u < j1) {
          a[u] = valid ? load_a_fp8(arow + (size_t)(j + u) * 128) : v8i{0, 0, 0, 0, 0, 0, 0, 0};
          sa[u] = valid ? (int)srow[(j + u) * 4] : 127;
        }
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        if (j + u < j1) {
#pragma unroll
          for (int t = 0; t < 2; ++t)
            acc[t] = mfma_fp8_fp4(a[u], widen_fp4(b[u][t]), acc[t], sa[u],
                                  (int)((sw[u] >> (8 * t)) & 0xFFu));
        }
      }
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) red[wave][t][lane] = acc[t];
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        v4f s = red[0][t][lane];
#pragma unroll
        for (int w = 1; w < kNW; ++w) s += red[w][t][lane];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int r = m0 + 4 * (lane >> 4) + v;
          if (r < seg1) O[(size_t)r * H + q2 * 32 + t * 16 + (lane & 15)] = s[v];
        }
      }
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_up_decode(const uint8_t* packed, const PackedLayout& L, const uint8_t* xq,
                            const uint8_t* xs, const int32_t* offsets,
                            const int32_t* sorted_pair, int k, uint8_t* hq, uint8_t* hs,
                            hipStream_t s) {
  const unsigned grid = (unsigned)L.E * (unsigned)(L.I / 32);
  hipLaunchKernelGGL(up_decode_kernel, dim3(grid), dim3(kNW * 64), 0, s, packed, L, xq, xs,
                     offsets, sorted_pair, k, hq, hs);
  return hipGetLastError();
}

hipError_t launch_down_decode(const uint8_t* packed, const PackedLayout& L, const uint8_t* hq,
                              const uint8_t* hs, const int32_t* offsets, float* O,
                              hipStream_t s) {
  const unsigned grid = (unsigned)L.E * (unsigned)(L.H / 32);
  hipLaunchKernelGGL(down_decode_kernel, dim3(grid), dim3(kNW * 64), 0, s, packed, L, hq, hs,
                     offsets, O);
  return hipGetLastError();
}

}  // namespace moe
