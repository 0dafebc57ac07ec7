// Decode path of the expert GEMMs: weight streaming for small token counts.
//
// With a handful of tokens per expert the layer is bound by reading the packed
// FP4 weights from HBM once.  One workgroup owns one expert and 32 output rows
// and streams those rows' packed tiles over the whole K range, its waves
// splitting K; each wave issues 128-bit loads of whole 1 KiB tiles (a tile is
// contiguous in the packed layout, so a wave's load is one 1 KiB run) plus one
// word per lane per K-step holding the tiles' E8M0 scales.  A wave's K-steps
// are taken in batches of kB whose loads are issued back to back, so each wave
// keeps a batch of weight bytes outstanding.  The dot products run on the gfx950 scaled MFMA
// (v_mfma_scale_f32_16x16x128_f8f6f4, MXFP8 activations as A, FP4 weights as
// B, one E8M0 scale per lane and operand), which applies the block scales in
// hardware: the token rows are padded to 16, compute is far below the
// roofline here.  The waves' partial sums are added in a fixed order through
// LDS (no atomics: pwwt.cn review, section 4.2), then wave 0 runs the epilogue
// -- SwiGLU and MXFP8 requantisation of h for the gate/up kernel, the bf16
// (round to nearest even) store of O for the down kernel.
#include "common.h"

namespace moe {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));

// The FP4 B operand occupies four registers; the builtin's operand is eight
// wide, the upper half is never read for the e2m1 format.
__device__ __forceinline__ v8i widen_fp4(uint4 b) {
  const v4i v = v4i{(int)b.x, (int)b.y, (int)b.z, (int)b.w};
  return __builtin_shufflevector(v, v, 0, 1, 2, 3, -1, -1, -1, -1);
}

__device__ __forceinline__ v4f mfma_fp8_fp4(v8i a, v8i b, v4f c, int sa, int sb) {
  // cbsz = 0: A is fp8 e4m3; blgp = 4: B is fp4 e2m1; scales taken from byte 0
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 4, 0, sa, 0, sb);
}

// Registers of one K-step: NT weight tiles and their scale word, plus the A
// fragment.  A operand (fp8) of the 16x16x128 scaled MFMA: lane l holds row
// l%16 and, for g = l/16, K elements [16g, 16g+16) in a0 and [64+16g,
// 64+16g+16) in a1 (measured on gfx950 with single-hot operands).  The A
// scale of (row m, 32-block b) is taken from lane 16b + m, i.e. lane l
// supplies the scale of block l/16 of its row.
// NG row groups of 16 share each loaded weight tile (NG MFMAs per tile).
template <int NT, int NG = 1>
struct Step {
  uint4 b[NT];
  uint32_t sw;
  v4u a0[NG], a1[NG];  // native vectors: arrays of them stay in registers
  uint32_t sa[NG];
};

// Per-wave streaming state: where the wave's tiles, scales and A rows start.
template <int NT, int NG = 1>
struct Stream {
  const uint8_t* w;       // packed tiles of K-step 0, this lane's 16 bytes
  const uint8_t* s;       // scale words of K-step 0, this lane's word
  const uint8_t* a[NG];   // activation row of this lane at K-step 0 (+16 * (lane / 16)), per row group
  const uint8_t* as[NG];  // activation scale of this lane at K-step 0 (+lane / 16)
  bool valid[NG];         // the lane's row is a real pair
};

template <int NT, int NG>
__device__ __forceinline__ void load_step(Step<NT, NG>& r, const Stream<NT, NG>& st, int j) {
  const uint8_t* wj = st.w + (size_t)j * (NT * 1024);
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    // streamed once per step: a non-temporal load keeps them from displacing
    // the activation rows in the caches
    const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(wj + t * 1024));
    r.b[t] = make_uint4(v.x, v.y, v.z, v.w);
  }
  if constexpr (NT == 4)
    r.sw = *reinterpret_cast<const uint32_t*>(st.s + (size_t)j * 256);
  else
    r.sw = *reinterpret_cast<const uint16_t*>(st.s + (size_t)j * 128);
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    if (st.valid[g]) {
      r.a0[g] = *reinterpret_cast<const v4u*>(st.a[g] + (size_t)j * 128);
      r.a1[g] = *reinterpret_cast<const v4u*>(st.a[g] + (size_t)j * 128 + 64);
      r.sa[g] = st.as[g][j * 4];
    } else {
      r.a0[g] = v4u{0u, 0u, 0u, 0u};
      r.a1[g] = v4u{0u, 0u, 0u, 0u};
      r.sa[g] = 127;
    }
  }
}

// acc[g * NT + t]: row group g, tile t
template <int NT, int NG>
__device__ __forceinline__ void mma_step(const Step<NT, NG>& r, v4f* acc) {
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    v8i a;
    a[0] = (int)r.a0[g][0]; a[1] = (int)r.a0[g][1]; a[2] = (int)r.a0[g][2]; a[3] = (int)r.a0[g][3];
    a[4] = (int)r.a1[g][0]; a[5] = (int)r.a1[g][1]; a[6] = (int)r.a1[g][2]; a[7] = (int)r.a1[g][3];
#pragma unroll
    for (int t = 0; t < NT; ++t)
      acc[g * NT + t] = mfma_fp8_fp4(a, widen_fp4(r.b[t]), acc[g * NT + t], (int)r.sa[g],
                                     (int)((r.sw >> (8 * t)) & 0xFFu));
  }
}

template <int NT, int NG, int kB>
__device__ __forceinline__ void load_batch(Step<NT, NG> (&r)[kB], const Stream<NT, NG>& st, int j,
                                           int j1) {
#pragma unroll
  for (int u = 0; u < kB; ++u)
    if (j + u < j1) load_step<NT, NG>(r[u], st, j + u);
}

template <int NT, int NG, int kB>
__device__ __forceinline__ void mma_batch(const Step<NT, NG> (&r)[kB], v4f* acc, int j, int j1) {
#pragma unroll
  for (int u = 0; u < kB; ++u)
    if (j + u < j1) mma_step<NT, NG>(r[u], acc);
}

// Multiply-accumulate K-steps [j0, j1) of one wave into acc, kB steps' loads
// issued back to back before their MFMAs.
template <int NT, int NG, int kB>
__device__ __forceinline__ void stream_k(const Stream<NT, NG>& st, int j0, int j1, v4f* acc) {
  for (int j = j0; j < j1; j += kB) {
    Step<NT, NG> r[kB];
    load_batch<NT, NG, kB>(r, st, j, j1);
    mma_batch<NT, NG, kB>(r, acc, j, j1);
  }
}

// Waves per workgroup and K-steps per load batch (one row group per pass;
// halved, rounded up, with two): measured over 2-8 waves and batches of 2-8.
constexpr int kUpNW = 4;
constexpr int kUpB = 4;
constexpr int kDnNW = 2;
constexpr int kDnB = 6;

// NG row groups of 16 per pass over the weights: NG = 1 for a handful of rows
// per expert, NG = 2 when the expected rows per expert fill more than one
// group (each weight tile then serves two MFMAs instead of being re-read).
template <int NG>
__global__ __launch_bounds__(kUpNW * 64) void up_decode_kernel(
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
  const int j0 = (wave * J) / kUpNW, j1 = ((wave + 1) * J) / kUpNW;
  __shared__ v4f red[kUpNW][NG * 4][64];

  for (int m0 = seg0; m0 < seg1; m0 += 16 * NG) {
    Stream<4, NG> st;
    st.w = packed + L.upw_block(e, q, 0) + lane * 16;
    st.s = packed + L.ups_block(e, q, 0) + lane * 4;
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const int row = m0 + 16 * g + (lane & 15);
      st.valid[g] = row < seg1;
      const int tok = st.valid[g] ? sorted_pair[row] / k : 0;
      st.a[g] = xq + (size_t)tok * H + (lane >> 4) * 16;
      st.as[g] = xs + (size_t)tok * (H / 32) + (lane >> 4);
    }
    v4f acc[NG * 4];
#pragma unroll
    for (int t = 0; t < NG * 4; ++t) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};
    // two row groups double the activation registers of a K-step: half the
    // K-steps per batch keeps the kernel within its registers
    stream_k<4, NG, NG == 2 ? (kUpB + 1) / 2 : kUpB>(st, j0, j1, acc);
#pragma unroll
    for (int t = 0; t < NG * 4; ++t) red[wave][t][lane] = acc[t];
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        v4f s[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          s[t] = red[0][g * 4 + t][lane];
#pragma unroll
          for (int w = 1; w < kUpNW; ++w) s[t] += red[w][g * 4 + t][lane];
        }
        // lane holds rows 4*(lane>>4)+v of the group, column lane&15 of each
        // 16-row tile: tiles 0/1 are G for i = 32q + c and 32q + 16 + c,
        // tiles 2/3 the matching U.
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float h0 = silu_mul(s[0][v], s[2][v]);
          const float h1 = silu_mul(s[1][v], s[3][v]);
          const float am = row16_max(fmaxf(fabsf(h0), fabsf(h1)));
          float mul;
          const uint32_t sc = mx_scale_from_amax(am, &mul);
          const int r = m0 + 16 * g + 4 * (lane >> 4) + v;
          if (r < seg1) {
            uint8_t* hrow = hq + (size_t)r * I + q * 32 + (lane & 15);
            const uint32_t c2 = f32x2_to_e4m3(h0 * mul, h1 * mul);
            hrow[0] = (uint8_t)c2;
            hrow[16] = (uint8_t)(c2 >> 8);
            if ((lane & 15) == 0) hs[(size_t)r * (I / 32) + q] = (uint8_t)sc;
          }
        }
      }
    }
    __syncthreads();
  }
}

template <int NG>
__global__ __launch_bounds__(kDnNW * 64) void down_decode_kernel(
    const uint8_t* __restrict__ packed, PackedLayout L, const uint8_t* __restrict__ hq,
    const uint8_t* __restrict__ hs, const int32_t* __restrict__ offsets, uint16_t* __restrict__ O) {
  const int QT2 = L.H / 32;
  const int e = blockIdx.x / QT2, q2 = blockIdx.x % QT2;
  const int seg0 = offsets[e], seg1 = offsets[e + 1];
  if (seg0 >= seg1) return;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int H = L.H, I = L.I, J2 = L.J2;
  const int j0 = (wave * J2) / kDnNW, j1 = ((wave + 1) * J2) / kDnNW;
  __shared__ v4f red[kDnNW][NG * 2][64];

  for (int m0 = seg0; m0 < seg1; m0 += 16 * NG) {
    Stream<2, NG> st;
    st.w = packed + L.dnw_block(e, q2, 0) + lane * 16;
    st.s = packed + L.dns_block(e, q2, 0) + lane * 2;
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const int row = m0 + 16 * g + (lane & 15);
      st.valid[g] = row < seg1;
      const int rr = st.valid[g] ? row : 0;
      st.a[g] = hq + (size_t)rr * I + (lane >> 4) * 16;
      st.as[g] = hs + (size_t)rr * (I / 32) + (lane >> 4);
    }
    v4f acc[NG * 2];
#pragma unroll
    for (int t = 0; t < NG * 2; ++t) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};
    stream_k<2, NG, NG == 2 ? (kDnB + 1) / 2 : kDnB>(st, j0, j1, acc);
#pragma unroll
    for (int t = 0; t < NG * 2; ++t) red[wave][t][lane] = acc[t];
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int g = 0; g < NG; ++g)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          v4f s = red[0][g * 2 + t][lane];
#pragma unroll
          for (int w = 1; w < kDnNW; ++w) s += red[w][g * 2 + t][lane];
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int r = m0 + 16 * g + 4 * (lane >> 4) + v;
            if (r < seg1) O[(size_t)r * H + q2 * 32 + t * 16 + (lane & 15)] = f32_to_bf16(s[v]);
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
                            int row_groups, hipStream_t s) {
  const unsigned grid = (unsigned)L.E * (unsigned)(L.I / 32);
  if (row_groups == 2)
    hipLaunchKernelGGL(up_decode_kernel<2>, dim3(grid), dim3(kUpNW * 64), 0, s, packed, L, xq, xs,
                       offsets, sorted_pair, k, hq, hs);
  else
    hipLaunchKernelGGL(up_decode_kernel<1>, dim3(grid), dim3(kUpNW * 64), 0, s, packed, L, xq, xs,
                       offsets, sorted_pair, k, hq, hs);
  return hipGetLastError();
}

hipError_t launch_down_decode(const uint8_t* packed, const PackedLayout& L, const uint8_t* hq,
                              const uint8_t* hs, const int32_t* offsets, uint16_t* O,
                              int row_groups, hipStream_t s) {
  const unsigned grid = (unsigned)L.E * (unsigned)(L.H / 32);
  if (row_groups == 2)
    hipLaunchKernelGGL(down_decode_kernel<2>, dim3(grid), dim3(kDnNW * 64), 0, s, packed, L, hq, hs,
                       offsets, O);
  else
    hipLaunchKernelGGL(down_decode_kernel<1>, dim3(grid), dim3(kDnNW * 64), 0, s, packed, L, hq, hs,
                       offsets, O);
  return hipGetLastError();
}

}  // namespace moe
