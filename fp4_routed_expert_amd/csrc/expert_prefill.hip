// Prefill path of the expert GEMMs: many tokens per expert, MFMA bound.
//
// The pages' prefill work on gfx90a used MFMA kernels with better reuse of the
// packed weights and retuned expert sorting ("DeepSeek-V4-Flash on AMD gfx90a:
// Correctness Recovery and Inference Performance Engineering", abstract); here
// the same reuse is a grouped GEMM on the gfx950 scaled MFMA
// (v_mfma_scale_f32_16x16x128_f8f6f4: MXFP8 activations x FP4 weights, the E8M0
// block scales applied by the instruction).
//
// Work list: a small kernel turns the expert offsets into a list of token tiles
// (expert, first sorted row) of up to kBM rows, on the device, so the grid can
// be sized from host-known bounds only (sum_e ceil(n_e/kBM) <= ceil(P/kBM) + E)
// and no count is ever read back to the host.  Workgroups past the tile count
// exit.  Each workgroup owns one token tile and one feature tile; the blockIdx
// -> work mapping is XCD aware: the dispatcher deals workgroups round-robin to
// the 8 XCDs, so consecutive work items (the feature tiles of one token tile,
// which share its activation rows) are placed on the same XCD and its L2.
//
// K loop: one K-step = 128 elements.  Per step the workgroup copies the
// gathered activation rows (kBM x 128 B, row stride padded to 144 B so that
// each group of 8 lanes of a 128-bit LDS read covers all banks) and the
// feature tile's packed weight tiles (16 KiB) global -> registers -> LDS,
// double-buffered so the next step's loads are in flight during this step's
// MFMAs.  4 waves in a 2x2 grid: each wave owns the interleaved 16-row
// sub-tiles {wm, wm+2, wm+4, wm+6} and half of the feature tile, and skips
// sub-tiles past the expert's last row (a tile of 16 rows costs 1/8 of a full
// one in MFMA issue).
#include "common.h"

namespace moe {
namespace {

constexpr int kBM = 128;                 // token rows per tile
constexpr int kAStride = 144;            // LDS bytes per activation row
constexpr int kABytes = kBM * kAStride;  // 18 KiB
constexpr int kBBytes = 16384;           // 16 weight tiles of 1 KiB per K-step
constexpr int kTileHdr = 256;            // tile count at offset 0, list at 256

__device__ __forceinline__ v8i load_a_lds(const uint8_t* p) {
  // same lane layout as the global loads of the decode path: bytes 0-15 hold
  // K [16g, 16g+16), bytes 16-31 hold K [64+16g, +16), g = lane/16
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
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 4, 0, sa, 0, sb);
}

// Workgroup b is dispatched to XCD b % 8; give each XCD a contiguous range of
// work items.  nb is a multiple of 8.
__device__ __forceinline__ int xcd_remap(int b, int nb) { return (b & 7) * (nb >> 3) + (b >> 3); }

__global__ __launch_bounds__(256) void build_tiles_kernel(const int32_t* __restrict__ offsets,
                                                          int E, int* __restrict__ hdr) {
  __shared__ int cnt[1024];
  __shared__ int wave_tot[4];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += 256) cnt[e] = (offsets[e + 1] - offsets[e] + kBM - 1) / kBM;
  __syncthreads();
  const int total = block_exclusive_scan256(cnt, E, wave_tot);
  int2* tiles = reinterpret_cast<int2*>(reinterpret_cast<uint8_t*>(hdr) + kTileHdr);
  for (int e = tid; e < E; e += 256) {
    const int o0 = offsets[e], n = (offsets[e + 1] - o0 + kBM - 1) / kBM;
    for (int i = 0; i < n; ++i) tiles[cnt[e] + i] = make_int2(e, o0 + i * kBM);
  }
  if (tid == 0) hdr[0] = total;
}

__global__ __launch_bounds__(256) void up_prefill_kernel(
    const uint8_t* __restrict__ packed, PackedLayout L, const uint8_t* __restrict__ xq,
    const uint8_t* __restrict__ xs, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ sorted_pair, int k, const int* __restrict__ hdr, int NF,
    int nblocks, uint8_t* __restrict__ hq, uint8_t* __restrict__ hs) {
  __shared__ __align__(16) uint8_t As[2][kABytes];
  __shared__ __align__(16) uint8_t Bs[2][kBBytes];
  __shared__ uint32_t Ss[2][kBM];  // activation scales of the K-step, 4 blocks per row
  __shared__ int tok_s[kBM];
  const int logical = xcd_remap(blockIdx.x, nblocks);
  const int tile = logical / NF, ft = logical % NF;
  if (tile >= hdr[0]) return;
  const int2 td = reinterpret_cast<const int2*>(reinterpret_cast<const uint8_t*>(hdr) + kTileHdr)[tile];
  const int e = td.x, m0 = td.y;
  const int rows = min(kBM, offsets[e + 1] - m0);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave & 1, wn = wave >> 1;
  const int H = L.H, I = L.I, J = L.J;
  for (int r = tid; r < kBM; r += 256) tok_s[r] = (r < rows) ? sorted_pair[m0 + r] / k : -1;
  __syncthreads();

  // copy assignment: activation chunk u of this thread = row (tid>>3) + 32u,
  // 16-byte column tid&7; weight chunk u = 4 KiB block of q-group 4ft+u, offset tid*16
  const uint8_t* asrc[4];
  bool aval[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int tok = tok_s[(tid >> 3) + 32 * u];
    aval[u] = tok >= 0;
    asrc[u] = xq + (size_t)(aval[u] ? tok : 0) * H + (tid & 7) * 16;
  }
  const uint8_t* bsrc[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) bsrc[u] = packed + L.upw_block(e, 4 * ft + u, 0) + tid * 16;
  const int stok = (tid < kBM) ? tok_s[tid] : -1;
  const uint32_t* ssrc = reinterpret_cast<const uint32_t*>(xs + (size_t)(stok >= 0 ? stok : 0) * (H / 32));

  uint4 ra[4], rb[4];
  uint32_t rs = 0;
  auto gload = [&](int j) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
      ra[u] = aval[u] ? *reinterpret_cast<const uint4*>(asrc[u] + (size_t)j * 128) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int u = 0; u < 4; ++u) rb[u] = *reinterpret_cast<const uint4*>(bsrc[u] + (size_t)j * 4096);
    if (tid < kBM) rs = (stok >= 0) ? ssrc[j] : 0x7F7F7F7Fu;
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
      *reinterpret_cast<uint4*>(&As[buf][((tid >> 3) + 32 * u) * kAStride + (tid & 7) * 16]) = ra[u];
#pragma unroll
    for (int u = 0; u < 4; ++u) *reinterpret_cast<uint4*>(&Bs[buf][u * 4096 + tid * 16]) = rb[u];
    if (tid < kBM) Ss[buf][tid] = rs;
  };

  int nact = 0;  // active sub-tiles of this wave form a prefix of i = 0..3
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (16 * (wm + 2 * i) < rows) nact = i + 1;
  // weight scales: one dword per lane per K-step for each of the wave's 2 q-groups
  const uint32_t* sbp[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
    sbp[qb] = reinterpret_cast<const uint32_t*>(packed + L.ups_block(e, 4 * ft + 2 * wn + qb, 0)) + lane;

  v4f acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[i][t] = v4f{0.f, 0.f, 0.f, 0.f};

  gload(0);
  lstore(0);
  __syncthreads();
  for (int j = 0; j < J; ++j) {
    const int buf = j & 1;
    if (j + 1 < J) gload(j + 1);
    uint32_t sbq[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) sbq[qb] = sbp[qb][(size_t)j * 64];
    v8i bf[8];
#pragma unroll
    for (int t = 0; t < 8; ++t)
      bf[t] = widen_fp4(*reinterpret_cast<const uint4*>(
          &Bs[buf][(2 * wn + (t >> 2)) * 4096 + (t & 3) * 1024 + lane * 16]));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i < nact) {
        const int row = 16 * (wm + 2 * i) + (lane & 15);
        const v8i a = load_a_lds(&As[buf][row * kAStride + (lane >> 4) * 16]);
        const int sa = (int)((Ss[buf][row] >> (8 * (lane >> 4))) & 0xFFu);
#pragma unroll
        for (int t = 0; t < 8; ++t)
          acc[i][t] = mfma_fp8_fp4(a, bf[t], acc[i][t], sa, (int)((sbq[t >> 2] >> (8 * (t & 3))) & 0xFFu));
      }
    }
    if (j + 1 < J) lstore(buf ^ 1);
    __syncthreads();
  }

  // epilogue: tiles t = 4*qb + {0: G rows 0-15, 1: G rows 16-31, 2: U 0-15, 3: U 16-31}
  // of q-group 4ft + 2wn + qb; lane holds rows 4*(lane>>4)+v, column lane&15.
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (i < nact) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const int q = 4 * ft + 2 * wn + qb;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float h0 = silu_mul(acc[i][4 * qb + 0][v], acc[i][4 * qb + 2][v]);
          const float h1 = silu_mul(acc[i][4 * qb + 1][v], acc[i][4 * qb + 3][v]);
          float am = fmaxf(fabsf(h0), fabsf(h1));
#pragma unroll
          for (int m = 1; m < 16; m <<= 1) am = fmaxf(am, __shfl_xor(am, m, 64));
          float mul;
          const uint32_t sc = mx_scale_from_amax(am, &mul);
          const int r = 16 * (wm + 2 * i) + 4 * (lane >> 4) + v;
          if (r < rows) {
            uint8_t* hrow = hq + (size_t)(m0 + r) * I + q * 32 + (lane & 15);
            hrow[0] = (uint8_t)f32_to_e4m3(h0 * mul);
            hrow[16] = (uint8_t)f32_to_e4m3(h1 * mul);
            if ((lane & 15) == 0) hs[(size_t)(m0 + r) * (I / 32) + q] = (uint8_t)sc;
          }
        }
      }
    }
  }
}

__global__ __launch_bounds__(256) void down_prefill_kernel(
    const uint8_t* __restrict__ packed, PackedLayout L, const uint8_t* __restrict__ hq,
    const uint8_t* __restrict__ hs, const int32_t* __restrict__ offsets,
    const int* __restrict__ hdr, int NF, int nblocks, float* __restrict__ O) {
  __shared__ __align__(16) uint8_t As[2][kABytes];
  __shared__ __align__(16) uint8_t Bs[2][kBBytes];
  __shared__ uint32_t Ss[2][kBM];
  const int logical = xcd_remap(blockIdx.x, nblocks);
  const int tile = logical / NF, ft = logical % NF;
  if (tile >= hdr[0]) return;
  const int2 td = reinterpret_cast<const int2*>(reinterpret_cast<const uint8_t*>(hdr) + kTileHdr)[tile];
  const int e = td.x, m0 = td.y;
  const int rows = min(kBM, offsets[e + 1] - m0);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave & 1, wn = wave >> 1;
  const int H = L.H, I = L.I, J2 = L.J2;
  const int QG = H / 32;  // 32-row groups of the down weights

  // activation rows are the expert's sorted rows m0.. (already contiguous)
  const uint8_t* asrc[4];
  bool aval[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int r = (tid >> 3) + 32 * u;
    aval[u] = r < rows;
    asrc[u] = hq + (size_t)(m0 + (aval[u] ? r : 0)) * I + (tid & 7) * 16;
  }
  // weight chunk u: q2-group 8ft + 2u + (tid>>7), offset (tid & 127) * 16 in its 2 KiB block
  const uint8_t* bsrc[4];
  bool bval[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int g = 8 * ft + 2 * u + (tid >> 7);
    bval[u] = g < QG;
    bsrc[u] = packed + L.dnw_block(e, bval[u] ? g : 0, 0) + (tid & 127) * 16;
  }
  const bool sval = tid < rows;
  const uint32_t* ssrc = reinterpret_cast<const uint32_t*>(hs + (size_t)(m0 + (sval ? tid : 0)) * (I / 32));

  uint4 ra[4], rb[4];
  uint32_t rs = 0;
  auto gload = [&](int j) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
      ra[u] = aval[u] ? *reinterpret_cast<const uint4*>(asrc[u] + (size_t)j * 128) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      rb[u] = bval[u] ? *reinterpret_cast<const uint4*>(bsrc[u] + (size_t)j * 2048) : make_uint4(0, 0, 0, 0);
    if (tid < kBM) rs = sval ? ssrc[j] : 0x7F7F7F7Fu;
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
      *reinterpret_cast<uint4*>(&As[buf][((tid >> 3) + 32 * u) * kAStride + (tid & 7) * 16]) = ra[u];
#pragma unroll
    for (int u = 0; u < 4; ++u) *reinterpret_cast<uint4*>(&Bs[buf][u * 4096 + tid * 16]) = rb[u];
    if (tid < kBM) Ss[buf][tid] = rs;
  };

  int nact = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (16 * (wm + 2 * i) < rows) nact = i + 1;
  // this wave's weight tiles: q2-groups 8ft + 4wn + qb (qb 0..3), 2 tiles each: t = 2qb + tt
  const uint16_t* sbp[4];
  bool gval[4];
#pragma unroll
  for (int qb = 0; qb < 4; ++qb) {
    const int g = 8 * ft + 4 * wn + qb;
    gval[qb] = g < QG;
    sbp[qb] = reinterpret_cast<const uint16_t*>(packed + L.dns_block(e, gval[qb] ? g : 0, 0)) + lane;
  }

  v4f acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[i][t] = v4f{0.f, 0.f, 0.f, 0.f};

  gload(0);
  lstore(0);
  __syncthreads();
  for (int j = 0; j < J2; ++j) {
    const int buf = j & 1;
    if (j + 1 < J2) gload(j + 1);
    uint32_t sbq[4];
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) sbq[qb] = sbp[qb][(size_t)j * 64];
    v8i bf[8];
#pragma unroll
    for (int t = 0; t < 8; ++t)
      bf[t] = widen_fp4(*reinterpret_cast<const uint4*>(
          &Bs[buf][(4 * wn + (t >> 1)) * 2048 + (t & 1) * 1024 + lane * 16]));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i < nact) {
        const int row = 16 * (wm + 2 * i) + (lane & 15);
        const v8i a = load_a_lds(&As[buf][row * kAStride + (lane >> 4) * 16]);
        const int sa = (int)((Ss[buf][row] >> (8 * (lane >> 4))) & 0xFFu);
#pragma unroll
        for (int t = 0; t < 8; ++t)
          acc[i][t] = mfma_fp8_fp4(a, bf[t], acc[i][t], sa, (int)((sbq[t >> 1] >> (8 * (t & 1))) & 0xFFu));
      }
    }
    if (j + 1 < J2) lstore(buf ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (i < nact) {
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        if (!gval[t >> 1]) continue;
        const int col = (8 * ft + 4 * wn + (t >> 1)) * 32 + (t & 1) * 16 + (lane & 15);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int r = 16 * (wm + 2 * i) + 4 * (lane >> 4) + v;
          if (r < rows) O[(size_t)(m0 + r) * H + col] = acc[i][t][v];
        }
      }
    }
  }
}

long max_tiles(long P, int E) { return (P + kBM - 1) / kBM + E; }

}  // namespace

size_t prefill_tile_bytes(long P, int E) { return kTileHdr + (size_t)max_tiles(P, E) * 8; }

hipError_t launch_up_prefill(const uint8_t* packed, const PackedLayout& L, const uint8_t* xq,
                             const uint8_t* xs, const int32_t* offsets,
                             const int32_t* sorted_pair, int T, int k, uint8_t* hq, uint8_t* hs,
                             void* tile_ws, hipStream_t s) {
  int* hdr = static_cast<int*>(tile_ws);
  hipLaunchKernelGGL(build_tiles_kernel, dim3(1), dim3(256), 0, s, offsets, L.E, hdr);
  const int NF = L.I / 128;
  const long nb = (max_tiles((long)T * k, L.E) * NF + 7) / 8 * 8;
  hipLaunchKernelGGL(up_prefill_kernel, dim3((unsigned)nb), dim3(256), 0, s, packed, L, xq, xs,
                     offsets, sorted_pair, k, hdr, NF, (int)nb, hq, hs);
  return hipGetLastError();
}

hipError_t launch_down_prefill(const uint8_t* packed, const PackedLayout& L, const uint8_t* hq,
                               const uint8_t* hs, const int32_t* offsets, int T, int k, float* O,
                               void* tile_ws, hipStream_t s) {
  int* hdr = static_cast<int*>(tile_ws);
  hipLaunchKernelGGL(build_tiles_kernel, dim3(1), dim3(256), 0, s, offsets, L.E, hdr);
  const int NF = (L.H + 255) / 256;
  const long nb = (max_tiles((long)T * k, L.E) * NF + 7) / 8 * 8;
  hipLaunchKernelGGL(down_prefill_kernel, dim3((unsigned)nb), dim3(256), 0, s, packed, L, hq, hs,
                     offsets, hdr, NF, (int)nb, O);
  return hipGetLastError();
}

}  // namespace moe
