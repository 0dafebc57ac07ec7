// Prefill path of the expert GEMMs: many tokens per expert, MFMA bound.
//
// The pages' prefill work on gfx90a used MFMA kernels with better reuse of the
// packed weights and retuned expert sorting ("DeepSeek-V4-Flash on AMD gfx90a:
// Correctness Recovery and Inference Performance Engineering", abstract); here
// the same reuse is a grouped GEMM on the gfx950 scaled MFMA
// (v_mfma_scale_f32_16x16x128_f8f6f4: MXFP8 activations x FP4 weights, the E8M0
// block scales applied by the instruction, FP8 issue rate).
//
// Work list: a small kernel turns the expert offsets into a list of token tiles
// (expert, first sorted row) of up to kBM rows, on the device, so the grid is
// sized from host-known bounds only (sum_e ceil(n_e/kBM) <= ceil(P/kBM) + E)
// and no count is ever read back to the host; workgroups past the tile count
// exit.  kBM = 192 covers a whole expert at the prefill shape (113-180 rows
// per expert), so each expert's packed weights stream from HBM once per
// feature tile; 16-row sub-tiles past the expert's last row are skipped, so a short
// tile costs MFMA issue in proportion to its real rows.
//
// Each workgroup (8 waves, two per SIMD) owns one token tile and one feature
// tile.  The blockIdx -> work mapping is XCD aware: the dispatcher deals
// workgroups round-robin to the 8 XCDs; each XCD gets an equal contiguous
// share of the work items that exist, so neighbouring items (the feature tiles
// of one token tile, which share its activation rows) sit on the same XCD and
// its L2, and no XCD idles when the real tile count is below the grid bound.
//
// K loop (one K-step = 128 elements): the activation rows (kBM x 128 B, stored
// with the 16-byte chunk index XOR-ed with the row's low 3 bits so that the
// 128-bit LDS reads and writes of 8 lanes cover all banks), the feature tile's
// packed weight tiles (16 KiB) and both operands' E8M0 scales travel global ->
// registers -> LDS, double-buffered: step j's global loads for stage j+1 are
// in flight during step j's MFMAs, then land in the other LDS buffer; one
// barrier per K-step.  Every access is visible to the compiler, which
// schedules the LDS reads among the MFMAs and waits on each load precisely.
//
// Waves form a 2 (tokens) x 4 (features) grid: each wave owns the 16-row
// sub-tiles {wm, wm+2, ..., wm+10} and 4 weight tiles (32 MFMAs per K-step
// when all its sub-tiles are live); for the gate/up GEMM a wave's 4 tiles are
// one 32-feature group of W1 and W3, so SwiGLU stays in its registers.  The number of live
// sub-tiles is a compile-time parameter of the loop body, selected once per
// wave, so the MFMA stream has no conditionals and only live accumulators are
// allocated.
#include "common.h"

namespace moe {
namespace {

constexpr int kBM = 192;                 // token rows per tile (12 sub-tiles of 16)
constexpr int kThreads = 512;            // 8 waves
constexpr int kABytes = kBM * 128;       // activation rows of one K-step
constexpr int kBBytes = 16384;           // 16 weight tiles of 1 KiB
constexpr int kTileHdr = 256;            // tile count at offset 0, list at 256

struct Stage {
  uint8_t a[kABytes];
  uint8_t b[kBBytes];
  uint32_t as[256];  // activation scales: 4 blocks of the K-step per row (rows < kBM)
  uint32_t bs[256];  // weight scales of the feature tile's tiles
};

typedef int v4i __attribute__((ext_vector_type(4)));

// The FP4 B operand occupies the low 4 registers of the 8-register operand;
// the upper half is left undefined so no registers are spent on it.
__device__ __forceinline__ v8i widen_fp4(uint4 b) {
  const v4i v = v4i{(int)b.x, (int)b.y, (int)b.z, (int)b.w};
  return __builtin_shufflevector(v, v, 0, 1, 2, 3, -1, -1, -1, -1);
}

__device__ __forceinline__ v4f mfma_fp8_fp4(v8i a, v8i b, v4f c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 4, 0, sa, 0, sb);
}

// Byte offset of 16-byte chunk c (0..7) of activation row r in a stage.
__device__ __forceinline__ int a_off(int r, int c) { return r * 128 + ((c ^ (r & 7)) << 4); }

// Workgroup b is dispatched to XCD b % 8.  Give each XCD an equal contiguous
// share of the W work items that exist (W is known on the device only; the
// grid is sized for the host-known bound, nb >= W, nb a multiple of 8), so
// that every XCD gets work and neighbouring items share one L2.  Returns -1
// for a workgroup with nothing to do.
__device__ __forceinline__ int xcd_work_item(int b, int W) {
  const int per = (W + 7) >> 3;
  const int r = b >> 3;
  const int w = (b & 7) * per + r;
  return (r < per && w < W) ? w : -1;
}

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

// Per-thread load plan and tile coordinates, computed once per workgroup.
struct Plan {
  const uint8_t* asrc[3];   // activation chunk sources (K-step 0)
  const uint8_t* bsrc[2];   // weight chunk sources (K-step 0)
  const uint32_t* sc;       // scale dword source (K-step 0): activation or weight
  size_t bstep;             // weight bytes per K-step per chunk source
  int bsstep;               // weight scale dwords per K-step
  int J;                    // K-steps
  int tid, wave, lane, wm, wn;
  int nrows;                // rows of the tile (chunks of later rows are not loaded)
};

// One stage in registers: 3 activation chunks, 2 weight chunks, 1 scale dword.
struct Regs {
  uint4 a[3], b[2];
  uint32_t s;
};

__device__ __forceinline__ void gload(const Plan& p, Regs& R, int j) {
#pragma unroll
  for (int u = 0; u < 2; ++u) R.b[u] = *reinterpret_cast<const uint4*>(p.bsrc[u] + (size_t)j * p.bstep);
#pragma unroll
  for (int u = 0; u < 3; ++u)
    R.a[u] = (64 * u + (p.tid >> 3) < p.nrows)
                 ? *reinterpret_cast<const uint4*>(p.asrc[u] + (size_t)j * 128) : make_uint4(0, 0, 0, 0);
  R.s = (p.tid < 256) ? p.sc[j] : p.sc[(size_t)j * p.bsstep];
}

// Activation chunk u of thread tid: row 64u + (tid >> 3), logical chunk tid & 7.
__device__ __forceinline__ void lstore(const Plan& p, Stage& s, const Regs& R) {
#pragma unroll
  for (int u = 0; u < 3; ++u)
    *reinterpret_cast<uint4*>(&s.a[a_off(64 * u + (p.tid >> 3), p.tid & 7)]) = R.a[u];
#pragma unroll
  for (int u = 0; u < 2; ++u) *reinterpret_cast<uint4*>(&s.b[(kThreads * u + p.tid) * 16]) = R.b[u];
  if (p.tid < 256) s.as[p.tid] = R.s; else s.bs[p.tid - 256] = R.s;
}

// One K-step of MFMAs for a wave with N live sub-tiles on LDS stage `cur`.
template <bool kUp, int N>
__device__ __forceinline__ void mfma_step(const Plan& p, const Stage& cur, v4f (&acc)[N][4]) {
  const int lane = p.lane, g = lane >> 4, wm = p.wm, wn = p.wn;
  // this wave's 4 weight tiles: up = q-group wn (W1 0-15, W1 16-31, W3 0-15,
  // W3 16-31); down = q2-groups 2wn, 2wn+1 (2 tiles each)
  v8i b[4];
  int sb[4];
  if (kUp) {
    const uint32_t w = cur.bs[wn * 64 + lane];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      sb[t] = (int)((w >> (8 * t)) & 0xFFu);
      b[t] = widen_fp4(*reinterpret_cast<const uint4*>(&cur.b[wn * 4096 + t * 1024 + lane * 16]));
    }
  } else {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int g2 = 2 * wn + (t >> 1);
      sb[t] = (int)((cur.bs[g2 * 32 + (lane >> 1)] >> (16 * (lane & 1) + 8 * (t & 1))) & 0xFFu);
      b[t] = widen_fp4(*reinterpret_cast<const uint4*>(&cur.b[g2 * 2048 + (t & 1) * 1024 + lane * 16]));
    }
  }
  // activation fragments one sub-tile ahead of the MFMAs; the scheduling
  // fences keep at most two fragments live (registers) while the next
  // fragment's LDS read overlaps this sub-tile's MFMAs
  auto read_a = [&](int i, v8i& a, int& sa) {
    const int row = 16 * (wm + 2 * i) + (lane & 15);
    const uint4 lo = *reinterpret_cast<const uint4*>(&cur.a[a_off(row, g)]);
    const uint4 hi = *reinterpret_cast<const uint4*>(&cur.a[a_off(row, g + 4)]);
    a = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    sa = (int)((cur.as[row] >> (8 * g)) & 0xFFu);
  };
  v8i a_cur, a_nxt;
  int sa_cur, sa_nxt;
  read_a(0, a_cur, sa_cur);
#pragma unroll
  for (int i = 0; i < N; ++i) {
    if (i + 1 < N) read_a(i + 1, a_nxt, sa_nxt);
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[i][t] = mfma_fp8_fp4(a_cur, b[t], acc[i][t], sa_cur, sb[t]);
    __builtin_amdgcn_sched_barrier(0);
    a_cur = a_nxt;
    sa_cur = sa_nxt;
  }
}

template <bool kUp, int N>
__device__ __forceinline__ void gemm_body(const Plan& p, Stage* st, int rows, int m0, int ft,
                                          int I, int H, int QG2, uint8_t* __restrict__ hq,
                                          uint8_t* __restrict__ hs, float* __restrict__ O) {
  const int J = p.J;
  v4f acc[N > 0 ? N : 1][4];
#pragma unroll
  for (int i = 0; i < N; ++i)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[i][t] = v4f{0.f, 0.f, 0.f, 0.f};

  // stage j+1 is loaded into registers while step j's MFMAs run, then written
  // to the other LDS buffer; one barrier per K-step
  Regs R;
  gload(p, R, 0);
  lstore(p, st[0], R);
  __syncthreads();
  for (int j = 0; j < J; ++j) {
    if (j + 1 < J) gload(p, R, j + 1);
    if constexpr (N > 0) mfma_step<kUp, N>(p, st[j & 1], acc);
    if (j + 1 < J) lstore(p, st[(j + 1) & 1], R);
    __syncthreads();
  }

  // lane holds rows 4*(lane>>4)+v of each 16-row sub-tile, column lane&15 of each tile
  const int lane = p.lane, wm = p.wm, wn = p.wn;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const int rbase = 16 * (wm + 2 * i) + 4 * (lane >> 4);
    if (kUp) {
      const int q = 4 * ft + wn;  // 32-feature group of I
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float h0 = silu_mul(acc[i][0][v], acc[i][2][v]);
        const float h1 = silu_mul(acc[i][1][v], acc[i][3][v]);
        float am = fmaxf(fabsf(h0), fabsf(h1));
#pragma unroll
        for (int m = 1; m < 16; m <<= 1) am = fmaxf(am, __shfl_xor(am, m, 64));
        float mul;
        const uint32_t sc = mx_scale_from_amax(am, &mul);
        const int r = rbase + v;
        if (r < rows) {
          uint8_t* hrow = hq + (size_t)(m0 + r) * I + q * 32 + (lane & 15);
          hrow[0] = (uint8_t)f32_to_e4m3(h0 * mul);
          hrow[16] = (uint8_t)f32_to_e4m3(h1 * mul);
          if ((lane & 15) == 0) hs[(size_t)(m0 + r) * (I / 32) + q] = (uint8_t)sc;
        }
      }
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int g2 = 8 * ft + 2 * wn + (t >> 1);
        if (g2 >= QG2) continue;
        const int col = g2 * 32 + (t & 1) * 16 + (lane & 15);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int r = rbase + v;
          if (r < rows) O[(size_t)(m0 + r) * H + col] = acc[i][t][v];
        }
      }
    }
  }
}

// kUp: gate/up GEMM (A = x rows gathered by token, K = H; B = W1/W3; epilogue
// SwiGLU + MXFP8 of h).  !kUp: down GEMM (A = h rows in sorted order, K = I;
// B = W2; epilogue fp32 store of O).
template <bool kUp>
__global__ __launch_bounds__(kThreads) void prefill_gemm_kernel(
    const uint8_t* __restrict__ packed, PackedLayout L, const uint8_t* __restrict__ act,
    const uint8_t* __restrict__ act_s, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ sorted_pair, int k, const int* __restrict__ hdr, int NF,
    int nblocks, uint8_t* __restrict__ hq, uint8_t* __restrict__ hs, float* __restrict__ O) {
  __shared__ __align__(16) Stage st[2];
  __shared__ int row_src[kBM];
  const int logical = xcd_work_item(blockIdx.x, hdr[0] * NF);
  if (logical < 0) return;
  const int tile = logical / NF, ft = logical % NF;
  const int2 td = reinterpret_cast<const int2*>(reinterpret_cast<const uint8_t*>(hdr) + kTileHdr)[tile];
  const int e = td.x, m0 = td.y;
  const int rows = min(kBM, offsets[e + 1] - m0);
  const int tid = threadIdx.x;
  const int H = L.H, I = L.I;
  const int K = kUp ? H : I;  // reduction length
  const int QG2 = H / 32;     // 32-row groups of the down weights
  if (tid < kBM) row_src[tid] = (tid < rows) ? (kUp ? sorted_pair[m0 + tid] / k : m0 + tid) : -1;
  __syncthreads();

  Plan p;
  p.tid = tid;
  p.nrows = rows;
  p.lane = tid & 63;
  p.wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar control flow
  p.wm = p.wave & 1;
  p.wn = p.wave >> 1;  // 0..3
  p.J = K / 128;
  // Activations: chunk u of thread tid = row 64u + (tid >> 3), logical 16-byte
  // chunk tid & 7 (rows past the tile are not loaded).
#pragma unroll
  for (int u = 0; u < 3; ++u) {
    const int r = 64 * u + (tid >> 3);
    const int src = row_src[r] >= 0 ? row_src[r] : row_src[0];
    p.asrc[u] = act + (size_t)src * K + (tid & 7) * 16;
  }
  // Weights: stage bytes (512u + tid) * 16, in packed-block order (up: 4 q-groups
  // of 4 KiB; down: 8 q2-groups of 2 KiB; groups past H read group 0, unused).
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int ci = kThreads * u + tid;
    if (kUp) {
      p.bsrc[u] = packed + L.upw_block(e, 4 * ft + (ci >> 8), 0) + (ci & 255) * 16;
    } else {
      const int g2 = 8 * ft + (ci >> 7);
      p.bsrc[u] = packed + L.dnw_block(e, g2 < QG2 ? g2 : 0, 0) + (ci & 127) * 16;
    }
  }
  p.bstep = kUp ? 4096 : 2048;
  // Scales: threads 0-255 fill as[tid] (activation scale dword of row tid, rows
  // past kBM unused); threads 256-511 fill bs[d], d = tid - 256 (up: q-group
  // d/64, lane d%64; down: q2-group d/32, lanes 2(d%32), 2(d%32)+1).
  p.bsstep = kUp ? 64 : 32;
  if (tid < 256) {
    const int src = (tid < kBM && row_src[tid] >= 0) ? row_src[tid] : row_src[0];
    p.sc = reinterpret_cast<const uint32_t*>(act_s + (size_t)src * (K / 32));
  } else {
    const int d = tid - 256;
    if (kUp) {
      p.sc = reinterpret_cast<const uint32_t*>(packed + L.ups_block(e, 4 * ft + (d >> 6), 0)) + (d & 63);
    } else {
      const int g2 = 8 * ft + (d >> 5);
      p.sc = reinterpret_cast<const uint32_t*>(packed + L.dns_block(e, g2 < QG2 ? g2 : 0, 0)) + (d & 31);
    }
  }

  const int nsub = (rows + 15) / 16;  // live 16-row sub-tiles of the tile
  int nact = 0;                       // this wave's live sub-tiles: i = 0..nact-1
#pragma unroll
  for (int i = 0; i < kBM / 32; ++i)
    if (p.wm + 2 * i < nsub) nact = i + 1;
  nact = __builtin_amdgcn_readfirstlane(nact);
  switch (nact) {
    case 0: gemm_body<kUp, 0>(p, st, rows, m0, ft, I, H, QG2, hq, hs, O); break;
    case 1: gemm_body<kUp, 1>(p, st, rows, m0, ft, I, H, QG2, hq, hs, O); break;
    case 2: gemm_body<kUp, 2>(p, st, rows, m0, ft, I, H, QG2, hq, hs, O); break;
    case 3: gemm_body<kUp, 3>(p, st, rows, m0, ft, I, H, QG2, hq, hs, O); break;
    case 4: gemm_body<kUp, 4>(p, st, rows, m0, ft, I, H, QG2, hq, hs, O); break;
    case 5: gemm_body<kUp, 5>(p, st, rows, m0, ft, I, H, QG2, hq, hs, O); break;
    default: gemm_body<kUp, 6>(p, st, rows, m0, ft, I, H, QG2, hq, hs, O); break;
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
  hipLaunchKernelGGL(prefill_gemm_kernel<true>, dim3((unsigned)nb), dim3(kThreads), 0, s, packed, L,
                     xq, xs, offsets, sorted_pair, k, hdr, NF, (int)nb, hq, hs, (float*)nullptr);
  return hipGetLastError();
}

hipError_t launch_down_prefill(const uint8_t* packed, const PackedLayout& L, const uint8_t* hq,
                               const uint8_t* hs, const int32_t* offsets, int T, int k, float* O,
                               void* tile_ws, hipStream_t s) {
  int* hdr = static_cast<int*>(tile_ws);
  hipLaunchKernelGGL(build_tiles_kernel, dim3(1), dim3(256), 0, s, offsets, L.E, hdr);
  const int NF = (L.H + 255) / 256;
  const long nb = (max_tiles((long)T * k, L.E) * NF + 7) / 8 * 8;
  hipLaunchKernelGGL(prefill_gemm_kernel<false>, dim3((unsigned)nb), dim3(kThreads), 0, s, packed,
                     L, hq, hs, offsets, (const int32_t*)nullptr, k, hdr, NF, (int)nb,
                     (uint8_t*)nullptr, (uint8_t*)nullptr, O);
  return hipGetLastError();
}

}  // namespace moe
