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
// feature tile; 16-row sub-tiles past the expert's last row are skipped, so a
// short tile costs MFMA issue in proportion to its real rows.
//
// Each workgroup (8 waves, two per SIMD) owns one token tile and one feature
// tile.  The blockIdx -> work mapping is XCD aware: the dispatcher deals
// workgroups round-robin to the 8 XCDs; each XCD gets an equal contiguous
// share of the work items that exist, so neighbouring items (the feature tiles
// of one token tile, which share its activation rows) sit on the same XCD and
// its L2, and no XCD idles when the real tile count is below the grid bound.
//
// K loop (one K-step = 128 elements): every operand of a K-step -- the
// activation rows (kBM x 128 B, the 16-byte chunk index XOR-ed with the row's
// low 3 bits so that 128-bit LDS reads of 8 lanes cover all banks), the
// feature tile's 16 packed weight tiles and both operands' E8M0 scales --
// travels from global memory straight into LDS with the gfx950 LDS-DMA loads
// (global_load_lds_dword / _dwordx4: lane l of a wave writes 4 or 16 bytes at
// M0 + 4l or M0 + 16l), into a ring of three stages, so no register is spent
// on staging.  Every wave issues the same six loads per stage (three
// activation row groups, two weight tiles, one scale dword) and one stage per
// K-step, past the last K-step too (the last stage again, never read), so the
// number of its loads outstanding after any stage is a constant and the wait
// for a stage is one fixed s_waitcnt vmcnt.  The DMA loads are issued from
// inline assembly so that the compiler, which cannot tell which LDS bytes a
// DMA writes, does not drain them before every LDS read.
//
// A K-step is software-pipelined across the LDS ring: its weight fragments
// and first half of activation fragments (the head) were read from LDS during
// the previous step; the rest (the tail) are read at its start, behind the
// head's MFMAs; midway, one barrier publishes the next stage and retires the
// current slot, which is refilled at once, and the next head is read behind
// the tail's MFMAs.  So LDS reads, DMA issue and the barrier all overlap
// MFMA work, and the loop body has no branches.
//
// Waves form a 2 (tokens) x 4 (features) grid, wm = wave / 4 so that each
// SIMD holds one wave of each token half: a wave owns the 16-row sub-tiles
// {wm, wm+2, ..., wm+10} and 4 weight tiles (up to 24 MFMAs per K-step); for
// the gate/up GEMM a wave's 4 tiles are one 32-feature group of W1 and W3, so
// SwiGLU stays in its registers.  The number of live sub-tiles is a
// compile-time parameter of the loop body, selected once per wave, so the
// MFMA stream has no conditionals and only live accumulators are allocated.
#include "common.h"

namespace moe {
namespace {

constexpr int kBM = 192;                 // token rows per tile (12 sub-tiles of 16)
constexpr int kThreads = 512;            // 8 waves
constexpr int kABytes = kBM * 128;       // activation rows of one K-step
constexpr int kBBytes = 16384;           // 16 weight tiles of 1 KiB
constexpr int kRing = 3;                 // LDS stages
constexpr int kTileHdr = 256;            // tile count at offset 0, list at 256
// DMA loads per wave per stage: 3 activation row groups and 2 weight tiles
// (dwordx4) on every wave, plus one scale load on waves 0-3 (activation scale
// dwords on waves 0-2, all weight scales as one dwordx4 on wave 3).  Waits use
// the smaller count, which can only over-wait.
constexpr int kOps = 5;

struct Stage {
  uint8_t a[kABytes];
  uint8_t b[kBBytes];
  uint32_t as[kBM];  // activation scales: the 4 blocks of the K-step, one dword per row
  uint32_t bs[256];  // weight scales of the feature tile's tiles
};
static_assert(sizeof(Stage) % 16 == 0, "stage alignment");

typedef int v4i __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;

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

// LDS-DMA: every lane of the wave loads 16 (or 4) bytes from its own global
// address; lane l's bytes land at LDS byte address lds + 16 l (or 4 l).  `lds`
// must be wave-uniform.  M0 carries the LDS address and is restored after; one
// wait state separates the M0 write from the load that reads it.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(g), "s"(lds)
      : "memory");
}

__device__ __forceinline__ void dma4(const void* g, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(g), "s"(lds)
      : "memory");
}

// Wait until at most N of this wave's vector-memory loads are outstanding
// (they complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

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

// One wave's share of the DMA loads of a stage, at K-step 0; every source
// advances by a fixed stride per K-step.  LDS offsets are relative to the
// stage and wave-uniform.
struct Dma {
  const uint8_t* a[3];  // this lane's activation chunk sources
  const uint8_t* b[2];  // this lane's weight bytes
  const uint8_t* s;     // this lane's scale source (4 or 16 bytes)
  uint32_t a_lds[3], b_lds[2], s_lds;
  int bstep;            // weight bytes per K-step
  size_t sstep;         // scale bytes per K-step
  int skind;            // 0: no scale load, 1: dword, 2: dwordx4 (wave-uniform)
};

__device__ __forceinline__ void issue_stage(const Dma& d, uint32_t stage_lds, int j) {
  if (d.skind == 1)
    dma4(d.s + (size_t)j * d.sstep, stage_lds + d.s_lds);
  else if (d.skind == 2)
    dma16(d.s + (size_t)j * d.sstep, stage_lds + d.s_lds);
#pragma unroll
  for (int u = 0; u < 3; ++u) dma16(d.a[u] + (size_t)j * 128, stage_lds + d.a_lds[u]);
#pragma unroll
  for (int u = 0; u < 2; ++u) dma16(d.b[u] + (size_t)j * d.bstep, stage_lds + d.b_lds[u]);
}

// Operand fragments of one K-step for a wave with N live sub-tiles: its 4
// weight tiles (up: q-group wn = W1 rows 0-15, W1 16-31, W3 0-15, W3 16-31;
// down: q2-groups 2wn, 2wn+1, 2 tiles each) and the activation fragments of
// its sub-tiles wm, wm+2, ...  A operand (fp8) of the 16x16x128 scaled MFMA:
// lane l holds row l%16, K bytes [16g, 16g+16) and [64+16g, 64+16g+16) for
// g = l/16, and supplies the E8M0 scale of the row's block g.  The head holds
// the weight fragments and the first kHead activation fragments, read one
// step ahead; the tail the remaining activation fragments, read at the start
// of the step that uses them.
template <int N>
struct FragsShape {
  static constexpr int kHead = (N + 1) / 2;
  static constexpr int kTail = N - kHead;
};

template <int N>
struct Head {
  uint4 b[4];
  int sb[4];
  v8i a[FragsShape<N>::kHead > 0 ? FragsShape<N>::kHead : 1];
  int sa[FragsShape<N>::kHead > 0 ? FragsShape<N>::kHead : 1];
};

template <int N>
struct Tail {
  v8i a[FragsShape<N>::kTail > 0 ? FragsShape<N>::kTail : 1];
  int sa[FragsShape<N>::kTail > 0 ? FragsShape<N>::kTail : 1];
};

__device__ __forceinline__ void read_a(v8i& a, int& sa, int lane, int row, const Stage& ca) {
  const int g = lane >> 4;
  const uint4 lo = *reinterpret_cast<const uint4*>(&ca.a[a_off(row, g)]);
  const uint4 hi = *reinterpret_cast<const uint4*>(&ca.a[a_off(row, g + 4)]);
  a = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  sa = (int)((ca.as[row] >> (8 * g)) & 0xFFu);
}

template <bool kUp, int N>
__device__ __forceinline__ void read_head(Head<N>& f, int lane, int wm, int wn, const Stage& c) {
  const Stage& ca = c;
  const Stage& cb = c;
  if (kUp) {
    const uint32_t w = cb.bs[wn * 64 + lane];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      f.sb[t] = (int)((w >> (8 * t)) & 0xFFu);
      f.b[t] = *reinterpret_cast<const uint4*>(&cb.b[wn * 4096 + t * 1024 + lane * 16]);
    }
  } else {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int g2 = 2 * wn + (t >> 1);
      f.sb[t] = (int)((cb.bs[g2 * 32 + (lane >> 1)] >> (16 * (lane & 1) + 8 * (t & 1))) & 0xFFu);
      f.b[t] = *reinterpret_cast<const uint4*>(&cb.b[g2 * 2048 + (t & 1) * 1024 + lane * 16]);
    }
  }
#pragma unroll
  for (int i = 0; i < FragsShape<N>::kHead; ++i)
    read_a(f.a[i], f.sa[i], lane, 16 * (wm + 2 * i) + (lane & 15), ca);
}

template <int N>
__device__ __forceinline__ void read_tail(Tail<N>& f, int lane, int wm, const Stage& ca) {
#pragma unroll
  for (int i = 0; i < FragsShape<N>::kTail; ++i)
    read_a(f.a[i], f.sa[i], lane, 16 * (wm + 2 * (FragsShape<N>::kHead + i)) + (lane & 15), ca);
}

template <int N>
__device__ __forceinline__ void mfma_head(const Head<N>& f, v4f (&acc)[N][4]) {
#pragma unroll
  for (int i = 0; i < FragsShape<N>::kHead; ++i)
#pragma unroll
    for (int t = 0; t < 4; ++t)
      acc[i][t] = mfma_fp8_fp4(f.a[i], widen_fp4(f.b[t]), acc[i][t], f.sa[i], f.sb[t]);
}

template <int N>
__device__ __forceinline__ void mfma_tail(const Head<N>& h, const Tail<N>& f, v4f (&acc)[N][4]) {
#pragma unroll
  for (int i = 0; i < FragsShape<N>::kTail; ++i)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      v4f& c = acc[FragsShape<N>::kHead + i][t];
      c = mfma_fp8_fp4(f.a[i], widen_fp4(h.b[t]), c, f.sa[i], h.sb[t]);
    }
}

template <bool kUp, int N>
__device__ __forceinline__ void gemm_body(const Dma& d, Stage* st, int J, int lane, int wm, int wn,
                                          int rows, int m0, int ft, int I, int H, int QG2,
                                          uint8_t* __restrict__ hq, uint8_t* __restrict__ hs,
                                          float* __restrict__ O) {
  v4f acc[N > 0 ? N : 1][4];
#pragma unroll
  for (int i = 0; i < N; ++i)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[i][t] = v4f{0.f, 0.f, 0.f, 0.f};

  const uint32_t ring = (uint32_t)(uintptr_t)(lds_u8*)st;
  // stage s goes to slot s % kRing; stages past the last load the last again
  auto issue = [&](int s) {
    issue_stage(d, ring + (uint32_t)(s % kRing) * (uint32_t)sizeof(Stage), min(s, J - 1));
  };
  // Step j multiplies stage j from registers (head hc read during step j-1,
  // tail read here).  Stages issued before its barrier run up to j + 2, so
  // stage j+1 is complete once at most one stage of this wave's loads is
  // outstanding; the barrier then publishes it to every wave and retires slot
  // j % kRing (every wave's reads of stage j precede it), which takes stage
  // j + 3.
  auto step = [&](int j, Head<N>& hc, Head<N>& hn) {
    Tail<N> tl;
    if constexpr (N > 0) read_tail<N>(tl, lane, wm, st[j % kRing]);
    if constexpr (N > 0) mfma_head<N>(hc, acc);
    wait_vmcnt<kOps>();
    __syncthreads();
    if constexpr (N > 0) read_head<kUp, N>(hn, lane, wm, wn, st[(j + 1) % kRing]);
    issue(j + kRing);
    if constexpr (N > 0) mfma_tail<N>(hc, tl, acc);
  };
  issue(0);
  issue(1);
  issue(2);
  Head<N> h0, h1;
  wait_vmcnt<2 * kOps>();
  __syncthreads();
  if constexpr (N > 0) read_head<kUp, N>(h0, lane, wm, wn, st[0]);
  int j = 0;
  if (J & 1) {  // odd J: one step first, so the loop below takes steps in pairs
    step(0, h0, h1);
    h0 = h1;
    j = 1;
  }
  for (; j < J; j += 2) {
    step(j, h0, h1);
    step(j + 1, h1, h0);
  }
  // no LDS-DMA may still be writing when the workgroup's LDS is released
  wait_vmcnt<0>();

  // lane holds rows 4*(lane>>4)+v of each 16-row sub-tile, column lane&15 of each tile
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

// Activation scales by K-step: sT[j][p] = the dword of E8M0 codes of K-step j
// (4 blocks of 32) of sorted row p, taken from row sorted_pair[p] / k of the
// token-order scales (gate/up), or from row p (down, sorted_pair null).  A
// tile's rows are consecutive sorted rows, so each K-step's scale loads then
// read one contiguous run instead of one dword from each of 192 rows.
__global__ __launch_bounds__(256) void scales_by_step_kernel(const uint32_t* __restrict__ src,
                                                             int J, const int32_t* __restrict__ sorted_pair,
                                                             int k, long P, uint32_t* __restrict__ sT) {
  const long p = (long)blockIdx.x * 256 + threadIdx.x;
  const int j = blockIdx.y;
  if (p >= P) return;
  const long row = sorted_pair ? (long)(sorted_pair[p] / k) : p;
  sT[(size_t)j * P + p] = src[(size_t)row * J + j];
}

// kUp: gate/up GEMM (A = x rows gathered by token, K = H; B = W1/W3; epilogue
// SwiGLU + MXFP8 of h).  !kUp: down GEMM (A = h rows in sorted order, K = I;
// B = W2; epilogue fp32 store of O).
template <bool kUp>
__global__ __launch_bounds__(kThreads) void prefill_gemm_kernel(
    const uint8_t* __restrict__ packed, PackedLayout L, const uint8_t* __restrict__ act,
    const uint32_t* __restrict__ sT, long P, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ sorted_pair, int k, const int* __restrict__ hdr, int NF,
    int nblocks, uint8_t* __restrict__ hq, uint8_t* __restrict__ hs, float* __restrict__ O) {
  __shared__ __align__(16) Stage st[kRing];
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
  // source row of each tile row; rows past the tile read row 0's data, whose
  // products land in output rows that are never stored
  if (tid < kBM) row_src[tid] = (tid < rows) ? (kUp ? sorted_pair[m0 + tid] / k : m0 + tid) : -1;
  __syncthreads();
  const int row0 = row_src[0];

  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar control flow
  const int wm = wave >> 2, wn = wave & 3;

  Dma d;
  // Activations: row group rg = wave + 8u (u < 3) holds rows 8rg..8rg+7,
  // 1 KiB at stage offset 1024 rg; lane l lands at row 8rg + l/8, physical
  // chunk l%8, which holds logical chunk (l%8) ^ (l/8) (the row's low 3 bits
  // are l/8).
#pragma unroll
  for (int u = 0; u < 3; ++u) {
    const int rg = wave + 8 * u;
    const int r = 8 * rg + (lane >> 3);
    const int src = row_src[r] >= 0 ? row_src[r] : row0;
    d.a[u] = act + (size_t)src * K + (((lane & 7) ^ (lane >> 3)) << 4);
    d.a_lds[u] = (uint32_t)(1024 * rg);
  }
  // Weights: stage tiles 2w, 2w+1 (1 KiB each, lane order = packed order).
  // up: tile index 4g + t = q-group 4ft + g, tile t; down: tile index
  // 2g2 + t = q2-group 8ft + g2, tile t (groups past H read group 0, whose
  // products are never stored).
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int ti = 2 * wave + u;
    if (kUp) {
      d.b[u] = packed + L.upw_block(e, 4 * ft + (ti >> 2), 0) + (ti & 3) * 1024 + lane * 16;
    } else {
      const int g2 = 8 * ft + (ti >> 1);
      d.b[u] = packed + L.dnw_block(e, g2 < QG2 ? g2 : 0, 0) + (ti & 1) * 1024 + lane * 16;
    }
    d.b_lds[u] = (uint32_t)(kABytes + 1024 * ti);
  }
  d.bstep = kUp ? 4096 : 2048;
  // Scales.  Waves 0-2: activation scale dwords of rows 64w..64w+63 (as[row])
  // from the by-step array, one contiguous run per K-step (rows past the
  // tile read its last row).  Wave 3: all weight scales of the K-step as one
  // dwordx4 load, 16 bytes per lane: up: lanes 16g..16g+15 take q-group
  // 4ft + g's 256 bytes (bs[64g + d]); down: lanes 8g2..8g2+7 take q2-group
  // 8ft + g2's 128 bytes (bs[32 g2 + d]).
  if (wave < 3) {
    const int r = 64 * wave + lane;
    d.s = reinterpret_cast<const uint8_t*>(sT + m0 + min(r, rows - 1));
    d.sstep = (size_t)P * 4;
    d.s_lds = (uint32_t)(kABytes + kBBytes + 256 * wave);
    d.skind = 1;
  } else if (wave == 3) {
    if (kUp) {
      d.s = packed + L.ups_block(e, 4 * ft + (lane >> 4), 0) + (lane & 15) * 16;
      d.sstep = 256;
    } else {
      const int g2 = 8 * ft + (lane >> 3);
      d.s = packed + L.dns_block(e, g2 < QG2 ? g2 : 0, 0) + (lane & 7) * 16;
      d.sstep = 128;
    }
    d.s_lds = (uint32_t)(kABytes + kBBytes + kBM * 4);
    d.skind = 2;
  } else {
    d.s = nullptr;
    d.sstep = 0;
    d.s_lds = 0;
    d.skind = 0;
  }

  const int J = K / 128;
  const int nsub = (rows + 15) / 16;  // live 16-row sub-tiles of the tile
  int nact = 0;                       // this wave's live sub-tiles: i = 0..nact-1
#pragma unroll
  for (int i = 0; i < kBM / 32; ++i)
    if (wm + 2 * i < nsub) nact = i + 1;
  nact = __builtin_amdgcn_readfirstlane(nact);
  switch (nact) {
    case 0: gemm_body<kUp, 0>(d, st, J, lane, wm, wn, rows, m0, ft, I, H, QG2, hq, hs, O); break;
    case 1: gemm_body<kUp, 1>(d, st, J, lane, wm, wn, rows, m0, ft, I, H, QG2, hq, hs, O); break;
    case 2: gemm_body<kUp, 2>(d, st, J, lane, wm, wn, rows, m0, ft, I, H, QG2, hq, hs, O); break;
    case 3: gemm_body<kUp, 3>(d, st, J, lane, wm, wn, rows, m0, ft, I, H, QG2, hq, hs, O); break;
    case 4: gemm_body<kUp, 4>(d, st, J, lane, wm, wn, rows, m0, ft, I, H, QG2, hq, hs, O); break;
    case 5: gemm_body<kUp, 5>(d, st, J, lane, wm, wn, rows, m0, ft, I, H, QG2, hq, hs, O); break;
    default: gemm_body<kUp, 6>(d, st, J, lane, wm, wn, rows, m0, ft, I, H, QG2, hq, hs, O); break;
  }
}

long max_tiles(long P, int E) { return (P + kBM - 1) / kBM + E; }

size_t align256_(size_t x) { return (x + 255) & ~(size_t)255; }

// workspace: tile header and list, then the by-step activation scales
size_t tile_list_bytes(long P, int E) { return align256_(kTileHdr + (size_t)max_tiles(P, E) * 8); }

}  // namespace

size_t prefill_stage_bytes(long P, int E, int H, int I) {
  const int Jmax = (H > I ? H : I) / 128;
  return tile_list_bytes(P, E) + align256_((size_t)P * Jmax * 4);
}

hipError_t launch_up_prefill(const uint8_t* packed, const PackedLayout& L, const uint8_t* xq,
                             const uint8_t* xs, const int32_t* offsets,
                             const int32_t* sorted_pair, int T, int k, uint8_t* hq, uint8_t* hs,
                             void* tile_ws, hipStream_t s) {
  const long P = (long)T * k;
  int* hdr = static_cast<int*>(tile_ws);
  uint32_t* sT = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(tile_ws) + tile_list_bytes(P, L.E));
  hipLaunchKernelGGL(build_tiles_kernel, dim3(1), dim3(256), 0, s, offsets, L.E, hdr);
  hipLaunchKernelGGL(scales_by_step_kernel, dim3((unsigned)((P + 255) / 256), (unsigned)L.J), dim3(256),
                     0, s, reinterpret_cast<const uint32_t*>(xs), L.J, sorted_pair, k, P, sT);
  const int NF = L.I / 128;
  const long nb = (max_tiles(P, L.E) * NF + 7) / 8 * 8;
  hipLaunchKernelGGL(prefill_gemm_kernel<true>, dim3((unsigned)nb), dim3(kThreads), 0, s, packed, L,
                     xq, sT, P, offsets, sorted_pair, k, hdr, NF, (int)nb, hq, hs, (float*)nullptr);
  return hipGetLastError();
}

hipError_t launch_down_prefill(const uint8_t* packed, const PackedLayout& L, const uint8_t* hq,
                               const uint8_t* hs, const int32_t* offsets, int T, int k, float* O,
                               void* tile_ws, hipStream_t s) {
  const long P = (long)T * k;
  int* hdr = static_cast<int*>(tile_ws);
  uint32_t* sT = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(tile_ws) + tile_list_bytes(P, L.E));
  hipLaunchKernelGGL(build_tiles_kernel, dim3(1), dim3(256), 0, s, offsets, L.E, hdr);
  hipLaunchKernelGGL(scales_by_step_kernel, dim3((unsigned)((P + 255) / 256), (unsigned)L.J2), dim3(256),
                     0, s, reinterpret_cast<const uint32_t*>(hs), L.J2, (const int32_t*)nullptr, k, P, sT);
  const int NF = (L.H + 255) / 256;
  const long nb = (max_tiles(P, L.E) * NF + 7) / 8 * 8;
  hipLaunchKernelGGL(prefill_gemm_kernel<false>, dim3((unsigned)nb), dim3(kThreads), 0, s, packed,
                     L, hq, sT, P, offsets, (const int32_t*)nullptr, k, hdr, NF, (int)nb,
                     (uint8_t*)nullptr, (uint8_t*)nullptr, O);
  return hipGetLastError();
}

}  // namespace moe
