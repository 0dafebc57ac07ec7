// Router logits ahead of the top-k: logits[t, e] = sum_h x[t, h] * Wg[e, h],
// x and Wg as bf16, accumulated in fp32 by the bf16 matrix cores.  The
// review's precision policy lets the first layers of the MoE gate network run
// at low precision while the top-k compare stays fp32 (pwwt.cn review,
// section 4.1, the operator classes and the row "MoE routing top-k").
//
// v_mfma_f32_16x16x32_bf16: lane l supplies 8 bf16 of row l%16 (A) or column
// l%16 (B); A and B use the same lane-to-K assignment, so each lane loads the
// 8 consecutive bf16 (16 bytes) at K offset k0 + 8*(l/16) of its row and one
// instruction covers 32 K.
//
// The GEMM is skinny (E <= 1024 columns, K = H up to 7168 and more), so the
// work is split along K as well as over output tiles, deterministically:
//   * a wave item is (token tile of 16*TM rows, 64-expert group, K slice s);
//     a wave accumulates its 16*TM x 64 block over its slice and writes it to
//     partial[s] (or straight to the logits when there is a single slice);
//   * a second pass adds the S partial blocks of every logit in slice order.
// The slice count S is a function of (T, H, E) only, so the summation order,
// hence every bit of the result, is fixed per shape.  Workgroup b works on
// slice b % S and lands on XCD b % 8: with S a multiple of 4 each XCD reads
// a fixed set of K columns of Wg into its L2 and reuses them for every token
// tile, and the four waves of a workgroup share their x rows in L1.
#include "lds_dma.h"
#include "stages.h"

namespace moe {
namespace {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

__device__ __forceinline__ v8bf as_bf8(uint4 v) { return __builtin_bit_cast(v8bf, v); }

// Chunks of 32 K in flight per wave (a chunk is TM + 4 16-byte loads per lane),
// for either token-tile count.
template <int TM>
constexpr int ring_depth() {
  return 3;
}

template <int TM>
struct Chunk {
  uint4 a[TM];
  uint4 b[4];
};

template <int TM>
__device__ __forceinline__ void load_chunk(Chunk<TM>& c, const uint16_t* const (&xrow)[TM],
                                           const uint16_t* const (&wrow)[4], int k) {
#pragma unroll
  for (int m = 0; m < TM; ++m) c.a[m] = *reinterpret_cast<const uint4*>(xrow[m] + k);
#pragma unroll
  for (int n = 0; n < 4; ++n) c.b[n] = *reinterpret_cast<const uint4*>(wrow[n] + k);
}

template <int TM>
__device__ __forceinline__ void mma_chunk(const Chunk<TM>& c, v4f (&acc)[TM][4]) {
#pragma unroll
  for (int m = 0; m < TM; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n)
      acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf8(c.a[m]), as_bf8(c.b[n]), acc[m][n],
                                                          0, 0, 0);
}

// out: partial[S][T][E] fp32 (S > 1) or the logits [T][E] (S == 1)
template <int TM>
__global__ __launch_bounds__(256) void router_partial_kernel(const uint16_t* __restrict__ x,
                                                             const uint16_t* __restrict__ wg, int T,
                                                             int H, int E, int S,
                                                             float* __restrict__ out) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int NT = (T + 16 * TM - 1) / (16 * TM), NE = (E + 63) / 64;
  const int s = (int)(blockIdx.x % (unsigned)S);
  const int q = (int)(blockIdx.x / (unsigned)S) * 4 + wave;  // (token tile, expert group)
  if (q >= NT * NE) return;                                   // whole wave leaves: no barriers
  const int tt = q / NE, eg = q % NE;
  const int t0 = 16 * TM * tt, e0 = 64 * eg;
  const int g = lane >> 4, r = lane & 15;
  // this lane's rows (clamped: rows past T or E are computed from the last
  // valid row and never stored)
  const uint16_t* xrow[TM];
  const uint16_t* wrow[4];
#pragma unroll
  for (int m = 0; m < TM; ++m) xrow[m] = x + (size_t)min(t0 + 16 * m + r, T - 1) * H + 8 * g;
#pragma unroll
  for (int n = 0; n < 4; ++n) wrow[n] = wg + (size_t)min(e0 + 16 * n + r, E - 1) * H + 8 * g;

  const int nchunk = H / 32;
  const int c0 = (int)(((long)s * nchunk) / S), c1 = (int)(((long)(s + 1) * nchunk) / S);
  v4f acc[TM][4];
#pragma unroll
  for (int m = 0; m < TM; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n) acc[m][n] = v4f{0.f, 0.f, 0.f, 0.f};

  // Ring of kRing chunks: chunk c + kRing - 1 loads while chunk c multiplies.
  // The steady-state loop has no branches (loads past the slice re-read its
  // last chunk and are never used), so the compiler's wait counts let the
  // younger loads stay in flight; the last chunks run in a plain tail loop.
  constexpr int kRing = ring_depth<TM>();
  Chunk<TM> ring[kRing];
  const int last = c1 - 1;
#pragma unroll
  for (int i = 0; i < kRing - 1; ++i) load_chunk(ring[i], xrow, wrow, 32 * min(c0 + i, last));
  int c = c0;
  for (; c + kRing <= c1; c += kRing) {
#pragma unroll
    for (int i = 0; i < kRing; ++i) {
      load_chunk(ring[(i + kRing - 1) % kRing], xrow, wrow, 32 * min(c + i + kRing - 1, last));
      __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of this chunk's MFMAs
      mma_chunk(ring[i], acc);
    }
  }
  // c1 - c < kRing chunks left; chunk c sits in ring[0], c + 1 in ring[1], ...
#pragma unroll
  for (int i = 0; i < kRing - 1; ++i)
    if (c + i < c1) mma_chunk(ring[i], acc);

  // lane holds rows 4*(lane>>4)+v of each token tile, column lane&15 of each expert tile
  float* o = out + (S > 1 ? (size_t)s * T * E : 0);
#pragma unroll
  for (int m = 0; m < TM; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const int e = e0 + 16 * n + r;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int t = t0 + 16 * m + 4 * g + v;
        if (t < T && e < E) o[(size_t)t * E + e] = acc[m][n][v];
      }
    }
}

// ------------------------------------------------ LDS-tiled GEMM, large T
// A workgroup (4 waves, 2 x 2) owns a 128-token x 128-expert tile and one K
// slice; per stage of 64 K it stages 16 KB of x rows and 16 KB of Wg rows in
// LDS (each row's eight 16-byte granules XOR-swizzled by row & 7 so that the
// fragment reads of 16 consecutive rows spread over the banks), double
// buffered: the next stage's global loads are in flight while the current
// stage's 32 MFMAs per wave run, and one barrier per stage separates the
// buffers' reuse.  Rows past T or E are clamped to the last valid row and
// never stored.
constexpr int kTB = 128;          // tile rows (tokens) = tile columns (experts)
constexpr int kTK = 64;           // K per stage
constexpr int kTStage = 2 * kTB * kTK * 2;  // bytes of one stage (x and Wg)

typedef uint32_t v4u __attribute__((ext_vector_type(4)));

struct TileLoad {
  v4u a[4], b[4];
};

__device__ __forceinline__ int swz(int row, int q) { return row * 128 + ((q ^ (row & 7)) << 4); }

__device__ __forceinline__ void tile_gload(TileLoad& r, const uint16_t* const (&ga)[4],
                                           const uint16_t* const (&gb)[4], int st) {
  const int k = st * kTK;
#pragma unroll
  for (int j = 0; j < 4; ++j) r.a[j] = *reinterpret_cast<const v4u*>(ga[j] + k);
#pragma unroll
  for (int j = 0; j < 4; ++j) r.b[j] = *reinterpret_cast<const v4u*>(gb[j] + k);
}

__device__ __forceinline__ void tile_lstore(const TileLoad& r, uint8_t* buf, int lr, int lq) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    *reinterpret_cast<v4u*>(buf + swz(32 * j + lr, lq)) = r.a[j];
    *reinterpret_cast<v4u*>(buf + kTB * 128 + swz(32 * j + lr, lq)) = r.b[j];
  }
}

// One stage's 2 x 16 MFMAs of a wave from the LDS buffer `cur`.
__device__ __forceinline__ void tile_compute(v4f (&acc)[4][4], const uint8_t* cur, int abase,
                                             int bbase, int fo0, int fo1) {
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    const int fo = kk ? fo1 : fo0;
    v8bf a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = *reinterpret_cast<const v8bf*>(cur + abase + 16 * 128 * i + fo);
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = *reinterpret_cast<const v8bf*>(cur + bbase + 16 * 128 * j + fo);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
  }
}

__global__ __launch_bounds__(256) void router_tiled_kernel(const uint16_t* __restrict__ x,
                                                           const uint16_t* __restrict__ wg, int T,
                                                           int H, int E, int S,
                                                           float* __restrict__ out) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int NTm = (T + kTB - 1) / kTB, NTn = (E + kTB - 1) / kTB;
  // block -> (slice, token tile, expert tile); slice-minor so that each XCD
  // (block % 8) keeps a fixed set of K slices of Wg in its L2
  const int s = (int)(blockIdx.x % (unsigned)S);
  const int tile = (int)(blockIdx.x / (unsigned)S);
  const int tm = tile / NTn, tn = tile % NTn;
  if (tm >= NTm) return;  // uniform per block: before any barrier
  const int m0 = tm * kTB, n0 = tn * kTB;
  const int nst = H / kTK;
  const int st0 = (int)(((long)s * nst) / S), st1 = (int)(((long)(s + 1) * nst) / S);

  // this thread's four x rows and four Wg rows (32 rows apart) and granule
  const int lr = tid >> 3, lq = tid & 7;
  const uint16_t* ga[4];
  const uint16_t* gb[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    ga[j] = x + (size_t)min(m0 + 32 * j + lr, T - 1) * H + 8 * lq;
    gb[j] = wg + (size_t)min(n0 + 32 * j + lr, E - 1) * H + 8 * lq;
  }
  // fragment offsets: row (16-row block base) + lane & 15, granule 4 kk + lane >> 4
  const int fr = lane & 15, fg = lane >> 4;
  const int fo0 = swz(fr, fg), fo1 = swz(fr, 4 + fg);
  const int abase = (64 * wm) * 128, bbase = kTB * 128 + (64 * wn) * 128;

  v4f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // Two register sets: stage st + 2 loads while stage st multiplies and stage
  // st + 1 (loaded one stage earlier) goes from registers to the idle LDS
  // buffer.  Loads past the slice re-read its last stage and are never used.
  const int last = st1 - 1;
  TileLoad p, q;
  tile_gload(p, ga, gb, st0);
  tile_gload(q, ga, gb, min(st0 + 1, last));
  tile_lstore(p, lds, lr, lq);
  __syncthreads();
  uint8_t* const buf0 = lds;
  uint8_t* const buf1 = lds + kTStage;
  int st = st0;
  for (; st + 2 <= st1; st += 2) {
    tile_gload(p, ga, gb, min(st + 2, last));
    tile_compute(acc, buf0, abase, bbase, fo0, fo1);
    tile_lstore(q, buf1, lr, lq);
    __syncthreads();
    tile_gload(q, ga, gb, min(st + 3, last));
    tile_compute(acc, buf1, abase, bbase, fo0, fo1);
    tile_lstore(p, buf0, lr, lq);
    __syncthreads();
  }
  if (st < st1) tile_compute(acc, buf0, abase, bbase, fo0, fo1);  // odd count: last stage in buf0

  float* o = out + (S > 1 ? (size_t)s * T * E : 0);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = n0 + 64 * wn + 16 * j + fr;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int t = m0 + 64 * wm + 16 * i + 4 * fg + v;
        if (t < T && e < E) o[(size_t)t * E + e] = acc[i][j][v];
      }
    }
}

// ------------------------------------------------ LDS-DMA GEMM, large T, E >= 256
// A workgroup (8 waves, 2 x 4) owns a 128-token x 256-expert tile and one K
// slice.  Per stage of 64 K the tile's x rows (16 KB) and Wg rows (32 KB)
// travel from global memory straight into LDS with LDS-DMA loads (every
// lane writes 16 bytes; no register holds staged data), into a ring of three
// stages.  A row's 128 bytes of a stage sit as eight 16-byte chunks, chunk c
// at position c ^ (row & 7), so that the fragment reads of 16 consecutive
// rows spread over the banks.  Each wave issues the same six loads per stage
// (two x row groups, four Wg row groups of 8 rows; past the slice, its last
// stage again, never read), so a stage is complete once at most six of the
// wave's loads issued after it are outstanding.  Wave (wm, wn) multiplies
// token rows 64 wm .. + 63 by expert rows 64 wn .. + 63: 4 x 4 blocks, two
// MFMAs of 32 K (the stage's halves) each.  The K loop is software-pipelined
// across the ring as in the FP4 expert GEMMs: a stage's first-half fragments
// (the head) are read during the previous step, its second half (the tail)
// at the start of its own step, behind the head's MFMAs; midway one barrier
// publishes the next stage and frees the current slot, which takes the stage
// three ahead, and the next head is read behind the tail's MFMAs.  Rows past
// T or E are clamped to the last valid row and never stored.
constexpr int kDM = 128;                       // tile rows (tokens)
constexpr int kDN = 256;                       // tile columns (experts)
constexpr int kDKB = 128;                      // bytes of a row per stage (64 bf16)
constexpr int kDStage = (kDM + kDN) * kDKB;    // 48 KB
constexpr int kDRing = 3;
constexpr int kDOps = 6;                       // DMA loads per wave per stage

struct RFrag {
  v8bf a[4], b[4];
};

__global__ __launch_bounds__(512) void router_dma_kernel(const uint16_t* __restrict__ x,
                                                         const uint16_t* __restrict__ wg, int T,
                                                         int H, int E, int S,
                                                         float* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kDRing * kDStage];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int NTm = (T + kDM - 1) / kDM, NTn = (E + kDN - 1) / kDN;
  // block -> (slice, token tile, expert tile), slice-minor as in the tiled kernel
  const int s = (int)(blockIdx.x % (unsigned)S);
  const int tile = (int)(blockIdx.x / (unsigned)S);
  const int tm = tile / NTn, tn = tile % NTn;
  if (tm >= NTm) return;  // uniform per block: before any barrier
  const int m0 = tm * kDM, n0 = tn * kDN;
  const int nst = H / 64;
  const int st0 = (int)(((long)s * nst) / S), n = (int)(((long)(s + 1) * nst) / S) - st0;

  // DMA sources: lane l of row group rg loads row 8 rg + l / 8, logical chunk
  // (l % 8) ^ (l / 8) (the row's low 3 bits are l / 8), which lands at
  // physical chunk l % 8.  Offsets are from the slice's first K byte.
  const uint32_t ch = (uint32_t)(((lane & 7) ^ (lane >> 3)) << 4);
  const uint32_t rowb = (uint32_t)H * 2u;
  uint32_t xo[2], wo[4];
#pragma unroll
  for (int u = 0; u < 2; ++u)
    xo[u] = (uint32_t)min(m0 + 8 * (wave + 8 * u) + (lane >> 3), T - 1) * rowb + ch;
#pragma unroll
  for (int u = 0; u < 4; ++u)
    wo[u] = (uint32_t)min(n0 + 8 * (wave + 8 * u) + (lane >> 3), E - 1) * rowb + ch;
  const uint8_t* xb = reinterpret_cast<const uint8_t*>(x) + (size_t)st0 * kDKB;
  const uint8_t* wb = reinterpret_cast<const uint8_t*>(wg) + (size_t)st0 * kDKB;
  const uint32_t ring = (uint32_t)(uintptr_t)(lds_u8*)lds;
  auto issue = [&](int j) {
    const int jj = min(j, n - 1);
    const uint32_t st = wave_u32(ring + (uint32_t)(j % kDRing) * (uint32_t)kDStage);
    const uint8_t* xs = wave_ptr(xb + (size_t)jj * kDKB);
    const uint8_t* ws = wave_ptr(wb + (size_t)jj * kDKB);
#pragma unroll
    for (int u = 0; u < 2; ++u) dma_x4(xs, xo[u], st + 1024u * (uint32_t)(wave + 8 * u));
#pragma unroll
    for (int u = 0; u < 4; ++u)
      dma_x4(ws, wo[u], st + (uint32_t)(kDM * kDKB) + 1024u * (uint32_t)(wave + 8 * u));
  };

  // fragment offsets: row 16-row block base + lane & 15, chunk g (first half
  // of the stage) or g + 4 (second half)
  const int fr = lane & 15, fg = lane >> 4;
  const int fo0 = (fr * 128) + ((fg ^ (fr & 7)) << 4);
  const int fo1 = (fr * 128) + (((fg + 4) ^ (fr & 7)) << 4);
  const int abase = (64 * wm) * kDKB, bbase = kDM * kDKB + (64 * wn) * kDKB;
  auto read = [&](RFrag& f, const uint8_t* S0, int fo) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f.a[i] = *reinterpret_cast<const v8bf*>(S0 + abase + 16 * kDKB * i + fo);
#pragma unroll
    for (int i = 0; i < 4; ++i) f.b[i] = *reinterpret_cast<const v8bf*>(S0 + bbase + 16 * kDKB * i + fo);
  };

  v4f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
  auto mma = [&](const RFrag& f) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        acc[i][q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.a[i], f.b[q], acc[i][q], 0, 0, 0);
  };

  // Step j: stages up to j + 2 were issued before its barrier, so stage j + 1
  // is complete once at most one stage of the wave's loads is outstanding.
  auto step = [&](int j, const RFrag& hc, RFrag& hn) {
    RFrag tl;
    read(tl, lds + (j % kDRing) * kDStage, fo1);
    mma(hc);
    wait_vmcnt<kDOps>();
    __syncthreads();  // stage j + 1 visible to all; every wave done with slot j
    read(hn, lds + ((j + 1) % kDRing) * kDStage, fo0);
    issue(j + kDRing);
    mma(tl);
  };
  issue(0);
  issue(1);
  issue(2);
  wait_vmcnt<2 * kDOps>();
  __syncthreads();
  RFrag h0, h1;
  read(h0, lds, fo0);
  int j = 0;
  if (n & 1) {  // odd count: one step first, so the loop below takes steps in pairs
    step(0, h0, h1);
    h0 = h1;
    j = 1;
  }
  for (; j < n; j += 2) {
    step(j, h0, h1);
    step(j + 1, h1, h0);
  }
  wait_vmcnt<0>();  // no LDS-DMA may still be writing when the workgroup's LDS is released

  float* o = out + (S > 1 ? (size_t)s * T * E : 0);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = n0 + 64 * wn + 16 * q + fr;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int t = m0 + 64 * wm + 16 * i + 4 * fg + v;
        if (t < T && e < E) o[(size_t)t * E + e] = acc[i][q][v];
      }
    }
}

// logits[i] = ((partial[0][i] + partial[1][i]) + ...) + partial[S-1][i], the
// same order in which the routing kernels sum the partials they read directly
__global__ __launch_bounds__(256) void router_reduce_kernel(const float* __restrict__ part, long n,
                                                            int S, float* __restrict__ logits) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  logits[i] = slice_sum(part, n, S, i);
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

int router_tm(int T) { return T <= 16 ? 1 : 4; }

// Token counts from which the LDS-tiled kernels run the GEMM; the LDS-DMA
// kernel takes over from 256 experts (its tile is 256 experts wide) while
// the per-lane byte offsets of x fit 32 bits.
constexpr int kTiledMinT = 128;
bool router_dma(int T, int H, int E) {
  return T >= kTiledMinT && E >= kDN && (long)T * H * 2 < (1L << 32) && (long)E * H * 2 < (1L << 32);
}
// The 128 x 128 LDS-tiled kernel from kTiledMinT tokens, and from 17 tokens
// when the experts fill two of its tiles or more (E >= 256: stand-alone it
// measured faster than the per-wave split-K kernel at every T from 16).
bool router_tiled(int T, int E) { return T >= kTiledMinT || (T > 16 && E >= 2 * kTB); }

}  // namespace

// Number of K slices, capped so that every slice keeps at least 4 steps of
// its kernel's K unit.  Decode (one token tile of 16): slices of about 16
// chunks of 32, rounded up to a multiple of 4 (each XCD then works on a fixed
// set of K ranges), a wave's whole slice in a few round trips while the
// partial planes stay few for the routing launch to add.  Medium T: none
// while the output tiles give the chip about 1024 waves, else enough slices
// for that (multiple of 4).  Tiled (large T): as many slices as keep the
// workgroups within one per compute unit (256).
int router_slices(int T, int H, int E) {
  if (router_dma(T, H, E)) {
    const long tiles = (long)((T + kDM - 1) / kDM) * ((E + kDN - 1) / kDN);
    const long want = 256 / tiles > 1 ? 256 / tiles : 1;
    const int smax = H / 64 / 4 > 1 ? H / 64 / 4 : 1;
    return (int)(want < smax ? want : smax);
  }
  if (router_tiled(T, E)) {
    const long tiles = (long)((T + kTB - 1) / kTB) * ((E + kTB - 1) / kTB);
    const long want = 256 / tiles > 1 ? 256 / tiles : 1;
    const int smax = H / kTK / 4 > 1 ? H / kTK / 4 : 1;
    return (int)(want < smax ? want : smax);
  }
  const int tm = router_tm(T);
  const int nchunk = H / 32;
  long want;
  if (tm == 1) {
    want = (nchunk + 15) / 16;
  } else {
    const long base = (long)((T + 16 * tm - 1) / (16 * tm)) * ((E + 63) / 64);
    want = (1024 + base - 1) / base;
  }
  if (want <= 1) return 1;
  const int smax = nchunk / 4 > 1 ? nchunk / 4 : 1;
  const long s4 = (want + 3) / 4 * 4;
  return (int)(s4 < smax ? s4 : smax);
}

size_t router_ws_bytes(int T, int H, int E) {
  const int S = router_slices(T, H, E);
  return S > 1 ? (size_t)S * T * E * sizeof(float) : 0;
}

hipError_t launch_identity_route(int T, int32_t* sorted_pair, int32_t* offsets, hipStream_t s) {
  hipLaunchKernelGGL(identity_route_kernel, dim3((unsigned)((T + 255) / 256)), dim3(256), 0, s, T,
                     sorted_pair, offsets);
  return hipGetLastError();
}

hipError_t launch_router_partials(const uint16_t* x, const uint16_t* wg, int T, int H, int E,
                                  float* logits, float* partial, hipStream_t s) {
  const int S = router_slices(T, H, E);
  if (router_dma(T, H, E)) {
    const long tiles = (long)((T + kDM - 1) / kDM) * ((E + kDN - 1) / kDN);
    hipLaunchKernelGGL(router_dma_kernel, dim3((unsigned)(tiles * S)), dim3(512), 0, s, x, wg, T,
                       H, E, S, S > 1 ? partial : logits);
    return hipGetLastError();
  }
  if (router_tiled(T, E)) {
    const long tiles = (long)((T + kTB - 1) / kTB) * ((E + kTB - 1) / kTB);
    hipLaunchKernelGGL(router_tiled_kernel, dim3((unsigned)(tiles * S)), dim3(256), 2 * kTStage, s,
                       x, wg, T, H, E, S, S > 1 ? partial : logits);
    return hipGetLastError();
  }
  const int tm = router_tm(T);
  const long items = (long)((T + 16 * tm - 1) / (16 * tm)) * ((E + 63) / 64);
  const unsigned nb = (unsigned)(S * ((items + 3) / 4));
  float* out = S > 1 ? partial : logits;
  if (tm == 1)
    hipLaunchKernelGGL(router_partial_kernel<1>, dim3(nb), dim3(256), 0, s, x, wg, T, H, E, S, out);
  else
    hipLaunchKernelGGL(router_partial_kernel<4>, dim3(nb), dim3(256), 0, s, x, wg, T, H, E, S, out);
  return hipGetLastError();
}

hipError_t launch_router(const uint16_t* x, const uint16_t* wg, int T, int H, int E, float* logits,
                         float* partial, hipStream_t s) {
  hipError_t e = launch_router_partials(x, wg, T, H, E, logits, partial, s);
  const int S = router_slices(T, H, E);
  if (e != hipSuccess || S == 1) return e;
  const long n = (long)T * E;
  hipLaunchKernelGGL(router_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                     partial, n, S, logits);
  return hipGetLastError();
}

}  // namespace moe
