// FP8 dense projection: y[t, n] = sum_k x[t, k] * W[n, k] with W in OCP e4m3
// and one E8M0 scale per 32 consecutive K elements of a row, x as the MXFP8
// rows of the path's activation quantiser, fp32 accumulation in the gfx950
// scaled MFMA (v_mfma_scale_f32_16x16x128_f8f6f4, both operands e4m3, the
// block scales applied in hardware) and y stored as bf16 (RNE).  The pages
// list "FP8 dense projections" beside the FP4 routed experts (abstract of the
// arxivdaily page) and name block-wise quantisation as the way FP8 pays off
// (pwwt.cn review, section 5.3); matrix-multiply outputs may be low precision
// while the accumulation stays fp32 (same review, section 4.1).
//
// Packed weights: tile (nt, j) = rows 16 nt .. +16, K 128 j .. +128, 2 KiB in
// the MFMA operand's lane order -- lane l = 16 g + r holds row r's K elements
// [16 g, 16 g + 16) in the first KiB and [64 + 16 g, +16) in the second (the
// e4m3 operand layout measured on gfx950), so a wave loads a tile with two
// fully contiguous 1 KiB runs; its 64 scale bytes follow the same lanes (lane
// l: row r, 32-block g).  The two tiles of a 32-row group are adjacent for
// each K-step, and a group's K-steps are consecutive.
//
// Decode (few tokens): weight streaming.  A workgroup owns one 32-row group
// (two tiles, so each activation fragment serves two MFMAs) and one 16-token
// tile, or two from 17 tokens (each weight tile then feeds the MFMAs of both
// token tiles); its 16 waves take the K-steps in turn (wave w: steps w, w + 16, ...),
// so at any moment they read neighbouring 4 KiB blocks, each keeping two steps
// in flight; partial sums meet in LDS in wave order.  Prefill: LDS-tiled
// GEMMs, 128 K per stage.  From a few thousand tokens (even K-step counts):
// 256 tokens x 256 rows per workgroup, one wave per SIMD, the operands moved
// by LDS-DMA (dense_dma_kernel); below that, or with an odd K-step count,
// 128 x 128 (4 waves) or 192 x 256 (8 waves) tiles staged through two
// register sets so that one stage loads while another multiplies.  The launch
// takes the geometry with the fewest rounds of workgroups weighted by each
// one's measured round time.
#include <atomic>

#include "lds_dma.h"

namespace moe {
namespace {

typedef uint32_t v4u __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v8i cat8(v4u lo, v4u hi) {
  return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

__device__ __forceinline__ v4f mfma_fp8_fp8(v8i a, v8i b, v4f c, int sa, int sb) {
  // cbsz = 0, blgp = 0: both operands e4m3; scale bytes from byte 0 of sa / sb
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}

// ----------------------------------------------------------------- prepack
// One thread per (tile, lane): canonical wq [N, K], ws [N, K/32] -> packed.
__global__ __launch_bounds__(256) void dense_pack_kernel(const uint8_t* __restrict__ wq,
                                                         const uint8_t* __restrict__ ws, int N,
                                                         int K, uint8_t* __restrict__ packed) {
  const DenseLayout L(N, K);
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  const long ntiles = (long)(N / 16) * L.J;
  if (i >= ntiles * 64) return;
  const long tile = i >> 6;
  const int lane = (int)(i & 63), r = lane & 15, g = lane >> 4;
  const int nt = (int)(tile / L.J), j = (int)(tile % L.J);
  const long row = 16L * nt + r;
  const uint8_t* src = wq + row * K + 128L * j;
  uint8_t* dst = packed + L.tile_off(nt, j);
  *reinterpret_cast<uint4*>(dst + lane * 16) = *reinterpret_cast<const uint4*>(src + 16 * g);
  *reinterpret_cast<uint4*>(dst + 1024 + lane * 16) = *reinterpret_cast<const uint4*>(src + 64 + 16 * g);
  packed[L.scale_off(nt, j) + lane] = ws[row * (K / 32) + 4L * j + g];
}

// ------------------------------------------------------------------ decode
// One K-step of a wave: NT weight tiles and their scale bytes, the activation
// fragment (token row r, the same two 16-byte pieces) and its scale byte.
// NG token tiles of 16 share each loaded weight tile (NG MFMAs per tile).
template <int NT, int NG = 1>
struct DStep {
  v4u b0[NT], b1[NT], a0[NG], a1[NG];
  uint32_t sb[NT], sa[NG];
};

// wt[t]/st[t]: this lane's bytes of tile (nt0 + t, 0) and its scale; K-step j
// is kTileStep * j further (scales: kScaleStep * j).
template <int NT, int NG>
__device__ __forceinline__ void dload(DStep<NT, NG>& s, const uint8_t* const (&wt)[NT],
                                      const uint8_t* const (&st)[NT], const uint8_t* const (&arow)[NG],
                                      const uint8_t* const (&as)[NG], int j) {
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const uint8_t* w = wt[t] + (size_t)j * DenseLayout::kTileStep;
    // weights are streamed once: non-temporal loads leave the caches to the activations
    s.b0[t] = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(w));
    s.b1[t] = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(w + 1024));
    s.sb[t] = st[t][(size_t)j * DenseLayout::kScaleStep];
  }
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    s.a0[g] = *reinterpret_cast<const v4u*>(arow[g] + (size_t)j * 128);
    s.a1[g] = *reinterpret_cast<const v4u*>(arow[g] + (size_t)j * 128 + 64);
    s.sa[g] = as[g][(size_t)j * 4];
  }
}

// acc[g * NT + t]: token tile g, weight tile t
template <int NT, int NG>
__device__ __forceinline__ void dmma(const DStep<NT, NG>& s, v4f (&acc)[NG * NT]) {
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const v8i a = cat8(s.a0[g], s.a1[g]);
#pragma unroll
    for (int t = 0; t < NT; ++t)
      acc[g * NT + t] = mfma_fp8_fp8(a, cat8(s.b0[t], s.b1[t]), acc[g * NT + t], (int)s.sa[g], (int)s.sb[t]);
  }
}

// NW waves split the K-steps: with kIlv wave w takes steps w, w + NW, ...
// (the workgroup's waves read neighbouring tiles at any moment), else one
// contiguous range each.  NT row tiles per workgroup share each activation
// fragment, NG token tiles of 16 each weight tile (the workgroup then covers
// tokens 16 NG mt .. +16 NG).
template <int NW, int kB, int NT, bool kIlv, int NG>
__global__ __launch_bounds__(64 * NW) void dense_decode_kernel(const uint8_t* __restrict__ packed,
                                                               const uint8_t* __restrict__ xq,
                                                               const uint8_t* __restrict__ xs,
                                                               int T, int N, int K,
                                                               uint16_t* __restrict__ y) {
  const DenseLayout L(N, K);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int nt0 = blockIdx.x * NT, mt = blockIdx.y;
  const int ntiles = N / 16;
  const int J = L.J;
  // step u of this wave is K-step js + jstep * u, u < nsteps
  int js, jstep, nsteps;
  if (kIlv) {
    js = wave;
    jstep = NW;
    nsteps = J > wave ? (J - wave + NW - 1) / NW : 0;
  } else {
    js = (wave * J) / NW;
    jstep = 1;
    nsteps = ((wave + 1) * J) / NW - js;
  }
  // this lane's pieces: weight tile lane offset (tiles past N clamped to the
  // last one, never stored), activation rows 16 (NG mt + tg) + r (clamped the
  // same way)
  const uint8_t* wt[NT];
  const uint8_t* st[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int ntc = min(nt0 + t, ntiles - 1);
    wt[t] = packed + L.tile_off(ntc, 0) + lane * 16;
    st[t] = packed + L.scale_off(ntc, 0) + lane;
  }
  const uint8_t* arow[NG];
  const uint8_t* as[NG];
#pragma unroll
  for (int tg = 0; tg < NG; ++tg) {
    const int trow = min(16 * (NG * mt + tg) + r, T - 1);
    arow[tg] = xq + (size_t)trow * K + 16 * g;
    as[tg] = xs + (size_t)trow * (K / 32) + g;
  }

  v4f acc[NG * NT];
#pragma unroll
  for (int t = 0; t < NG * NT; ++t) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};
  DStep<NT, NG> s[kB];
  int u = 0;
  // whole batches: kB steps' loads back to back, then their MFMAs
  for (; u + kB <= nsteps; u += kB) {
#pragma unroll
    for (int b = 0; b < kB; ++b) dload<NT, NG>(s[b], wt, st, arow, as, js + jstep * (u + b));
#pragma unroll
    for (int b = 0; b < kB; ++b) dmma<NT, NG>(s[b], acc);
  }
  for (; u < nsteps; ++u) {
    dload<NT, NG>(s[0], wt, st, arow, as, js + jstep * u);
    dmma<NT, NG>(s[0], acc);
  }

  // fixed-order sum of the waves' partials, then bf16 stores of the valid tokens
  __shared__ v4f red[NW][NG * NT][64];
#pragma unroll
  for (int t = 0; t < NG * NT; ++t) red[wave][t][lane] = acc[t];
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int tg = 0; tg < NG; ++tg)
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (nt0 + t >= ntiles) break;
      v4f a = red[0][tg * NT + t][lane];
#pragma unroll
      for (int w = 1; w < NW; ++w) a += red[w][tg * NT + t][lane];
      const int n = 16 * (nt0 + t) + r;  // D column = weight row
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int tk = 16 * (NG * mt + tg) + 4 * g + v;  // D row = token
        if (tk < T) y[(size_t)tk * N + n] = f32_to_bf16(a[v]);
      }
    }
}

// ----------------------------------------------------------------- prefill
// Tile geometry: kWM x kWN waves, each owning kSM 16-token sub-tiles x 4
// weight tiles (64 rows); the workgroup tile is BM tokens x 16 BT weight rows.
// Per stage of 128 K the LDS holds A = BM x-rows (128 bytes each, swizzled),
// B = BT packed weight tiles, then one dword per thread: the scale dwords of
// the BM x rows, the 16 BT 4-byte runs of weight-tile scales, padding.
template <int kWM, int kWN, int kSM>
struct DCfg {
  static constexpr int NT = 64 * kWM * kWN;
  static constexpr int BM = kWM * 16 * kSM;
  static constexpr int BT = kWN * 4;
  static constexpr int A = BM * 128;
  static constexpr int B = BT * 2048;
  static constexpr int SA = BM * 4;
  static constexpr int STAGE = A + B + 4 * NT;
  static constexpr int RA = BM * 8 / NT;    // 16-byte x chunks per thread and stage
  static constexpr int RB = BT * 128 / NT;  // 16-byte weight chunks per thread and stage
  static_assert(BM + 16 * BT <= NT, "one scale dword per thread at most");
  static_assert(RA * NT == BM * 8 && RB * NT == BT * 128, "whole rounds of chunks");
};

template <class C>
struct DLoad {
  v4u a[C::RA], b[C::RB];
  uint32_t sc;  // threads < BM: x row tid's scale dword; others: 4 scale bytes of a weight tile
};

__device__ __forceinline__ int dswz(int row, int q) { return row * 128 + ((q ^ (row & 7)) << 4); }

// Global sources of one thread at K-step 0 (byte offsets, all < 2^32): x rows
// (tid >> 3) + (NT / 8) i at granule tid & 7; 16 bytes (tid & 127) of weight
// tiles (tid >> 7) + (NT / 128) i; one scale dword.
template <class C>
struct DSrc {
  uint32_t a[C::RA], b[C::RB];
  const uint8_t* sbase;    // xs (threads < BM) or packed
  uint32_t soff, sstep;    // scale dword offset at K-step 0, bytes per K-step
};

// Loads K-step min(j, J - 1); a step j >= J (the padding step of an odd
// count) is zeroed instead, so its products are exact zeros.
template <class C>
__device__ __forceinline__ void dense_gload(DLoad<C>& d, const uint8_t* __restrict__ xq,
                                            const uint8_t* __restrict__ packed, const DSrc<C>& g,
                                            int j, int J) {
  const uint32_t live = j < J ? ~0u : 0u;  // uniform: a mask, not a branch
  const uint32_t jj = (uint32_t)min(j, J - 1);
#pragma unroll
  for (int i = 0; i < C::RA; ++i)
    d.a[i] = *reinterpret_cast<const v4u*>(xq + (g.a[i] + 128u * jj)) & live;
#pragma unroll
  for (int i = 0; i < C::RB; ++i)
    d.b[i] = *reinterpret_cast<const v4u*>(packed + (g.b[i] + (uint32_t)DenseLayout::kTileStep * jj)) &
             live;
  d.sc = *reinterpret_cast<const uint32_t*>(g.sbase + (g.soff + g.sstep * jj));
}

template <class C>
__device__ __forceinline__ void dense_lstore(const DLoad<C>& d, uint8_t* buf, int tid) {
  const int lr = tid >> 3, lq = tid & 7;
#pragma unroll
  for (int i = 0; i < C::RA; ++i)
    *reinterpret_cast<v4u*>(buf + dswz(C::NT / 8 * i + lr, lq)) = d.a[i];
#pragma unroll
  for (int i = 0; i < C::RB; ++i)
    *reinterpret_cast<v4u*>(buf + C::A + ((tid >> 7) + C::NT / 128 * i) * 2048 + 16 * (tid & 127)) =
        d.b[i];
  *reinterpret_cast<uint32_t*>(buf + C::A + C::B + 4 * tid) = d.sc;
}

// One stage's 4 kSM MFMAs of a wave (kSM token sub-tiles x 4 weight tiles).
template <class C, int kSM>
__device__ __forceinline__ void dense_compute(v4f (&acc)[kSM][4], const uint8_t* cur, int wm,
                                              int wn, int lane) {
  const int r = lane & 15, g = lane >> 4;
  v8i b[4];
  int sb[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const uint8_t* tb = cur + C::A + (4 * wn + t) * 2048 + 16 * lane;
    b[t] = cat8(*reinterpret_cast<const v4u*>(tb), *reinterpret_cast<const v4u*>(tb + 1024));
    sb[t] = cur[C::A + C::B + C::SA + (4 * wn + t) * 64 + lane];
  }
#pragma unroll
  for (int i = 0; i < kSM; ++i) {
    const int row = 16 * kSM * wm + 16 * i + r;
    const v8i a = cat8(*reinterpret_cast<const v4u*>(cur + dswz(row, g)),
                       *reinterpret_cast<const v4u*>(cur + dswz(row, 4 + g)));
    const int sa = cur[C::A + C::B + 4 * row + g];
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[i][t] = mfma_fp8_fp8(a, b[t], acc[i][t], sa, sb[t]);
  }
}

// kSplit groups of kWM x kWN waves split the K-steps of one tile: group g
// runs the whole pipeline below on its own share with its own two LDS
// stages, and the groups' partial sums are added in group order at the end
// (for tiles too few to give every CU one).
// XCD-aware tile walk.  Workgroup b is dispatched to XCD b % 8; XCD x owns
// the contiguous run [x per, (x + 1) per) (per = ceil(tiles / 8)) of the
// tiles in panel order: column panels of SN = ceil(NTn / 4) weight-row tiles,
// row-major inside a panel.  So the tiles an XCD runs at once form a compact
// block (at 24 x 28 tiles: 12 token tiles x 7 row tiles per XCD) whose x rows
// and weight rows its L2 shares, instead of every XCD reading every token
// tile.  The grid is 8 per; a workgroup whose position is past the tiles
// returns at once (false).
__device__ __forceinline__ bool dense_tile_of(int NTm, int NTn, int b, int& bm, int& bn) {
  const int tiles = NTm * NTn, per = (tiles + 7) / 8;
  const int P = (b & 7) * per + (b >> 3);
  if (P >= tiles) return false;
  const int SN = (NTn + 3) / 4;
  const int sc = P / (NTm * SN), q = P - sc * (NTm * SN);
  const int w = min(SN, NTn - sc * SN);
  bm = q / w;
  bn = sc * SN + q % w;
  return true;
}

long dense_grid(long tiles) { return 8 * ((tiles + 7) / 8); }

template <int kWM, int kWN, int kSM, int kSets, int kSplit>
__global__ __launch_bounds__(64 * kWM * kWN * kSplit) void dense_prefill_kernel(
    const uint8_t* __restrict__ packed, const uint8_t* __restrict__ xq,
    const uint8_t* __restrict__ xs, int T, int N, int K, uint16_t* __restrict__ y) {
  using C = DCfg<kWM, kWN, kSM>;
  static_assert(kSplit == 1 || kSplit == 2, "one or two K groups");
  static_assert(kSplit == 1 || kWM * kWN * kSM * 4 * 64 * 16 <= 2 * C::STAGE,
                "a group's partial sums fit its two stages");
  __shared__ __attribute__((aligned(16))) uint8_t lds[kSplit * 2 * C::STAGE];
  const DenseLayout L(N, K);
  // (compile-time zero / identity without a split: the unsplit kernel keeps
  // its register count, and with it two workgroups per CU)
  const int grp = kSplit == 1 ? 0 : (int)threadIdx.x / C::NT;                 // K group
  const int tid = kSplit == 1 ? (int)threadIdx.x : (int)threadIdx.x % C::NT;  // thread in the group
  const int lane = tid & 63, wave = tid >> 6;   // wave within the group
  const int wm = wave / kWN, wn = wave % kWN;
  const int NTn = (N + 16 * C::BT - 1) / (16 * C::BT);
  const int NTm = (T + C::BM - 1) / C::BM;
  int bm, bn;
  if (!dense_tile_of(NTm, NTn, (int)blockIdx.x, bm, bn)) return;  // uniform: before any barrier
  const int m0 = bm * C::BM, nt0 = bn * C::BT;  // first token, first 16-row weight tile
  const int ntiles = N / 16;
  // this group's K-steps [j0, J) (J re-based as its end); steps past it load
  // zeros, like the padding step of an odd count
  const int Jg = kSplit == 1 ? L.J : (L.J + kSplit - 1) / kSplit;
  const int j0 = kSplit == 1 ? 0 : grp * Jg;
  const int J = kSplit == 1 ? L.J : min(L.J, j0 + Jg);

  DSrc<C> src;
#pragma unroll
  for (int i = 0; i < C::RA; ++i)
    src.a[i] = (uint32_t)min(m0 + C::NT / 8 * i + (tid >> 3), T - 1) * (uint32_t)K + 16 * (tid & 7);
  // weight tiles past N are clamped to the last one (their columns are never
  // stored), so each chunk keeps its own base
#pragma unroll
  for (int i = 0; i < C::RB; ++i)
    src.b[i] = (uint32_t)L.tile_off(min(nt0 + (tid >> 7) + C::NT / 128 * i, ntiles - 1), 0) +
               16 * (tid & 127);
  if (tid < C::BM) {
    src.sbase = xs;
    src.soff = (uint32_t)min(m0 + tid, T - 1) * (uint32_t)(K / 32);
    src.sstep = 4;
  } else {
    // weight-tile scales; threads past the last run re-read tile run 0 into the padding
    const int u = tid - C::BM < 16 * C::BT ? tid - C::BM : 0;
    src.sbase = packed;
    src.soff = (uint32_t)L.scale_off(min(nt0 + (u >> 4), ntiles - 1), 0) + 4 * (u & 15);
    src.sstep = (uint32_t)DenseLayout::kScaleStep;
  }

  v4f acc[kSM][4];
#pragma unroll
  for (int i = 0; i < kSM; ++i)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[i][t] = v4f{0.f, 0.f, 0.f, 0.f};

  // kSets = 2: stage j + 2 loads while j multiplies and j + 1 goes to the
  // idle buffer; kSets = 1: stage j + 1 loads while j multiplies.  The steps
  // run in pairs; an odd count gets a zero padding step (a step left over
  // after the loop would make the compiler rename the accumulators, doubling
  // their registers).
  // every group takes the same number of loop trips (the barriers are the
  // workgroup's): Jg rounded up to even
  const int J2 = Jg + (Jg & 1);
  uint8_t* const buf0 = kSplit == 1 ? lds : lds + grp * 2 * C::STAGE;
  uint8_t* const buf1 = buf0 + C::STAGE;
  if constexpr (kSets == 2) {
    DLoad<C> p, q;
    dense_gload<C>(p, xq, packed, src, j0, J);
    dense_gload<C>(q, xq, packed, src, j0 + 1, J);
    dense_lstore<C>(p, buf0, tid);
    __syncthreads();
    for (int j = j0; j < j0 + J2; j += 2) {
      dense_gload<C>(p, xq, packed, src, j + 2, J);
      dense_compute<C, kSM>(acc, buf0, wm, wn, lane);
      dense_lstore<C>(q, buf1, tid);
      __syncthreads();
      dense_gload<C>(q, xq, packed, src, j + 3, J);
      dense_compute<C, kSM>(acc, buf1, wm, wn, lane);
      dense_lstore<C>(p, buf0, tid);
      __syncthreads();
    }
  } else {
    DLoad<C> p;
    dense_gload<C>(p, xq, packed, src, j0, J);
    dense_lstore<C>(p, buf0, tid);
    __syncthreads();
    for (int j = j0; j < j0 + J2; j += 2) {
      dense_gload<C>(p, xq, packed, src, j + 1, J);
      dense_compute<C, kSM>(acc, buf0, wm, wn, lane);
      dense_lstore<C>(p, buf1, tid);
      __syncthreads();
      dense_gload<C>(p, xq, packed, src, j + 2, J);
      dense_compute<C, kSM>(acc, buf1, wm, wn, lane);
      dense_lstore<C>(p, buf0, tid);
      __syncthreads();
    }
  }
  if constexpr (kSplit == 2) {
    // group 1 parks its sums in its own (now idle) stages, group 0 adds them
    v4f* part = reinterpret_cast<v4f*>(lds + 2 * C::STAGE) + (wave * kSM * 4) * 64 + lane;
    if (grp == 1) {
#pragma unroll
      for (int i = 0; i < kSM; ++i)
#pragma unroll
        for (int t = 0; t < 4; ++t) part[(i * 4 + t) * 64] = acc[i][t];
    }
    __syncthreads();
    if (grp == 1) return;
#pragma unroll
    for (int i = 0; i < kSM; ++i)
#pragma unroll
      for (int t = 0; t < 4; ++t) acc[i][t] += part[(i * 4 + t) * 64];
  }

  // the wave's 4 tiles are 64 consecutive outputs of a token row: its 128
  // bytes go out in 4 consecutive stores (t inner)
  const int r = lane & 15, g = lane >> 4;
  const int n0 = 16 * (nt0 + 4 * wn);
#pragma unroll
  for (int i = 0; i < kSM; ++i)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int tok = m0 + 16 * kSM * wm + 16 * i + 4 * g + v;
      if (tok < T) {
        uint16_t* yrow = y + (size_t)tok * N + n0 + r;
#pragma unroll
        for (int t = 0; t < 4; ++t)
          if (n0 + 16 * t < N) yrow[16 * t] = f32_to_bf16(acc[i][t][v]);
      }
    }
}

// ------------------------------------------------- prefill, LDS-DMA ring
// 256 tokens x 256 weight rows per workgroup, 4 waves (one per SIMD, up to
// 512 registers each) in a 2 x 2 grid: wave (wm, wn) owns tokens 128 wm ..
// +128 (8 sub-tiles of 16) and weight tiles 8 wn .. 8 wn + 7 (128 rows), 64
// MFMAs per K-step on 256 fp32 accumulators (AGPRs).  Against the
// register-staged kernels a wave's tile is 2.7x larger, so the LDS fragment
// reads per flop drop by a third, and the operands of a K-step travel from
// global memory to LDS by LDS-DMA (no staging registers).  Two stages of
// 66 KiB: the activation rows (row r's 16-byte chunk c at physical chunk
// c ^ (r & 7), as in the expert GEMMs), the 16 weight tiles in packed order,
// the rows' scale dwords and the tiles' scale bytes.
// A K-step runs in two phases of 8 MFMA rows: phase 0 multiplies A fragment
// n with weight tiles 0-3, phase 1 fragment n with tiles 4-7, so only half of
// the weight fragments are live at a time.  Phase 1 opens with the step's one
// barrier (after two MFMAs, so the pipe stays busy across it): it publishes
// stage j + 1 and frees stage j's slot, whose refill (18 LDS-DMA loads per
// wave) is spread over the following rows, three loads per row -- with one
// wave per SIMD, any instruction that is not an MFMA keeps the matrix pipe
// idle unless an MFMA is in flight (issuing the loads at once after the
// barrier measured 11 % slower).  The next step's fragments are read in
// phase 1 as their registers free up, six or more rows before their use.
namespace dd {
constexpr int kBM = 256, kBN = 256;
constexpr int kA = kBM * 128;           // activation rows of a K-step
constexpr int kB = kBN * 128;           // 16 weight tiles of 2 KiB
constexpr int kSA = kBM * 4;            // a scale dword per row
constexpr int kSB = (kBN / 32) * 128;   // 8 weight-tile pairs x 128 scale bytes
constexpr int kStage = kA + kB + kSA + kSB;
constexpr int kLoads = 18;              // DMA loads per wave per stage
static_assert(kStage % 16 == 0, "stage alignment");
}  // namespace dd

// A wave's share of one stage's DMA: activation row groups w + 4u (u < 8, 8
// rows of 128 B each), weight pairs 2w, 2w + 1 (4 KiB each as four 1 KiB
// loads), the scale dwords of rows 64w .. 64w + 63 and the scale bytes of
// weight pairs 2w, 2w + 1.  Few registers: the activation offsets are formed
// at issue from the lane's first row (rows past T read row T - 1), the weight
// pairs' offsets live in scalar bases.
struct DDma {
  const uint8_t* b0;  // weight pair 2w (or the last pair), K-step 0
  const uint8_t* b1;  // weight pair 2w + 1
  int row;            // the lane's activation row in group w (tile-relative token + m0)
  uint32_t ach;       // the lane's 16-byte chunk: logical chunk (l%8) ^ (l/8) -- physical l%8
  uint32_t sa, sb;    // scale offsets
};

// Load k (< 18) of the wave's share of K-step j's stage: 0-7 activation row
// groups, 8-15 weight quarters, 16 row scales, 17 weight scales.
__device__ __forceinline__ void dd_issue1(const DDma& d, const uint8_t* xq, const uint8_t* xs,
                                          const uint8_t* psc, int T, int K, int j, uint32_t S,
                                          int wave, int lane, int k) {
  if (k < 8) {
    dma_x4(wave_ptr(xq + (size_t)j * 128), (uint32_t)min(d.row + 32 * k, T - 1) * (uint32_t)K + d.ach,
           S + 1024u * (uint32_t)(wave + 4 * k));
  } else if (k < 16) {
    const int u = k - 8;
    dma_x4(wave_ptr((u < 4 ? d.b0 : d.b1) + (size_t)j * DenseLayout::kTileStep + 1024 * (u & 3)),
           16u * (uint32_t)lane,
           S + (uint32_t)dd::kA + 4096u * (uint32_t)(2 * wave + (u >> 2)) + 1024u * (uint32_t)(u & 3));
  } else if (k == 16) {
    dma_x1(wave_ptr(xs + (size_t)j * 4), d.sa, S + (uint32_t)(dd::kA + dd::kB) + 256u * (uint32_t)wave);
  } else {
    dma_x1(wave_ptr(psc + (size_t)j * DenseLayout::kScaleStep), d.sb,
           S + (uint32_t)(dd::kA + dd::kB + dd::kSA) + 256u * (uint32_t)wave);
  }
}

__device__ __forceinline__ void dd_issue(const DDma& d, const uint8_t* xq, const uint8_t* xs,
                                         const uint8_t* psc, int T, int K, int j,
                                         uint32_t stage_lds, int wave, int lane) {
  const uint32_t S = wave_u32(stage_lds);
#pragma unroll
  for (int k = 0; k < dd::kLoads; ++k) dd_issue1(d, xq, xs, psc, T, K, j, S, wave, lane, k);
}

struct DDB {  // four weight fragments of a wave and their scale bytes
  v8i b[4];
  int sb[4];
};

// Per-lane LDS addresses of one stage slot, each the base of reads at small
// constant offsets (the DS offset field holds 16 bits; the slots reach past
// 64 KiB).  Laundered through an empty asm so that the compiler keeps them
// as bases instead of folding them into one address with large offsets.
struct DDAddr {
  uint32_t alo, ahi;  // A row 128 wm + lane % 16, chunks g and g + 4 (sub-tile i at +2048 i)
  uint32_t sa;        // its scale byte g (sub-tile i at +64 i)
  uint32_t b;         // weight tile 8 wn, this lane's 16 bytes (tile t at +2048 t, second KiB +1024)
  uint32_t sb;        // its scale byte (tile t at +64 t)
};

__device__ __forceinline__ uint32_t opaque(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}

// The accumulating MFMA with its C operand tied to an AGPR tuple: with 256
// accumulators per wave the compiler, left to itself, gives part of the
// MFMAs a fresh destination and copies the accumulator (four moves and a
// hazard wait per MFMA).  The asm is volatile and ordered with memory, so
// that the MFMAs keep their order with the barrier and the DMA issue and every
// LDS read stays where the loop below puts it: its A, B and scale operands
// are read at issue, and each register is overwritten only a row of MFMAs or
// more after its last use, so no wait states are needed inside the loop; the
// epilogue waits before reading the accumulators.
__device__ __forceinline__ void dd_mfma(v4f& c, const v8i& a, const v8i& b, int sa, int sb) {
  asm volatile("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0]"
               : "+a"(c)
               : "v"(a), "v"(b), "v"(sa), "v"(sb)
               : "memory");
}

__device__ __forceinline__ DDAddr dd_addr(uint32_t slot, int wm, int wn, int lane) {
  const int r = lane & 15, g = lane >> 4;
  const int row = 128 * wm + r;
  DDAddr a;
  a.alo = opaque(slot + (uint32_t)dswz(row, g));
  a.ahi = opaque(slot + (uint32_t)dswz(row, g + 4));
  a.sa = opaque(slot + (uint32_t)(dd::kA + dd::kB + 4 * row + g));
  a.b = opaque(slot + (uint32_t)(dd::kA + 16384 * wn + 16 * lane));
  a.sb = opaque(slot + (uint32_t)(dd::kA + dd::kB + dd::kSA + 512 * wn + lane));
  return a;
}

__device__ __forceinline__ v4u lds_v4(uint32_t addr) {
  return *reinterpret_cast<const __attribute__((address_space(3))) v4u*>((uintptr_t)addr);
}
__device__ __forceinline__ int lds_u8v(uint32_t addr) {
  return *reinterpret_cast<const __attribute__((address_space(3))) uint8_t*>((uintptr_t)addr);
}

// weight tiles 4h .. 4h + 3 of the wave
__device__ __forceinline__ void dd_read_b(DDB& f, const DDAddr& a, int h) {
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    f.b[t] = cat8(lds_v4(a.b + 2048 * (4 * h + t)), lds_v4(a.b + 2048 * (4 * h + t) + 1024));
    f.sb[t] = lds_u8v(a.sb + 64 * (4 * h + t));
  }
}

__device__ __forceinline__ void dd_read_a(v8i& av, int& sa, const DDAddr& a, int i) {
  av = cat8(lds_v4(a.alo + 2048 * i), lds_v4(a.ahi + 2048 * i));
  sa = lds_u8v(a.sa + 64 * i);
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void dense_dma_kernel(
    const uint8_t* __restrict__ packed, const uint8_t* __restrict__ xq,
    const uint8_t* __restrict__ xs, int T, int N, int K, uint16_t* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * dd::kStage];
  const DenseLayout L(N, K);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int NTn = (N + dd::kBN - 1) / dd::kBN, NTm = (T + dd::kBM - 1) / dd::kBM;
  int bm, bn;
  if (!dense_tile_of(NTm, NTn, (int)blockIdx.x, bm, bn)) return;  // uniform: before any barrier
  const int m0 = bm * dd::kBM, g0 = bn * (dd::kBN / 32);  // first token, first 32-row weight pair
  const int ngroups = N / 32, J = L.J;

  DDma d;
  d.row = m0 + 8 * wave + (lane >> 3);
  d.ach = (uint32_t)(((lane & 7) ^ (lane >> 3)) << 4);
  // weight pairs past N read the last pair (their columns are never stored)
  d.b0 = wave_ptr(packed + (size_t)min(g0 + 2 * wave, ngroups - 1) * J * DenseLayout::kTileStep);
  d.b1 = wave_ptr(packed + (size_t)min(g0 + 2 * wave + 1, ngroups - 1) * J * DenseLayout::kTileStep);
  d.sa = (uint32_t)min(m0 + 64 * wave + lane, T - 1) * (uint32_t)(K / 32);
  {
    const int gg = min(g0 + 2 * wave + (lane >> 5), ngroups - 1);
    d.sb = (uint32_t)((size_t)gg * J * DenseLayout::kScaleStep) + 4u * (uint32_t)(lane & 31);
  }
  const uint8_t* psc = packed + L.s_off;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_u8*)lds;

  v4f acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[i][t] = v4f{0.f, 0.f, 0.f, 0.f};

  dd_issue(d, xq, xs, psc, T, K, 0, lds0, wave, lane);
  dd_issue(d, xq, xs, psc, T, K, 1, lds0 + dd::kStage, wave, lane);
  wait_vmcnt<dd::kLoads>();
  __syncthreads();
  const DDAddr ad0 = dd_addr(lds0, wm, wn, lane), ad1 = dd_addr(lds0 + dd::kStage, wm, wn, lane);
  // Registers: the step's 8 A fragments, blo = weight tiles 0-3, bhi = tiles
  // 4-7.  Phase 0 (rows n = 0..7) multiplies fragment n with tiles 0-3,
  // phase 1 (n = 8..15) fragment n - 8 with tiles 4-7.  bhi is read at the
  // second row; after it nothing reads stage j but fragments 6 and 7 (read at
  // the first two rows), so phase 1 opens with the step's barrier and the
  // refill of stage j's slot, then reads the next step's tiles 0-3 (blo is
  // free) and its fragments one by one, each a row after its register's last
  // use (fragment f at row 10 + f; 6 and 7 at the next step's rows 0 and 1),
  // so every fragment is read six or more rows of MFMAs before it is used.
  DDB blo, bhi;
  v8i af[8];
  int sf[8];
  dd_read_b(blo, ad0, 0);
#pragma unroll
  for (int f = 0; f < 6; ++f) dd_read_a(af[f], sf[f], ad0, f);

  auto step = [&](int j) {
    const DDAddr& S = (j & 1) ? ad1 : ad0;
    const DDAddr& Sn = (j & 1) ? ad0 : ad1;
#pragma unroll
    for (int n = 0; n < 16; ++n) {
      const int ph = n >> 3, i = n & 7;
      if (n < 2) dd_read_a(af[6 + n], sf[6 + n], S, 6 + n);
      if (n == 1) dd_read_b(bhi, S, 1);
      if (n == 8) wait_vmcnt<0>();  // stage j + 1, the last one issued
      if (n >= 10) dd_read_a(af[n - 10], sf[n - 10], Sn, n - 10);
      const DDB& bb = ph ? bhi : blo;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        dd_mfma(acc[i][4 * ph + t], af[i], bb.b[t], sf[i], bb.sb[t]);
        if (n == 8 && t == 1) {
          // two MFMAs in the pipe across the barrier, which publishes stage
          // j + 1 and frees stage j's slot; then the next step's tiles 0-3
          // (past the last K-step the last stage is loaded again and read,
          // never used: the step has no branch)
          __syncthreads();
          dd_read_b(blo, Sn, 0);
        }
        // the refill of stage j's slot: three of its 18 loads after the
        // second MFMA of each of phase 1's first six rows
        if (n >= 8 && n < 14 && t == 1) {
          const int jn = min(j + 2, J - 1);
          const uint32_t Sl = wave_u32(lds0 + (uint32_t)((j & 1) * dd::kStage));
          const int k0 = 3 * (n - 8);
#pragma unroll
          for (int k = k0; k < k0 + 3; ++k) dd_issue1(d, xq, xs, psc, T, K, jn, Sl, wave, lane, k);
        }
      }
    }
  };
  for (int j = 0; j < J; j += 2) {
    step(j);
    step(j + 1);
  }
  // the last MFMAs' results are read below: 48 wait states (more than any
  // MFMA's read-after-write distance), then the DMA of the stage loaded
  // past the last K-step
  asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 15\n\ts_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int t = 0; t < 8; ++t) asm volatile("" : "+a"(acc[i][t]));

  // lane holds tokens 4g + v of column r of each 16 x 16 block; a token row's
  // 256 bytes of the wave go out in 8 consecutive stores (t inner)
  const int r = lane & 15, g = lane >> 4;
  const int n0 = 32 * g0 + 128 * wn;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int tok = m0 + 128 * wm + 16 * i + 4 * g + v;
      if (tok < T) {
        uint16_t* yrow = y + (size_t)tok * N + n0 + r;
#pragma unroll
        for (int t = 0; t < 8; ++t)
          if (n0 + 16 * t < N) yrow[16 * t] = f32_to_bf16(acc[i][t][v]);
      }
    }
}

// The two geometries: 128 x 128 (4 waves) and 192 x 256 (8 waves; 256 x 256 does
// not fit 2 waves per SIMD without spills).  The large tile stages fewer bytes
// per flop (11 % faster on 4604 tokens) but a workgroup of either runs its
// whole K range, so below a few thousand tokens the time is set by how many
// rounds of workgroups the CUs take: two small workgroups share a CU, one
// large one fills it, and a round of large tiles measured 1.16x a round of
// small ones (K 16384, N 7168; T from 97 to 4604).
constexpr int kLWM = 2, kLWN = 4, kLSM = 6, kLSets = 2;
using DSmall = DCfg<2, 2, 4>;
using DLarge = DCfg<kLWM, kLWN, kLSM>;

// Resident workgroups per CU of each geometry and the CU count, once per device.
struct DenseOccupancy {
  int ncu = 0, small = 0, large = 0;
};

// (Packed in one atomic word per device: concurrent first calls from several
// host threads store the same value.)
DenseOccupancy dense_occupancy() {
  static std::atomic<uint64_t> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  const uint64_t w = cached[dev].load(std::memory_order_relaxed);
  if (w != 0) {
    DenseOccupancy o;
    o.ncu = (int)(w & 0xFFFFFu);
    o.small = (int)((w >> 20) & 0xFFFFFu);
    o.large = (int)(w >> 40);
    return o;
  }
  {
    DenseOccupancy n;
    if (hipDeviceGetAttribute(&n.ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n.ncu < 1)
      n.ncu = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &n.small, reinterpret_cast<const void*>(&dense_prefill_kernel<2, 2, 4, 2, 1>), DSmall::NT,
            0) != hipSuccess || n.small < 1)
      n.small = 1;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &n.large,
            reinterpret_cast<const void*>(&dense_prefill_kernel<kLWM, kLWN, kLSM, kLSets, 1>),
            DLarge::NT, 0) != hipSuccess || n.large < 1)
      n.large = 1;
    cached[dev].store((uint64_t)(n.ncu & 0xFFFFF) | ((uint64_t)(n.small & 0xFFFFF) << 20) |
                          ((uint64_t)n.large << 40),
                      std::memory_order_relaxed);
    return n;
  }
}

}  // namespace

hipError_t launch_dense_pack(const uint8_t* wq, const uint8_t* ws, int N, int K, uint8_t* packed,
                             hipStream_t s) {
  const long threads = (long)(N / 16) * (K / 128) * 64;
  hipLaunchKernelGGL(dense_pack_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s,
                     wq, ws, N, K, packed);
  return hipGetLastError();
}

hipError_t launch_dense_decode(const uint8_t* packed, const uint8_t* xq, const uint8_t* xs, int T,
                               int N, int K, uint16_t* y, hipStream_t s) {
  constexpr int kNW = 16, kBt = 2, kNT = 2;
  constexpr bool kIl = true;
  // from 17 tokens two token tiles share each pass over the weights
  if (T > 16) {
    const dim3 grid((unsigned)((N / 16 + kNT - 1) / kNT), (unsigned)((T + 31) / 32));
    hipLaunchKernelGGL((dense_decode_kernel<kNW, kBt, kNT, kIl, 2>), grid, dim3(64 * kNW), 0, s,
                       packed, xq, xs, T, N, K, y);
  } else {
    const dim3 grid((unsigned)((N / 16 + kNT - 1) / kNT), (unsigned)((T + 15) / 16));
    hipLaunchKernelGGL((dense_decode_kernel<kNW, kBt, kNT, kIl, 1>), grid, dim3(64 * kNW), 0, s,
                       packed, xq, xs, T, N, K, y);
  }
  return hipGetLastError();
}

hipError_t launch_dense_prefill(const uint8_t* packed, const uint8_t* xq, const uint8_t* xs, int T,
                                int N, int K, uint16_t* y, hipStream_t s) {
  const DenseOccupancy occ = dense_occupancy();
  const long wg_small = (long)((T + DSmall::BM - 1) / DSmall::BM) *
                        ((N + 16 * DSmall::BT - 1) / (16 * DSmall::BT));
  const long wg_large = (long)((T + DLarge::BM - 1) / DLarge::BM) *
                        ((N + 16 * DLarge::BT - 1) / (16 * DLarge::BT));
  const long wg_dma = (long)((T + dd::kBM - 1) / dd::kBM) * ((N + dd::kBN - 1) / dd::kBN);
  const long slots_small = (long)occ.small * occ.ncu, slots_large = (long)occ.large * occ.ncu;
  const long rounds_small = (wg_small + slots_small - 1) / slots_small;
  const long rounds_large = (wg_large + slots_large - 1) / slots_large;
  const long rounds_dma = (wg_dma + occ.ncu - 1) / occ.ncu;  // one per CU (its LDS)
  // Each geometry's time is its rounds of workgroups times its round time,
  // measured at K 16384, N 7168 against a round of small tiles: 1.16 for the
  // 192 x 256 tiles, 1.06 for the 256 x 256 LDS-DMA kernel (which needs an
  // even K-step count).
  const long t_small = 100 * rounds_small, t_large = 116 * rounds_large;
  if ((K / 128) % 2 == 0 && 106 * rounds_dma < (t_small < t_large ? t_small : t_large)) {
    hipLaunchKernelGGL(dense_dma_kernel, dim3((unsigned)dense_grid(wg_dma)), dim3(256), 0, s, packed, xq,
                       xs, T, N, K, y);
  } else if (t_large < t_small) {
    hipLaunchKernelGGL((dense_prefill_kernel<kLWM, kLWN, kLSM, kLSets, 1>), dim3((unsigned)dense_grid(wg_large)),
                       dim3(DLarge::NT), 0, s, packed, xq, xs, T, N, K, y);
  } else if (wg_small <= occ.ncu) {
    // fewer small tiles than CUs: each tile's K-steps split over two wave groups
    hipLaunchKernelGGL((dense_prefill_kernel<2, 2, 4, 2, 2>), dim3((unsigned)dense_grid(wg_small)),
                       dim3(2 * DSmall::NT), 0, s, packed, xq, xs, T, N, K, y);
  } else {
    hipLaunchKernelGGL((dense_prefill_kernel<2, 2, 4, 2, 1>), dim3((unsigned)dense_grid(wg_small)),
                       dim3(DSmall::NT), 0, s, packed, xq, xs, T, N, K, y);
  }
  return hipGetLastError();
}

}  // namespace moe
