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
// (expert, first sorted row) of up to kBM rows, on the device; no count is
// ever read back to the host.  A work item is a (token tile, feature tile)
// pair.  kBM = 192 covers a whole expert at the prefill shape (113-180 rows
// per expert), so each expert's packed weights stream from HBM once per
// feature tile; 16-row sub-tiles past the expert's last row are skipped, so a
// short tile costs MFMA issue in proportion to its real rows.
//
// Persistent workgroups: one per compute unit (its LDS ring allows no
// second), 8 waves, two per SIMD.  The dispatcher deals workgroups
// round-robin to the 8 XCDs; each XCD owns an equal contiguous share of the
// items that exist, so the feature tiles of one token tile (which share its
// activation rows) sit on one XCD and its L2, and a workgroup walks its XCD's
// share with a fixed stride.  The LDS ring runs on across items: the last
// three K-steps of an item already load the next item's first three stages
// (and the row sources of the item after that), so the ring never drains and
// the epilogue of one item overlaps the next item's first loads.
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
// head's MFMAs; midway, one barrier publishes the next stage and frees the
// current slot, which is refilled, and the next head is read -- before the
// tail's MFMAs by one wave of each SIMD, after them by the other, so that
// the two waves' LDS reads and DMA issue do not coincide and one of them
// keeps the matrix pipe busy.  So LDS reads, DMA issue and the barrier all
// overlap MFMA work; the loop's only branches are on the wave's token half.
//
// Waves form a 2 (tokens) x 4 (features) grid, wm = wave / 4 so that each
// SIMD holds one wave of each token half: a wave owns the 16-row sub-tiles
// {wm, wm+2, ..., wm+10} and 4 weight tiles (up to 24 MFMAs per K-step); for
// the gate/up GEMM a wave's 4 tiles are one 32-feature group of W1 and W3, so
// SwiGLU stays in its registers.  The number of live sub-tiles is a
// compile-time parameter of the loop body, selected once per wave, so the
// MFMA stream has no conditionals and only live accumulators are allocated.
#include <atomic>

#include "lds_dma.h"

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

// An FP4 operand occupies the low 4 registers of the 8-register operand;
// the upper half is left undefined so no registers are spent on it.
__device__ __forceinline__ v8i widen_fp4(uint4 b) {
  const v4i v = v4i{(int)b.x, (int)b.y, (int)b.z, (int)b.w};
  return __builtin_shufflevector(v, v, 0, 1, 2, 3, -1, -1, -1, -1);
}


// The five 16-byte loads of a wave's stage (three activation row groups from
// one base, two weight tiles from another) in one block, M0 saved once.
__device__ __forceinline__ void dma_stage5(const uint8_t* abase, uint32_t a0, uint32_t a1,
                                           uint32_t a2, const uint8_t* bbase, uint32_t b0,
                                           uint32_t b1, uint32_t la0, uint32_t la1, uint32_t la2,
                                           uint32_t lb0, uint32_t lb1) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %8\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %4\n\t"
      "s_mov_b32 m0, %9\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, %4\n\t"
      "s_mov_b32 m0, %10\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %3, %4\n\t"
      "s_mov_b32 m0, %11\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %5, %7\n\t"
      "s_mov_b32 m0, %12\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %6, %7\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(a0), "v"(a1), "v"(a2), "s"(abase), "v"(b0), "v"(b1), "s"(bbase), "s"(la0),
        "s"(la1), "s"(la2), "s"(lb0), "s"(lb1)
      : "memory");
}

// The token-tile list, built by one wave: tiles of kBM sorted rows, expert by
// expert in order (tile (e, o0 + i kBM) for i < ceil(rows_e / kBM)); the
// count at hdr[0], the (expert, first row) pairs from byte kTileHdr.  Round j
// takes experts 64 j .. 64 j + 63, one per lane: a wave-wide inclusive scan of
// their tile counts, on top of the rounds before, places each expert's tiles;
// then the wave writes the round's tiles 64 at a time, each lane finding the
// expert of its tile by binary search over the scan (an expert with many
// tiles is not left to one lane).
__device__ void build_tiles_wave(const int32_t* __restrict__ offsets, int E, int* __restrict__ hdr) {
  const int lane = threadIdx.x & 63;
  int2* tiles = reinterpret_cast<int2*>(reinterpret_cast<uint8_t*>(hdr) + kTileHdr);
  // every round's offsets in one batch of loads (E <= 1024: at most 16 rounds)
  constexpr int kRounds = 16;
  int lo_off[kRounds], hi_off[kRounds];
#pragma unroll
  for (int j = 0; j < kRounds; ++j) {
    lo_off[j] = offsets[min(64 * j + lane, E)];
    hi_off[j] = offsets[min(64 * j + lane + 1, E)];
  }
  int base = 0;
#pragma unroll
  for (int j = 0; j < kRounds; ++j) {
    const int e0 = 64 * j;
    if (e0 >= E) break;
    const int o0 = lo_off[j];
    const int m = (hi_off[j] - o0 + kBM - 1) / kBM;  // 0 past the last expert
    int incl = m;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int v = __shfl_up(incl, d);
      if (lane >= d) incl += v;
    }
    const int n = __shfl(incl, 63);
    for (int i0 = 0; i0 < n; i0 += 64) {  // uniform: every lane takes part in the shuffles
      const int i = i0 + lane;
      int lo = 0;  // first lane whose inclusive count exceeds i (63 when i >= n)
#pragma unroll
      for (int step = 32; step > 0; step >>= 1)
        if (__shfl(incl, lo + step - 1) <= i) lo += step;
      const int first = __shfl(incl - m, lo), row0 = __shfl(o0, lo);
      if (i < n) tiles[base + i] = make_int2(e0 + lo, row0 + (i - first) * kBM);
    }
    base += n;
  }
  if (lane == 0) hdr[0] = base;
}

// One wave's share of the DMA loads of a stage, the part that changes from
// one work item to the next: bases at K-step 0 (each advances by a fixed
// stride per K-step) and per-lane source offsets.  The LDS destinations and
// strides follow from the wave index (issue_stage).
struct Dma {
  const uint8_t* abase;  // activation rows
  const uint8_t* bbase;  // the wave's first weight tile
  const uint8_t* sbase;  // scales (waves 0-3)
  uint32_t aoff[3];      // this lane's chunk of row groups w, w+8, w+16
  uint32_t soff;         // this lane's scale bytes
};

// The per-wave constant part of the DMA: which scale load the wave issues
// (0: none, 1: activation scale dwords, 2: weight scales as dwordx4), its
// K-step stride and LDS offset within a stage, and the lane's weight offset.
struct WaveDma {
  int skind;
  long sstep;
  uint32_t ls;
  uint32_t boff0;
};

// Stage j of descriptor d into the stage at LDS address stage_lds.  Wave w
// writes activation row groups w, w+8, w+16 (1 KiB each at 1024 rg), weight
// tiles 2w, 2w+1 (at kABytes + 1024 t), and its scale load (see WaveDma).
template <bool kUp>
__device__ __forceinline__ void issue_stage(const Dma& d, const WaveDma& c, uint32_t stage_lds_,
                                            int j, int wave) {
  const uint32_t stage_lds = wave_u32(stage_lds_);
  if (c.skind == 1)
    dma_x1(wave_ptr(d.sbase + (size_t)j * c.sstep), d.soff, stage_lds + c.ls);
  else if (c.skind == 2)
    dma_x4(wave_ptr(d.sbase + (size_t)j * c.sstep), d.soff, stage_lds + c.ls);
  const uint32_t la = stage_lds + (uint32_t)(1024 * wave);
  const uint32_t lb = stage_lds + (uint32_t)(kABytes + 2048 * wave);
  dma_stage5(wave_ptr(d.abase + (size_t)j * 128), d.aoff[0], d.aoff[1], d.aoff[2],
             wave_ptr(d.bbase + (size_t)j * (kUp ? 4096 : 2048)), c.boff0, c.boff0 + 1024u, la,
             la + 8192u, la + 16384u, lb, lb + 1024u);
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
  uint32_t sb[2];  // up: sb[0] holds the 4 tiles' scale bytes; down: sb[u] the pair of q2-group u
  v8i a[FragsShape<N>::kHead > 0 ? FragsShape<N>::kHead : 1];
  uint32_t sa[FragsShape<N>::kHead > 0 ? FragsShape<N>::kHead : 1];
};

template <int N>
struct Tail {
  v8i a[FragsShape<N>::kTail > 0 ? FragsShape<N>::kTail : 1];
  uint32_t sa[FragsShape<N>::kTail > 0 ? FragsShape<N>::kTail : 1];
};

// Per-lane LDS byte offsets (within a stage) of the wave's fragments; the
// fragment of sub-tile i, weight tile t is at a fixed distance from them, so
// every LDS read of a step is one base plus an immediate offset.
struct Lds {
  int a_lo, a_hi;  // activation row 16 wm + l%16, K chunks g and g+4 (swizzled)
  int a_s;         // that row's scale byte of block g (a byte read: no unpacking)
  int b;           // weight tile 0 of the wave, this lane's 16 bytes
  int b_s;         // up: the lane's scale dword; down: its 16-bit scale pair in q2-group 2wn
};

__device__ __forceinline__ void read_a(v8i& a, uint32_t& sa, const uint8_t* S, const Lds& o, int i) {
  const uint4 lo = *reinterpret_cast<const uint4*>(S + o.a_lo + 4096 * i);
  const uint4 hi = *reinterpret_cast<const uint4*>(S + o.a_hi + 4096 * i);
  a = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  sa = S[o.a_s + 128 * i];
}

template <bool kUp, int N>
__device__ __forceinline__ void read_head(Head<N>& f, const uint8_t* S, const Lds& o) {
#pragma unroll
  for (int t = 0; t < 4; ++t)
    f.b[t] = *reinterpret_cast<const uint4*>(S + o.b + (kUp ? 1024 * t : 2048 * (t >> 1) + 1024 * (t & 1)));
  if (kUp) {
    f.sb[0] = *reinterpret_cast<const uint32_t*>(S + o.b_s);
  } else {
    f.sb[0] = *reinterpret_cast<const uint16_t*>(S + o.b_s);
    f.sb[1] = *reinterpret_cast<const uint16_t*>(S + o.b_s + 128);
  }
#pragma unroll
  for (int i = 0; i < FragsShape<N>::kHead; ++i) read_a(f.a[i], f.sa[i], S, o, i);
}

template <int N>
__device__ __forceinline__ void read_tail(Tail<N>& f, const uint8_t* S, const Lds& o) {
#pragma unroll
  for (int i = 0; i < FragsShape<N>::kTail; ++i)
    read_a(f.a[i], f.sa[i], S, o, FragsShape<N>::kHead + i);
}

// One 16x16 block of the product.  Gate/up computes the transposed block:
// the weight tile is the MFMA's A operand (FP4, 16 features x 128 K) and the
// activation fragment its B operand (FP8, 128 K x 16 tokens) -- the two
// operands' lane layouts are the same (lane l: row or column l%16, K block
// l/16), so a fragment serves either way round -- and the result holds
// features 4(l/16)..4(l/16)+3 of token l%16 in lane l, so the epilogue
// writes each token's 4 fp8 codes as one dword.  Down keeps activations as A:
// lane l holds tokens 4(l/16)..+3 of feature l%16, and its bf16 stores of 16
// lanes fill 32 bytes of 4 rows -- measured faster than 8-byte stores that
// touch 16 rows each.  Weight tile t's scale: byte t of the up dword, byte
// t&1 of the down pair of q2-group t>>1 -- selected by the MFMA's scale
// operand byte select.
template <bool kUp, int T>
__device__ __forceinline__ v4f mfma_t(v8i a, uint32_t sa, uint4 b, const uint32_t* sb, v4f c) {
  if (kUp)
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(widen_fp4(b), a, c, 4, 0, T, (int)sb[0], 0, (int)sa);
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, widen_fp4(b), c, 0, 4, 0, (int)sa, T & 1,
                                                          (int)sb[T >> 1]);
}

template <bool kUp, int N>
__device__ __forceinline__ void mfma_row(v8i a, uint32_t sa, const Head<N>& h, v4f (&acc)[4]) {
  acc[0] = mfma_t<kUp, 0>(a, sa, h.b[0], h.sb, acc[0]);
  acc[1] = mfma_t<kUp, 1>(a, sa, h.b[1], h.sb, acc[1]);
  acc[2] = mfma_t<kUp, 2>(a, sa, h.b[2], h.sb, acc[2]);
  acc[3] = mfma_t<kUp, 3>(a, sa, h.b[3], h.sb, acc[3]);
}

template <bool kUp, int N>
__device__ __forceinline__ void mfma_head(const Head<N>& f, v4f (&acc)[N][4]) {
#pragma unroll
  for (int i = 0; i < FragsShape<N>::kHead; ++i) mfma_row<kUp, N>(f.a[i], f.sa[i], f, acc[i]);
}

template <bool kUp, int N>
__device__ __forceinline__ void mfma_tail(const Head<N>& h, const Tail<N>& f, v4f (&acc)[N][4]) {
#pragma unroll
  for (int i = 0; i < FragsShape<N>::kTail; ++i)
    mfma_row<kUp, N>(f.a[i], f.sa[i], h, acc[FragsShape<N>::kHead + i]);
}

// Launch constants of a GEMM.  The kernel's prologue parks them in LDS and
// each work item re-reads them there, so none holds a register across the
// K-loop.  Weight block (e, g, j) (g: 32-row group, j: K-step) starts at
// wbase + ((e*QG + g)*J + j) * 4096 (gate/up) or 2048 (down) bytes, its scales
// at sbase + (...) * 256 or 128.
struct KArgs {
  const uint8_t* wbase;
  const uint8_t* sbase;
  const uint8_t* act;         // activations: x (gate/up) or h (down), fp8 rows of K bytes
  const uint32_t* sT;         // activation scales by K-step
  const int32_t* sorted_pair;
  const int32_t* offsets;
  const int* hdr;             // tile count, then the tile list at kTileHdr
  uint8_t* hq;
  uint8_t* hs;
  uint16_t* O;
  long P;
  int k, NF, H, I, QG, J;
  int hs_by_step;             // gate/up: hs in the down GEMM's K-step layout (sT)
};

// One work item of a workgroup: a token tile (expert e, sorted rows m0 ..
// m0 + rows) and a feature tile ft, with this wave's DMA descriptor for it.
struct Item {
  Dma d;
  int e, m0, rows, ft;
};

// Tile of work item `it`: expert, first sorted row, rows, feature tile.  The
// tile list and the offsets are not written by the GEMM kernels, so they are
// read as constant memory: uniform scalar loads, whose wait is not the
// vector-memory count (a vector load's wait would also wait for the ring's
// DMA).
__device__ __forceinline__ void item_tile(const int* __restrict__ hdr,
                                          const int32_t* __restrict__ offsets, int NF, int it,
                                          int& e, int& m0, int& rows, int& ft) {
  typedef __attribute__((address_space(4))) const int32_t cint;  // read-only here
  const int tile = __builtin_amdgcn_readfirstlane(it / NF);
  ft = it - tile * NF;
  cint* tl = (cint*)(reinterpret_cast<const uint8_t*>(hdr) + kTileHdr);
  e = tl[2 * tile];
  m0 = tl[2 * tile + 1];
  rows = min(kBM, ((cint*)offsets)[e + 1] - m0);
}

// A pointer re-read from LDS, known again to address global memory, so that
// accesses through it are global (not flat) instructions.
template <class T>
__device__ __forceinline__ __attribute__((address_space(1))) T* as_global(T* p) {
  return (__attribute__((address_space(1))) T*)p;
}

// The wave's DMA descriptor of an item.  rsrc (LDS, gate/up only) holds the
// sorted pair index of each tile row, rows past the tile repeating the last
// one; the token row is the pair index / k.  Down reads rows m0 .. of h in
// sorted order, rows past the tile repeating the last.
template <bool kUp>
__device__ __forceinline__ void make_dma(Item& it, const int* rsrc, const KArgs& a, int wave,
                                         int lane_) {
  // Down GEMM: the lane index recomputed here from the exec mask (all lanes
  // are active; the asm is not hoisted), so that no register carries it
  // across the K loop -- the down kernel's register budget is full.
  int lane = lane_;
  if (!kUp) asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane));
  Dma& d = it.d;
  const int K = kUp ? a.H : a.I;
  const int e = it.e, m0 = it.m0, rows = it.rows, ft = it.ft;
  // Activations: row group rg = wave + 8u (u < 3) holds rows 8rg..8rg+7,
  // 1 KiB at stage offset 1024 rg; lane l lands at row 8rg + l/8, physical
  // chunk l%8, which holds logical chunk (l%8) ^ (l/8) (the row's low 3 bits
  // are l/8).  Offsets are from the activation base (token rows for gate/up,
  // the tile's first sorted row for down); rows past the tile load the last
  // row again, and their products land in output rows that are never stored.
  d.abase = kUp ? a.act : a.act + (size_t)m0 * K;
#pragma unroll
  for (int u = 0; u < 3; ++u) {
    const int r = 8 * (wave + 8 * u) + (lane >> 3);
    const size_t src = kUp ? (size_t)(rsrc[r] / a.k) : (size_t)min(r, rows - 1);
    d.aoff[u] = (uint32_t)(src * K) + (uint32_t)(((lane & 7) ^ (lane >> 3)) << 4);
  }
  // Weights: stage tiles 2w, 2w+1 (1 KiB each, lane order = packed order),
  // adjacent in the packed layout.  up: tile index 4g + t = q-group 4ft + g,
  // tile t; down: tile index 2g2 + t = q2-group 8ft + g2, tile t (groups past
  // H read group 0, whose products are never stored).
  const size_t eJ = (size_t)e * a.QG;
  if (kUp) {
    d.bbase = a.wbase + (eJ + 4 * ft + (wave >> 1)) * a.J * 4096 + (size_t)(2 * (wave & 1)) * 1024;
  } else {
    const int g2 = 8 * ft + wave;
    d.bbase = a.wbase + (eJ + (g2 < a.QG ? g2 : 0)) * a.J * 2048;
  }
  // Scales.  Waves 0-2: activation scale dwords of rows 64w..64w+63 (as[row])
  // from the by-step array, one contiguous run per K-step (rows past the
  // tile read its last row).  Wave 3: all weight scales of the K-step as one
  // dwordx4 load, 16 bytes per lane: up: lanes 16g..16g+15 take q-group
  // 4ft + g's 256 bytes (bs[64g + d]); down: lanes 8g2..8g2+7 take q2-group
  // 8ft + g2's 128 bytes (bs[32 g2 + d]).
  if (wave < 3) {
    d.sbase = reinterpret_cast<const uint8_t*>(a.sT + m0);
    d.soff = (uint32_t)(min(64 * wave + lane, rows - 1) * 4);
  } else if (wave == 3) {
    if (kUp) {
      d.sbase = a.sbase + (eJ + 4 * ft) * a.J * 256;
      d.soff = (uint32_t)((lane >> 4) * a.J * 256 + (lane & 15) * 16);
    } else {
      const int g2 = 8 * ft + (lane >> 3);
      d.sbase = a.sbase + (eJ + 8 * ft) * a.J * 128;
      d.soff = (uint32_t)((g2 < a.QG ? (lane >> 3) : 0) * a.J * 128 + (lane & 7) * 16);
    }
  } else {
    d.sbase = a.wbase;
    d.soff = 0;
  }
  // the bases are uniform: keep them in scalar registers
  d.abase = wave_ptr(d.abase);
  d.bbase = wave_ptr(d.bbase);
  d.sbase = wave_ptr(d.sbase);
}

// One work item with N live sub-tiles on this wave.  The K-loop keeps three
// stages of the ring in flight (stage s of the item in ring slot
// (base + s) % kRing).  Stages s >= J are the next item's stages s - J when
// chain is set (the next item then starts primed: its stages 0-2 issued and
// stage 0 published by this item's last barrier), else the last stage again,
// never read.
template <bool kUp, int N>
__device__ __forceinline__ void run_item(const Item& cur, const Item& nxt, int base, bool primed,
                                         bool chain, const Lds& o, const WaveDma& wd, Stage* st,
                                         int J, int lane, int wave, const KArgs& ka) {
  const int wm = wave >> 2, wn = wave & 3;
  v4f acc[N > 0 ? N : 1][4];
#pragma unroll
  for (int i = 0; i < N; ++i)
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[i][t] = v4f{0.f, 0.f, 0.f, 0.f};

  const uint32_t ring = (uint32_t)(uintptr_t)(lds_u8*)st;
  auto issue = [&](int s) {
    const bool nx = s >= J && chain;
    Dma d;
    d.abase = nx ? nxt.d.abase : cur.d.abase;
    d.bbase = nx ? nxt.d.bbase : cur.d.bbase;
    d.sbase = nx ? nxt.d.sbase : cur.d.sbase;
#pragma unroll
    for (int u = 0; u < 3; ++u) d.aoff[u] = nx ? nxt.d.aoff[u] : cur.d.aoff[u];
    d.soff = nx ? nxt.d.soff : cur.d.soff;
    issue_stage<kUp>(d, wd, ring + (uint32_t)((base + s) % kRing) * (uint32_t)sizeof(Stage),
                     s < J ? s : (nx ? s - J : J - 1), wave);
  };
  // Step j multiplies stage j from registers (head hc read during step j-1,
  // tail read here).  Stages issued before its barrier run up to j + 2, so
  // stage j+1 is complete once at most one stage of this wave's loads is
  // outstanding (loads issued after it only lengthen the wait); the barrier
  // then publishes it to every wave and retires the slot of stage j (every
  // wave's reads of stage j precede it), which takes stage j + 3.
  auto step = [&](int j, Head<N>& hc, Head<N>& hn) {
    Tail<N> tl;
    const uint8_t* Sc = reinterpret_cast<const uint8_t*>(&st[(base + j) % kRing]);
    const uint8_t* Sn = reinterpret_cast<const uint8_t*>(&st[(base + j + 1) % kRing]);
    if constexpr (N > 0) read_tail<N>(tl, Sc, o);
    if constexpr (N > 0) mfma_head<kUp, N>(hc, acc);
    wait_vmcnt<kOps>();
    __syncthreads();
    // The two waves of a SIMD (token halves wm 0 and 1) take the memory work
    // of the step at different points: wm 0 reads the next head and issues
    // its DMA right after the barrier, then runs the tail MFMAs; wm 1 runs
    // its tail MFMAs first.  So while one wave of a SIMD waits on LDS reads
    // and DMA issue the other keeps the matrix pipe busy, instead of all 8
    // waves doing both at the same moment after the barrier.
    if (wm == 0) {
      if constexpr (N > 0) read_head<kUp, N>(hn, Sn, o);
      issue(j + kRing);
    }
    if constexpr (N > 0) mfma_tail<kUp, N>(hc, tl, acc);
    if (wm != 0) {
      if constexpr (N > 0) read_head<kUp, N>(hn, Sn, o);
      issue(j + kRing);
    }
  };
  if (!primed) {  // cold start: fill the ring and wait for stage 0
    issue(0);
    issue(1);
    issue(2);
    wait_vmcnt<2 * kOps>();
    __syncthreads();
  }
  Head<N> h0, h1;
  if constexpr (N > 0) read_head<kUp, N>(h0, reinterpret_cast<const uint8_t*>(&st[base % kRing]), o);
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

  const int H = ka.H, I = ka.I, QG2 = ka.H / 32;
  auto* __restrict__ hq = as_global(ka.hq);
  auto* __restrict__ hs = as_global(ka.hs);
  auto* __restrict__ O = as_global(ka.O);
  const int g = lane >> 4;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    if (kUp) {
      // lane holds token row 16 (wm + 2i) + lane%16 and h features 4g + v
      // (tiles 0 and 2: W1 and W3 rows 0-15) and 16 + 4g + v (tiles 1 and 3)
      // of q-group q, v < 4; one E8M0 scale per token over its 32 features,
      // which lie in lanes l, l^16, l^32, l^48
      const int r = 16 * (wm + 2 * i) + (lane & 15);
      const int q = 4 * cur.ft + wn;
      float h0[4], h1[4];
      float am = 0.0f;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        h0[v] = silu_mul(acc[i][0][v], acc[i][2][v]);
        h1[v] = silu_mul(acc[i][1][v], acc[i][3][v]);
        am = fmaxf(am, fmaxf(fabsf(h0[v]), fabsf(h1[v])));
      }
      am = max_lanes_xor16_32(am);
      float mul;
      const uint32_t sc = mx_scale_from_amax(am, &mul);
      if (r < cur.rows) {
        auto* hrow = hq + (size_t)(cur.m0 + r) * I + q * 32 + 4 * g;
        *reinterpret_cast<__attribute__((address_space(1))) uint32_t*>(hrow) =
            f32x4_to_e4m3(h0[0] * mul, h0[1] * mul, h0[2] * mul, h0[3] * mul);
        *reinterpret_cast<__attribute__((address_space(1))) uint32_t*>(hrow + 16) =
            f32x4_to_e4m3(h1[0] * mul, h1[1] * mul, h1[2] * mul, h1[3] * mul);
        // [P, I/32] row-major, or by K-step of the down GEMM: the dword of
        // K-step q/4 of row p at dword (q/4) P + p, byte q % 4
        const size_t p = (size_t)(cur.m0 + r);
        const size_t at = ka.hs_by_step ? ((size_t)(q >> 2) * (size_t)ka.P + p) * 4 + (q & 3)
                                        : p * (I / 32) + q;
        if (g == 0) hs[at] = (uint8_t)sc;
      }
    } else {
      // lane holds token rows 16 (wm + 2i) + 4g + v, v < 4, column lane%16 of
      // each tile.  The wave's 4 tiles are 64 consecutive columns (q2-groups
      // g2, g2 + 1; H/32 is a multiple of 4, so both exist or neither does).
      // Each row's 128 bytes are written by 4 consecutive stores (t inner),
      // which measured 4 % faster on the whole GEMM than finishing one
      // tile's 4 rows at a time.
      const int rbase = 16 * (wm + 2 * i) + 4 * g;
      const int g2 = 8 * cur.ft + 2 * wn;
      if (g2 < QG2) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int r = rbase + v;
          if (r < cur.rows) {
            auto* orow = O + (size_t)(cur.m0 + r) * H + g2 * 32 + (lane & 15);
#pragma unroll
            for (int t = 0; t < 4; ++t) orow[16 * t] = f32_to_bf16(acc[i][t][v]);
          }
        }
      }
    }
  }
}



// Activation scales by K-step: sT[j][p] = the dword of E8M0 codes of K-step j
// (4 blocks of 32) of sorted row p, taken from row sorted_pair[p] / k of the
// token-order scales (gate/up), or from row p (down, sorted_pair null).  A
// tile's rows are consecutive sorted rows, so each K-step's scale loads then
// read one contiguous run instead of one dword from each of 192 rows.  One
// thread per sorted row reads the row's J dwords (16 bytes at a time when
// vec: J a multiple of 4 and src 16-byte aligned, so every row is) and
// writes K-step j's dword at sT[j][p], consecutive across the wave's lanes.
// With hdr set, the launch's first workgroup builds the token-tile list
// instead (hdr null: the list is already built).
__global__ __launch_bounds__(64) void scales_by_step_kernel(const uint32_t* __restrict__ src,
                                                            int J, bool vec,
                                                            const int32_t* __restrict__ sorted_pair,
                                                            int k, long P, uint32_t* __restrict__ sT,
                                                            const int32_t* __restrict__ offsets,
                                                            int E, int* __restrict__ hdr) {
  if (hdr && blockIdx.x == 0) {
    build_tiles_wave(offsets, E, hdr);
    return;
  }
  const long p = (long)(blockIdx.x - (hdr ? 1 : 0)) * 64 + threadIdx.x;
  if (p >= P) return;
  const long row = sorted_pair ? (long)(sorted_pair[p] / k) : p;
  const uint32_t* s = src + (size_t)row * J;
  uint32_t* d = sT + p;
  if (vec) {
#pragma unroll 4
    for (int j = 0; j < J; j += 4) {
      const uint4 v = *reinterpret_cast<const uint4*>(s + j);
      d[(size_t)j * P] = v.x;
      d[(size_t)(j + 1) * P] = v.y;
      d[(size_t)(j + 2) * P] = v.z;
      d[(size_t)(j + 3) * P] = v.w;
    }
  } else {
    for (int j = 0; j < J; ++j) d[(size_t)j * P] = s[j];
  }
}

// kUp: gate/up GEMM (A = x rows gathered by token, K = H; B = W1/W3; epilogue
// SwiGLU + MXFP8 of h).  !kUp: down GEMM (A = h rows in sorted order, K = I;
// B = W2; epilogue bf16 store of O).  Persistent: one workgroup per CU walks
// its share of the work items.  Workgroup b is dispatched to XCD b % 8; XCD x
// owns items [x*per, (x+1)*per) (per = ceil(W/8), W known on the device
// only), so the feature tiles of one token tile, which share its activation
// rows, stay on one XCD and its L2; its r-th workgroup takes items
// x*per + r, + G/8, ... (G = the grid).
template <bool kUp>
__global__ __launch_bounds__(kThreads) void prefill_gemm_kernel(KArgs args) {
  __shared__ __align__(16) Stage st[kRing];
  __shared__ int rsrc[3][kBM];
  __shared__ KArgs ka;
  const int tid = threadIdx.x, lane = tid & 63;
  if (tid == 0) ka = args;
  const int W = args.hdr[0] * args.NF;
  const int per = (W + 7) >> 3;
  const int xcd = blockIdx.x & 7, stride = gridDim.x >> 3;
  const int end = min((xcd + 1) * per, W);
  int it = xcd * per + (int)(blockIdx.x >> 3);
  if (it >= end) return;

  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar control flow
  const int wm = wave >> 2, wn = wave & 3;
  const int J = args.J;
  const long P = args.P;

  // Row sources (gate/up): rsrc[q % 3] holds those of the workgroup's q-th
  // item.  The first two come by plain loads; with chaining, item q + 2's
  // come by one LDS-DMA dword per lane from waves 0-2 at the start of item q,
  // before its stage 3, so item q's step-1 wait and barrier cover them before
  // item q + 1 builds its successor's descriptor from them.
  Item cur, nxt;
  item_tile(args.hdr, args.offsets, args.NF, it, cur.e, cur.m0, cur.rows, cur.ft);
  if (kUp) {
    if (tid < kBM) rsrc[0][tid] = args.sorted_pair[cur.m0 + min(tid, cur.rows - 1)];
    if (it + stride < end) {
      int e1, m1, r1, f1;
      item_tile(args.hdr, args.offsets, args.NF, it + stride, e1, m1, r1, f1);
      if (tid < kBM) rsrc[1][tid] = args.sorted_pair[m1 + min(tid, r1 - 1)];
    }
  }
  __syncthreads();
  make_dma<kUp>(cur, rsrc[0], args, wave, lane);

  // LDS read offsets of this lane's fragments (see Lds)
  Lds o;
  {
    const int l15 = lane & 15, g = lane >> 4;
    const int row = 16 * wm + l15;
    o.a_lo = row * 128 + ((g ^ (l15 & 7)) << 4);
    o.a_hi = row * 128 + (((g + 4) ^ (l15 & 7)) << 4);
    o.a_s = kABytes + kBBytes + row * 4 + g;
    if (kUp) {
      o.b = kABytes + wn * 4096 + lane * 16;
      o.b_s = kABytes + kBBytes + kBM * 4 + (wn * 64 + lane) * 4;
    } else {
      o.b = kABytes + 2 * wn * 2048 + lane * 16;
      o.b_s = kABytes + kBBytes + kBM * 4 + (2 * wn * 32 + (lane >> 1)) * 4 + 2 * (lane & 1);
    }
  }

  WaveDma wd;
  wd.skind = wave < 3 ? 1 : (wave == 3 ? 2 : 0);
  wd.sstep = wave < 3 ? P * 4 : (kUp ? 256 : 128);
  wd.ls = (uint32_t)(wave < 3 ? kABytes + kBBytes + 256 * wave : kABytes + kBBytes + kBM * 4);
  wd.boff0 = (uint32_t)(lane * 16);

  int base = 0;
  bool primed = false;
  for (int q = 0;; ++q) {
    const int nit = it + stride;
    const bool has_next = nit < end;
    const bool chain = has_next && J >= 4;
    if (has_next) {
      item_tile(args.hdr, args.offsets, args.NF, nit, nxt.e, nxt.m0, nxt.rows, nxt.ft);
      if (kUp && !chain && q > 0) {  // short K, no chaining: plain loads
        if (tid < kBM) rsrc[(q + 1) % 3][tid] = as_global(ka.sorted_pair)[nxt.m0 + min(tid, nxt.rows - 1)];
        __syncthreads();
      }
      make_dma<kUp>(nxt, rsrc[(q + 1) % 3], ka, wave, lane);
    }
    if (kUp && chain && nit + stride < end && wave < 3) {
      int e2, m2, r2, f2;
      item_tile(args.hdr, args.offsets, args.NF, nit + stride, e2, m2, r2, f2);
      dma_x1(wave_ptr(reinterpret_cast<const uint8_t*>(ka.sorted_pair + m2)),
             (uint32_t)(min(64 * wave + lane, r2 - 1) * 4),
             wave_u32((uint32_t)(uintptr_t)(lds_u8*)rsrc[(q + 2) % 3] + 256u * (uint32_t)wave));
    }
    const int nsub = (cur.rows + 15) / 16;  // live 16-row sub-tiles of the tile
    int nact = 0;                           // this wave's live sub-tiles: i = 0..nact-1
#pragma unroll
    for (int i = 0; i < kBM / 32; ++i)
      if (wm + 2 * i < nsub) nact = i + 1;
    nact = __builtin_amdgcn_readfirstlane(nact);
#define MOE_RUN(NN) run_item<kUp, NN>(cur, nxt, base, primed, chain, o, wd, st, J, lane, wave, ka)
    switch (nact) {
      case 0: MOE_RUN(0); break;
      case 1: MOE_RUN(1); break;
      case 2: MOE_RUN(2); break;
      case 3: MOE_RUN(3); break;
      case 4: MOE_RUN(4); break;
      case 5: MOE_RUN(5); break;
      default: MOE_RUN(6); break;
    }
#undef MOE_RUN
    if (!has_next) break;
    base = (base + J) % kRing;
    primed = chain;
    cur = nxt;
    it = nit;
  }
  // no LDS-DMA may still be writing when the workgroup's LDS is released
  wait_vmcnt<0>();
}

long max_tiles(long P, int E) { return (P + kBM - 1) / kBM + E; }

size_t align256_(size_t x) { return (x + 255) & ~(size_t)255; }

// workspace: tile header and list, then the by-step activation scales
size_t tile_list_bytes(long P, int E) { return align256_(kTileHdr + (size_t)max_tiles(P, E) * 8); }

// One workgroup per compute unit (the kernel's LDS allows no more), rounded
// down to whole rounds of the 8 XCDs; queried once per device.
// (Atomic: concurrent first calls from several host threads store the same value.)
unsigned persistent_grid() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  int v = cached[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    int ncu = 0;
    if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu < 8)
      ncu = 256;
    v = ncu / 8 * 8;
    cached[dev].store(v, std::memory_order_relaxed);
  }
  return (unsigned)v;
}

}  // namespace

size_t prefill_stage_bytes(long P, int E, int H, int I) {
  const int Jmax = (H > I ? H : I) / 128;
  return tile_list_bytes(P, E) + align256_((size_t)P * Jmax * 4);
}

hipError_t launch_up_prefill(const uint8_t* packed, const PackedLayout& L, const uint8_t* xq,
                             const uint8_t* xs, const int32_t* offsets,
                             const int32_t* sorted_pair, int T, int k, uint8_t* hq, uint8_t* hs,
                             bool hs_by_step, void* tile_ws, hipStream_t s) {
  const long P = (long)T * k;
  int* hdr = static_cast<int*>(tile_ws);
  uint32_t* sT = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(tile_ws) + tile_list_bytes(P, L.E));
  hipLaunchKernelGGL(scales_by_step_kernel, dim3((unsigned)((P + 63) / 64 + 1)), dim3(64), 0, s,
                     reinterpret_cast<const uint32_t*>(xs), L.J, L.J % 4 == 0 && (uintptr_t)xs % 16 == 0,
                     sorted_pair, k, P, sT, offsets, L.E, hdr);
  const int NF = L.I / 128;
  KArgs a;
  a.wbase = packed + L.upw_off;
  a.sbase = packed + L.ups_off;
  a.act = xq;
  a.sT = sT;
  a.sorted_pair = sorted_pair;
  a.offsets = offsets;
  a.hdr = hdr;
  a.hq = hq;
  a.hs = hs;
  a.O = nullptr;
  a.P = P;
  a.k = k;
  a.NF = NF;
  a.H = L.H;
  a.I = L.I;
  a.QG = L.I / 32;
  a.J = L.J;
  a.hs_by_step = hs_by_step ? 1 : 0;
  hipLaunchKernelGGL(prefill_gemm_kernel<true>, dim3(persistent_grid()), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_down_prefill(const uint8_t* packed, const PackedLayout& L, const uint8_t* hq,
                               const uint8_t* hs, const int32_t* offsets, int T, int k, uint16_t* O,
                               void* tile_ws, bool chained, hipStream_t s) {
  const long P = (long)T * k;
  int* hdr = static_cast<int*>(tile_ws);
  uint32_t* sT = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(tile_ws) + tile_list_bytes(P, L.E));
  if (chained)  // the gate/up launch built the tile list and wrote hs by K-step
    sT = reinterpret_cast<uint32_t*>(const_cast<uint8_t*>(hs));
  else
    hipLaunchKernelGGL(scales_by_step_kernel, dim3((unsigned)((P + 63) / 64 + 1)), dim3(64), 0, s,
                       reinterpret_cast<const uint32_t*>(hs), L.J2,
                       L.J2 % 4 == 0 && (uintptr_t)hs % 16 == 0, (const int32_t*)nullptr, k, P, sT,
                       offsets, L.E, hdr);
  const int NF = (L.H + 255) / 256;
  KArgs a;
  a.wbase = packed + L.dnw_off;
  a.sbase = packed + L.dns_off;
  a.act = hq;
  a.sT = sT;
  a.sorted_pair = nullptr;
  a.offsets = offsets;
  a.hdr = hdr;
  a.hq = nullptr;
  a.hs = nullptr;
  a.O = O;
  a.P = P;
  a.k = k;
  a.NF = NF;
  a.H = L.H;
  a.I = L.I;
  a.QG = L.H / 32;
  a.J = L.J2;
  a.hs_by_step = 0;
  hipLaunchKernelGGL(prefill_gemm_kernel<false>, dim3(persistent_grid()), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
