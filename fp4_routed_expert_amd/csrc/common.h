// Internal header of the gfx950 MoE library: device helpers, the packed
// weight layout, and the launchers each kernel file provides to moe_api.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ---------------------------------------------------------------- MXFP8
// OCP MX conversion of one 32-element block: shared exponent
// X = floor(log2 amax) - 8, X = -127 when amax is zero or below the fp32
// normal range, scale code X + 127.  Returned: the scale code; *mul is the
// exact power of two 2^-X to multiply each element by before rounding.
__host__ __device__ __forceinline__ uint32_t mx_scale_from_amax(float amax, float* mul) {
  uint32_t ua;
  __builtin_memcpy(&ua, &amax, 4);
  const uint32_t ef = (ua >> 23) & 0xFFu;  // amax >= 0
  int X = (ef == 0u) ? -127 : (int)ef - 135;
  if (X < -127) X = -127;  // ef <= 254 keeps X <= 119
  const uint32_t um = (uint32_t)(127 - X) << 23;
  __builtin_memcpy(mul, &um, 4);
  return (uint32_t)(X + 127);
}

// Round an fp32 value (|a| < 512 after scaling) to an OCP e4m3fn code:
// nearest, ties to even, saturating at 448, sign kept.  The three ranges are
// all computed and one selected, so the conversion has no branches.
__host__ __device__ __forceinline__ uint32_t f32_to_e4m3(float a) {
  uint32_t u;
  __builtin_memcpy(&u, &a, 4);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t mag = u & 0x7FFFFFFFu;
  // below 2^-6 the codes step by 2^-9: round |a| * 512 (exact) to an integer 0..8
  const uint32_t mag_sub = (mag < 0x3C800000u) ? mag : 0u;  // other ranges: a dummy 0
  float m;
  __builtin_memcpy(&m, &mag_sub, 4);
  const uint32_t sub = (uint32_t)(int)__builtin_rintf(m * 512.0f);
  // normal: keep 3 of the 23 mantissa bits, round to nearest even on the bit
  // pattern; a carry moves into the exponent field, which is the correct next
  // binade; then rebias 127 -> 7
  const uint32_t nrm = ((mag + 0x7FFFFu + ((mag >> 20) & 1u)) >> 20) - (120u << 3);
  uint32_t c = (mag < 0x3C800000u) ? sub : nrm;
  c = (mag >= 0x43E00000u) ? 0x7Eu : c;  // >= 448
  return sign | c;
}

// The same codes from the gfx950 conversion instruction (v_cvt_pk_fp8_f32:
// OCP e4m3fn, round to nearest even) after a clamp to +-448, which makes the
// overflow saturate as above; equal to f32_to_e4m3 for every |a| < 512
// (tests/native/cvt_equivalence.hip checks each of those inputs).  Two
// values give bytes 0 and 1; four give a whole dword, a in byte 0.
__device__ __forceinline__ float e4m3_clamp(float a) { return __builtin_fminf(__builtin_fmaxf(a, -448.0f), 448.0f); }
__device__ __forceinline__ uint32_t f32x2_to_e4m3(float a, float b) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(a), e4m3_clamp(b), 0, false) & 0xFFFFu;
}
__device__ __forceinline__ uint32_t f32x4_to_e4m3(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(a), e4m3_clamp(b), 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(c), e4m3_clamp(d), lo, true);
}

// fp32 -> bf16 bits, round to nearest even (finite inputs): the gfx950
// conversion instruction (v_cvt_pk_bf16_f32), equal for every finite input
// to rounding the bit pattern, (u + 0x7FFF + ((u >> 16) & 1)) >> 16
// (tests/native/cvt_equivalence.hip checks each of them).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
__device__ __forceinline__ uint32_t f32x2_to_bf16(float a, float b) {
  const bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// SiLU(g) * u with the hardware exponential and reciprocal (fp32, about one
// ulp each): the result is rounded to fp8 right after.
__device__ __forceinline__ float silu_mul(float g, float u) {
  return g * u * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
}

// One DPP lane permutation (no LDS traffic); every source lane is inside the
// destination's row of 16, so no lane reads outside the wave.
template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF, false));
}

// Maximum over lanes l, l^16, l^32, l^48 (the same lane of the wave's four
// rows of 16), returned to all four: the gfx950 row swaps (v_permlane32_swap
// pairs lane l with l^32, v_permlane16_swap pairs l with l^16), no LDS.
__device__ __forceinline__ float max_lanes_xor16_32(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Maximum over each quad of 4 lanes, returned to every lane of the quad.
__device__ __forceinline__ float quad_max(float v) {
  v = fmaxf(v, dpp_f32<0xB1>(v));  // quad_perm [1,0,3,2]
  return fmaxf(v, dpp_f32<0x4E>(v));  // quad_perm [2,3,0,1]
}

// Maximum over each row of 16 lanes, returned to every lane of the row: the
// quad maximum, then the half-row mirror (lane i <-> 7-i of each 8) joins the
// two quads of a half and the row mirror (i <-> 15-i) the two halves.
__device__ __forceinline__ float row16_max(float v) {
  v = quad_max(v);
  v = fmaxf(v, dpp_f32<0x141>(v));  // row_half_mirror
  return fmaxf(v, dpp_f32<0x140>(v));  // row_mirror
}

// ------------------------------------------------------------------ scans
__device__ __forceinline__ int wave_inclusive_scan(int x, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  return x;
}

// Exclusive scan of a[0..n) in LDS (n <= 1024) by a 256-thread block; returns
// the total.  Each thread owns 4 consecutive entries; wave_tot is LDS [4].
__device__ __forceinline__ int block_exclusive_scan256(int* a, int n, int* wave_tot) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int v[4], s = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int idx = 4 * tid + i;
    v[i] = idx < n ? a[idx] : 0;
    s += v[i];
  }
  const int incl = wave_inclusive_scan(s, lane);
  if (lane == 63) wave_tot[w] = incl;
  __syncthreads();
  int before = 0, total = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    before += (i < w) ? wave_tot[i] : 0;
    total += wave_tot[i];
  }
  int run = before + incl - s;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int idx = 4 * tid + i;
    if (idx < n) a[idx] = run;
    run += v[i];
  }
  __syncthreads();
  return total;
}

// ------------------------------------------------------ packed weight layout
// Every weight tile is the B operand of one v_mfma_scale_f32_16x16x128_f8f6f4:
// 16 output rows x 128 K, 1 KiB, stored in lane order: lane l holds row
// (l & 15) and K elements [32*(l >> 4), +32) as 16 consecutive bytes (even K
// in the low nibble), i.e. exactly one 32-element scale block per lane (the B
// operand's lane layout and its per-lane scale were measured on gfx950).
//
// Region UPW (gate/up weights): per expert e, per 32-row group q of I, per
//   K-step j of H/128: 4 tiles of 1 KiB = [W1 rows 32q..+16, W1 rows 32q+16..+16,
//                                          W3 rows 32q..+16, W3 rows 32q+16..+16]
// Region UPS (their scales): per (e, q, j): 64 lanes x 4 B; byte t of lane l's
//   dword is the E8M0 scale of lane l's block in tile t.
// Region DNW (down weights): per expert e, per 32-row group q2 of H, per
//   K-step j2 of I/128: 2 tiles = [W2 rows 32q2..+16, 32q2+16..+16].
// Region DNS (their scales): per (e, q2, j2): 64 lanes x 2 B (byte t = tile t).
struct PackedLayout {
  int E, H, I;
  int J;   // gate/up K-steps (H/128)
  int J2;  // down K-steps (I/128)
  size_t upw_off, ups_off, dnw_off, dns_off, total;

  __host__ __device__ static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

  __host__ __device__ PackedLayout(int E_, int H_, int I_) : E(E_), H(H_), I(I_) {
    J = H / 128;
    J2 = I / 128;
    const size_t upw = (size_t)E * (I / 32) * J * 4096;
    const size_t ups = (size_t)E * (I / 32) * J * 256;
    const size_t dnw = (size_t)E * (H / 32) * J2 * 2048;
    const size_t dns = (size_t)E * (H / 32) * J2 * 128;
    upw_off = 0;
    ups_off = align256(upw_off + upw);
    dnw_off = align256(ups_off + ups);
    dns_off = align256(dnw_off + dnw);
    total = align256(dns_off + dns);
  }
  // byte offset of the 4 KiB gate/up block (e, q, j) and of its 256 B of scales
  __host__ __device__ size_t upw_block(int e, int q, int j) const {
    return upw_off + (((size_t)e * (I / 32) + q) * J + j) * 4096;
  }
  __host__ __device__ size_t ups_block(int e, int q, int j) const {
    return ups_off + (((size_t)e * (I / 32) + q) * J + j) * 256;
  }
  // byte offset of the 2 KiB down block (e, q2, j2) and of its 128 B of scales
  __host__ __device__ size_t dnw_block(int e, int q2, int j2) const {
    return dnw_off + (((size_t)e * (H / 32) + q2) * J2 + j2) * 2048;
  }
  __host__ __device__ size_t dns_block(int e, int q2, int j2) const {
    return dns_off + (((size_t)e * (H / 32) + q2) * J2 + j2) * 128;
  }
};

// ------------------------------------------------- FP8 dense weight layout
// Tile (nt, j): weight rows 16 nt .. +16, K 128 j .. +128, 2 KiB in the e4m3
// MFMA operand's lane order (lane l = 16 g + r: row r, K [16 g, +16) in the
// first KiB, K [64 + 16 g, +16) in the second).  The two tiles of a 32-row
// group sit side by side for each K-step (4 KiB), and a group's K-steps are
// consecutive.  Scales: 64 bytes per tile, byte l = row r, block g, grouped
// the same way (128 bytes per group and K-step).
struct DenseLayout {
  int N, K, J;
  size_t s_off, total;
  static constexpr size_t kTileStep = 4096;   // bytes from K-step j to j + 1 of a tile
  static constexpr size_t kScaleStep = 128;   // the same for its scales
  __host__ __device__ DenseLayout(int N_, int K_) : N(N_), K(K_), J(K_ / 128) {
    s_off = PackedLayout::align256((size_t)(N / 16) * J * 2048);
    total = PackedLayout::align256(s_off + (size_t)(N / 16) * J * 64);
  }
  __host__ __device__ size_t tile_off(int nt, int j) const {
    return ((size_t)(nt >> 1) * J + j) * kTileStep + (size_t)(nt & 1) * 2048;
  }
  __host__ __device__ size_t scale_off(int nt, int j) const {
    return s_off + ((size_t)(nt >> 1) * J + j) * kScaleStep + (size_t)(nt & 1) * 64;
  }
};

// ------------------------------------------------------------- launchers
// Each returns the hipError_t of its launch(es).
// Token counts taken by the fused front kernel: at 24 and 32 tokens the
// stand-alone routing, sort and quantisation measured faster (one workgroup
// routes every token in the fused kernel), at 16 and below the two are equal.
constexpr int kFrontMaxT = 16;
int route_keys_per_lane(int E);
// The routing launchers read S logit planes T*E floats apart and sum them in
// plane order (S = 1: plain logits), route over E experts and append ns shared
// slots (experts E .. E+ns-1, weight 1) after the k routed ones per token.
hipError_t launch_front_small(const float* logits, int S, const uint16_t* x, int T, int H, int E,
                              int k, int ns, int32_t* ids, float* gates, int32_t* counts,
                              int32_t* offsets, int32_t* sorted_pair, int32_t* pair_pos,
                              uint8_t* xq, uint8_t* xs, hipStream_t s);
hipError_t launch_route_topk(const float* logits, int S, int T, int E, int k, int ns,
                             int32_t* ids, float* gates, hipStream_t s);
// Routing (as launch_route_topk) and MXFP8 quantisation of x [T, H] (as
// launch_quant_mxfp8) in one launch, for batches above kFrontMaxT.
hipError_t launch_front_route_quant(const float* logits, int S, const uint16_t* x, int T, int H,
                                    int E, int k, int ns, int32_t* ids, float* gates, uint8_t* xq,
                                    uint8_t* xs, hipStream_t s);
size_t sort_workspace_bytes(int T, int E, int k);
hipError_t launch_sort_permute(const int32_t* ids, int T, int E, int k, int32_t* counts,
                               int32_t* offsets, int32_t* sorted_pair, int32_t* pair_pos,
                               void* ws, hipStream_t s);
hipError_t launch_quant_mxfp8(const uint16_t* x, long M, int K, uint8_t* q, uint8_t* sc,
                              hipStream_t s);
hipError_t launch_prepack(const uint8_t* w1, const uint8_t* s1, const uint8_t* w3,
                          const uint8_t* s3, const uint8_t* w2, const uint8_t* s2,
                          const PackedLayout& L, uint8_t* packed, hipStream_t s);
// row_groups (1 or 2): 16-row groups of an expert's pairs per pass over its
// weights.
hipError_t launch_up_decode(const uint8_t* packed, const PackedLayout& L, const uint8_t* xq,
                            const uint8_t* xs, const int32_t* offsets,
                            const int32_t* sorted_pair, int k, uint8_t* hq, uint8_t* hs,
                            int row_groups, hipStream_t s);
hipError_t launch_down_decode(const uint8_t* packed, const PackedLayout& L, const uint8_t* hq,
                              const uint8_t* hs, const int32_t* offsets, uint16_t* O,
                              int row_groups, hipStream_t s);
size_t prefill_stage_bytes(long P, int E, int H, int I);
hipError_t launch_up_prefill(const uint8_t* packed, const PackedLayout& L, const uint8_t* xq,
                             const uint8_t* xs, const int32_t* offsets,
                             const int32_t* sorted_pair, int T, int k, uint8_t* hq, uint8_t* hs,
                             bool hs_by_step, void* tile_ws, hipStream_t s);
// hs_by_step: hs [P, I/32] is written in the down GEMM's scale layout instead
// (the dword of K-step j of row p at dword j P + p), for a chained down call.
// chained: launch_up_prefill(hs_by_step) just ran on this tile_ws and these
// offsets, so the token-tile list is there and hs is already by K-step.
hipError_t launch_down_prefill(const uint8_t* packed, const PackedLayout& L, const uint8_t* hq,
                               const uint8_t* hs, const int32_t* offsets, int T, int k, uint16_t* O,
                               void* tile_ws, bool chained, hipStream_t s);
hipError_t launch_combine(const uint16_t* O, const float* gates, const int32_t* pair_pos,
                          const uint16_t* O_shared, int T, int k, int H, float* y, hipStream_t s);
// partial: router_ws_bytes(T, H, E) bytes of fp32 K-slice partial sums
// (unused, may be null, when that is 0)
int router_slices(int T, int H, int E);
size_t router_ws_bytes(int T, int H, int E);
hipError_t launch_router(const uint16_t* x, const uint16_t* wg, int T, int H, int E, float* logits,
                         float* partial, hipStream_t s);
// Only the GEMM: writes the logits when router_slices() == 1, else the S
// partial planes in `partial` (for a routing launch that sums them itself).
hipError_t launch_router_partials(const uint16_t* x, const uint16_t* wg, int T, int H, int E,
                                  float* logits, float* partial, hipStream_t s);
hipError_t launch_identity_route(int T, int32_t* sorted_pair, int32_t* offsets, hipStream_t s);
hipError_t launch_dense_pack(const uint8_t* wq, const uint8_t* ws, int N, int K, uint8_t* packed,
                             hipStream_t s);
hipError_t launch_dense_decode(const uint8_t* packed, const uint8_t* xq, const uint8_t* xs, int T,
                               int N, int K, uint16_t* y, hipStream_t s);
hipError_t launch_dense_prefill(const uint8_t* packed, const uint8_t* xq, const uint8_t* xs, int T,
                                int N, int K, uint16_t* y, hipStream_t s);

}  // namespace moe
