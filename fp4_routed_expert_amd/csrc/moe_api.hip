// C ABI of the library (declared in include/moe_fp4.h): host-side argument
// checks, workspace carving and path selection.  Every check runs before any
// launch, so a failing call enqueues nothing and touches no output.
#include <atomic>

#include "common.h"
#include "../../include/moe_fp4.h"

using namespace moe;

namespace {

thread_local int g_last_hip_error = 0;

// Every launch records its result for moe_last_hip_error (0 on success).
moe_status_t hip_status(hipError_t e) {
  g_last_hip_error = (int)e;
  return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

constexpr int kMaxE = 1024;
constexpr int kMaxK = 32;
// dense projection: weight streaming up to 3 passes of two token tiles
// (streaming measured faster than the tiled GEMM up to T = 96 at K 16384,
// N 7168: 99 vs 116 us; 133 vs 119 us at T = 128)
constexpr int kDenseDecodeMaxT = 96;
// expert GEMMs: weight streaming while T*k <= this many rows per expert (the
// measured crossover of the two paths at the decode-sized expert shapes)
constexpr int64_t kDecodeRowsPerExpert = 16;

// Common checks of (T, E, k): negative or zero sizes are invalid, shapes
// outside the kernels' coverage unsupported.
moe_status_t check_tek(int32_t T, int32_t E, int32_t k) {
  if (T < 0 || E < 1 || k < 1) return MOE_ERR_INVALID_ARGUMENT;
  if (E > kMaxE || k > kMaxK || k > E) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)T * k >= ((int64_t)1 << 31)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

moe_status_t check_hi(int32_t H, int32_t I) {
  if (H < 1 || I < 1) return MOE_ERR_INVALID_ARGUMENT;
  if (H % 128 != 0 || I % 128 != 0) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)H > (1 << 20) || (int64_t)I > (1 << 20)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

moe_status_t check_weights(const moe_fp4_weights_t* w) {
  if (!w || !w->packed) return MOE_ERR_INVALID_ARGUMENT;
  if (w->layout_version != MOE_FP4_LAYOUT_VERSION) return MOE_ERR_INVALID_ARGUMENT;
  if (w->E < 1 || w->E > kMaxE) return MOE_ERR_INVALID_ARGUMENT;
  moe_status_t st = check_hi(w->H, w->I);
  if (st != MOE_OK) return st;
  if (!aligned(w->packed, 256)) return MOE_ERR_INVALID_ARGUMENT;
  if (w->packed_bytes < PackedLayout(w->E, w->H, w->I).total) return MOE_ERR_INVALID_ARGUMENT;
  return MOE_OK;
}

// Row groups per weight pass of the decode kernels, from host-known sizes:
// two once the pairs average 12 or more per expert (experts over 16 rows are
// then common, and one pass serves 32 rows instead of re-reading the weights;
// at 8-12 rows per expert the two measured within 3 %).
int decode_row_groups(int64_t P, int E) { return P >= 12 * (int64_t)E ? 2 : 1; }

// Path choice from host-known sizes only.  0 = decode, 1 = prefill, -1 = bad flags.
int select_path(int64_t P, int E, uint32_t flags) {
  const bool fd = flags & MOE_FLAG_FORCE_DECODE, fp = flags & MOE_FLAG_FORCE_PREFILL;
  if ((flags & ~(MOE_FLAG_FORCE_DECODE | MOE_FLAG_FORCE_PREFILL)) != 0) return -1;
  if (fd && fp) return -1;
  if (fd) return 0;
  if (fp) return 1;
  return P <= kDecodeRowsPerExpert * (int64_t)E ? 0 : 1;
}

size_t stage_ws_bytes(int32_t T, int32_t k, int32_t E, int32_t H, int32_t I) {
  return align256(prefill_stage_bytes((long)T * k, E, H, I));
}

struct FwdCarve {
  size_t hq, hs, O, stage, total;
};

FwdCarve carve(int32_t T, int32_t k, int32_t E, int32_t H, int32_t I) {
  const size_t P = (size_t)T * (size_t)k;
  FwdCarve c;
  c.hq = 0;
  c.hs = align256(c.hq + P * I);
  c.O = align256(c.hs + P * (I / 32));
  c.stage = align256(c.O + P * H * sizeof(uint16_t));
  c.total = align256(c.stage + stage_ws_bytes(T, k, E, H, I));
  return c;
}

struct LayerCarve {
  size_t ids, gates, counts, offsets, sorted, pos, sort_ws, xq, xs, fwd, fwd_bytes, total;
};

LayerCarve layer_carve(int32_t T, int32_t k, int32_t E, int32_t H, int32_t I) {
  const size_t P = (size_t)T * (size_t)k;
  LayerCarve c;
  c.ids = 0;
  c.gates = align256(c.ids + P * 4);
  c.counts = align256(c.gates + P * 4);
  c.offsets = align256(c.counts + (size_t)E * 4);
  c.sorted = align256(c.offsets + ((size_t)E + 1) * 4);
  c.pos = align256(c.sorted + P * 4);
  c.sort_ws = align256(c.pos + P * 4);
  c.xq = align256(c.sort_ws + sort_workspace_bytes(T, E, k));
  c.xs = align256(c.xq + (size_t)T * H);
  c.fwd = align256(c.xs + (size_t)T * (H / 32));
  c.fwd_bytes = carve(T, k, E, H, I).total;
  c.total = align256(c.fwd + c.fwd_bytes);
  return c;
}

// Steps 1-3 of the layer into the carve's buffers: one fused launch for
// T <= kFrontMaxT, else routing and quantisation in one launch, then the
// sort.  The logits are S planes summed in order (S = 1: plain logits);
// routing is over E experts, with ns shared experts (E .. E+ns-1, weight 1)
// appended as slots k .. k+ns-1 of every token; c is the carve for k + ns
// slots and E + ns experts.
moe_status_t run_front(const float* logits, int S, const uint16_t* x_bf16, int32_t T, int32_t H,
                       int32_t E, int32_t k, int32_t ns, uint8_t* ws, const LayerCarve& c,
                       hipStream_t stream) {
  int32_t* ids = reinterpret_cast<int32_t*>(ws + c.ids);
  float* gates = reinterpret_cast<float*>(ws + c.gates);
  int32_t* counts = reinterpret_cast<int32_t*>(ws + c.counts);
  int32_t* offsets = reinterpret_cast<int32_t*>(ws + c.offsets);
  int32_t* sorted = reinterpret_cast<int32_t*>(ws + c.sorted);
  int32_t* pos = reinterpret_cast<int32_t*>(ws + c.pos);
  uint8_t* xq = ws + c.xq;
  uint8_t* xs = ws + c.xs;
  if (T <= kFrontMaxT)
    return hip_status(launch_front_small(logits, S, x_bf16, T, H, E, k, ns, ids, gates, counts,
                                         offsets, sorted, pos, xq, xs, stream));
  moe_status_t st = hip_status(
      launch_front_route_quant(logits, S, x_bf16, T, H, E, k, ns, ids, gates, xq, xs, stream));
  if (st == MOE_OK)
    st = hip_status(launch_sort_permute(ids, T, E + ns, k + ns, counts, offsets, sorted, pos,
                                        ws + c.sort_ws, stream));
  return st;
}

// Workspace of the shared expert: its trivial routing (pair = token), its h
// and the GEMM stages' workspace.
struct SharedCarve {
  size_t sorted, offsets, hq, hs, stage, total;
};

SharedCarve shared_carve(int32_t T, int32_t H, int32_t Is) {
  SharedCarve c;
  c.sorted = 0;
  c.offsets = align256(c.sorted + (size_t)T * 4);
  c.hq = align256(c.offsets + 2 * 4);
  c.hs = align256(c.hq + (size_t)T * Is);
  c.stage = align256(c.hs + (size_t)T * (Is / 32));
  c.total = align256(c.stage + stage_ws_bytes(T, 1, 1, H, Is));
  return c;
}

// Workspace of the layer from hidden states: the router's output (its S
// K-slice planes, or the logits when S == 1) and the layer's own carve for
// k + ns slots over E experts (E = routed + shared).
struct FullCarve {
  size_t rout, layer, total;
  LayerCarve lc;
};

FullCarve full_carve(int32_t T, int32_t k, int32_t E, int32_t H, int32_t I, int32_t ns) {
  FullCarve c;
  const int32_t Er = E - ns;
  c.rout = 0;
  c.layer = align256(c.rout + (size_t)router_slices(T, H, Er) * T * Er * 4);
  c.lc = layer_carve(T, k + ns, E, H, I);
  c.total = align256(c.layer + c.lc.total);
  return c;
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status_t s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARGUMENT: return "MOE_ERR_INVALID_ARGUMENT";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
  }
  return "MOE_ERR_UNKNOWN";
}

int moe_last_hip_error(void) { return g_last_hip_error; }

moe_status_t moe_route_topk(const float* logits, int32_t T, int32_t E, int32_t k,
                            int32_t* topk_ids, float* topk_gates, hipStream_t stream) {
  moe_status_t st = check_tek(T, E, k);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (!logits || !topk_ids || !topk_gates) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned(logits, 4) || !aligned(topk_ids, 4) || !aligned(topk_gates, 4))
    return MOE_ERR_INVALID_ARGUMENT;
  return hip_status(launch_route_topk(logits, 1, T, E, k, 0, topk_ids, topk_gates, stream));
}

size_t moe_sort_permute_workspace_size(int32_t T, int32_t E, int32_t k) {
  if (check_tek(T, E, k) != MOE_OK) return 0;
  return align256(sort_workspace_bytes(T, E, k));
}

moe_status_t moe_sort_permute(const int32_t* topk_ids, int32_t T, int32_t E, int32_t k,
                              int32_t* expert_counts, int32_t* expert_offsets,
                              int32_t* sorted_pair, int32_t* pair_pos, void* workspace,
                              size_t workspace_bytes, hipStream_t stream) {
  moe_status_t st = check_tek(T, E, k);
  if (st != MOE_OK) return st;
  if (!expert_counts || !expert_offsets) return MOE_ERR_INVALID_ARGUMENT;
  if (T > 0 && (!topk_ids || !sorted_pair || !pair_pos)) return MOE_ERR_INVALID_ARGUMENT;
  const size_t need = moe_sort_permute_workspace_size(T, E, k);
  if (need > 0 && (!workspace || workspace_bytes < need)) return MOE_ERR_WORKSPACE;
  if (workspace && !aligned(workspace, 256)) return MOE_ERR_INVALID_ARGUMENT;
  // T == 0 still defines counts = 0 and offsets = 0 (the small kernel writes them)
  return hip_status(launch_sort_permute(topk_ids, T, E, k, expert_counts, expert_offsets,
                                        sorted_pair, pair_pos, workspace, stream));
}

moe_status_t moe_quant_act_mxfp8(const uint16_t* x_bf16, int32_t M, int32_t K, uint8_t* q,
                                 uint8_t* s, hipStream_t stream) {
  if (M < 0 || K < 1) return MOE_ERR_INVALID_ARGUMENT;
  if (K % 32 != 0) return MOE_ERR_UNSUPPORTED;
  if (M == 0) return MOE_OK;
  if (!x_bf16 || !q || !s) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned(x_bf16, 16) || !aligned(q, 16)) return MOE_ERR_INVALID_ARGUMENT;
  if ((int64_t)M * K / 8 >= ((int64_t)1 << 40)) return MOE_ERR_UNSUPPORTED;
  return hip_status(launch_quant_mxfp8(x_bf16, M, K, q, s, stream));
}

size_t moe_fp4_packed_weight_bytes(int32_t E, int32_t H, int32_t I) {
  if (E < 1 || E > kMaxE || check_hi(H, I) != MOE_OK) return 0;
  return PackedLayout(E, H, I).total;
}

moe_status_t moe_fp4_prepack_weights(const uint8_t* w1, const uint8_t* s1, const uint8_t* w3,
                                     const uint8_t* s3, const uint8_t* w2, const uint8_t* s2,
                                     int32_t E, int32_t H, int32_t I, void* packed,
                                     size_t packed_bytes, moe_fp4_weights_t* desc,
                                     hipStream_t stream) {
  if (E < 1) return MOE_ERR_INVALID_ARGUMENT;
  if (E > kMaxE) return MOE_ERR_UNSUPPORTED;
  moe_status_t st = check_hi(H, I);
  if (st != MOE_OK) return st;
  if (!w1 || !s1 || !w3 || !s3 || !w2 || !s2 || !packed || !desc) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned(w1, 16) || !aligned(w3, 16) || !aligned(w2, 16) || !aligned(packed, 256))
    return MOE_ERR_INVALID_ARGUMENT;
  const PackedLayout L(E, H, I);
  if (packed_bytes < L.total) return MOE_ERR_INVALID_ARGUMENT;
  st = hip_status(launch_prepack(w1, s1, w3, s3, w2, s2, L, static_cast<uint8_t*>(packed), stream));
  if (st != MOE_OK) return st;
  desc->E = E;
  desc->H = H;
  desc->I = I;
  desc->layout_version = MOE_FP4_LAYOUT_VERSION;
  desc->packed = packed;
  desc->packed_bytes = packed_bytes;
  return MOE_OK;
}

size_t moe_fp4_stage_workspace_size(int32_t T, int32_t E, int32_t k, int32_t H, int32_t I) {
  if (check_tek(T, E, k) != MOE_OK || check_hi(H, I) != MOE_OK) return 0;
  return stage_ws_bytes(T, k, E, H, I);
}

}  // extern "C"

// The gate/up stage; hs_by_step: on the prefill path, hs is written in the
// down GEMM's scale layout for a chained expert_down call of the same chain.
static moe_status_t expert_up(const moe_fp4_weights_t* w, const uint8_t* xq, const uint8_t* xs,
                              const int32_t* expert_offsets, const int32_t* sorted_pair, int32_t T,
                              int32_t k, uint8_t* hq, uint8_t* hs, void* workspace,
                              size_t workspace_bytes, uint32_t flags, bool hs_by_step,
                              hipStream_t stream) {
  moe_status_t st = check_weights(w);
  if (st != MOE_OK) return st;
  st = check_tek(T, w->E, k);
  if (st != MOE_OK) return st;
  const int path = select_path((int64_t)T * k, w->E, flags);
  if (path < 0) return MOE_ERR_INVALID_ARGUMENT;
  if (T == 0) return MOE_OK;
  if (!xq || !xs || !expert_offsets || !sorted_pair || !hq || !hs) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned(xq, 16) || !aligned(hq, 16) || !aligned(xs, 4) || !aligned(hs, 4))
    return MOE_ERR_INVALID_ARGUMENT;
  if (!workspace || workspace_bytes < stage_ws_bytes(T, k, w->E, w->H, w->I)) return MOE_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return MOE_ERR_INVALID_ARGUMENT;
  const PackedLayout L(w->E, w->H, w->I);
  const uint8_t* pk = static_cast<const uint8_t*>(w->packed);
  // the prefill kernel addresses activation rows with 32-bit offsets
  if (path == 1 && (int64_t)T * w->H >= ((int64_t)1 << 32)) return MOE_ERR_UNSUPPORTED;
  if (path == 1)
    return hip_status(launch_up_prefill(pk, L, xq, xs, expert_offsets, sorted_pair, T, k, hq, hs,
                                        hs_by_step, workspace, stream));
  return hip_status(launch_up_decode(pk, L, xq, xs, expert_offsets, sorted_pair, k, hq, hs,
                                     decode_row_groups((int64_t)T * k, w->E), stream));
}

extern "C" {

moe_status_t moe_fp4_expert_up(const moe_fp4_weights_t* w, const uint8_t* xq, const uint8_t* xs,
                               const int32_t* expert_offsets, const int32_t* sorted_pair,
                               int32_t T, int32_t k, uint8_t* hq, uint8_t* hs, void* workspace,
                               size_t workspace_bytes, uint32_t flags, hipStream_t stream) {
  return expert_up(w, xq, xs, expert_offsets, sorted_pair, T, k, hq, hs, workspace,
                   workspace_bytes, flags, false, stream);
}

}  // extern "C"

// The down stage; chained: expert_up(hs_by_step) of the same chain just ran
// with this workspace and these offsets, so its token-tile list is reused and
// hs is already in the down GEMM's scale layout.
static moe_status_t expert_down(const moe_fp4_weights_t* w, const uint8_t* hq, const uint8_t* hs,
                                const int32_t* expert_offsets, int32_t T, int32_t k, uint16_t* O,
                                void* workspace, size_t workspace_bytes, uint32_t flags,
                                bool chained, hipStream_t stream) {
  moe_status_t st = check_weights(w);
  if (st != MOE_OK) return st;
  st = check_tek(T, w->E, k);
  if (st != MOE_OK) return st;
  const int path = select_path((int64_t)T * k, w->E, flags);
  if (path < 0) return MOE_ERR_INVALID_ARGUMENT;
  if (T == 0) return MOE_OK;
  if (!hq || !hs || !expert_offsets || !O) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned(hq, 16) || !aligned(O, 16) || !aligned(hs, 4)) return MOE_ERR_INVALID_ARGUMENT;
  if (!workspace || workspace_bytes < stage_ws_bytes(T, k, w->E, w->H, w->I)) return MOE_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return MOE_ERR_INVALID_ARGUMENT;
  const PackedLayout L(w->E, w->H, w->I);
  const uint8_t* pk = static_cast<const uint8_t*>(w->packed);
  if (path == 1)
    return hip_status(launch_down_prefill(pk, L, hq, hs, expert_offsets, T, k, O, workspace,
                                          chained, stream));
  return hip_status(launch_down_decode(pk, L, hq, hs, expert_offsets, O,
                                       decode_row_groups((int64_t)T * k, w->E), stream));
}

extern "C" {

moe_status_t moe_fp4_expert_down(const moe_fp4_weights_t* w, const uint8_t* hq, const uint8_t* hs,
                                 const int32_t* expert_offsets, int32_t T, int32_t k, uint16_t* O,
                                 void* workspace, size_t workspace_bytes, uint32_t flags,
                                 hipStream_t stream) {
  return expert_down(w, hq, hs, expert_offsets, T, k, O, workspace, workspace_bytes, flags, false,
                     stream);
}

moe_status_t moe_combine(const uint16_t* O, const float* topk_gates, const int32_t* pair_pos,
                         int32_t T, int32_t k, int32_t H, float* y, hipStream_t stream) {
  if (T < 0 || k < 1 || H < 1) return MOE_ERR_INVALID_ARGUMENT;
  if (k > kMaxK || H % 4 != 0) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!O || !topk_gates || !pair_pos || !y) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned(O, 8) || !aligned(y, 16)) return MOE_ERR_INVALID_ARGUMENT;
  return hip_status(launch_combine(O, topk_gates, pair_pos, nullptr, T, k, H, y, stream));
}

size_t moe_fp4_forward_workspace_size(int32_t T, int32_t E, int32_t k, int32_t H, int32_t I,
                                      uint32_t flags) {
  (void)flags;
  if (check_tek(T, E, k) != MOE_OK || check_hi(H, I) != MOE_OK) return 0;
  return carve(T, k, E, H, I).total;
}

moe_status_t moe_fp4_grouped_forward(const moe_fp4_weights_t* w, const uint8_t* xq,
                                     const uint8_t* xs, const float* topk_gates,
                                     const int32_t* expert_offsets, const int32_t* sorted_pair,
                                     const int32_t* pair_pos, int32_t T, int32_t k, float* y,
                                     void* workspace, size_t workspace_bytes, uint32_t flags,
                                     hipStream_t stream) {
  moe_status_t st = check_weights(w);
  if (st != MOE_OK) return st;
  st = check_tek(T, w->E, k);
  if (st != MOE_OK) return st;
  if (select_path((int64_t)T * k, w->E, flags) < 0) return MOE_ERR_INVALID_ARGUMENT;
  if (T == 0) return MOE_OK;
  if (!xq || !xs || !topk_gates || !expert_offsets || !sorted_pair || !pair_pos || !y)
    return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned(xq, 16) || !aligned(y, 16) || !aligned(xs, 4)) return MOE_ERR_INVALID_ARGUMENT;
  const FwdCarve c = carve(T, k, w->E, w->H, w->I);
  if (!workspace || workspace_bytes < c.total) return MOE_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return MOE_ERR_INVALID_ARGUMENT;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  uint8_t* hq = ws + c.hq;
  uint8_t* hs = ws + c.hs;
  uint16_t* O = reinterpret_cast<uint16_t*>(ws + c.O);
  void* stage = ws + c.stage;
  const size_t stage_bytes = c.total - c.stage;
  st = expert_up(w, xq, xs, expert_offsets, sorted_pair, T, k, hq, hs, stage, stage_bytes, flags,
                 true, stream);
  if (st != MOE_OK) return st;
  st = expert_down(w, hq, hs, expert_offsets, T, k, O, stage, stage_bytes, flags, true, stream);
  if (st != MOE_OK) return st;
  return moe_combine(O, topk_gates, pair_pos, T, k, w->H, y, stream);
}

}  // extern "C"

extern "C" {

size_t moe_fp4_layer_workspace_size(int32_t T, int32_t E, int32_t k, int32_t H, int32_t I,
                                    uint32_t flags) {
  (void)flags;
  if (check_tek(T, E, k) != MOE_OK || check_hi(H, I) != MOE_OK) return 0;
  return layer_carve(T, k, E, H, I).total;
}

moe_status_t moe_fp4_layer_forward(const moe_fp4_weights_t* w, const uint16_t* x_bf16,
                                   const float* logits, int32_t T, int32_t k, float* y,
                                   void* workspace, size_t workspace_bytes, uint32_t flags,
                                   hipStream_t stream) {
  moe_status_t st = check_weights(w);
  if (st != MOE_OK) return st;
  st = check_tek(T, w->E, k);
  if (st != MOE_OK) return st;
  if (select_path((int64_t)T * k, w->E, flags) < 0) return MOE_ERR_INVALID_ARGUMENT;
  if (T == 0) return MOE_OK;
  if (!x_bf16 || !logits || !y) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned(x_bf16, 16) || !aligned(logits, 4) || !aligned(y, 16))
    return MOE_ERR_INVALID_ARGUMENT;
  const int32_t E = w->E, H = w->H, I = w->I;
  const LayerCarve c = layer_carve(T, k, E, H, I);
  if (!workspace || workspace_bytes < c.total) return MOE_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return MOE_ERR_INVALID_ARGUMENT;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  st = run_front(logits, 1, x_bf16, T, H, E, k, 0, ws, c, stream);
  if (st != MOE_OK) return st;
  return moe_fp4_grouped_forward(w, ws + c.xq, ws + c.xs,
                                 reinterpret_cast<const float*>(ws + c.gates),
                                 reinterpret_cast<const int32_t*>(ws + c.offsets),
                                 reinterpret_cast<const int32_t*>(ws + c.sorted),
                                 reinterpret_cast<const int32_t*>(ws + c.pos), T, k, y, ws + c.fwd,
                                 c.fwd_bytes, flags, stream);
}

}  // extern "C"

// ------------------------------------------------- the no-allocation layer
// The workspace of moe_fp4_layer_forward_noalloc: a fixed array in device
// memory, one copy per GPU, held until the process ends.  In host code its
// name is only a stand-in for the symbol; kernels get its device address,
// fetched once per device with that device current.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];

// Device address of `scratch` on the current device (the first call on a
// device looks it up; concurrent first calls store the same address).
hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_addr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return hipSuccess;
}

}  // namespace

extern "C" {

moe_status_t moe_fp4_layer_forward_noalloc(const moe_fp4_weights_t* w, const uint16_t* x_bf16,
                                           const float* logits, int32_t T, int32_t k, float* y,
                                           uint32_t flags, hipStream_t stream) {
  moe_status_t st = check_weights(w);
  if (st != MOE_OK) return st;
  st = check_tek(T, w->E, k);
  if (st != MOE_OK) return st;
  if (select_path((int64_t)T * k, w->E, flags) < 0) return MOE_ERR_INVALID_ARGUMENT;
  if (T == 0) return MOE_OK;
  if (!x_bf16 || !logits || !y) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned(x_bf16, 16) || !aligned(logits, 4) || !aligned(y, 16))
    return MOE_ERR_INVALID_ARGUMENT;
  const size_t need = layer_carve(T, k, w->E, w->H, w->I).total;
  if (need > (size_t)MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
  void* ws = nullptr;
  st = hip_status(scratch_address(&ws));
  if (st != MOE_OK) return st;
  return moe_fp4_layer_forward(w, x_bf16, logits, T, k, y, ws, MOE_NOALLOC_SCRATCH_BYTES, flags,
                               stream);
}

}  // extern "C"

// ------------------------------------------- router GEMM and shared expert
extern "C" {

static moe_status_t check_router(int32_t T, int32_t H, int32_t E) {
  if (T < 0 || H < 1 || E < 1) return MOE_ERR_INVALID_ARGUMENT;
  if (H % 128 != 0 || H > (1 << 20) || E > kMaxE) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)T * E * router_slices(T > 0 ? T : 1, H, E) >= ((int64_t)1 << 31))
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

size_t moe_router_workspace_size(int32_t T, int32_t H, int32_t E) {
  if (check_router(T, H, E) != MOE_OK || T == 0) return 0;
  return router_ws_bytes(T, H, E);
}

moe_status_t moe_router_logits(const uint16_t* x_bf16, const uint16_t* router_w, int32_t T,
                               int32_t H, int32_t E, float* logits, void* workspace,
                               size_t workspace_bytes, hipStream_t stream) {
  moe_status_t st = check_router(T, H, E);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (!x_bf16 || !router_w || !logits) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned(x_bf16, 16) || !aligned(router_w, 16) || !aligned(logits, 4))
    return MOE_ERR_INVALID_ARGUMENT;
  const size_t need = router_ws_bytes(T, H, E);
  if (need > 0 && (!workspace || workspace_bytes < need)) return MOE_ERR_WORKSPACE;
  if (need > 0 && !aligned(workspace, 256)) return MOE_ERR_INVALID_ARGUMENT;
  return hip_status(
      launch_router(x_bf16, router_w, T, H, E, logits, static_cast<float*>(workspace), stream));
}

size_t moe_fp4_shared_workspace_size(int32_t T, int32_t H, int32_t I_shared, uint32_t flags) {
  (void)flags;
  if (check_tek(T, 1, 1) != MOE_OK || check_hi(H, I_shared) != MOE_OK) return 0;
  return shared_carve(T, H, I_shared).total;
}

moe_status_t moe_fp4_shared_expert(const moe_fp4_weights_t* w, const uint8_t* xq, const uint8_t* xs,
                                   int32_t T, uint16_t* O_shared, void* workspace,
                                   size_t workspace_bytes, uint32_t flags, hipStream_t stream) {
  moe_status_t st = check_weights(w);
  if (st != MOE_OK) return st;
  if (w->E != 1) return MOE_ERR_INVALID_ARGUMENT;
  st = check_tek(T, 1, 1);
  if (st != MOE_OK) return st;
  if (select_path(T, 1, flags) < 0) return MOE_ERR_INVALID_ARGUMENT;
  if (T == 0) return MOE_OK;
  if (!xq || !xs || !O_shared) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned(xq, 16) || !aligned(xs, 4) || !aligned(O_shared, 16)) return MOE_ERR_INVALID_ARGUMENT;
  const SharedCarve c = shared_carve(T, w->H, w->I);
  if (!workspace || workspace_bytes < c.total) return MOE_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return MOE_ERR_INVALID_ARGUMENT;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  int32_t* sorted = reinterpret_cast<int32_t*>(ws + c.sorted);
  int32_t* offsets = reinterpret_cast<int32_t*>(ws + c.offsets);
  st = hip_status(launch_identity_route(T, sorted, offsets, stream));
  if (st != MOE_OK) return st;
  st = expert_up(w, xq, xs, offsets, sorted, T, 1, ws + c.hq, ws + c.hs, ws + c.stage,
                 c.total - c.stage, flags, true, stream);
  if (st != MOE_OK) return st;
  return expert_down(w, ws + c.hq, ws + c.hs, offsets, T, 1, O_shared, ws + c.stage,
                     c.total - c.stage, flags, true, stream);
}

moe_status_t moe_combine_shared(const uint16_t* O, const float* topk_gates, const int32_t* pair_pos,
                                const uint16_t* O_shared, int32_t T, int32_t k, int32_t H, float* y,
                                hipStream_t stream) {
  if (T < 0 || k < 1 || H < 1) return MOE_ERR_INVALID_ARGUMENT;
  if (k > kMaxK || H % 4 != 0) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!O || !topk_gates || !pair_pos || !O_shared || !y) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned(O, 8) || !aligned(O_shared, 8) || !aligned(y, 16)) return MOE_ERR_INVALID_ARGUMENT;
  return hip_status(launch_combine(O, topk_gates, pair_pos, O_shared, T, k, H, y, stream));
}

static moe_status_t check_full(int32_t T, int32_t k, int32_t E, int32_t H, int32_t ns) {
  if (ns < 0 || ns >= E) return MOE_ERR_INVALID_ARGUMENT;
  moe_status_t st = check_tek(T, E - ns, k);
  if (st != MOE_OK) return st;
  if (k + ns > kMaxK) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)T * (k + ns) >= ((int64_t)1 << 31)) return MOE_ERR_UNSUPPORTED;
  return check_router(T, H, E - ns);
}

size_t moe_fp4_layer_full_workspace_size(int32_t T, int32_t E, int32_t k, int32_t H, int32_t I,
                                         int32_t n_shared, uint32_t flags) {
  (void)flags;
  if (E < 1 || E > kMaxE || check_hi(H, I) != MOE_OK) return 0;
  if (check_full(T, k, E, H, n_shared) != MOE_OK) return 0;
  return full_carve(T, k, E, H, I, n_shared).total;
}

moe_status_t moe_fp4_layer_forward_full(const moe_fp4_weights_t* w, int32_t n_shared,
                                        const uint16_t* router_w, const uint16_t* x_bf16,
                                        int32_t T, int32_t k, float* y, void* workspace,
                                        size_t workspace_bytes, uint32_t flags,
                                        hipStream_t stream) {
  moe_status_t st = check_weights(w);
  if (st != MOE_OK) return st;
  st = check_full(T, k, w->E, w->H, n_shared);
  if (st != MOE_OK) return st;
  const int32_t E = w->E, H = w->H, I = w->I, ns = n_shared, Er = E - ns, kk = k + ns;
  if (select_path((int64_t)T * kk, E, flags) < 0) return MOE_ERR_INVALID_ARGUMENT;
  if (T == 0) return MOE_OK;
  if (!router_w || !x_bf16 || !y) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned(router_w, 16) || !aligned(x_bf16, 16) || !aligned(y, 16))
    return MOE_ERR_INVALID_ARGUMENT;
  const FullCarve c = full_carve(T, k, E, H, I, ns);
  if (!workspace || workspace_bytes < c.total) return MOE_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return MOE_ERR_INVALID_ARGUMENT;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  float* rout = reinterpret_cast<float*>(ws + c.rout);
  const int S = router_slices(T, H, Er);
  uint8_t* lw = ws + c.layer;
  const LayerCarve& lc = c.lc;
  // the router GEMM leaves S planes; the routing launch sums them in plane order
  st = hip_status(launch_router_partials(x_bf16, router_w, T, H, Er, rout, rout, stream));
  if (st == MOE_OK) st = run_front(rout, S, x_bf16, T, H, Er, k, ns, lw, lc, stream);
  if (st != MOE_OK) return st;
  return moe_fp4_grouped_forward(w, lw + lc.xq, lw + lc.xs,
                                 reinterpret_cast<const float*>(lw + lc.gates),
                                 reinterpret_cast<const int32_t*>(lw + lc.offsets),
                                 reinterpret_cast<const int32_t*>(lw + lc.sorted),
                                 reinterpret_cast<const int32_t*>(lw + lc.pos), T, kk, y,
                                 lw + lc.fwd, lc.fwd_bytes, flags, stream);
}

}  // extern "C"

// ------------------------------------------------------- FP8 dense projection
extern "C" {

static moe_status_t check_dense_nk(int32_t N, int32_t K) {
  if (N < 1 || K < 1) return MOE_ERR_INVALID_ARGUMENT;
  if (N % 32 != 0 || K % 128 != 0 || N > (1 << 20) || K > (1 << 20)) return MOE_ERR_UNSUPPORTED;
  if (DenseLayout(N, K).total >= ((size_t)1 << 32)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

size_t moe_fp8_dense_packed_bytes(int32_t N, int32_t K) {
  if (check_dense_nk(N, K) != MOE_OK) return 0;
  return DenseLayout(N, K).total;
}

moe_status_t moe_fp8_dense_prepack(const uint8_t* wq, const uint8_t* ws, int32_t N, int32_t K,
                                   void* packed, size_t packed_bytes, moe_fp8_dense_weights_t* desc,
                                   hipStream_t stream) {
  moe_status_t st = check_dense_nk(N, K);
  if (st != MOE_OK) return st;
  if (!wq || !ws || !packed || !desc) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned(wq, 16) || !aligned(packed, 256)) return MOE_ERR_INVALID_ARGUMENT;
  const DenseLayout L(N, K);
  if (packed_bytes < L.total) return MOE_ERR_INVALID_ARGUMENT;
  st = hip_status(launch_dense_pack(wq, ws, N, K, static_cast<uint8_t*>(packed), stream));
  if (st != MOE_OK) return st;
  desc->N = N;
  desc->K = K;
  desc->layout_version = MOE_FP8_DENSE_LAYOUT_VERSION;
  desc->packed = packed;
  desc->packed_bytes = packed_bytes;
  return MOE_OK;
}

moe_status_t moe_fp8_dense_forward(const moe_fp8_dense_weights_t* w, const uint8_t* xq,
                                   const uint8_t* xs, int32_t T, uint16_t* y, uint32_t flags,
                                   hipStream_t stream) {
  if (!w) return MOE_ERR_INVALID_ARGUMENT;
  if (w->layout_version != MOE_FP8_DENSE_LAYOUT_VERSION || !w->packed) return MOE_ERR_INVALID_ARGUMENT;
  moe_status_t st = check_dense_nk(w->N, w->K);
  if (st != MOE_OK) return st;
  if (w->packed_bytes < DenseLayout(w->N, w->K).total || !aligned(w->packed, 256))
    return MOE_ERR_INVALID_ARGUMENT;
  if (T < 0) return MOE_ERR_INVALID_ARGUMENT;
  const bool fd = flags & MOE_FLAG_FORCE_DECODE, fp = flags & MOE_FLAG_FORCE_PREFILL;
  if ((flags & ~(MOE_FLAG_FORCE_DECODE | MOE_FLAG_FORCE_PREFILL)) != 0 || (fd && fp))
    return MOE_ERR_INVALID_ARGUMENT;
  if ((int64_t)T * w->K >= ((int64_t)1 << 32)) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!xq || !xs || !y) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned(xq, 16) || !aligned(xs, 4) || !aligned(y, 2)) return MOE_ERR_INVALID_ARGUMENT;
  const uint8_t* pk = static_cast<const uint8_t*>(w->packed);
  const bool decode = fd || (!fp && T <= kDenseDecodeMaxT);
  if (decode) return hip_status(launch_dense_decode(pk, xq, xs, T, w->N, w->K, y, stream));
  return hip_status(launch_dense_prefill(pk, xq, xs, T, w->N, w->K, y, stream));
}

}  // extern "C"
