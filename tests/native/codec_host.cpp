// Test harness, not part of the library: the library's own MXFP8 codec
// helpers (fp4_routed_expert_amd/csrc/common.h) compiled for the host, so the
// CPU tests can run them on every rounding boundary against the oracle.
#include "../../fp4_routed_expert_amd/csrc/common.h"

extern "C" {

// e4m3 code of each a[i] (|a| < 512), as the kernels' quantisers compute it.
void host_f32_to_e4m3(const float* a, long n, uint8_t* out) {
  for (long i = 0; i < n; ++i) out[i] = (uint8_t)moe::f32_to_e4m3(a[i]);
}

// E8M0 scale code and power-of-two multiplier of each block maximum amax[i] >= 0.
void host_mx_scale(const float* amax, long n, uint8_t* code, float* mul) {
  for (long i = 0; i < n; ++i) code[i] = (uint8_t)moe::mx_scale_from_amax(amax[i], &mul[i]);
}

// One MXFP8 block of 32 fp32 values the way the kernels quantise it: amax,
// scale from it, each element times the multiplier rounded to e4m3.
void host_quant_block32(const float* v, uint8_t* q, uint8_t* scale) {
  float amax = 0.0f;
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  float mul;
  *scale = (uint8_t)moe::mx_scale_from_amax(amax, &mul);
  for (int i = 0; i < 32; ++i) q[i] = (uint8_t)moe::f32_to_e4m3(v[i] * mul);
}

}  // extern "C"
