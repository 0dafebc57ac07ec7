/*
 * Seeded synthetic inputs for the FP4 routed-expert MoE layer.
 *
 * This module is shared by the CPU oracle tests and by the GPU path's tests and
 * benchmark.  It only draws random numbers and lays them out in the storage
 * formats of the layer's inputs; it holds none of the layer's arithmetic
 * (no routing, no quantisation, no matrix products).
 *
 * Generator: counter-based SplitMix64 (G. Steele, D. Lea, C. Flood, "Fast
 * splittable pseudorandom number generators", OOPSLA 2014; finaliser constants
 * as published by S. Vigna).  Every tensor gets its own key derived from
 * (seed, tensor id); element n of that tensor is mix(key + n), so any element
 * can be drawn independently and in parallel.
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#include <string.h>

#define SYNTH_GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t x) {
  uint64_t z = x + SYNTH_GAMMA;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

uint64_t synth_mix64(uint64_t x) { return mix64(x); }

uint64_t synth_key(uint64_t seed, uint64_t tensor_id) {
  return mix64(mix64(seed) ^ tensor_id);
}

uint64_t synth_draw(uint64_t key, uint64_t n) { return mix64(key + n); }

/* Uniform random bytes: byte n is byte (n mod 8) of draw n/8. */
void synth_bytes(uint64_t seed, uint64_t tensor_id, uint8_t* out, size_t n) {
  const uint64_t key = synth_key(seed, tensor_id);
  const size_t nw = n / 8;
#pragma omp parallel for schedule(static)
  for (size_t w = 0; w < nw; ++w) {
    uint64_t r = mix64(key + w);
    memcpy(out + 8 * w, &r, 8);
  }
  if (n % 8) {
    uint64_t r = mix64(key + nw);
    memcpy(out + 8 * nw, &r, n % 8);
  }
}

/* Uniform integers in [lo, hi] (the small modulo bias is irrelevant here). */
void synth_uniform_codes(uint64_t seed, uint64_t tensor_id, uint8_t* out, size_t n,
                         int lo, int hi) {
  const uint64_t key = synth_key(seed, tensor_id);
  const uint64_t span = (uint64_t)(hi - lo + 1);
#pragma omp parallel for schedule(static)
  for (size_t i = 0; i < n; ++i) out[i] = (uint8_t)(lo + (int)(mix64(key + i) % span));
}

/* Gaussian N(0, sigma^2) in fp32 by the Box-Muller transform (cosine branch),
 * with both uniforms taken as 24-bit fields of one draw; u1 lies in (0, 1]. */
void synth_normal_f32(uint64_t seed, uint64_t tensor_id, float* out, size_t n, double sigma) {
  const uint64_t key = synth_key(seed, tensor_id);
  const double two_pi = 6.283185307179586476925286766559;
#pragma omp parallel for schedule(static)
  for (size_t i = 0; i < n; ++i) {
    uint64_t r = mix64(key + i);
    double u1 = ((double)(r >> 40) + 1.0) / 16777216.0;
    double u2 = (double)((r >> 16) & 0xFFFFFFu) / 16777216.0;
    out[i] = (float)(sigma * sqrt(-2.0 * log(u1)) * cos(two_pi * u2));
  }
}

/* fp32 -> bf16 storage with round-to-nearest-even (inputs are finite). */
void synth_f32_to_bf16(const float* in, uint16_t* out, size_t n) {
#pragma omp parallel for schedule(static)
  for (size_t i = 0; i < n; ++i) {
    uint32_t b;
    memcpy(&b, &in[i], 4);
    b += 0x7FFFu + ((b >> 16) & 1u);
    out[i] = (uint16_t)(b >> 16);
  }
}

/* Per-expert router bias from a Zipf(s) popularity ranking: a seeded random
 * permutation gives expert e the rank r_e in 1..E, its popularity is
 * p_e = r_e^-s / sum_j j^-s, and the bias added to its logit is ln(E * p_e). */
void synth_zipf_bias(uint64_t seed, uint64_t tensor_id, int E, double s, float* bias) {
  const uint64_t key = synth_key(seed, tensor_id);
  int rank[4096];
  if (E > 4096) return;
  for (int e = 0; e < E; ++e) rank[e] = e + 1;
  for (int i = E - 1; i > 0; --i) { /* Fisher-Yates */
    int j = (int)(mix64(key + (uint64_t)i) % (uint64_t)(i + 1));
    int tmp = rank[i]; rank[i] = rank[j]; rank[j] = tmp;
  }
  double norm = 0.0;
  for (int r = 1; r <= E; ++r) norm += pow((double)r, -s);
  for (int e = 0; e < E; ++e) {
    double p = pow((double)rank[e], -s) / norm;
    bias[e] = (float)log((double)E * p);
  }
}

/* Add a per-column bias to a [rows, cols] fp32 matrix. */
void synth_add_col_bias(float* m, const float* bias, size_t rows, int cols) {
#pragma omp parallel for schedule(static)
  for (size_t r = 0; r < rows; ++r)
    for (int c = 0; c < cols; ++c) m[r * (size_t)cols + c] += bias[c];
}

/* Identity-structured down-projection weights: element (e, r, i) holds the
 * e2m1 code of +1.0 (0x2) where i == (r + e) mod I and +0 elsewhere; two
 * elements per byte along i, even i in the low nibble; every block scale code
 * is 127 (2^0). */
void synth_w2_probe(int E, int H, int I, uint8_t* w2, uint8_t* s2) {
  const size_t rowb = (size_t)I / 2;
  memset(w2, 0, (size_t)E * H * rowb);
  memset(s2, 127, (size_t)E * H * (I / 32));
#pragma omp parallel for schedule(static)
  for (long er = 0; er < (long)E * H; ++er) {
    int e = (int)(er / H), r = (int)(er % H);
    int i = (r + e) % I;
    w2[(size_t)er * rowb + i / 2] |= (uint8_t)(0x2 << (4 * (i & 1)));
  }
}
