/*
 * CPU ORACLE for the FP4 routed mixture-of-experts layer.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is built into liboracle.so, which only
 * the tests, the smoke check and the benchmark's CPU-baseline leg load.  The
 * GPU library never links, includes or calls it, and it shares no code, table
 * or constant with the GPU library.
 *
 * What it computes: one routed-expert MoE layer with 4-bit e2m1 weights and
 * per-32 E8M0 block scales, MXFP8 (e4m3) activations, SwiGLU between the
 * gate/up and down projections, and a gate-weighted combine.  The pages name
 * this as the "FP4 routed mixture-of-experts computation" whose W2 (down
 * projection) layout had to be repaired ("DeepSeek-V4-Flash on AMD gfx90a:
 * Correctness Recovery and Inference Performance Engineering", abstract);
 * the MoE top-k must compare in FP32 with a fixed tie-break (pwwt.cn review,
 * section 4.1 table, row "MoE routing top-k"), ties go by expert id and never
 * by memory address (same page, section 4.2); MI355X uses the OCP FP8 dialect,
 * not fnuz (aijianwen.com MI300X log, FP8 section); the experts run through an
 * MXFP4 MoE path (same log, profiling section).  The 4-bit/8-bit element
 * formats and the E8M0 scale are those of the OCP Microscaling (MX) v1.0
 * format family.
 *
 * Arithmetic: every decode is exact.  Dot products, SwiGLU, softmax and the
 * combine run in plain ascending index order in the accumulation type acc_t:
 * fp32 by default (the precision the method fixes: products of the decoded
 * values, which are exact, summed in fp32; exp in fp32), or fp64 when built
 * with -DORC_ACC_FP64, a diagnostic build that measures the fp32 build's own
 * rounding.  The one place where a floating value decides an integer code
 * inside the layer (requantising the SwiGLU output h) takes that decision on
 * h in fp32, the precision the GPU kernels hold h in, in both builds.
 * Routing compares the fp32 logits themselves.  The router logits are the
 * exact sums (fp64) in both builds: they are compared against a bound.
 *
 * Beside the layer: the router logits and the shared expert around it, and
 * the FP8 dense projection (FP8 weights with per-32 E8M0 scales times MXFP8
 * activations), each at the end of this file.
 *
 * No blocking, no reordering: each function is the definition written out.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef ORC_ACC_FP64
typedef double acc_t;
#define ACC_EXP exp
#define ORC_PRECISION "fp64"
#else
typedef float acc_t;
#define ACC_EXP expf
#define ORC_PRECISION "fp32"
#endif

/* The accumulation type this build was compiled with: "fp32" or "fp64". */
const char* orc_precision(void) { return ORC_PRECISION; }

/* ---------------------------------------------------------------- decoders */

/* e2m1: 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit; exponent field 0
 * is subnormal (value = m * 0.5).  Codes 0..7 are 0, .5, 1, 1.5, 2, 3, 4, 6. */
double orc_e2m1(unsigned code) {
  unsigned s = (code >> 3) & 1u, e = (code >> 1) & 3u, m = code & 1u;
  double mag = (e == 0) ? 0.5 * (double)m : ldexp(1.0 + 0.5 * (double)m, (int)e - 1);
  return s ? -mag : mag;
}

/* E8M0: an unsigned biased exponent, value 2^(code-127); code 255 is NaN. */
double orc_e8m0(unsigned code) {
  if (code == 255u) return NAN;
  return ldexp(1.0, (int)code - 127);
}

/* OCP e4m3fn: 1 sign, 4 exponent bits (bias 7), 3 mantissa bits, no infinity;
 * exponent 0 is subnormal (m * 2^-9); S.1111.111 is NaN; max finite 448. */
double orc_e4m3(unsigned byte) {
  unsigned s = (byte >> 7) & 1u, e = (byte >> 3) & 15u, m = byte & 7u;
  double mag;
  if (e == 15u && m == 7u) return NAN;
  if (e == 0u) mag = ldexp((double)m, -9);
  else mag = ldexp(1.0 + (double)m / 8.0, (int)e - 7);
  return s ? -mag : mag;
}

/* bf16 storage -> value (exact). */
double orc_bf16(uint16_t bits) {
  uint32_t b = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &b, 4);
  return (double)f;
}

/* Row `row` of a packed weight matrix with K elements per row, decoded into
 * out[0..K): each element is its nibble's e2m1 value (even K index in the low
 * half of the byte) times its 32-block's E8M0 scale (the product is exact). */
static void decode_weight_row(const uint8_t* w, const uint8_t* s, int K, long row, double* out) {
  double e2m1_of[16];
  for (unsigned n = 0; n < 16; ++n) e2m1_of[n] = orc_e2m1(n);
  for (int b = 0; b < K / 32; ++b) {
    const double scale = orc_e8m0(s[row * (K / 32) + b]);
    for (int c = 32 * b; c < 32 * b + 32; ++c) {
      const uint8_t byte = w[row * (K / 2) + c / 2];
      const unsigned nib = (c & 1) ? (byte >> 4) : (byte & 15u);
      out[c] = e2m1_of[nib] * scale;
    }
  }
}

void orc_decode_fp4_matrix(const uint8_t* w, const uint8_t* s, long rows, int K, double* out) {
#pragma omp parallel for schedule(static)
  for (long r = 0; r < rows; ++r) decode_weight_row(w, s, K, r, out + r * K);
}

void orc_decode_mxfp8(const uint8_t* q, const uint8_t* s, long rows, int K, double* out) {
#pragma omp parallel for schedule(static)
  for (long r = 0; r < rows; ++r)
    for (long c = 0; c < K; ++c)
      out[r * K + c] = orc_e4m3(q[r * K + c]) * orc_e8m0(s[r * (K / 32) + c / 32]);
}

/* ------------------------------------------------------------ quantisation */

/* Round |a| to the OCP e4m3fn grid, nearest value, ties to the code with an
 * even (zero) mantissa LSB, saturating at 448; the sign bit is always kept, so
 * a negative input that rounds to zero gives 0x80.  Done by a binary search
 * over the 127 finite non-negative codes, which are increasing in value. */
unsigned orc_e4m3_rne_sat(double a) {
  unsigned sign = signbit(a) ? 0x80u : 0u;
  double m = fabs(a);
  if (m >= 448.0) return sign | 0x7Eu;
  unsigned lo = 0, hi = 0x7E; /* invariant: e4m3(lo) <= m < e4m3(hi) */
  while (hi - lo > 1) {
    unsigned mid = (lo + hi) / 2;
    if (orc_e4m3(mid) <= m) lo = mid; else hi = mid;
  }
  double dlo = m - orc_e4m3(lo), dhi = orc_e4m3(hi) - m;
  unsigned c;
  if (dlo < dhi) c = lo;
  else if (dhi < dlo) c = hi;
  else c = (lo & 1u) ? hi : lo;
  return sign | c;
}

/* MXFP8 quantisation of one block of 32 values (OCP MX v1.0 conversion rule):
 * shared exponent X = floor(log2(max|v|)) - 8, where 8 is the largest e4m3
 * exponent; X = -127 for an all-zero block; X clamped to [-127, 127]; the
 * scale code is X + 127; each element is v * 2^-X rounded by orc_e4m3_rne_sat
 * (the multiply by a power of two is exact). */
void orc_quant_block32(const double* v, uint8_t* q, uint8_t* scale) {
  double amax = 0.0;
  for (int i = 0; i < 32; ++i) if (fabs(v[i]) > amax) amax = fabs(v[i]);
  int X;
  if (amax == 0.0) {
    X = -127;
  } else {
    int ex;
    frexp(amax, &ex);           /* amax = f * 2^ex, f in [0.5, 1) */
    X = (ex - 1) - 8;           /* floor(log2 amax) - 8 */
    if (X < -127) X = -127;
    if (X > 127) X = 127;
  }
  *scale = (uint8_t)(X + 127);
  for (int i = 0; i < 32; ++i) q[i] = (uint8_t)orc_e4m3_rne_sat(ldexp(v[i], -X));
}

/* Quantise rows of bf16 activations [M, K] to e4m3 bytes [M, K] and scale
 * codes [M, K/32]. */
void orc_quant_mxfp8_bf16(const uint16_t* x, long M, int K, uint8_t* q, uint8_t* s) {
#pragma omp parallel for schedule(static)
  for (long r = 0; r < M; ++r) {
    double v[32];
    for (int b = 0; b < K / 32; ++b) {
      for (int i = 0; i < 32; ++i) v[i] = orc_bf16(x[r * K + b * 32 + i]);
      orc_quant_block32(v, q + r * K + b * 32, s + r * (K / 32) + b);
    }
  }
}

/* Same for fp32 rows. */
void orc_quant_mxfp8_f32(const float* x, long M, int K, uint8_t* q, uint8_t* s) {
#pragma omp parallel for schedule(static)
  for (long r = 0; r < M; ++r) {
    double v[32];
    for (int b = 0; b < K / 32; ++b) {
      for (int i = 0; i < 32; ++i) v[i] = (double)x[r * K + b * 32 + i];
      orc_quant_block32(v, q + r * K + b * 32, s + r * (K / 32) + b);
    }
  }
}

/* ----------------------------------------------------------------- routing */

/* Top-k routing of one token: slot j holds the expert with the j-th largest
 * logit, ties going to the lower expert index (fixed tie-break on expert id,
 * pwwt.cn review sections 4.1-4.2).  The fp32 logits are compared as fp32
 * values (so -0 equals +0).  Gates are a softmax over the k selected logits:
 * g_j = exp(l_j - l_0) / sum_i exp(l_i - l_0), the sum in slot order. */
void orc_route_token(const float* logit, int E, int k, int32_t* ids, float* gates) {
  unsigned char* taken = (unsigned char*)calloc((size_t)E, 1);
  for (int j = 0; j < k; ++j) {
    int best = -1;
    for (int e = 0; e < E; ++e) {
      if (taken[e]) continue;
      if (best < 0 || logit[e] > logit[best]) best = e;
    }
    taken[best] = 1;
    ids[j] = best;
  }
  free(taken);
  const acc_t l0 = (acc_t)logit[ids[0]];
  acc_t den = 0;
  for (int j = 0; j < k; ++j) den += ACC_EXP((acc_t)logit[ids[j]] - l0);
  for (int j = 0; j < k; ++j) gates[j] = (float)(ACC_EXP((acc_t)logit[ids[j]] - l0) / den);
}

void orc_route(const float* logits, long T, int E, int k, int32_t* ids, float* gates) {
#pragma omp parallel for schedule(static)
  for (long t = 0; t < T; ++t) orc_route_token(logits + t * E, E, k, ids + t * k, gates + t * k);
}

/* --------------------------------------------------------- sort / permute */

/* Expert grouping of the P = T*k (token, slot) pairs, pair p = t*k + j:
 * counts[e] = number of pairs routed to e; offsets = exclusive prefix sum
 * (offsets[E] = P); sorted_pair lists the pairs of expert 0, then expert 1,
 * ..., each group in ascending p (a stable order: unstable sorting is ruled
 * out, pwwt.cn review section 4.2); pair_pos is its inverse. */
void orc_sort(const int32_t* ids, long P, int E, int32_t* counts, int32_t* offsets,
              int32_t* sorted_pair, int32_t* pair_pos) {
  for (int e = 0; e < E; ++e) counts[e] = 0;
  for (long p = 0; p < P; ++p) counts[ids[p]] += 1;
  offsets[0] = 0;
  for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  long pos = 0;
  for (int e = 0; e < E; ++e)
    for (long p = 0; p < P; ++p)
      if (ids[p] == e) sorted_pair[pos++] = (int32_t)p;
  for (long s = 0; s < P; ++s) pair_pos[sorted_pair[s]] = (int32_t)s;
}

/* ------------------------------------------------------------ expert FFN */

/* Gate/up projections of one MXFP8 activation row through expert weights
 * W1, W3 ([I, H] packed): G[i] = sum_h x[h] W1[i,h], U[i] likewise with W3,
 * summed in ascending h in acc_t (each product of an e4m3 and an e2m1 value
 * with power-of-two scales is exact in either type).  G, U are returned as
 * doubles holding the acc_t values. */
void orc_expert_gate_up(const uint8_t* xq, const uint8_t* xs, int H, int I,
                        const uint8_t* w1, const uint8_t* s1,
                        const uint8_t* w3, const uint8_t* s3, double* G, double* U) {
  acc_t* xd = (acc_t*)malloc(sizeof(acc_t) * (size_t)H);
  for (int h = 0; h < H; ++h) xd[h] = (acc_t)(orc_e4m3(xq[h]) * orc_e8m0(xs[h / 32]));
#pragma omp parallel
  {
    double* r1 = (double*)malloc(sizeof(double) * (size_t)H);
    double* r3 = (double*)malloc(sizeof(double) * (size_t)H);
#pragma omp for schedule(static)
    for (int i = 0; i < I; ++i) {
      decode_weight_row(w1, s1, H, i, r1);
      decode_weight_row(w3, s3, H, i, r3);
      acc_t g = 0, u = 0;
      for (int h = 0; h < H; ++h) {
        g += xd[h] * (acc_t)r1[h];
        u += xd[h] * (acc_t)r3[h];
      }
      G[i] = (double)g;
      U[i] = (double)u;
    }
    free(r1);
    free(r3);
  }
  free(xd);
}

/* SwiGLU h = silu(G) * U with silu(z) = z / (1 + e^-z), evaluated in acc_t,
 * then MXFP8 requantisation of h per 32 along I.  h is rounded to fp32 first. */
void orc_swiglu_requant(const double* G, const double* U, int I, float* h,
                        uint8_t* hq, uint8_t* hs) {
  for (int i = 0; i < I; ++i) {
    const acc_t g = (acc_t)G[i], u = (acc_t)U[i];
    h[i] = (float)(g / ((acc_t)1 + ACC_EXP(-g)) * u);
  }
  double v[32];
  for (int b = 0; b < I / 32; ++b) {
    for (int i = 0; i < 32; ++i) v[i] = (double)h[b * 32 + i];
    orc_quant_block32(v, hq + b * 32, hs + b);
  }
}

/* Down projection: O[r] = sum_i h[i] W2[r,i], W2 packed [H, I], summed in
 * ascending i in acc_t. */
void orc_expert_down(const uint8_t* hq, const uint8_t* hs, int H, int I,
                     const uint8_t* w2, const uint8_t* s2, double* O) {
  acc_t* hd = (acc_t*)malloc(sizeof(acc_t) * (size_t)I);
  for (int i = 0; i < I; ++i) hd[i] = (acc_t)(orc_e4m3(hq[i]) * orc_e8m0(hs[i / 32]));
#pragma omp parallel
  {
    double* r2 = (double*)malloc(sizeof(double) * (size_t)I);
#pragma omp for schedule(static)
    for (int r = 0; r < H; ++r) {
      decode_weight_row(w2, s2, I, r, r2);
      acc_t o = 0;
      for (int i = 0; i < I; ++i) o += hd[i] * (acc_t)r2[i];
      O[r] = (double)o;
    }
    free(r2);
  }
  free(hd);
}

/* ------------------------------------------------------------ whole layer */

/* The layer for a list of tokens, each computed on its own (the plain
 * per-token definition): route, quantise x_t, run each selected expert's
 * FFN, then y_t = sum_{j=0..k-1, in order} g_j * O_j.
 * y is [ntok, H]; optional per-pair outputs (h, hq, hs: [ntok*k, I] etc.)
 * may be NULL. */
void orc_layer_tokens(const uint16_t* x, const float* logits, int H, int I, int E, int k,
                      const uint8_t* w1, const uint8_t* s1, const uint8_t* w3, const uint8_t* s3,
                      const uint8_t* w2, const uint8_t* s2,
                      const int32_t* tokens, long ntok, float* y,
                      float* h_out, uint8_t* hq_out, uint8_t* hs_out) {
  const size_t wup = (size_t)I * (H / 2), sup = (size_t)I * (H / 32);
  const size_t wdn = (size_t)H * (I / 2), sdn = (size_t)H * (I / 32);
  int32_t* ids = (int32_t*)malloc(sizeof(int32_t) * (size_t)k);
  float* gates = (float*)malloc(sizeof(float) * (size_t)k);
  uint8_t* xq = (uint8_t*)malloc((size_t)H);
  uint8_t* xs = (uint8_t*)malloc((size_t)H / 32);
  double* G = (double*)malloc(sizeof(double) * (size_t)I);
  double* U = (double*)malloc(sizeof(double) * (size_t)I);
  float* h = (float*)malloc(sizeof(float) * (size_t)I);
  uint8_t* hq = (uint8_t*)malloc((size_t)I);
  uint8_t* hs = (uint8_t*)malloc((size_t)I / 32);
  double* O = (double*)malloc(sizeof(double) * (size_t)H);
  acc_t* acc = (acc_t*)malloc(sizeof(acc_t) * (size_t)H);
  for (long n = 0; n < ntok; ++n) {
    long t = tokens[n];
    orc_route_token(logits + t * E, E, k, ids, gates);
    orc_quant_mxfp8_bf16(x + t * (long)H, 1, H, xq, xs);
    for (int r = 0; r < H; ++r) acc[r] = 0;
    for (int j = 0; j < k; ++j) {
      size_t e = (size_t)ids[j];
      orc_expert_gate_up(xq, xs, H, I, w1 + e * wup, s1 + e * sup, w3 + e * wup, s3 + e * sup, G, U);
      orc_swiglu_requant(G, U, I, h, hq, hs);
      orc_expert_down(hq, hs, H, I, w2 + e * wdn, s2 + e * sdn, O);
      for (int r = 0; r < H; ++r) acc[r] += (acc_t)gates[j] * (acc_t)O[r];
      if (h_out) memcpy(h_out + ((size_t)n * k + j) * I, h, sizeof(float) * (size_t)I);
      if (hq_out) memcpy(hq_out + ((size_t)n * k + j) * I, hq, (size_t)I);
      if (hs_out) memcpy(hs_out + ((size_t)n * k + j) * (I / 32), hs, (size_t)I / 32);
    }
    for (int r = 0; r < H; ++r) y[n * (long)H + r] = (float)acc[r];
  }
  free(ids); free(gates); free(xq); free(xs); free(G); free(U);
  free(h); free(hq); free(hs); free(O); free(acc);
}

/* The layer's per-pair intermediates for a list of (token, slot) pairs
 * p = t*k + j, by the same steps as orc_layer_tokens: route token t, take its
 * slot-j expert e, quantise x_t, run that expert's gate/up projections,
 * SwiGLU and requantisation, and its down projection.  Per listed pair n:
 * expert[n] = e, h[n, I] (fp32), hq[n, I], hs[n, I/32], and O[n, H] (the
 * down projection before the gate, as doubles holding acc_t values).  The
 * outputs may be NULL except O. */
void orc_layer_pairs(const uint16_t* x, const float* logits, int H, int I, int E, int k,
                     const uint8_t* w1, const uint8_t* s1, const uint8_t* w3, const uint8_t* s3,
                     const uint8_t* w2, const uint8_t* s2, const int32_t* pairs, long npairs,
                     int32_t* expert_out, float* h_out, uint8_t* hq_out, uint8_t* hs_out,
                     double* O) {
  const size_t wup = (size_t)I * (H / 2), sup = (size_t)I * (H / 32);
  const size_t wdn = (size_t)H * (I / 2), sdn = (size_t)H * (I / 32);
  int32_t* ids = (int32_t*)malloc(sizeof(int32_t) * (size_t)k);
  float* gates = (float*)malloc(sizeof(float) * (size_t)k);
  uint8_t* xq = (uint8_t*)malloc((size_t)H);
  uint8_t* xs = (uint8_t*)malloc((size_t)H / 32);
  double* G = (double*)malloc(sizeof(double) * (size_t)I);
  double* U = (double*)malloc(sizeof(double) * (size_t)I);
  float* h = (float*)malloc(sizeof(float) * (size_t)I);
  uint8_t* hq = (uint8_t*)malloc((size_t)I);
  uint8_t* hs = (uint8_t*)malloc((size_t)I / 32);
  for (long n = 0; n < npairs; ++n) {
    const long t = pairs[n] / k;
    const int j = (int)(pairs[n] % k);
    orc_route_token(logits + t * E, E, k, ids, gates);
    orc_quant_mxfp8_bf16(x + t * (long)H, 1, H, xq, xs);
    const size_t e = (size_t)ids[j];
    orc_expert_gate_up(xq, xs, H, I, w1 + e * wup, s1 + e * sup, w3 + e * wup, s3 + e * sup, G, U);
    orc_swiglu_requant(G, U, I, h, hq, hs);
    orc_expert_down(hq, hs, H, I, w2 + e * wdn, s2 + e * sdn, O + (size_t)n * H);
    if (expert_out) expert_out[n] = (int32_t)e;
    if (h_out) memcpy(h_out + (size_t)n * I, h, sizeof(float) * (size_t)I);
    if (hq_out) memcpy(hq_out + (size_t)n * I, hq, (size_t)I);
    if (hs_out) memcpy(hs_out + (size_t)n * (I / 32), hs, (size_t)I / 32);
  }
  free(ids); free(gates); free(xq); free(xs); free(G); free(U);
  free(h); free(hq); free(hs);
}

/* --------------------------------------------- router and shared expert */

/* Router logits ahead of the top-k (the gate network's first layer, which the
 * pwwt.cn review, section 4.1, lets run at low precision while the top-k
 * compare stays fp32): logit[t,e] = sum_h x[t,h] * Wg[e,h] with x and Wg in
 * bf16.  Each product of two bf16 values is exact in fp64 and the sum is
 * taken in fp64 in index order.  absum[t,e] = sum_h |x[t,h] * Wg[e,h]| bounds
 * the rounding error of any fp32 evaluation of the same sum. */
void orc_router_logits(const uint16_t* x, const uint16_t* wg, long T, int H, int E,
                       double* logit, double* absum) {
#pragma omp parallel for schedule(static)
  for (long t = 0; t < T; ++t) {
    for (int e = 0; e < E; ++e) {
      double s = 0.0, a = 0.0;
      for (int h = 0; h < H; ++h) {
        const double p = orc_bf16(x[t * (long)H + h]) * orc_bf16(wg[(long)e * H + h]);
        s += p;
        a += fabs(p);
      }
      logit[t * E + e] = s;
      absum[t * E + e] = a;
    }
  }
}

/* The layer with a shared expert: the routed part exactly as orc_layer_tokens,
 * then one more expert FFN (weights w1s..s2s, intermediate size Is) on the same
 * MXFP8 row x_t, added with weight 1 after the k routed slots:
 * y_t = sum_{j=0..k-1, in order} g_j * O_j + O_shared.  y is [ntok, H]. */
void orc_layer_tokens_shared(const uint16_t* x, const float* logits, int H, int I, int E, int k,
                             const uint8_t* w1, const uint8_t* s1, const uint8_t* w3,
                             const uint8_t* s3, const uint8_t* w2, const uint8_t* s2, int Is,
                             const uint8_t* w1s, const uint8_t* s1s, const uint8_t* w3s,
                             const uint8_t* s3s, const uint8_t* w2s, const uint8_t* s2s,
                             const int32_t* tokens, long ntok, float* y) {
  const size_t wup = (size_t)I * (H / 2), sup = (size_t)I * (H / 32);
  const size_t wdn = (size_t)H * (I / 2), sdn = (size_t)H * (I / 32);
  const int Imax = I > Is ? I : Is;
  int32_t* ids = (int32_t*)malloc(sizeof(int32_t) * (size_t)k);
  float* gates = (float*)malloc(sizeof(float) * (size_t)k);
  uint8_t* xq = (uint8_t*)malloc((size_t)H);
  uint8_t* xs = (uint8_t*)malloc((size_t)H / 32);
  double* G = (double*)malloc(sizeof(double) * (size_t)Imax);
  double* U = (double*)malloc(sizeof(double) * (size_t)Imax);
  float* h = (float*)malloc(sizeof(float) * (size_t)Imax);
  uint8_t* hq = (uint8_t*)malloc((size_t)Imax);
  uint8_t* hs = (uint8_t*)malloc((size_t)Imax / 32);
  double* O = (double*)malloc(sizeof(double) * (size_t)H);
  acc_t* acc = (acc_t*)malloc(sizeof(acc_t) * (size_t)H);
  for (long n = 0; n < ntok; ++n) {
    long t = tokens[n];
    orc_route_token(logits + t * E, E, k, ids, gates);
    orc_quant_mxfp8_bf16(x + t * (long)H, 1, H, xq, xs);
    for (int r = 0; r < H; ++r) acc[r] = 0;
    for (int j = 0; j < k; ++j) {
      size_t e = (size_t)ids[j];
      orc_expert_gate_up(xq, xs, H, I, w1 + e * wup, s1 + e * sup, w3 + e * wup, s3 + e * sup, G, U);
      orc_swiglu_requant(G, U, I, h, hq, hs);
      orc_expert_down(hq, hs, H, I, w2 + e * wdn, s2 + e * sdn, O);
      for (int r = 0; r < H; ++r) acc[r] += (acc_t)gates[j] * (acc_t)O[r];
    }
    if (w1s) {
      orc_expert_gate_up(xq, xs, H, Is, w1s, s1s, w3s, s3s, G, U);
      orc_swiglu_requant(G, U, Is, h, hq, hs);
      orc_expert_down(hq, hs, H, Is, w2s, s2s, O);
      for (int r = 0; r < H; ++r) acc[r] += (acc_t)O[r];
    }
    for (int r = 0; r < H; ++r) y[n * (long)H + r] = (float)acc[r];
  }
  free(ids); free(gates); free(xq); free(xs); free(G); free(U);
  free(h); free(hq); free(hs); free(O); free(acc);
}

/* ------------------------------------------------- FP8 dense projection */

/* A dense (non-expert) linear layer with FP8 weights, the pages' second
 * quantised workload ("FP8 dense projections": abstract of the arxivdaily
 * page; the pwwt.cn review, section 5.3, names block-wise quantisation as the
 * way FP8 pays off).  Weights W [N, K] are OCP e4m3 codes with one E8M0 scale per 32
 * consecutive K elements of a row, activations the MXFP8 rows xq/xs of the
 * path's own quantiser; y[t, n] = sum_k x[t, k] * W[n, k] over the decoded
 * values, summed in acc_t in index order (each product of two scaled e4m3
 * values is exact in fp64; in fp32 too while the product's scale stays in
 * the normal range, as at every scale the path produces).  tokens lists the rows of x to compute; y is
 * [ntok, N]. */
void orc_dense_fp8(const uint8_t* xq, const uint8_t* xs, const uint8_t* wq, const uint8_t* ws,
                   int N, int K, const int32_t* tokens, long ntok, double* y) {
  acc_t* xd = (acc_t*)malloc(sizeof(acc_t) * (size_t)ntok * (size_t)K);
  for (long i = 0; i < ntok; ++i) {
    const long t = tokens[i];
    for (int k = 0; k < K; ++k)
      xd[i * K + k] = (acc_t)(orc_e4m3(xq[t * K + k]) * orc_e8m0(xs[t * (K / 32) + k / 32]));
  }
#pragma omp parallel for schedule(static)
  for (int n = 0; n < N; ++n) {
    acc_t* wd = (acc_t*)malloc(sizeof(acc_t) * (size_t)K);
    for (int k = 0; k < K; ++k)
      wd[k] = (acc_t)(orc_e4m3(wq[(long)n * K + k]) * orc_e8m0(ws[(long)n * (K / 32) + k / 32]));
    for (long i = 0; i < ntok; ++i) {
      acc_t acc = 0;
      for (int k = 0; k < K; ++k) acc += xd[i * K + k] * wd[k];
      y[i * N + n] = (double)acc;
    }
    free(wd);
  }
  free(xd);
}
