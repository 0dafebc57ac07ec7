// Expert sort / permute of the (token, slot) pairs: counting sort by expert.
//
// Counts come from LDS integer atomics (order-free, so exact and deterministic).
// Positions never come from atomics: a pair's rank among the pairs of its expert
// is the number of earlier pairs with the same expert, computed from wavefront
// ballots (equal-id lane masks) and a per-wave table in LDS, so the order
// inside each expert is ascending pair index -- a stable sort, as required by
// pwwt.cn review section 4.2 (no unstable sorting; ties by expert id).
//
// P <= kSmall pairs: one workgroup does histogram, scan and scatter.
// Larger P: (1) per-chunk histograms, (2) one workgroup scans them in
// (expert, chunk) order, (3) each chunk scatters from its own base.
#include "stages.h"

namespace moe {
namespace {

constexpr int kThreads = 256;           // 4 waves
constexpr int kWaves = kThreads / 64;
constexpr int kSmall = 4096;            // up to this many pairs: one workgroup

// Pairs per workgroup above kSmall: the power of two nearest above P / 64 in
// [1024, 4096], so that about 64 workgroups histogram and scatter while the
// scan's walk over the chunks stays short (c3 sizes: 24.6 -> 16.5 us, c4:
// 32.5 -> 20.7 us against fixed 4096-pair chunks and an unbatched scan).
int sort_chunk(long P) {
  int c = 1024;
  while (c < 4096 && (long)c * 64 < P) c *= 2;
  return c;
}

__global__ __launch_bounds__(kThreads) void sort_small_kernel(
    const int32_t* __restrict__ ids, int P, int E, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_pair,
    int32_t* __restrict__ pair_pos) {
  __shared__ SortSmallLds sm;
  sort_small_body(ids, P, E, sm, counts, offsets, sorted_pair, pair_pos);
}

__global__ __launch_bounds__(kThreads) void sort_hist_kernel(const int32_t* __restrict__ ids,
                                                             int P, int E, int chunk,
                                                             int32_t* __restrict__ chunk_counts) {
  __shared__ int hist[kMaxE];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += kThreads) hist[e] = 0;
  __syncthreads();
  const int p0 = blockIdx.x * chunk, p1 = min(P, p0 + chunk);
  for (int p = p0 + tid; p < p1; p += kThreads) atomicAdd(&hist[ids[p]], 1);
  __syncthreads();
  for (int e = tid; e < E; e += kThreads) chunk_counts[(size_t)blockIdx.x * E + e] = hist[e];
}

// chunk_counts[b][e] -> the number of pairs of expert e in chunks before b
// (the scatter adds offsets[e]); counts and offsets of the whole sort.  The
// chunk counts of an expert are loaded eight at a time, so the walk over the
// chunks costs one memory round trip per eight chunks.
__global__ __launch_bounds__(kThreads) void sort_scan_kernel(int nchunks, int P, int E,
                                                             int32_t* __restrict__ chunk_counts,
                                                             int32_t* __restrict__ counts,
                                                             int32_t* __restrict__ offsets) {
  __shared__ int tot[kMaxE];
  __shared__ int wave_tot[kWaves];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += kThreads) {
    int run = 0;
    for (int b0 = 0; b0 < nchunks; b0 += 8) {
      int c[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        c[u] = b0 + u < nchunks ? chunk_counts[(size_t)(b0 + u) * E + e] : 0;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (b0 + u < nchunks) chunk_counts[(size_t)(b0 + u) * E + e] = run;
        run += c[u];
      }
    }
    tot[e] = run;
    counts[e] = run;
  }
  __syncthreads();
  const int total = block_exclusive_scan256(tot, E, wave_tot);
  for (int e = tid; e < E; e += kThreads) offsets[e] = tot[e];
  if (tid == 0) offsets[E] = total;
}

__global__ __launch_bounds__(kThreads) void sort_scatter_kernel(
    const int32_t* __restrict__ ids, int P, int E, int chunk, const int32_t* __restrict__ chunk_base,
    const int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_pair,
    int32_t* __restrict__ pair_pos) {
  __shared__ int base[kMaxE];
  __shared__ int table[kWaves * kMaxE];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += kThreads)
    base[e] = offsets[e] + chunk_base[(size_t)blockIdx.x * E + e];
  for (int i = tid; i < kWaves * E; i += kThreads) table[i] = 0;
  __syncthreads();
  const int p0 = blockIdx.x * chunk, p1 = min(P, p0 + chunk);
  stable_scatter<kThreads>(ids, p0, p1, E, base, table, sorted_pair, pair_pos);
}

}  // namespace

size_t sort_workspace_bytes(int T, int E, int k) {
  const long P = (long)T * k;
  const int chunk = sort_chunk(P);
  const long nchunks = (P + chunk - 1) / chunk;
  return P <= kSmall ? 0 : (size_t)nchunks * E * sizeof(int32_t);
}

hipError_t launch_sort_permute(const int32_t* ids, int T, int E, int k, int32_t* counts,
                               int32_t* offsets, int32_t* sorted_pair, int32_t* pair_pos,
                               void* ws, hipStream_t s) {
  const int P = T * k;
  const int chunk = sort_chunk(P);
  const int nchunks = (P + chunk - 1) / chunk;
  if (P <= kSmall) {
    hipLaunchKernelGGL(sort_small_kernel, dim3(1), dim3(kThreads), 0, s, ids, P, E, counts,
                       offsets, sorted_pair, pair_pos);
    return hipGetLastError();
  }
  int32_t* chunk_counts = static_cast<int32_t*>(ws);
  hipLaunchKernelGGL(sort_hist_kernel, dim3(nchunks), dim3(kThreads), 0, s, ids, P, E, chunk,
                     chunk_counts);
  hipLaunchKernelGGL(sort_scan_kernel, dim3(1), dim3(kThreads), 0, s, nchunks, P, E,
                     chunk_counts, counts, offsets);
  hipLaunchKernelGGL(sort_scatter_kernel, dim3(nchunks), dim3(kThreads), 0, s, ids, P, E, chunk,
                     chunk_counts, offsets, sorted_pair, pair_pos);
  return hipGetLastError();
}

}  // namespace moe
