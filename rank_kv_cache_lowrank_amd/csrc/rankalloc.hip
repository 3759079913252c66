// Global rank allocation (TraceKV abstract; ai4snews Synopsis and Interpretation: the rank budget
// is allocated globally across the KV states rather than uniformly per layer).
//
// Rule (the pages name the step, not its rule): ranks start at r_min and grow by granules of g up
// to r_max; while the budget allows, the granule with the largest marginal energy gain
// sum_{k=r}^{r+g-1} sigma_m[k]^2 is added, equal gains going to the lower matrix index. For
// non-increasing spectra a matrix's gains never increase, so that greedy choice equals taking
// the n = min(floor((budget - M r_min) / g), M nb) best granules of the whole model under the
// order (gain descending, then granule index m * nb + j ascending): the chosen granules of each
// matrix are a prefix, and its rank is r_min + g * (their number).
//
// lr_rank_gains    one thread per granule: its gain in float64 (squares of the float32
//                  spectrum summed in index order; each square is exact in float64), stored as
//                  the bits of the double (non-negative doubles order like their bits), and its
//                  count reset; one thread per matrix also resets its rank to r_min.
// lr_rank_count    grid (granules / 256, key chunks of 256): each thread counts the chunk's
//                  granules ahead of its own in that order (the chunk is read with wave-uniform
//                  loads) and adds the count to its granule's (integer atomics: the total does
//                  not depend on their order).
// lr_rank_select   one thread per matrix: rank = r_min + g * (its granules with fewer than n
//                  granules ahead).
#include "device_common.h"
#include "internal.h"

namespace lr {

struct RankArgs {
  const float* sigma;
  unsigned long long* keys;
  int32_t* ahead;
  int32_t* ranks;
  int n_mat, sigma_ld, r_min, g, nb, N;
  long long n_take;
};

__global__ __launch_bounds__(256) void lr_rank_gains(RankArgs a) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= a.N) return;
  const int m = i / a.nb, j = i - m * a.nb;
  const float* row = a.sigma + (size_t)m * a.sigma_ld + a.r_min + j * a.g;
  double acc = 0.0;
  for (int k = 0; k < a.g; ++k) {
    const double s = (double)row[k];
    acc = acc + s * s;
  }
  a.keys[i] = (unsigned long long)__builtin_bit_cast(long long, acc);
  a.ahead[i] = 0;
  if (j == 0) a.ranks[m] = a.r_min;
}

constexpr int kRankChunk = 256;

__global__ __launch_bounds__(256) void lr_rank_count(RankArgs a) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  const bool mine = i < a.N;
  const unsigned long long ki = mine ? a.keys[i] : 0ull;
  const int t0 = blockIdx.y * kRankChunk;
  const int t1 = min(t0 + kRankChunk, a.N);
  int ahead = 0;
#pragma unroll 8
  for (int t = t0; t < t1; ++t) {
    const unsigned long long kj = a.keys[t];   // the same address in every lane
    ahead += (kj > ki) || (kj == ki && t < i);
  }
  if (mine && ahead > 0) atomicAdd(&a.ahead[i], ahead);
}

__global__ __launch_bounds__(256) void lr_rank_select(RankArgs a) {
  const int m = blockIdx.x * 256 + threadIdx.x;
  if (m >= a.n_mat) return;
  int taken = 0;
  for (int j = 0; j < a.nb; ++j) taken += a.ahead[m * a.nb + j] < a.n_take;
  a.ranks[m] = a.r_min + a.g * taken;
}

hipError_t launch_rank_allocate(const float* sigma, int n_mat, int sigma_ld, long long n_take, int r_min,
                                int g, int nb, int32_t* ranks, void* ws, hipStream_t st) {
  RankArgs a;
  a.sigma = sigma;
  a.keys = (unsigned long long*)ws;
  a.ranks = ranks;
  a.n_mat = n_mat;
  a.sigma_ld = sigma_ld;
  a.r_min = r_min;
  a.g = g;
  a.nb = nb;
  a.N = n_mat * nb;
  a.ahead = (int32_t*)(a.keys + (a.N > n_mat ? a.N : n_mat));
  a.n_take = n_take;
  if (a.N == 0) {
    // no granule to hand out: every rank is r_min (one thread per matrix)
    a.nb = 1;
    a.N = n_mat;
    a.g = 0;
    a.n_take = 0;
    hipLaunchKernelGGL(lr_rank_gains, dim3((n_mat + 255) / 256), dim3(256), 0, st, a);
    return hipGetLastError();
  }
  const unsigned nblk = (unsigned)((a.N + 255) / 256);
  hipLaunchKernelGGL(lr_rank_gains, dim3(nblk), dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(lr_rank_count, dim3(nblk, (unsigned)((a.N + kRankChunk - 1) / kRankChunk)), dim3(256), 0, st, a);
  hipLaunchKernelGGL(lr_rank_select, dim3((n_mat + 255) / 256), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace lr
