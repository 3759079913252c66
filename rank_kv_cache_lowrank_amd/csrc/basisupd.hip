// Block-incremental basis update of a low-rank KV matrix (iS-KV, "iS-KV: Online Low-Rank KV Cache
// Compression via Block-Incremental SVD", English abstract and method summary: the low-rank basis
// evolves incrementally as blocks of older states are folded into the bounded-rank history, and
// the stored coordinates are synchronised with it).
//
// The history is kept as U diag(sigma) B (B [r, D] orthonormal rows). Folding a block of dense
// rows Y [n, D] takes the rank-r' SVD of M = [ diag(sigma) B ; Y ]: its right singular vectors
// and values are those of the whole history stacked with the block (incremental SVD). Here M's
// r + n rows are staged as bf16 matrix-core operands and factorised with the weighted-SVD kernels
// (Gram on the matrix cores, block Jacobi; unit weights), so the result is the top-r' right
// singular vectors of exactly those rows:
//
//   lr_bu_stage    rows i < r: bf16(sigma_i * B_i) (float32 product, one rounding);
//                  rows r + j: Y_j (bf16 already); unit weights
//   (sens_svd)     B' (float32) and the spectrum of the staged rows
//   lr_bu_finish   basis_new = B' in the basis dtype, sigma_new = the top r' singular values,
//                  W = B' B^T [r', round_up(r, 8)] in the basis dtype (float32 accumulation over
//                  D; pad columns 0): the coordinate sync z' = z W^T of lowrank_kv_rebase, since
//                  B' has orthonormal rows (pinv(B') = B'^T).
#include <math.h>

#include "device_common.h"
#include "internal.h"

namespace lr {

struct BuArgs {
  const void* basis;     // [r][D], f32 or bf16
  const float* sigma;    // [r]
  const __bf16* rows;    // [n][D]
  __bf16* x;             // staged rows [r + n][D]
  float* w;              // [r + n] unit weights
  const float* bnew32;   // B' [r'][D] float32 (from the SVD)
  const float* sig_all;  // [D] spectrum of the staged rows
  void* basis_new;       // [r'][D], basis dtype
  float* sigma_new;      // [r']
  void* wout;            // [r'][ldw], basis dtype
  int r, n, D, r_new, ldw, f32;
};

__device__ __forceinline__ float basis_at(const BuArgs& a, size_t i) {
  return a.f32 ? ((const float*)a.basis)[i] : (float)((const __bf16*)a.basis)[i];
}

// grid (r + n), 256 threads: one staged row per workgroup
__global__ __launch_bounds__(256) void lr_bu_stage(BuArgs a) {
  const int i = blockIdx.x;
  __bf16* dst = a.x + (size_t)i * a.D;
  if (i < a.r) {
    const float s = a.sigma[i];
    for (int c = threadIdx.x; c < a.D; c += 256) dst[c] = (__bf16)(s * basis_at(a, (size_t)i * a.D + c));
  } else {
    const __bf16* src = a.rows + (size_t)(i - a.r) * a.D;
    for (int c = threadIdx.x; c < a.D; c += 256) dst[c] = src[c];
  }
  if (threadIdx.x == 0) a.w[i] = 1.f;
}

// grid (r', ceil(ldw / 64)), 256 threads. Workgroup (k, cb): wave v forms W[k][c] for the 16
// columns c = 64 cb + 16 v + i: lane l sums B'[k][d] B[c][d] over d = l, l + 64, ... (coalesced
// rows), then the wave adds its lanes' sums (fixed order). Workgroups with cb == 0 also write
// basis row k and sigma_new[k].
__global__ __launch_bounds__(256) void lr_bu_finish(BuArgs a) {
  const int k = blockIdx.x, cb = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, v = tid >> 6;
  const float* bn = a.bnew32 + (size_t)k * a.D;
  float bk[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) bk[u] = (lane + 64 * u < a.D) ? bn[lane + 64 * u] : 0.f;
  for (int i = 0; i < 16; ++i) {
    const int col = cb * 64 + v * 16 + i;
    if (col >= a.ldw) break;                       // wave-uniform
    float acc = 0.f;
    if (col < a.r) {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int d = lane + 64 * u;
        if (d < a.D) acc += bk[u] * basis_at(a, (size_t)col * a.D + d);
      }
    }
    for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
    if (lane == 0) {
      if (a.f32) ((float*)a.wout)[(size_t)k * a.ldw + col] = acc;
      else ((__bf16*)a.wout)[(size_t)k * a.ldw + col] = (__bf16)acc;
    }
  }
  if (cb == 0) {
    for (int c = tid; c < a.D; c += 256) {
      if (a.f32) ((float*)a.basis_new)[(size_t)k * a.D + c] = bn[c];
      else ((__bf16*)a.basis_new)[(size_t)k * a.D + c] = (__bf16)bn[c];
    }
    if (tid == 0) a.sigma_new[k] = a.sig_all[k];
  }
}

static inline size_t bu_align(size_t x) { return (x + 255) & ~(size_t)255; }

hipError_t launch_basis_update(const void* basis, int f32, const float* sigma, int r, const void* rows, int n, int D,
                               int r_new, int sweeps, void* basis_new, float* sigma_new, void* w, void* ws,
                               hipStream_t st) {
  const int m = r + n;
  unsigned char* p = (unsigned char*)ws;
  BuArgs a;
  a.basis = basis;
  a.sigma = sigma;
  a.rows = (const __bf16*)rows;
  a.x = (__bf16*)p;
  p += bu_align((size_t)m * D * 2);
  a.w = (float*)p;
  p += bu_align((size_t)m * 4);
  void* svd_ws = p;
  p += bu_align(svd_workspace_bytes(m, D));
  float* bnew32 = (float*)p;
  p += bu_align((size_t)D * D * 4);
  float* sig_all = (float*)p;
  a.bnew32 = bnew32;
  a.sig_all = sig_all;
  a.basis_new = basis_new;
  a.sigma_new = sigma_new;
  a.wout = w;
  a.r = r;
  a.n = n;
  a.D = D;
  a.r_new = r_new;
  a.ldw = (r + 7) / 8 * 8;
  a.f32 = f32;
  hipLaunchKernelGGL(lr_bu_stage, dim3(m), dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_sens_svd(a.x, a.w, 1, m, D, r_new, sweeps, bnew32, 1, sig_all, svd_ws, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(lr_bu_finish, dim3(r_new, (a.ldw + 63) / 64), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace lr
