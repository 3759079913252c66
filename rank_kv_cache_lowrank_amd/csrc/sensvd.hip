// Sensitivity-weighted SVD basis construction (TraceKV abstract; ai4snews Synopsis and
// Interpretation: each KV state is weighted by its sensitivity before the SVD).
//
// For KV samples x_n [D] (bf16) and sensitivities w_n >= 0 the basis is the top-r right singular
// vectors of diag(sqrt(w)) X, and the spectrum its singular values. With y_n = bf16(sqrt(w_n) x_n)
// (float32 product, one rounding: the matrix-core operand) they are the eigenvectors and the
// square roots of the eigenvalues of G = Y^T Y [D, D]:
//
//   lr_svd_gram     partial Grams: workgroup (64x64 tile of the upper triangle, sample range);
//                   32 samples at a time are weighted, rounded and staged in LDS row-major, and
//                   both 16x16x32 bf16 matrix-core operands (K = samples) come from the gfx950
//                   transpose read; float32 accumulation.
//   lr_svd_reduce   G = sum of the partials in range order (deterministic), mirrored; V = I.
//   lr_jacobi_rows  block Jacobi, one workgroup per pair of 16-index blocks of a round (circle
//   lr_jacobi_cols  ordering, D/16 - 1 rounds per sweep): the pair's 32x32 block of G is
//                   diagonalised in LDS by cyclic scalar Jacobi (rotations as in Golub and Van
//                   Loan's symmetric Schur step), its rotation U [32, 32] then updates the pair's
//                   rows of G (U^T G), and after the launch boundary its columns of G and V
//                   (G U, V U). Pairs of a round touch disjoint rows and columns.
//   lr_svd_finish   eigenvalues from diag(G) sorted descending (bitonic, index breaks ties),
//                   sigma = sqrt(max(lambda, 0)), basis rows = the matching columns of V,
//                   normalised, with the largest-magnitude component made positive.
#include <math.h>

#include "device_common.h"
#include "internal.h"

namespace lr {

typedef __attribute__((__vector_size__(4 * sizeof(short)))) short svd_s16x4;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 svd_bf16x4;

constexpr int kSvdTile = 64;             // Gram tile (64 x 64)
constexpr int kSvdK = 32;                // samples per matrix-core step
constexpr int kSvdStride = 128 * 2 + 32; // LDS row stride (bytes) of the staged [32][128] tile

// 16x16x32 operand with K = staged rows: lane (g, j) gets column c0 + j of rows 8g .. 8g+7.
// Through the transpose read, lane 16g + 4e + q supplies the address of row 8g + e (+4 for the
// second read), columns c0 + 4q .. +3; lane j of the group receives column j of those 4 rows.
__device__ __forceinline__ bf16x8 svd_operand(const unsigned char* tile, int c0, int lane) {
  const int g = lane >> 4, e = (lane >> 2) & 3, q = lane & 3;
  const unsigned char* p = tile + (8 * g + e) * kSvdStride + (c0 + 4 * q) * 2;
  const svd_s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) svd_s16x4*)(p));
  const svd_s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) svd_s16x4*)(p + 4 * kSvdStride));
  bf16x8 r;
  const svd_bf16x4 a = __builtin_bit_cast(svd_bf16x4, lo), b = __builtin_bit_cast(svd_bf16x4, hi);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r[i] = a[i];
    r[4 + i] = b[i];
  }
  return r;
}

struct SvdArgs {
  const __bf16* x;
  const float* w;
  float* part;       // [nsplit][D][D]
  float* G;          // [D][D]
  float* V;          // [D][D]
  float* U;          // [npairs][32][32]
  void* basis;       // [rank][D]
  float* sigma;      // [D]
  int n, D, nsplit, rank, basis_f32, round;
};

__global__ __launch_bounds__(256) void lr_svd_gram(SvdArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char tile[kSvdK * kSvdStride];
  // upper-triangle tile index -> (I, J), I <= J
  const int nbt = a.D / kSvdTile;
  int t = blockIdx.x, I = 0;
  while (t >= nbt - I) {
    t -= nbt - I;
    ++I;
  }
  const int J = I + t;
  const int s = blockIdx.y;
  const int n0 = (int)((long long)a.n * s / a.nsplit), n1 = (int)((long long)a.n * (s + 1) / a.nsplit);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lg = lane >> 4, li = lane & 15;
  const int ci = (wave >> 1) * 32, cj = 64 + (wave & 1) * 32;   // this wave's 32x32 quadrant
  f32x4 acc[2][2];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int v = 0; v < 2; ++v) acc[u][v] = f32x4{0.f, 0.f, 0.f, 0.f};

  // staging: thread -> (row r = tid / 8, 16-byte granule c = tid % 8 of the I block, then J)
  const int sr = tid >> 3, sc = (tid & 7) * 8;
  for (int b0 = n0; b0 < n1; b0 += kSvdK) {
    const int n = b0 + sr;
    u32x4 vi = {0u, 0u, 0u, 0u}, vj = {0u, 0u, 0u, 0u};
    if (n < n1) {
      const float sw = sqrtf(a.w[n]);
      const __bf16* row = a.x + (size_t)n * a.D;
      const bf16x8 xi = *(const bf16x8*)(row + I * kSvdTile + sc);
      const bf16x8 xj = *(const bf16x8*)(row + J * kSvdTile + sc);
      bf16x8 yi, yj;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        yi[e] = (__bf16)(sw * (float)xi[e]);
        yj[e] = (__bf16)(sw * (float)xj[e]);
      }
      vi = __builtin_bit_cast(u32x4, yi);
      vj = __builtin_bit_cast(u32x4, yj);
    }
    __syncthreads();
    *(u32x4*)(tile + sr * kSvdStride + sc * 2) = vi;
    *(u32x4*)(tile + sr * kSvdStride + (64 + sc) * 2) = vj;
    __syncthreads();
    bf16x8 av[2], bv[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      av[u] = svd_operand(tile, ci + 16 * u, lane);
      bv[u] = svd_operand(tile, cj + 16 * u, lane);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int v = 0; v < 2; ++v) acc[u][v] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[u], bv[v], acc[u][v], 0, 0, 0);
  }
  // C[row 4lg + i][col li] of block (u, v)
  float* out = a.part + (size_t)s * a.D * a.D;
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int v = 0; v < 2; ++v)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int gi = I * kSvdTile + ci + 16 * u + 4 * lg + i;
        const int gj = J * kSvdTile + (cj - 64) + 16 * v + li;
        out[(size_t)gi * a.D + gj] = acc[u][v][i];
      }
}

__global__ __launch_bounds__(256) void lr_svd_reduce(SvdArgs a) {
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long long)a.D * a.D) return;
  const int i = (int)(idx / a.D), j = (int)(idx - (long long)i * a.D);
  const bool upper = (i / kSvdTile) <= (j / kSvdTile);
  const size_t src = upper ? (size_t)i * a.D + j : (size_t)j * a.D + i;
  float g = 0.f;
  for (int s = 0; s < a.nsplit; ++s) g += a.part[(size_t)s * a.D * a.D + src];
  a.G[idx] = g;
  a.V[idx] = (i == j) ? 1.f : 0.f;
}

// circle-method pairing: round r of n (even) players, pair k -> (lo, hi) player indices
__device__ __forceinline__ void circle_pair(int n, int r, int k, int& p, int& q) {
  const int m = n - 1;
  if (k == 0) {
    p = r % m;
    q = m;
  } else {
    p = (r + k) % m;
    q = (r + m - k) % m;
  }
}

constexpr int kJb = 16;                   // Jacobi block size
constexpr int kJs = 2 * kJb;              // pair subproblem size (32)
constexpr int kJacobiInner = 3;           // cyclic sweeps over a pair's 32x32 block

__device__ __forceinline__ void jacobi_rotation(float app, float aqq, float apq, float& c, float& s) {
  // Golub and Van Loan, symmetric Schur step: J = [[c, s], [-s, c]] on (p, q) zeroes J^T A J (p, q)
  if (apq == 0.f || fabsf(apq) <= 1e-30f) {
    c = 1.f;
    s = 0.f;
    return;
  }
  const float tau = (aqq - app) / (2.f * apq);
  const float t = (tau >= 0.f ? 1.f : -1.f) / (fabsf(tau) + sqrtf(1.f + tau * tau));
  c = 1.f / sqrtf(1.f + t * t);
  s = t * c;
}

__global__ __launch_bounds__(256) void lr_jacobi_rows(SvdArgs a) {
  extern __shared__ float jsm[];
  float* S = jsm;                         // [32][33]
  float* Ul = S + kJs * (kJs + 1);        // [32][33]
  float* cs = Ul + kJs * (kJs + 1);       // [16][2]
  float* rows = cs + 2 * kJb;             // [32][D]
  const int tid = threadIdx.x;
  const int nb = a.D / kJb;
  int pb, qb;
  circle_pair(nb, a.round, blockIdx.x, pb, qb);
  auto gidx = [&](int l) { return l < kJb ? pb * kJb + l : qb * kJb + (l - kJb); };
  for (int e = tid; e < kJs * kJs; e += 256) {
    const int r = e / kJs, c = e - r * kJs;
    S[r * (kJs + 1) + c] = a.G[(size_t)gidx(r) * a.D + gidx(c)];
    Ul[r * (kJs + 1) + c] = (r == c) ? 1.f : 0.f;
  }
  __syncthreads();
  for (int sw = 0; sw < kJacobiInner; ++sw) {
    for (int rr = 0; rr < kJs - 1; ++rr) {
      if (tid < kJb) {
        int p, q;
        circle_pair(kJs, rr, tid, p, q);
        float c, s;
        jacobi_rotation(S[p * (kJs + 1) + p], S[q * (kJs + 1) + q], S[p * (kJs + 1) + q], c, s);
        cs[2 * tid] = c;
        cs[2 * tid + 1] = s;
      }
      __syncthreads();
      for (int e = tid; e < kJb * kJs; e += 256) {      // rows p, q of S
        const int k = e / kJs, col = e - k * kJs;
        int p, q;
        circle_pair(kJs, rr, k, p, q);
        const float c = cs[2 * k], s = cs[2 * k + 1];
        const float rp = S[p * (kJs + 1) + col], rq = S[q * (kJs + 1) + col];
        S[p * (kJs + 1) + col] = c * rp - s * rq;
        S[q * (kJs + 1) + col] = s * rp + c * rq;
      }
      __syncthreads();
      for (int e = tid; e < kJb * kJs; e += 256) {      // columns p, q of S and of Ul
        const int k = e / kJs, row = e - k * kJs;
        int p, q;
        circle_pair(kJs, rr, k, p, q);
        const float c = cs[2 * k], s = cs[2 * k + 1];
        const float sp = S[row * (kJs + 1) + p], sq = S[row * (kJs + 1) + q];
        S[row * (kJs + 1) + p] = c * sp - s * sq;
        S[row * (kJs + 1) + q] = s * sp + c * sq;
        const float up = Ul[row * (kJs + 1) + p], uq = Ul[row * (kJs + 1) + q];
        Ul[row * (kJs + 1) + p] = c * up - s * uq;
        Ul[row * (kJs + 1) + q] = s * up + c * uq;
      }
      __syncthreads();
    }
  }
  float* Ug = a.U + (size_t)blockIdx.x * kJs * kJs;
  for (int e = tid; e < kJs * kJs; e += 256) Ug[e] = Ul[(e / kJs) * (kJs + 1) + (e % kJs)];
  // rows of G: new row a = sum_b U[b][a] * old row b
  for (int e = tid; e < kJs * a.D; e += 256) {
    const int r = e / a.D, c = e - r * a.D;
    rows[e] = a.G[(size_t)gidx(r) * a.D + c];
  }
  __syncthreads();
  for (int e = tid; e < kJs * a.D; e += 256) {
    const int r = e / a.D, c = e - r * a.D;
    float v = 0.f;
    for (int b = 0; b < kJs; ++b) v = fmaf(Ul[b * (kJs + 1) + r], rows[b * a.D + c], v);
    a.G[(size_t)gidx(r) * a.D + c] = v;
  }
}

__global__ __launch_bounds__(256) void lr_jacobi_cols(SvdArgs a) {
  extern __shared__ float jsm[];
  float* Ul = jsm;                        // [32][33]
  float* cols = Ul + kJs * (kJs + 1);     // [D][33]
  const int tid = threadIdx.x;
  const int nb = a.D / kJb;
  int pb, qb;
  circle_pair(nb, a.round, blockIdx.x, pb, qb);
  auto gidx = [&](int l) { return l < kJb ? pb * kJb + l : qb * kJb + (l - kJb); };
  const float* Ug = a.U + (size_t)blockIdx.x * kJs * kJs;
  for (int e = tid; e < kJs * kJs; e += 256) Ul[(e / kJs) * (kJs + 1) + (e % kJs)] = Ug[e];
  for (int m = 0; m < 2; ++m) {
    float* M = m == 0 ? a.G : a.V;
    __syncthreads();
    for (int e = tid; e < a.D * kJs; e += 256) {
      const int r = e / kJs, l = e - r * kJs;
      cols[r * (kJs + 1) + l] = M[(size_t)r * a.D + gidx(l)];
    }
    __syncthreads();
    for (int e = tid; e < a.D * kJs; e += 256) {
      const int r = e / kJs, l = e - r * kJs;
      float v = 0.f;
      for (int b = 0; b < kJs; ++b) v = fmaf(cols[r * (kJs + 1) + b], Ul[b * (kJs + 1) + l], v);
      M[(size_t)r * a.D + gidx(l)] = v;
    }
  }
}

__global__ __launch_bounds__(512) void lr_svd_finish(SvdArgs a) {
  __shared__ float key[512];
  __shared__ int idx[512];
  const int tid = threadIdx.x;
  int P = 1;
  while (P < a.D) P <<= 1;
  for (int i = tid; i < P; i += 512) {
    key[i] = i < a.D ? a.G[(size_t)i * a.D + i] : -INFINITY;
    idx[i] = i;
  }
  __syncthreads();
  // bitonic sort, descending by eigenvalue, ascending index on ties
  for (int k = 2; k <= P; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < P; i += 512) {
        const int l = i ^ j;
        if (l > i) {
          const bool desc = (i & k) == 0;
          const float ki = key[i], kl = key[l];
          const int ii = idx[i], il = idx[l];
          const bool i_first = ki > kl || (ki == kl && ii < il);   // i belongs before l
          if (desc ? !i_first : i_first) {
            key[i] = kl;
            key[l] = ki;
            idx[i] = il;
            idx[l] = ii;
          }
        }
      }
      __syncthreads();
    }
  }
  for (int i = tid; i < a.D; i += 512) a.sigma[i] = sqrtf(fmaxf(key[i], 0.f));
  for (int k = tid; k < a.rank; k += 512) {
    const int col = idx[k];
    int best = 0;
    float bv = -1.f;
    double nrm = 0.0;
    for (int c = 0; c < a.D; ++c) {
      const float x = a.V[(size_t)c * a.D + col];
      const float v = fabsf(x);
      nrm += (double)x * (double)x;
      if (v > bv) {
        bv = v;
        best = c;
      }
    }
    // the rotations keep the columns orthogonal to float32 precision but let their norms drift
    // (a few 1e-4 after many sweeps): each basis row is normalised here
    const float sg = (a.V[(size_t)best * a.D + col] < 0.f ? -1.f : 1.f) / (float)sqrt(nrm > 0.0 ? nrm : 1.0);
    for (int c = 0; c < a.D; ++c) {
      const float v = sg * a.V[(size_t)c * a.D + col];
      if (a.basis_f32) ((float*)a.basis)[(size_t)k * a.D + c] = v;
      else ((__bf16*)a.basis)[(size_t)k * a.D + c] = (__bf16)v;
    }
  }
}

int svd_nsplit(int n) {
  int s = (n + 255) / 256;
  return s < 1 ? 1 : (s > 64 ? 64 : s);
}

size_t svd_workspace_bytes(int n, int D) {
  const size_t dd = (size_t)D * D * 4;
  return (size_t)svd_nsplit(n) * dd + 2 * dd + (size_t)(D / kJs) * kJs * kJs * 4 + 1024;
}

hipError_t launch_sens_svd(const void* x, const float* w, int n, int D, int rank, int sweeps, void* basis,
                           int basis_f32, float* sigma, void* ws, hipStream_t st) {
  SvdArgs a;
  a.x = (const __bf16*)x;
  a.w = w;
  a.D = D;
  a.n = n;
  a.nsplit = svd_nsplit(n);
  a.rank = rank;
  a.basis = basis;
  a.basis_f32 = basis_f32;
  a.sigma = sigma;
  unsigned char* p = (unsigned char*)ws;
  const size_t dd = (size_t)D * D * 4;
  a.part = (float*)p;
  a.G = (float*)(p + (size_t)a.nsplit * dd);
  a.V = (float*)(p + (size_t)a.nsplit * dd + dd);
  a.U = (float*)(p + (size_t)a.nsplit * dd + 2 * dd);
  a.round = 0;
  const int nbt = D / kSvdTile;
  hipLaunchKernelGGL(lr_svd_gram, dim3(nbt * (nbt + 1) / 2, a.nsplit), dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(lr_svd_reduce, dim3((unsigned)(((long long)D * D + 255) / 256)), dim3(256), 0, st, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nb = D / kJb, npairs = nb / 2;
  const size_t lds_rows = (size_t)(2 * kJs * (kJs + 1) + 2 * kJb + kJs * D) * 4;
  const size_t lds_cols = (size_t)(kJs * (kJs + 1) + D * (kJs + 1)) * 4;
  static bool attr[64] = {};
  int dev = 0;
  e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < 64 && !attr[dev]) {
    e = hipFuncSetAttribute((const void*)lr_jacobi_rows, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute((const void*)lr_jacobi_cols, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
    if (e != hipSuccess) return e;
    attr[dev] = true;
  }
  for (int sw = 0; sw < sweeps; ++sw) {
    for (int r = 0; r < nb - 1; ++r) {
      a.round = r;
      hipLaunchKernelGGL(lr_jacobi_rows, dim3(npairs), dim3(256), lds_rows, st, a);
      hipLaunchKernelGGL(lr_jacobi_cols, dim3(npairs), dim3(256), lds_cols, st, a);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(lr_svd_finish, dim3(1), dim3(512), 0, st, a);
  return hipGetLastError();
}

}  // namespace lr
