// Sensitivity-weighted SVD basis construction (TraceKV abstract; ai4snews Synopsis and
// Interpretation: each KV state is weighted by its sensitivity before the SVD).
//
// (A batch of matrices of one shape runs as one: every kernel takes the matrix index from a spare
// grid dimension and its pointers from svd_at.)
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
//   lr_svd_reduce   G = sum of the partials in range order (deterministic), per upper tile,
//                   mirrored through LDS, and a copy G0 of it; V = I.
//   lr_jacobi_pair  block Jacobi over 16-index blocks, circle ordering (D/16 - 1 rounds per
//   lr_jacobi_apply sweep): one workgroup per block pair reduces the pair's 32x32 block of G in
//                   LDS by one cyclic sweep of scalar Jacobi (rotations as in Golub and Van
//                   Loan's symmetric Schur step), accumulating U [32, 32]; then one launch
//                   applies all pairs' U: G <- Q^T G Q block by block (U_i^T G_ij U_j) and
//                   V <- V Q. Pairs of a round touch disjoint rows and columns.
//   lr_svd_rayleigh eigenvalues as Rayleigh quotients of the columns of V on the unrotated G
//                   (the sweeps' accumulated rounding in diag(G) stays out of them: the
//                   quotient's error is second order in the eigenvector's).
//   lr_svd_sort     eigenvalues sorted descending (bitonic, index breaks ties),
//                   sigma = sqrt(max(lambda, 0)).
//   lr_svd_basis    basis rows = the matching columns of V, normalised, with the
//                   largest-magnitude component made positive.
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
  float* G;          // [D][D], rotated in place by the Jacobi sweeps
  float* G0;         // [D][D], the Gram as reduced (kept for the Rayleigh quotients)
  float* V;          // [D][D]
  double* rq;        // [D / 64 + 1][D]: partial quadratic forms of the columns of V, then their norms
  int* ord;          // [D]: column of V of each basis row
  float* U;          // [npairs][32][32]
  void* basis;       // [rank][D]
  float* sigma;      // [D]
  int n, D, nsplit, rank, basis_f32, round;
  size_t ws_stride;  // workspace bytes per matrix of a batch
};

// The arguments of matrix m of a batch: inputs [m][n][D] and [m][n], outputs [m][rank][D] and
// [m][D], and the m-th workspace slice.
__device__ __forceinline__ SvdArgs svd_at(SvdArgs a, int m) {
  const size_t nd = (size_t)a.n * a.D;
  a.x += (size_t)m * nd;
  a.w += (size_t)m * a.n;
  const size_t wo = (size_t)m * a.ws_stride;
  a.part = (float*)((unsigned char*)a.part + wo);
  a.G = (float*)((unsigned char*)a.G + wo);
  a.G0 = (float*)((unsigned char*)a.G0 + wo);
  a.V = (float*)((unsigned char*)a.V + wo);
  a.U = (float*)((unsigned char*)a.U + wo);
  a.rq = (double*)((unsigned char*)a.rq + wo);
  a.ord = (int*)((unsigned char*)a.ord + wo);
  const size_t bo = (size_t)m * a.rank * a.D * (a.basis_f32 ? 4 : 2);
  a.basis = (void*)((unsigned char*)a.basis + bo);
  a.sigma += (size_t)m * a.D;
  return a;
}

__global__ __launch_bounds__(256) void lr_svd_gram(SvdArgs a) {
  a = svd_at(a, blockIdx.z);
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

// One workgroup per 64x64 tile (I, J), I <= J, of the upper triangle (the tiles the partial
// Grams hold): each entry is the sum of the partials in range order (coalesced rows, eight
// loads issued ahead of their additions), written to G and G0 at (I, J) and, through LDS, at
// the mirrored tile (J, I); V = I.
__global__ __launch_bounds__(256) void lr_svd_reduce(SvdArgs a) {
  a = svd_at(a, blockIdx.y);
  __shared__ float T[kSvdTile][kSvdTile + 1];
  const int nbt = a.D / kSvdTile;
  int t = blockIdx.x, I = 0;
  while (t >= nbt - I) {
    t -= nbt - I;
    ++I;
  }
  const int J = I + t;
  const size_t dd = (size_t)a.D * a.D;
  for (int e = threadIdx.x; e < kSvdTile * kSvdTile; e += 256) {
    const int r = e / kSvdTile, c = e - r * kSvdTile;
    const size_t src = (size_t)(I * kSvdTile + r) * a.D + J * kSvdTile + c;
    float g = 0.f;
    int s = 0;
    for (; s + 8 <= a.nsplit; s += 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = a.part[(size_t)(s + u) * dd + src];
#pragma unroll
      for (int u = 0; u < 8; ++u) g += v[u];
    }
    for (; s < a.nsplit; ++s) g += a.part[(size_t)s * dd + src];
    a.G[src] = g;
    a.G0[src] = g;
    a.V[src] = (I == J && r == c) ? 1.f : 0.f;
    T[r][c] = g;
  }
  if (I == J) return;                            // a diagonal tile holds both triangles
  __syncthreads();
  for (int e = threadIdx.x; e < kSvdTile * kSvdTile; e += 256) {
    const int r = e / kSvdTile, c = e - r * kSvdTile;
    const size_t dst = (size_t)(J * kSvdTile + r) * a.D + I * kSvdTile + c;
    a.G[dst] = T[c][r];
    a.G0[dst] = T[c][r];
    a.V[dst] = 0.f;
  }
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

constexpr int kJacobiInner = 1;           // cyclic sweeps over a pair's 32x32 block per round

// One workgroup per block pair: the pair's 32x32 block S of G is diagonalised in LDS by cyclic
// scalar Jacobi (circle ordering of the 32 indices: 16 disjoint rotations per step). Thread
// (a, b) of 16 x 16 owns, in one step, the 2x2 block of S at rows (p_a, q_a) and columns
// (p_b, q_b) of the step's rotation pairs a and b: S' = J_a^T S J_b there, with both rotations
// formed by the thread itself from the diagonal of S (every thread forming rotation a reads the
// same three entries and runs the same instructions, so all get the same one). The same thread
// rotates U's columns (p_b, q_b) in rows (p_a, q_a): U' = U J. The blocks of a step partition S
// and U, so each step is one pass from one half of a double buffer into the other. Rotations use
// the hardware square root and reciprocal: the angles need not be correctly rounded, only
// orthogonal to float precision (the basis rows are normalised at the end and the eigenvalues
// are Rayleigh quotients). The accumulated U goes to the workspace.
// Golub and Van Loan's symmetric Schur step: J = [[c, s], [-s, c]] on (p, q) zeroes (J^T A J)[p][q].
__device__ __forceinline__ void jacobi_rotation_fast(float app, float aqq, float apq, float& c, float& s) {
  // branch-free: a negligible apq gives the identity by selection (with apq replaced by 1 the
  // arithmetic stays finite), so the caller's loads need not wait on a branch
  const bool skip = fabsf(apq) <= 1e-30f;
  const float tau = (aqq - app) * __builtin_amdgcn_rcpf(2.f * (skip ? 1.f : apq));
  const float t = (tau >= 0.f ? 1.f : -1.f) * __builtin_amdgcn_rcpf(fabsf(tau) + __builtin_amdgcn_sqrtf(fmaf(tau, tau, 1.f)));
  const float cc = __builtin_amdgcn_rsqf(fmaf(t, t, 1.f));
  c = skip ? 1.f : cc;
  s = skip ? 0.f : t * cc;
}

__global__ __launch_bounds__(256) void lr_jacobi_pair(SvdArgs a) {
  a = svd_at(a, blockIdx.y);
  // row stride 48: in the circle ordering p + q is the same for every pair of a step, so with a
  // stride of 33 the pairs' (p, q) entries would all fall in one bank; 48 spreads them and the
  // two rows of a half-wave's blocks over different banks
  constexpr int LD = 48;
  __shared__ float S[2][kJs * LD];
  __shared__ float Ul[2][kJs * LD];
  const int tid = threadIdx.x;
  const int nb = a.D / kJb;
  int pb, qb;
  circle_pair(nb, a.round, blockIdx.x, pb, qb);
  auto gidx = [&](int l) { return l < kJb ? pb * kJb + l : qb * kJb + (l - kJb); };
  for (int e = tid; e < kJs * kJs; e += 256) {
    const int r = e / kJs, c = e - r * kJs;
    S[0][r * LD + c] = a.G[(size_t)gidx(r) * a.D + gidx(c)];
    Ul[0][r * LD + c] = (r == c) ? 1.f : 0.f;
  }
  __syncthreads();
  const int ta = tid >> 4, tb = tid & 15;
  int p0, q0, p1, q1;
  circle_pair(kJs, 0, ta, p0, q0);
  circle_pair(kJs, 0, tb, p1, q1);
  int cur = 0;
  for (int sw = 0; sw < kJacobiInner; ++sw) {
    for (int rr = 0; rr < kJs - 1; ++rr) {
      const float* Sc = S[cur];
      const float* Uc = Ul[cur];
      float* Sn = S[cur ^ 1];
      float* Un = Ul[cur ^ 1];
      // all loads of the step first: the two rotations' inputs, the S and U blocks
      const float a_pp = Sc[p0 * LD + p0], a_qq = Sc[q0 * LD + q0], a_pq = Sc[p0 * LD + q0];
      const float b_pp = Sc[p1 * LD + p1], b_qq = Sc[q1 * LD + q1], b_pq = Sc[p1 * LD + q1];
      const float xpp = Sc[p0 * LD + p1], xpq = Sc[p0 * LD + q1];
      const float xqp = Sc[q0 * LD + p1], xqq = Sc[q0 * LD + q1];
      const float upp = Uc[p0 * LD + p1], upq = Uc[p0 * LD + q1];
      const float uqp = Uc[q0 * LD + p1], uqq = Uc[q0 * LD + q1];
      float c0, s0, c1, s1;
      jacobi_rotation_fast(a_pp, a_qq, a_pq, c0, s0);
      jacobi_rotation_fast(b_pp, b_qq, b_pq, c1, s1);
      // J restricted to a pair (p, q): J[p][p] = c, J[p][q] = s, J[q][p] = -s, J[q][q] = c
      // T = S_blk J_b
      const float tpp = xpp * c1 - xpq * s1, tpq = xpp * s1 + xpq * c1;
      const float tqp = xqp * c1 - xqq * s1, tqq = xqp * s1 + xqq * c1;
      // S' = J_a^T T
      Sn[p0 * LD + p1] = c0 * tpp - s0 * tqp;
      Sn[p0 * LD + q1] = c0 * tpq - s0 * tqq;
      Sn[q0 * LD + p1] = s0 * tpp + c0 * tqp;
      Sn[q0 * LD + q1] = s0 * tpq + c0 * tqq;
      Un[p0 * LD + p1] = upp * c1 - upq * s1;
      Un[p0 * LD + q1] = upp * s1 + upq * c1;
      Un[q0 * LD + p1] = uqp * c1 - uqq * s1;
      Un[q0 * LD + q1] = uqp * s1 + uqq * c1;
      __syncthreads();
      cur ^= 1;
      // next step of the circle ordering: every index except the fixed 31 advances by one mod 31
      p0 = p0 == kJs - 2 ? 0 : p0 + 1;
      p1 = p1 == kJs - 2 ? 0 : p1 + 1;
      q0 = q0 == kJs - 1 ? q0 : (q0 == kJs - 2 ? 0 : q0 + 1);
      q1 = q1 == kJs - 1 ? q1 : (q1 == kJs - 2 ? 0 : q1 + 1);
    }
  }
  float* Ug = a.U + (size_t)blockIdx.x * kJs * kJs;
  for (int e = tid; e < kJs * kJs; e += 256) Ug[e] = Ul[cur][(e / kJs) * LD + (e % kJs)];
}

// One round's update G <- Q^T G Q, V <- V Q, with Q the block-diagonal (in permuted order) of the
// pairs' U. Output block (pair i rows, pair j columns) of G is U_i^T G_ij U_j: it depends on its
// own input block only, so each workgroup updates its block in place. Workgroups 0 .. np(np+1)/2
// - 1 take the G blocks with i <= j and write the result and its transpose (G stays exactly
// symmetric); the rest take 32-row blocks of V times U_j. Thread (r, c4): row r, columns
// c4 .. c4+3 (inside one 16-index block, so the global accesses are 16-byte vectors).
__global__ __launch_bounds__(256) void lr_jacobi_apply(SvdArgs a) {
  a = svd_at(a, blockIdx.y);
  constexpr int LD = kJs + 1;
  __shared__ float B[kJs * LD];
  __shared__ float Ui[kJs * LD];
  __shared__ float Uj[kJs * LD];
  __shared__ float T[kJs * LD];
  const int tid = threadIdx.x;
  const int nb = a.D / kJb, np = nb / 2;
  const int ng = np * (np + 1) / 2;
  const int r = tid >> 3, c4 = (tid & 7) * 4;
  int i = 0, j = 0, rb = 0;
  const bool gblk = (int)blockIdx.x < ng;
  if (gblk) {
    int rem = blockIdx.x;
    while (rem >= np - i) {
      rem -= np - i;
      ++i;
    }
    j = i + rem;
  } else {
    const int v = blockIdx.x - ng;
    j = v % np;
    rb = v / np;
  }
  int pi, qi, pj, qj;
  circle_pair(nb, a.round, i, pi, qi);
  circle_pair(nb, a.round, j, pj, qj);
  auto gi = [&](int l) { return l < kJb ? pi * kJb + l : qi * kJb + (l - kJb); };
  auto gj = [&](int l) { return l < kJb ? pj * kJb + l : qj * kJb + (l - kJb); };
  const f32x4 uj = *(const f32x4*)(a.U + (size_t)j * kJs * kJs + r * kJs + c4);
  float* src = gblk ? a.G + (size_t)gi(r) * a.D + gj(c4) : a.V + (size_t)(rb * kJs + r) * a.D + gj(c4);
  const f32x4 bv = *(const f32x4*)src;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    B[r * LD + c4 + k] = bv[k];
    Uj[r * LD + c4 + k] = uj[k];
  }
  if (gblk) {
    const f32x4 ui = *(const f32x4*)(a.U + (size_t)i * kJs * kJs + r * kJs + c4);
#pragma unroll
    for (int k = 0; k < 4; ++k) Ui[r * LD + c4 + k] = ui[k];
  }
  __syncthreads();
  float t[4] = {0.f, 0.f, 0.f, 0.f};
  for (int l = 0; l < kJs; ++l) {
    const float bl = B[r * LD + l];
#pragma unroll
    for (int k = 0; k < 4; ++k) t[k] = fmaf(bl, Uj[l * LD + c4 + k], t[k]);
  }
  if (!gblk) {
    *(f32x4*)src = f32x4{t[0], t[1], t[2], t[3]};
    return;
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) T[r * LD + c4 + k] = t[k];
  __syncthreads();
  float o[4] = {0.f, 0.f, 0.f, 0.f};
  for (int l = 0; l < kJs; ++l) {
    const float u = Ui[l * LD + r];
#pragma unroll
    for (int k = 0; k < 4; ++k) o[k] = fmaf(u, T[l * LD + c4 + k], o[k]);
  }
  *(f32x4*)src = f32x4{o[0], o[1], o[2], o[3]};
  if (i == j) return;
  // the transpose block (pair j rows, pair i columns), staged through LDS
#pragma unroll
  for (int k = 0; k < 4; ++k) B[(c4 + k) * LD + r] = o[k];
  __syncthreads();
  *(f32x4*)(a.G + (size_t)gj(r) * a.D + gi(c4)) =
      f32x4{B[r * LD + c4], B[r * LD + c4 + 1], B[r * LD + c4 + 2], B[r * LD + c4 + 3]};
}

constexpr int kRqCols = 16;   // columns of V per workgroup in lr_svd_rayleigh

// lambda_k = v_k^T G0 v_k / v_k^T v_k for the columns v_k of V, as D / 64 partial quadratic
// forms: workgroup (column group k0 .. k0+15, row range j0 .. j0+63) sums
// v_k[i] G0[j][i] v_k[j] over all i and its j (G0 is exactly symmetric, so thread t reads row j
// at columns t and t + 256, coalesced) into rq[j0 / 64][k] (float64); range 0 also writes
// v_k^T v_k. lr_svd_sort adds the partials in range order.
__global__ __launch_bounds__(256) void lr_svd_rayleigh(SvdArgs a) {
  a = svd_at(a, blockIdx.z);
  __shared__ __attribute__((aligned(16))) float Vs[512 * kRqCols];
  __shared__ double red[4][2 * kRqCols];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int k0 = blockIdx.x * kRqCols, j0 = blockIdx.y * kRqRows;
  for (int e = tid; e < a.D * kRqCols; e += 256) {
    const int r = e / kRqCols, c = e - r * kRqCols;
    Vs[e] = a.V[(size_t)r * a.D + k0 + c];
  }
  __syncthreads();
  const int i0 = tid, i1 = tid + 256;
  const bool h0 = i0 < a.D, h1 = i1 < a.D;
  float t0[kRqCols], t1[kRqCols];
#pragma unroll
  for (int c = 0; c < kRqCols; ++c) t0[c] = t1[c] = 0.f;
  for (int jj = 0; jj < kRqRows; jj += 8) {
    float g0[8], g1[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      g0[u] = h0 ? a.G0[(size_t)(j0 + jj + u) * a.D + i0] : 0.f;
      g1[u] = h1 ? a.G0[(size_t)(j0 + jj + u) * a.D + i1] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
#pragma unroll
      for (int c4 = 0; c4 < kRqCols / 4; ++c4) {
        const f32x4 v = *(const f32x4*)(Vs + (j0 + jj + u) * kRqCols + 4 * c4);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          t0[4 * c4 + q] = fmaf(g0[u], v[q], t0[4 * c4 + q]);
          t1[4 * c4 + q] = fmaf(g1[u], v[q], t1[4 * c4 + q]);
        }
      }
    }
  }
#pragma unroll
  for (int c = 0; c < kRqCols; ++c) {
    const double v0 = h0 ? Vs[i0 * kRqCols + c] : 0.f, v1 = h1 ? Vs[i1 * kRqCols + c] : 0.f;
    double num = v0 * (double)t0[c] + v1 * (double)t1[c];
    double den = v0 * v0 + v1 * v1;
    for (int o = 32; o > 0; o >>= 1) {
      num += __shfl_down(num, o);
      den += __shfl_down(den, o);
    }
    if (lane == 0) {
      red[wv][2 * c] = num;
      red[wv][2 * c + 1] = den;
    }
  }
  __syncthreads();
  if (tid < kRqCols) {
    double num = 0.0, den = 0.0;
    for (int w = 0; w < 4; ++w) {
      num += red[w][2 * tid];
      den += red[w][2 * tid + 1];
    }
    a.rq[(size_t)blockIdx.y * a.D + k0 + tid] = num;
    if (blockIdx.y == 0) a.rq[(size_t)(a.D / kRqRows) * a.D + k0 + tid] = den;
  }
}

// eigenvalues (the Rayleigh quotients) sorted descending by a bitonic network in LDS, equal
// values ordered by column index; sigma = sqrt(max(lambda, 0)); the first rank column indices
// go to ord.
__global__ __launch_bounds__(512) void lr_svd_sort(SvdArgs a) {
  a = svd_at(a, blockIdx.x);
  __shared__ float key[512];
  __shared__ int idx[512];
  const int tid = threadIdx.x;
  int P = 1;
  while (P < a.D) P <<= 1;
  const int nr = a.D / kRqRows;
  for (int i = tid; i < P; i += 512) {
    float k = -INFINITY;
    if (i < a.D) {
      double num = 0.0;
      for (int y = 0; y < nr; ++y) num += a.rq[(size_t)y * a.D + i];
      const double den = a.rq[(size_t)nr * a.D + i];
      k = den > 0.0 ? (float)(num / den) : 0.f;
    }
    key[i] = k;
    idx[i] = i;
  }
  __syncthreads();
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
  for (int k = tid; k < a.rank; k += 512) a.ord[k] = idx[k];
}

// basis row k (one workgroup each) = column ord[k] of V, normalised (the rotations keep the
// columns orthogonal to float precision but let their norms drift by a few 1e-4 over the
// sweeps), its largest-magnitude component (lowest index among equal magnitudes) made positive.
__global__ __launch_bounds__(256) void lr_svd_basis(SvdArgs a) {
  a = svd_at(a, blockIdx.y);
  __shared__ double rn[4];
  __shared__ float rv[4];
  __shared__ int ri[4];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int k = blockIdx.x, col = a.ord[k];
  const int c0 = tid, c1 = tid + 256;
  const float x0 = c0 < a.D ? a.V[(size_t)c0 * a.D + col] : 0.f;
  const float x1 = c1 < a.D ? a.V[(size_t)c1 * a.D + col] : 0.f;
  double nrm = (double)x0 * x0 + (double)x1 * x1;
  float bv = fabsf(x0);
  int bi = c0;
  if (c1 < a.D && fabsf(x1) > bv) {
    bv = fabsf(x1);
    bi = c1;
  }
  for (int o = 32; o > 0; o >>= 1) {
    nrm += __shfl_down(nrm, o);
    const float ov = __shfl_down(bv, o);
    const int oi = __shfl_down(bi, o);
    if (ov > bv || (ov == bv && oi < bi)) {
      bv = ov;
      bi = oi;
    }
  }
  if (lane == 0) {
    rn[wv] = nrm;
    rv[wv] = bv;
    ri[wv] = bi;
  }
  __syncthreads();
  double n = 0.0;
  float v = -1.f;
  int best = 0;
  for (int w = 0; w < 4; ++w) {
    n += rn[w];
    if (rv[w] > v || (rv[w] == v && ri[w] < best)) {
      v = rv[w];
      best = ri[w];
    }
  }
  const float sg = (a.V[(size_t)best * a.D + col] < 0.f ? -1.f : 1.f) / (float)sqrt(n > 0.0 ? n : 1.0);
  if (a.basis_f32) {
    float* row = (float*)a.basis + (size_t)k * a.D;
    if (c0 < a.D) row[c0] = sg * x0;
    if (c1 < a.D) row[c1] = sg * x1;
  } else {
    __bf16* row = (__bf16*)a.basis + (size_t)k * a.D;
    if (c0 < a.D) row[c0] = (__bf16)(sg * x0);
    if (c1 < a.D) row[c1] = (__bf16)(sg * x1);
  }
}

hipError_t launch_sens_svd(const void* x, const float* w, int n_mat, int n, int D, int rank, int sweeps, void* basis,
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
  a.ws_stride = svd_workspace_stride(n, D);
  unsigned char* p = (unsigned char*)ws;
  const size_t dd = (size_t)D * D * 4;
  a.part = (float*)p;
  a.G = (float*)(p + (size_t)a.nsplit * dd);
  a.G0 = (float*)(p + (size_t)a.nsplit * dd + dd);
  a.V = (float*)(p + (size_t)a.nsplit * dd + 2 * dd);
  a.U = (float*)(p + (size_t)a.nsplit * dd + 3 * dd);
  a.rq = (double*)(a.U + (size_t)(D / kJs) * kJs * kJs);
  a.ord = (int*)(a.rq + (size_t)(D / kRqRows + 1) * D);
  a.round = 0;
  const int nbt = D / kSvdTile;
  const unsigned M = (unsigned)n_mat;
  hipLaunchKernelGGL(lr_svd_gram, dim3(nbt * (nbt + 1) / 2, a.nsplit, M), dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(lr_svd_reduce, dim3(nbt * (nbt + 1) / 2, M), dim3(256), 0, st, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nb = D / kJb, npairs = nb / 2;
  for (int sw = 0; sw < sweeps; ++sw) {
    for (int r = 0; r < nb - 1; ++r) {
      a.round = r;
      hipLaunchKernelGGL(lr_jacobi_pair, dim3(npairs, M), dim3(256), 0, st, a);
      hipLaunchKernelGGL(lr_jacobi_apply, dim3(npairs * (npairs + 1) / 2 + npairs * (D / kJs), M), dim3(256), 0, st,
                         a);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(lr_svd_rayleigh, dim3(D / kRqCols, D / kRqRows, M), dim3(256), 0, st, a);
  hipLaunchKernelGGL(lr_svd_sort, dim3(M), dim3(512), 0, st, a);
  if (rank > 0) hipLaunchKernelGGL(lr_svd_basis, dim3(rank, M), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace lr
