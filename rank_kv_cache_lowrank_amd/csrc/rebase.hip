// Historical-coordinate sync after a basis update.
//
// iS-KV ("iS-KV: Online Low-Rank KV Cache Compression via Block-Incremental SVD", English
// abstract; method summary): as the low-rank basis evolves during decoding, the coordinates of
// the stored history are synchronised with it, or the history drifts. Every stored latent row z
// becomes its least-squares coordinates in the new basis,
//     z' = z B pinv(B') = z W^T,     W [r_new][r_old] computed by the caller,
// stored in the cache dtype (bf16: round to nearest even, as the append path stores z).
//
// bf16 kernel: W (one chunk of its rows, i.e. of the new coordinates) is staged once per
// workgroup of 8 waves in LDS with padded rows; each wave then takes 32-row groups of one
// sequence, holds
// their two 16-row tiles in registers and runs 16x16x32 bf16 matrix-core products with
// A = 16 rows of W (new coordinates) and B = the tile's rows transposed (tokens), so a lane's
// accumulator holds 4 consecutive new coordinates of one token (8-byte stores). Every W read
// from LDS feeds both tiles. HBM traffic per token: the old row read once per chunk and the new
// row written once.
#include "device_common.h"
#include "internal.h"

namespace lr {

struct RebaseArgs {
  const unsigned char* src[2];   // K, V stored latents
  unsigned char* dst[2];
  const void* w[2];              // [r_new][ldw] row-major, ldw = round_up(r_old, 8)
  const int32_t* lat_len;
  long long src_tcap, dst_tcap;
  int src_ld[2], dst_ld[2];      // row strides in elements
  int r_old[2], r_new[2];
  int ldw[2];
  int B, max_len, groups_per_seq;
  int col_chunk[2];              // bf16: new coordinates per workgroup chunk (multiple of 16)
};

__device__ __forceinline__ bf16x8 zero8() { return __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u}); }

// AND-mask keeping elements c0 .. c0+7 of a 16-byte bf16 granule that are < n.
__device__ __forceinline__ u32x4 keep_below(int c0, int n) {
  u32x4 m;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    m[i] = (c0 + 2 * i < n ? 0x0000FFFFu : 0u) | (c0 + 2 * i + 1 < n ? 0xFFFF0000u : 0u);
  return m;
}

constexpr int kRebaseRows = 32;      // rows per wave group (two 16-row tiles)
constexpr int kRebaseWaves = 8;      // waves per workgroup, all sharing the staged W chunk

__host__ __device__ constexpr int rebase_ws(int nks) { return nks * 64 + 16; }   // W row stride (B)

template <int NKS>
__global__ __launch_bounds__(kRebaseWaves * 64) void lr_rebase_bf16(RebaseArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char wsm[];
  const int kv = blockIdx.y, chunk = blockIdx.z;
  const int r_old = a.r_old[kv], r_new = a.r_new[kv];
  const int j0 = chunk * a.col_chunk[kv];
  if (j0 >= r_new) return;                              // workgroup-uniform
  const int jc = min(a.col_chunk[kv], r_new - j0);
  const int nblk = (jc + 15) >> 4;                      // 16-coordinate output blocks
  const int nks = (r_old + 31) >> 5;                    // K steps over the old coordinates
  const int ws = rebase_ws(nks);                        // +16 B per row spreads rows over banks
  const int tid = threadIdx.x;

  // W rows j0 .. j0 + 16*nblk - 1 into LDS; rows past r_new and columns past r_old are zero
  {
    const __bf16* wg = (const __bf16*)a.w[kv];
    const int ldw = a.ldw[kv];
    for (int i = tid; i < nblk * 16 * nks * 4; i += kRebaseWaves * 64) {
      const int row = i / (nks * 4), g = i - row * (nks * 4);
      const int j = j0 + row, c = g * 8;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (j < r_new && c < r_old) v = *(const u32x4*)(wg + (size_t)j * ldw + c) & keep_below(c, r_old);
      *(u32x4*)(wsm + row * ws + g * 16) = v;
    }
  }
  __syncthreads();

  const int wave = tid >> 6, lane = tid & 63, lg = lane >> 4, li = lane & 15;
  const __bf16* src = (const __bf16*)a.src[kv];
  __bf16* dst = (__bf16*)a.dst[kv];
  const int sld = a.src_ld[kv], dld = a.dst_ld[kv];
  const long long cap = a.src_tcap < a.dst_tcap ? a.src_tcap : a.dst_tcap;
  const int total = a.B * a.groups_per_seq;

  for (int gi = blockIdx.x * kRebaseWaves + wave; gi < total; gi += gridDim.x * kRebaseWaves) {
    const int b = gi / a.groups_per_seq;
    const int t0 = (gi - b * a.groups_per_seq) * kRebaseRows;
    long long Lb = a.lat_len[b];
    Lb = Lb < 0 ? 0 : (Lb > a.max_len ? a.max_len : Lb);
    Lb = Lb > cap ? cap : Lb;
    const int L = (int)Lb;
    if (t0 >= L) continue;                              // wave-uniform

    // the group's two 16-row tiles as the B operand: lane (lg, li) holds row li's old
    // coordinates 32*ks + 8*lg .. +7. Only granules that start below r_old are read (they end
    // inside the row: the row stride is a multiple of 8 and >= r_old); the last one is masked.
    bf16x8 zb[2][NKS];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int row = t0 + 16 * tt + li;
      const bool valid = row < L;
      const __bf16* zr = src + ((size_t)b * a.src_tcap + (valid ? row : 0)) * sld + lg * 8;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const int c = ks * 32 + lg * 8;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (valid && c < r_old) {
          v = *(const u32x4*)(zr + ks * 32);
          if (c + 8 > r_old) v &= keep_below(c, r_old);
        }
        zb[tt][ks] = __builtin_bit_cast(bf16x8, v);
      }
    }

    for (int n = 0; n < nblk; ++n) {
      f32x4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = {0.f, 0.f, 0.f, 0.f};
      const unsigned char* wrow = wsm + (n * 16 + li) * ws + lg * 16;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        if (ks < nks) {
          const bf16x8 av = *(const bf16x8*)(wrow + ks * 64);
          c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, zb[0][ks], c0, 0, 0, 0);
          c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, zb[1][ks], c1, 0, 0, 0);
        }
      }
      // C[new coordinate n*16 + 4*lg + i][token li]
      const int jb = j0 + n * 16 + 4 * lg;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int row = t0 + 16 * tt + li;
        if (row >= L) continue;
        const f32x4 c = tt == 0 ? c0 : c1;
        __bf16* out = dst + ((size_t)b * a.dst_tcap + row) * dld + jb;
        if (jb + 4 <= r_new) {
          u32x2 o;
          o[0] = (unsigned)__builtin_bit_cast(unsigned short, (__bf16)c[0]) |
                 ((unsigned)__builtin_bit_cast(unsigned short, (__bf16)c[1]) << 16);
          o[1] = (unsigned)__builtin_bit_cast(unsigned short, (__bf16)c[2]) |
                 ((unsigned)__builtin_bit_cast(unsigned short, (__bf16)c[3]) << 16);
          *(u32x2*)out = o;
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (jb + i < r_new) out[i] = (__bf16)c[i];
        }
      }
    }
  }
}

// float32 latents (small caches): one thread per new coordinate, float32 sums in index order.
__global__ __launch_bounds__(256) void lr_rebase_f32(RebaseArgs a) {
  const int kv = blockIdx.y;
  const int r_old = a.r_old[kv], r_new = a.r_new[kv];
  const float* src = (const float*)a.src[kv];
  float* dst = (float*)a.dst[kv];
  const float* w = (const float*)a.w[kv];
  const long long cap = a.src_tcap < a.dst_tcap ? a.src_tcap : a.dst_tcap;
  const long long total = (long long)a.B * a.max_len;
  // rows are read completely before any of their new coordinates is written: one workgroup
  // owns a row (its threads stride over the new coordinates) and stages it in LDS first
  __shared__ float zrow[512];
  for (long long rr = blockIdx.x; rr < total; rr += gridDim.x) {
    const int b = (int)(rr / a.max_len), t = (int)(rr - (long long)b * a.max_len);
    long long Lb = a.lat_len[b];
    Lb = Lb < 0 ? 0 : (Lb > a.max_len ? a.max_len : Lb);
    Lb = Lb > cap ? cap : Lb;
    if (t >= Lb) continue;                              // workgroup-uniform
    const float* zs = src + ((size_t)b * a.src_tcap + t) * a.src_ld[kv];
    __syncthreads();
    for (int i = threadIdx.x; i < r_old; i += 256) zrow[i] = zs[i];
    __syncthreads();
    float* zd = dst + ((size_t)b * a.dst_tcap + t) * a.dst_ld[kv];
    for (int j = threadIdx.x; j < r_new; j += 256) {
      const float* wr = w + (size_t)j * a.ldw[kv];
      float acc = 0.f;
      for (int i = 0; i < r_old; ++i) acc = __builtin_fmaf(zrow[i], wr[i], acc);
      zd[j] = acc;
    }
  }
}

static int rebase_nks_max(int r_old) { return r_old <= 256 ? 8 : (r_old <= 384 ? 12 : 16); }

int rebase_col_chunk(int r_old, int r_new) {
  const int ws = rebase_ws((r_old + 31) >> 5);
  const int rows = ((kLdsBytes - 1024) / ws) & ~15;
  const int need = (r_new + 15) & ~15;
  return need < rows ? need : rows;
}

hipError_t launch_rebase(const RebasePlan& p, const lr_layer_cache* src, const lr_layer_cache* dst,
                         const void* wk, const void* wv, hipStream_t st) {
  RebaseArgs a;
  a.src[0] = (const unsigned char*)src->zk;
  a.src[1] = (const unsigned char*)src->zv;
  a.dst[0] = (unsigned char*)dst->zk;
  a.dst[1] = (unsigned char*)dst->zv;
  a.w[0] = wk;
  a.w[1] = wv;
  a.lat_len = src->lat_len;
  a.src_tcap = src->t_cap;
  a.dst_tcap = dst->t_cap;
  a.src_ld[0] = src->ld_k;
  a.src_ld[1] = src->ld_v;
  a.dst_ld[0] = dst->ld_k;
  a.dst_ld[1] = dst->ld_v;
  a.r_old[0] = p.rk;
  a.r_old[1] = p.rv;
  a.r_new[0] = p.rk_new;
  a.r_new[1] = p.rv_new;
  a.ldw[0] = (p.rk + 7) / 8 * 8;
  a.ldw[1] = (p.rv + 7) / 8 * 8;
  a.B = p.B;
  a.max_len = p.max_len;
  a.groups_per_seq = (p.max_len + kRebaseRows - 1) / kRebaseRows;
  a.col_chunk[0] = a.col_chunk[1] = 0;
  if (p.B == 0 || p.max_len == 0) return hipSuccess;
  if (p.latent == LR_F32) {
    const long long rows = (long long)p.B * p.max_len;
    const unsigned gx = (unsigned)(rows < 65535 ? rows : 65535);
    hipLaunchKernelGGL(lr_rebase_f32, dim3(gx, 2), dim3(256), 0, st, a);
    return hipGetLastError();
  }
  // one launch for K (blockIdx.y = 0) and V (1); blockIdx.z = chunk of the new coordinates
  const int r_max = p.rk > p.rv ? p.rk : p.rv;
  const int nmax = rebase_nks_max(r_max);
  size_t lds = 0;
  int nchunk = 1;
  for (int kv = 0; kv < 2; ++kv) {
    const int r_old = kv == 0 ? p.rk : p.rv, r_new = kv == 0 ? p.rk_new : p.rv_new;
    const int chunk = rebase_col_chunk(r_old, r_new);
    const int n = (r_new + chunk - 1) / chunk;
    const size_t l = (size_t)chunk * rebase_ws((r_old + 31) >> 5);
    a.col_chunk[kv] = chunk;
    if (n > nchunk) nchunk = n;
    if (l > lds) lds = l;
  }
  // workgroups per CU allowed by LDS (two at most: 8 waves each, up to ~225 VGPRs per lane)
  const int per_cu = kLdsBytes / lds >= 2 ? 2 : 1;
  const long long groups = (long long)p.B * a.groups_per_seq;
  long long gx = (groups + kRebaseWaves - 1) / kRebaseWaves;
  long long cap = (long long)device_cu_count() * per_cu / (2 * nchunk);
  cap = cap < 8 ? 8 : cap & ~7LL;   // a multiple of 8: the workgroups of one row range share an XCD
  if (gx > cap) gx = cap;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  static bool attr[64][3] = {};
  const void* fn = nmax == 8 ? (const void*)lr_rebase_bf16<8>
                 : nmax == 12 ? (const void*)lr_rebase_bf16<12> : (const void*)lr_rebase_bf16<16>;
  const int vi = nmax == 8 ? 0 : (nmax == 12 ? 1 : 2);
  if (dev >= 0 && dev < 64 && !attr[dev][vi]) {
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
    if (e != hipSuccess) return e;
    attr[dev][vi] = true;
  }
  const dim3 grid((unsigned)gx, 2, (unsigned)nchunk), block(kRebaseWaves * 64);
  if (nmax == 8) hipLaunchKernelGGL(lr_rebase_bf16<8>, grid, block, lds, st, a);
  else if (nmax == 12) hipLaunchKernelGGL(lr_rebase_bf16<12>, grid, block, lds, st, a);
  else hipLaunchKernelGGL(lr_rebase_bf16<16>, grid, block, lds, st, a);
  return hipGetLastError();
}

}  // namespace lr
