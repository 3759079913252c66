// Historical-coordinate sync after a basis update.
//
// iS-KV ("iS-KV: Online Low-Rank KV Cache Compression via Block-Incremental SVD", English
// abstract; method summary): as the low-rank basis evolves during decoding, the coordinates of
// the stored history are synchronised with it, or the history drifts. Every stored latent row z
// becomes its least-squares coordinates in the new basis,
//     z' = z B pinv(B') = z W^T,     W [r_new][r_old] computed by the caller,
// stored in the cache dtype (bf16: round to nearest even, as the append path stores z).
//
// bf16 kernel (W-stationary): each consumer wave of a workgroup holds a few 16-row blocks of W
// (new coordinates x all old coordinates) in registers for the whole launch; two producer waves
// stream 16-row tiles of stored rows through an LDS ring with direct-to-LDS loads, and every
// tile read from LDS feeds all of a consumer's blocks in 16x16x32 matrix-core products. HBM
// traffic per row: the old coordinates read once (once per chunk of new coordinates when W
// does not fit one workgroup's registers; the chunks of a row range run on one XCD and share
// its L2) and the new coordinates written once.
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
  int stages;                    // bf16: LDS ring depth in tiles
  int kv0;                       // bf16: matrix of blockIdx.y == 0 (0 = K, 1 = V)
  int sub;                       // bf16: 16-row tiles per ring step
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

__device__ __forceinline__ unsigned pack_bf16(float lo, float hi) {   // round to nearest even
  return (unsigned)__builtin_bit_cast(unsigned short, (__bf16)lo) |
         ((unsigned)__builtin_bit_cast(unsigned short, (__bf16)hi) << 16);
}

constexpr int kRbTile = 16;          // rows per tile (the MFMA's N)
constexpr int kRbProducers = 2;      // waves 0..1 stream the tiles into LDS
constexpr int kRbThreads = (kRbProducers + kRbConsumers) * 64;
constexpr int rb_threads(bool all) { return all ? kRbAllWaves * 64 : kRbThreads; }
constexpr int kRbMaxStages = 32;

// 16-byte granule order inside an LDS tile row. A consumer's read of one K step takes granule
// 4*ks + lg of rows li = 0..15; with G granules per row (G = 4 * K steps) the swizzle makes
// every 8 consecutive lanes hit 8 different 16-byte bank groups.
__device__ __forceinline__ int rb_swz(int row, int G) { return (G & 7) ? ((row >> 1) & 3) : (row & 7); }

// New coordinate (relative to a wave's first) of row r of its block nb. Blocks are paired so
// that the accumulator rows a lane holds (4 from each block of a pair) are 8 consecutive
// coordinates: one 16-byte store. Block 2p covers 8m + 0..3, block 2p+1 covers 8m + 4..7 of
// the pair's 32 coordinates (m = r / 4); an unpaired last block covers 16 in order.
__host__ __device__ constexpr int rb_coord(int nb, int NB, int r) {
  return nb < (NB & ~1) ? 32 * (nb >> 1) + 8 * (r >> 2) + 4 * (nb & 1) + (r & 3) : 16 * nb + r;
}

// Walks the steps (16 * sub rows of one sequence) of the linear range [lo, hi) that hold stored
// rows; every wave of a workgroup walks the same sequence. lat_len is read once per sequence.
struct RbIter {
  int idx, hi, sps, b, s, L;   // linear step, end, steps per sequence, sequence, step in it
  int cb, t0, cL;              // current step: sequence, first row, stored rows of the sequence
};
__device__ __forceinline__ void rb_init(RbIter& it, int lo, int hi, int sps) {
  it.idx = lo;
  it.hi = hi;
  it.sps = sps;
  it.b = lo / sps;
  it.s = lo - it.b * sps;
  it.L = -1;
}
__device__ __forceinline__ bool rb_next(RbIter& it, const RebaseArgs& a, long long cap, int step_rows) {
  while (it.idx < it.hi) {
    if (it.L < 0) {
      long long Lb = a.lat_len[it.b];
      Lb = Lb < 0 ? 0 : (Lb > a.max_len ? a.max_len : Lb);
      it.L = (int)(Lb > cap ? cap : Lb);
    }
    const int t0 = it.s * step_rows;
    if (t0 < it.L) {
      it.cb = it.b;
      it.t0 = t0;
      it.cL = it.L;
      ++it.idx;
      if (++it.s == it.sps) {
        it.s = 0;
        ++it.b;
        it.L = -1;
      }
      return true;
    }
    it.idx += it.sps - it.s;                // rest of this sequence is empty
    it.s = 0;
    ++it.b;
    it.L = -1;
  }
  return false;
}

// bf16 latents. blockIdx.y = K/V, blockIdx.z = chunk of the new coordinates, blockIdx.x = a
// contiguous range of steps (sub 16-row tiles of one sequence) over (sequence, position). Each
// consumer wave keeps its NB 16-row blocks of W (new coordinates) x all old coordinates in
// registers for the whole launch and runs 16x16x32 bf16 products with A = W block, B = tile
// rows read from LDS, so every LDS read of a tile feeds NB matrix-core products. Waves 0-1
// stream the steps through an LDS ring with direct-to-LDS loads and exact vmcnt waits (two
// producers double the loads one wave may keep in flight); one barrier per step.
// ALL: 8 waves that each hold NB blocks of W (twice the new coordinates of one workgroup, for
// ranks whose W blocks leave room for only 3 per wave) and each load their share of every
// step: a wave waits for its own loads of step c, the barrier publishes the step and frees the
// stage of step c - 1, and the wave then issues step c + stages - 1 into it.
template <int NKS, int NB, bool ALL>
__global__ __launch_bounds__(rb_threads(ALL)) void lr_rebase_bf16(RebaseArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char ring[];
  const int kv = a.kv0 + blockIdx.y;
  const int r_old = a.r_old[kv], r_new = a.r_new[kv];
  const int nks = (r_old + 31) >> 5;                    // K steps, in (NKS - 4, NKS]
  const int G = nks * 4;                                // granules per tile row
  const int tile_bytes = kRbTile * G * 16;
  const int sub = a.sub, step_rows = kRbTile * sub, step_bytes = tile_bytes * sub;
  const int nst = a.stages;
  const int sps = a.groups_per_seq;                     // steps per sequence
  const long long cap = a.src_tcap < a.dst_tcap ? a.src_tcap : a.dst_tcap;
  const int NT = a.B * sps;
  const int lo = (int)((long long)NT * blockIdx.x / gridDim.x);
  const int hi = (int)((long long)NT * (blockIdx.x + 1) / gridDim.x);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int sld = a.src_ld[kv];

  // ---- loads: rows -> LDS ring, by the NL loading waves (the producers, or with ALL every
  // wave). Instruction k of a 16-row tile (k = lw, lw + NL, ...) fills LDS slots 64k .. 64k+63
  // (16 B each) of the tile; slot s holds row s / G, granule (s % G) ^ swizzle(row). Granules past
  // the rank load granule 0 instead (in bounds, finite; their W columns are zero). Every tile of a
  // step is loaded (rows past the sequence's end repeat its last row), so each step costs every
  // loading wave the same number of loads.
  constexpr int NL = ALL ? kRbAllWaves : kRbProducers;
  constexpr int KP = (NKS + NL - 1) / NL;
  const int lw = wave < NL ? wave : 0;                  // this wave's loader index
  const int my_cnt = (nks - lw + NL - 1) / NL;          // loads per tile
  const __bf16* src = (const __bf16*)a.src[kv];
  int rowk[KP], colk[KP];
#pragma unroll
  for (int u = 0; u < KP; ++u) {
    const int k = lw + NL * u;
    const int sl = 64 * k + lane;
    const int row = sl / G, pos = sl - row * G;
    const int gr = pos ^ rb_swz(row, G);
    rowk[u] = row;
    colk[u] = gr * 8 < r_old ? gr * 8 : 0;
  }
  auto issue = [&](const RbIter& t, int stage) {
    const __bf16* base = src + (size_t)t.cb * a.src_tcap * sld;
    unsigned char* dstl = ring + stage * step_bytes + lw * 1024;
    for (int q = 0; q < sub; ++q) {
#pragma unroll
      for (int u = 0; u < KP; ++u) {
        if (u < my_cnt) {
          int row = t.t0 + q * kRbTile + rowk[u];
          row = row < t.cL ? row : t.cL - 1;
          dma16(base + (size_t)row * sld + colk[u], dstl + q * tile_bytes + NL * u * 1024);
        }
      }
    }
  };
  const int per_step = my_cnt * sub;

  if (!ALL && wave < kRbProducers) {
    RbIter ii, ci;
    rb_init(ii, lo, hi, sps);
    rb_init(ci, lo, hi, sps);
    int issued = 0;
    for (int s = 0; s < nst - 1; ++s) {
      if (!rb_next(ii, a, cap, step_rows)) break;
      issue(ii, issued % nst);
      ++issued;
    }
    for (int c = 0; rb_next(ci, a, cap, step_rows); ++c) {
      wait_vmcnt((issued - c - 1) * per_step);          // this wave's part of the step landed
      barrier_lds();                                    // ... for every consumer; stage c-1 is free
      if (rb_next(ii, a, cap, step_rows)) {
        issue(ii, issued % nst);
        ++issued;
      }
    }
    return;
  }

  // ---- consumers
  const int cw = ALL ? wave : wave - kRbProducers, lg = lane >> 4, li = lane & 15;
  const int jw = blockIdx.z * a.col_chunk[kv] + cw * NB * 16;   // first new coordinate of this wave
  const int jend = min(r_new, (blockIdx.z + 1) * a.col_chunk[kv]);
  // W rows -> registers. Every load is issued (rows and columns clamped into the matrix) and
  // then masked, so the loads overlap: rows past this chunk and columns past r_old are zero.
  bf16x8 w[NB][NKS];
  {
    const __bf16* wg = (const __bf16*)a.w[kv];
    const int ldw = a.ldw[kv];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int j = jw + rb_coord(nb, NB, li);
      const int jc = j < r_new ? j : r_new - 1;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const int c = ks * 32 + lg * 8;
        const int cc = c < ldw - 8 ? c : ldw - 8;
        u32x4 v = *(const u32x4*)(wg + (size_t)jc * ldw + cc);
        v &= keep_below(c, j < jend ? r_old : 0);
        w[nb][ks] = __builtin_bit_cast(bf16x8, v);
      }
    }
  }
  // z operand: K steps below NKS - 4 always exist. When r_old is not a multiple of 8, the step
  // holding r_old - 1 keeps only the columns below r_old (its granule carries pad columns, which
  // may hold anything); steps past nks are zero and skip their products. (Granules wholly past
  // r_old hold granule 0, finite, against zero W columns.)
  const u32x4 last_mask = keep_below((nks - 1) * 32 + lg * 8, r_old);
  const bool fix_tail = (r_old & 7) != 0 || nks < NKS;
  const int rsw = rb_swz(li, G);
  __bf16* dst = (__bf16*)a.dst[kv];
  const int dld = a.dst_ld[kv];
  constexpr int KF = NKS > 4 ? NKS - 4 : 0;             // K steps that always exist
  RbIter t;
  rb_init(t, lo, hi, sps);
  RbIter ii;                                            // ALL: the next step to load
  int issued = 0;
  if constexpr (ALL) {
    // W is in registers before any ring load goes out, so no wait inside the loop is ever for it
    LR_WAIT_VM(0);
    rb_init(ii, lo, hi, sps);
    for (int s2 = 0; s2 < nst - 1; ++s2) {
      if (!rb_next(ii, a, cap, step_rows)) break;
      issue(ii, issued % nst);
      ++issued;
    }
  }
  for (int c = 0; rb_next(t, a, cap, step_rows); ++c) {
    if constexpr (ALL) {
      // this wave's loads of step c landed (a conservative count: this wave's result stores are
      // counted too, and they only make it wait longer)
      wait_vmcnt((issued - c - 1) * per_step);
    }
    barrier_lds();
    if constexpr (ALL) {
      if (rb_next(ii, a, cap, step_rows)) {               // into the stage step c - 1 left
        issue(ii, issued % nst);
        ++issued;
      }
    }
    const unsigned char* stp = ring + (c % nst) * step_bytes + li * G * 16;
    for (int q = 0; q < sub; ++q) {
      const int row = t.t0 + q * kRbTile + li;
      if (t.t0 + q * kRbTile >= t.cL) break;            // step-uniform
      const unsigned char* st = stp + q * tile_bytes;
      f32x4 acc[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
      // the tile's z operands, all K steps at once (ALL: in halves, for the registers the loads
      // of the ring take); the products add the K steps in order either way
      constexpr int ZC = ALL ? (NKS + 1) / 2 : NKS;
#pragma unroll
      for (int ks0 = 0; ks0 < NKS; ks0 += ZC) {
        u32x4 zv[ZC];
#pragma unroll
        for (int u = 0; u < ZC; ++u) {
          const int ks = ks0 + u;
          const int kk = (ks < KF || ks < nks) ? ks : nks - 1;
          if (ks < NKS) zv[u] = *(const u32x4*)(st + (((4 * kk + lg) ^ rsw) << 4));
        }
        if (fix_tail) {
#pragma unroll
          for (int u = 0; u < ZC; ++u) {
            const int ks = ks0 + u;
            if (ks >= KF && ks < NKS && ks == nks - 1) zv[u] &= last_mask;
          }
        }
#pragma unroll
        for (int u = 0; u < ZC; ++u) {
          const int ks = ks0 + u;
          if (ks < NKS && (ks < KF || ks < nks)) {
            const bf16x8 zo = __builtin_bit_cast(bf16x8, zv[u]);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w[nb][ks], zo, acc[nb], 0, 0, 0);
          }
        }
      }
      // C[block row 4lg + i][token li]: pairs give 8 consecutive coordinates jp + 8lg + 0..7
      if (row < t.cL) {
        __bf16* out = dst + ((size_t)t.cb * a.dst_tcap + row) * dld;
#pragma unroll
        for (int pb = 0; pb < NB / 2; ++pb) {
          const int jb = jw + 32 * pb + 8 * lg;
          const f32x4 v0 = acc[2 * pb], v1 = acc[2 * pb + 1];
          if (jb + 8 <= jend) {
            u32x4 o;
            o[0] = pack_bf16(v0[0], v0[1]);
            o[1] = pack_bf16(v0[2], v0[3]);
            o[2] = pack_bf16(v1[0], v1[1]);
            o[3] = pack_bf16(v1[2], v1[3]);
            *(u32x4*)(out + jb) = o;
          } else if (jb < jend) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              if (jb + i < jend) out[jb + i] = (__bf16)v0[i];
              if (jb + 4 + i < jend) out[jb + 4 + i] = (__bf16)v1[i];
            }
          }
        }
        if constexpr ((NB & 1) != 0) {
          const int jb = jw + 16 * (NB - 1) + 4 * lg;
          const f32x4 v = acc[NB - 1];
          if (jb + 4 <= jend) {
            u32x2 o;
            o[0] = pack_bf16(v[0], v[1]);
            o[1] = pack_bf16(v[2], v[3]);
            *(u32x2*)(out + jb) = o;
          } else if (jb < jend) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (jb + i < jend) out[jb + i] = (__bf16)v[i];
          }
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

// Launch shape shared by K and V: K-step bound NKS (template), blocks of 16 new coordinates
// per consumer NB (template; bounded by registers), chunks of new coordinates (each chunk is
// one workgroup's consumers; every chunk re-reads the rows).
static hipError_t launch_rebase_bf16(int nks_t, int nb, bool all, dim3 grid, size_t lds, hipStream_t st,
                                     const RebaseArgs& a) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  static bool attr[64][24] = {};
  int vi = 0;
#define LR_RB_CASES(X) X(4, 1) X(4, 2) X(4, 3) X(4, 4) X(4, 5) X(4, 6) X(4, 7) X(4, 8) \
                       X(8, 1) X(8, 2) X(8, 3) X(8, 4) X(12, 1) X(12, 2) X(12, 3) X(16, 1) X(16, 2)
#define LR_RB_LAUNCH(K, N)                                                                      \
  if (nks_t == K && nb == N && !all) {                                                          \
    if (dev >= 0 && dev < 64 && !attr[dev][vi]) {                                               \
      e = hipFuncSetAttribute((const void*)lr_rebase_bf16<K, N, false>,                         \
                              hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);           \
      if (e != hipSuccess) return e;                                                            \
      attr[dev][vi] = true;                                                                     \
    }                                                                                           \
    hipLaunchKernelGGL((lr_rebase_bf16<K, N, false>), grid, dim3(rb_threads(false)), lds, st, a); \
    return hipGetLastError();                                                                   \
  }                                                                                             \
  ++vi;
  LR_RB_CASES(LR_RB_LAUNCH)
#undef LR_RB_LAUNCH
#undef LR_RB_CASES
  // the all-waves form: 8 waves of the most W blocks their registers hold
#define LR_RB_ALL(K, N, I)                                                                        \
  if (nks_t == K && nb == N && all) {                                                             \
    if (dev >= 0 && dev < 64 && !attr[dev][I]) {                                                  \
      e = hipFuncSetAttribute((const void*)lr_rebase_bf16<K, N, true>,                            \
                              hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);             \
      if (e != hipSuccess) return e;                                                              \
      attr[dev][I] = true;                                                                        \
    }                                                                                             \
    hipLaunchKernelGGL((lr_rebase_bf16<K, N, true>), grid, dim3(rb_threads(true)), lds, st, a);   \
    return hipGetLastError();                                                                     \
  }
  LR_RB_ALL(8, 4, 21) LR_RB_ALL(12, 3, 22) LR_RB_ALL(16, 2, 23)
#undef LR_RB_ALL
  return hipErrorInvalidValue;
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
  a.groups_per_seq = 0;
  a.stages = 0;
  a.col_chunk[0] = a.col_chunk[1] = 0;
  a.kv0 = 0;
  a.sub = 1;
  if (p.B == 0 || p.max_len == 0) return hipSuccess;
  if (p.latent == LR_F32) {
    const long long rows = (long long)p.B * p.max_len;
    const unsigned gx = (unsigned)(rows < 65535 ? rows : 65535);
    hipLaunchKernelGGL(lr_rebase_f32, dim3(gx, 2), dim3(256), 0, st, a);
    return hipGetLastError();
  }
  // K and V share one launch (blockIdx.y = matrix) when their kernel shapes agree
  RebaseShape sh[2];
  rebase_shape(p.rk, p.rk_new, &sh[0]);
  rebase_shape(p.rv, p.rv_new, &sh[1]);
  a.col_chunk[0] = sh[0].col_chunk;
  a.col_chunk[1] = sh[1].col_chunk;
  const bool together = sh[0].nks_t == sh[1].nks_t && sh[0].nb == sh[1].nb && sh[0].all == sh[1].all;
  for (int kv0 = 0; kv0 < 2; kv0 += together ? 2 : 1) {
    const int nmat = together ? 2 : 1;
    const int kv1 = kv0 + nmat - 1;
    const int nchunk = sh[kv0].nchunk > sh[kv1].nchunk ? sh[kv0].nchunk : sh[kv1].nchunk;
    // steps of sub 16-row tiles; ring depth: a producer's outstanding loads ((stages - 1) steps
    // of its share of the instructions) stay within the 6-bit vmcnt; LDS bounds it too
    const int r_max = (kv0 == 0 ? p.rk : p.rv) > (kv1 == 0 ? p.rk : p.rv) ? (kv0 == 0 ? p.rk : p.rv)
                                                                          : (kv1 == 0 ? p.rk : p.rv);
    const int nks = (r_max + 31) / 32;
    const int sub = nks <= 8 ? 4 : 2;
    const int step_bytes = kRbTile * nks * 4 * 16 * sub;
    const int nl = sh[kv0].all ? kRbAllWaves : kRbProducers;   // waves that load the ring
    const int per_wave = (nks + nl - 1) / nl * sub;
    int stages = 63 / per_wave + 1;
    if (stages > kRbMaxStages) stages = kRbMaxStages;
    if (stages * step_bytes > kLdsBytes) stages = kLdsBytes / step_bytes;
    RebaseArgs ak = a;
    ak.stages = stages;
    ak.sub = sub;
    ak.kv0 = kv0;
    ak.groups_per_seq = (p.max_len + kRbTile * sub - 1) / (kRbTile * sub);
    const size_t lds = (size_t)stages * step_bytes;
    const long long steps = (long long)p.B * ak.groups_per_seq;
    long long gx = device_cu_count() / (nmat * nchunk);
    gx = gx < 4 ? 4 : gx & ~3LL;      // 2*gx a multiple of 8: the chunks of one range share an XCD
    if (gx > steps) gx = steps;
    hipError_t e = launch_rebase_bf16(sh[kv0].nks_t, sh[kv0].nb, sh[kv0].all != 0,
                                      dim3((unsigned)gx, nmat, (unsigned)nchunk), lds, st, ak);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace lr
