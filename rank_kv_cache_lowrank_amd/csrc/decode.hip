// Decode attention over a low-rank latent KV cache: fold, split-token latent decode, combine.
//
// Method (TraceKV, "TraceKV: Policy-Preserving Low-Rank KV Cache Compression for Reasoning
// Vision-Language Models", abstract: the cache holds low-dimensional latents of the KV states
// and attention runs on them; iS-KV, "iS-KV: Online Low-Rank KV Cache Compression via
// Block-Incremental SVD", abstract: an exact recent window sits beside the latent history).
// Because (q Bk^T) Zk^T = q (Zk Bk)^T and (p Zv) Bv = p (Zv Bv), attending over the latents
// and up-projecting once gives the same result as attending over reconstructed keys/values.
//
// Kernels, in stream order:
//   lr_fold     qt[b, j, :] = (sm_scale * log2 e) * q[b, j, :] Bk[:, g(j)]^T  as bf16, heads
//               padded to 32 and the rank padded to a multiple of 32 with zeros.
//   lr_decode   one workgroup per (sequence, token range). The latent rows of the range stream
//               through a ring of LDS stages filled by 16-byte direct-to-LDS loads; per 32-token
//               tile: S = Zk qt^T on the matrix cores (16x16x32 bf16), online softmax in base 2,
//               A += P Zv on the matrix cores. All 28 query heads share the one latent stream,
//               so every latent byte is read from HBM once. Writes (m, l, A) per range.
//               Extra workgroups (first in the grid) attend over the exact window, if any.
//   lr_combine  one workgroup per (sequence, head): merges the ranges and the window partial
//               and up-projects through Bv[:, g(j)].
#include "device_common.h"
#include "internal.h"

#include <math.h>

namespace lr {

enum { LT_F32 = 0, LT_BF16 = 1, LT_I4 = 2 };

struct DecodeArgs {
  const unsigned char* zk;
  const unsigned char* zv;
  const unsigned char* zkq;
  const unsigned char* zvq;
  const __bf16* qt;
  const int32_t* lat_len;
  const int32_t* win_len;
  float* part_ml;
  float* part_acc;
  float* win_part;
  const void* q;
  const __bf16* kwin;
  const __bf16* vwin;
  long long t_cap;
  int row_bytes_k, row_bytes_v, qp_bytes_k, qp_bytes_v;
  int rk, rv, rk_pad, nks, nrb, rv_pad16;
  int nsplit, split_tokens, max_len;
  int Hq, Hkv, d, D, window;
  float wscale;
  int n_win_blocks;
  int stage_bytes, zv_off, qpk_off, qpv_off, nst;
};

__device__ __forceinline__ bf16x8 zero_bf16x8() {
  return __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
}

// ---------------------------------------------------------------------------------------------
// Matrix-core operands from the LDS tile.
// 16x16x32 bf16 layout (gfx950): A row = lane % 16, B column = lane % 16, and the 8 operand
// slots of lane group lg = lane / 16 pair A with B on the same K index; C row 4*lg + i,
// column lane % 16.
// Scores (S^T = Zk qt^T): A = Zk rows (token = lane % 16), K = latent index lg*8 + e.
// Values (A^T += Zv^T P^T): A = Zv^T (row = latent index), K = token; slot e of lane group lg
// holds token 4*lg + e (e < 4) or 16 + 4*lg + e - 4 (e >= 4), which is exactly how the score
// tiles of the two 16-token halves land in the C layout, so P needs no shuffle.
// ---------------------------------------------------------------------------------------------
template <int LT>
__device__ __forceinline__ bf16x8 k_operand(const unsigned char* row, int k0) {
  if constexpr (LT == LT_F32) {
    const f32x4 x0 = *(const f32x4*)(row + k0 * 4);
    const f32x4 x1 = *(const f32x4*)(row + k0 * 4 + 16);
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) { r[e] = (__bf16)x0[e]; r[4 + e] = (__bf16)x1[e]; }
    return r;
  } else {
    return *(const bf16x8*)(row + k0 * 2);
  }
}

__device__ __forceinline__ int slot_token(int lg, int e) {
  return e < 4 ? 4 * lg + e : 16 + 4 * lg + (e - 4);
}

template <int LT>
__device__ __forceinline__ bf16x8 v_operand(const unsigned char* sv, int row_bytes, int rv, int lg) {
  if constexpr (LT == LT_F32) {
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      r[e] = (__bf16)(*(const float*)(sv + slot_token(lg, e) * row_bytes + rv * 4));
    return r;
  } else {
    unsigned short h[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
      h[e] = *(const unsigned short*)(sv + slot_token(lg, e) * row_bytes + rv * 2);
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = (unsigned)h[2 * i] | ((unsigned)h[2 * i + 1] << 16);
    return __builtin_bit_cast(bf16x8, w);
  }
}

// ---------------------------------------------------------------------------------------------
// Exact-window workgroup: dense attention of every head over the live window slots of one
// sequence (iS-KV abstract: the recent window is kept exact). Writes (Aw[d], m, l) per head,
// in base-2 softmax units like the latent partials.
// ---------------------------------------------------------------------------------------------
template <int LT>
__device__ void window_block(const DecodeArgs& a, unsigned char* smem) {
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int Hq = a.Hq, d = a.d, D = a.D, W = a.window;
  const int grp = Hq / a.Hkv;
  int L = a.lat_len[b];
  L = L < 0 ? 0 : L;
  int wl = a.win_len[b];
  wl = wl < 0 ? 0 : (wl > W ? W : wl);

  float* qs = (float*)smem;                              // [Hq][d]
  __bf16* kc = (__bf16*)(qs + Hq * d);                   // [32][D]
  __bf16* vc = kc + 32 * D;                              // [32][D]
  float* sc = (float*)(vc + 32 * D);                     // [Hq][32]
  float* st = sc + Hq * 32;                              // [Hq][3]: m, l, alpha

  for (int i = tid; i < Hq * d; i += kDecodeThreads) {
    float qv;
    if constexpr (LT == LT_F32) qv = ((const float*)a.q)[(size_t)b * Hq * d + i];
    else qv = (float)((const __bf16*)a.q)[(size_t)b * Hq * d + i];
    qs[i] = qv * a.wscale;
  }
  for (int j = tid; j < Hq; j += kDecodeThreads) { st[j * 3] = -INFINITY; st[j * 3 + 1] = 0.f; }

  constexpr int kMaxAcc = 16;                            // Hq*d <= 32*128 = 16 * 256
  float acc[kMaxAcc];
#pragma unroll
  for (int u = 0; u < kMaxAcc; ++u) acc[u] = 0.f;
  const int nout = Hq * d;

  for (int c0 = 0; c0 < wl; c0 += 32) {
    const int n = (wl - c0) < 32 ? (wl - c0) : 32;
    __syncthreads();
    // stage n window rows (16 bytes per thread per step)
    const int vec_per_row = D / 8;
    for (int i = tid; i < n * vec_per_row; i += kDecodeThreads) {
      const int u = i / vec_per_row, c = i - u * vec_per_row;
      const int slot = (L + c0 + u) % W;
      const size_t src = ((size_t)b * W + slot) * D + c * 8;
      *(u32x4*)(kc + u * D + c * 8) = *(const u32x4*)(a.kwin + src);
      *(u32x4*)(vc + u * D + c * 8) = *(const u32x4*)(a.vwin + src);
    }
    __syncthreads();
    for (int i = tid; i < Hq * 32; i += kDecodeThreads) {
      const int j = i >> 5, u = i & 31;
      float s = -INFINITY;
      if (u < n) {
        const int g = j / grp;
        const float* qj = qs + j * d;
        const __bf16* kr = kc + u * D + g * d;
        s = 0.f;
        for (int c = 0; c < d; ++c) s += qj[c] * (float)kr[c];
        s = (s != s) ? INFINITY : s;   // NaN propagates to this head only (see latent_block)
      }
      sc[i] = s;
    }
    __syncthreads();
    for (int j = tid; j < Hq; j += kDecodeThreads) {
      float mx = -INFINITY;
      for (int u = 0; u < n; ++u) mx = fmaxf(mx, sc[j * 32 + u]);
      const float mold = st[j * 3];
      const float mnew = fmaxf(mold, mx);
      const float alpha = (mnew == -INFINITY) ? 1.f : fast_exp2(mold - mnew);
      float ps = 0.f;
      for (int u = 0; u < 32; ++u) {
        const float p = (u < n && mnew != -INFINITY) ? fast_exp2(sc[j * 32 + u] - mnew) : 0.f;
        sc[j * 32 + u] = p;
        ps += p;
      }
      st[j * 3] = mnew;
      st[j * 3 + 1] = st[j * 3 + 1] * alpha + ps;
      st[j * 3 + 2] = alpha;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kMaxAcc; ++u) {
      const int o = tid + u * kDecodeThreads;
      if (o < nout) {
        const int j = o / d, c = o - j * d;
        const int g = j / grp;
        float v = acc[u] * st[j * 3 + 2];
        for (int t = 0; t < n; ++t) v += sc[j * 32 + t] * (float)vc[t * D + g * d + c];
        acc[u] = v;
      }
    }
  }
  __syncthreads();
  float* wp = a.win_part + (size_t)b * Hq * (d + 2);
#pragma unroll
  for (int u = 0; u < kMaxAcc; ++u) {
    const int o = tid + u * kDecodeThreads;
    if (o < nout) {
      const int j = o / d, c = o - j * d;
      wp[j * (d + 2) + c] = acc[u];
    }
  }
  for (int j = tid; j < Hq; j += kDecodeThreads) {
    wp[j * (d + 2) + d] = st[j * 3];
    wp[j * (d + 2) + d + 1] = st[j * 3 + 1];
  }
}

// ---------------------------------------------------------------------------------------------
// Latent workgroup: one (sequence b, token range s).
// KS: compile-time bound on K steps of 32 (rank_k); RB: bound on value blocks per wave.
// ---------------------------------------------------------------------------------------------
template <int KS, int RB, int LT>
__device__ __forceinline__ void latent_block(const DecodeArgs& a, unsigned char* smem, int wg) {
  const int b = wg / a.nsplit;
  const int s = wg - b * a.nsplit;
  const int tid = threadIdx.x, lane = tid & 63, lg = lane >> 4, li = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform

  int L = a.lat_len[b];
  L = L < 0 ? 0 : (L > a.max_len ? a.max_len : L);
  const int t_begin = s * a.split_tokens;
  const int t_end = min(t_begin + a.split_tokens, L);
  const int ntiles = t_end > t_begin ? (t_end - t_begin + kTileTokens - 1) / kTileTokens : 0;

  unsigned char* ring = smem;
  float* sx = (float*)(smem + a.nst * a.stage_bytes + kLdsPad);

  const unsigned char* gk = a.zk + ((size_t)b * a.t_cap + t_begin) * a.row_bytes_k;
  const unsigned char* gv = a.zv + ((size_t)b * a.t_cap + t_begin) * a.row_bytes_v;

  // Per-wave count of direct-to-LDS instructions for a tile of `rows` rows.
  auto wave_chunks = [&](int bytes) {
    const int nch = (bytes + 1023) >> 10;
    return nch > wave ? (nch - wave + 3) >> 2 : 0;
  };
  const int rows_last = ntiles > 0 ? t_end - (t_begin + (ntiles - 1) * kTileTokens) : 0;
  const int cpw_full = wave_chunks(kTileTokens * a.row_bytes_k) + wave_chunks(kTileTokens * a.row_bytes_v);
  const int cpw_last = wave_chunks(rows_last * a.row_bytes_k) + wave_chunks(rows_last * a.row_bytes_v);

  auto issue = [&](int t) {
    unsigned char* stg = ring + (t % a.nst) * a.stage_bytes;
    const int t0 = t * kTileTokens;
    const int rows = min(kTileTokens, t_end - t_begin - t0);
    const int bk = rows * a.row_bytes_k;
    const unsigned char* srck = gk + (size_t)t0 * a.row_bytes_k;
    for (int c = wave; c * 1024 < bk; c += 4) {
      const int off = c * 1024 + lane * 16;
      if (off < bk) dma16(srck + off, stg + c * 1024);
    }
    const int bv = rows * a.row_bytes_v;
    const unsigned char* srcv = gv + (size_t)t0 * a.row_bytes_v;
    unsigned char* stv = stg + a.zv_off;
    for (int c = wave; c * 1024 < bv; c += 4) {
      const int off = c * 1024 + lane * 16;
      if (off < bv) dma16(srcv + off, stv + c * 1024);
    }
  };

  // Prologue: the first nst-1 tiles, then the folded query of this wave's head block.
  const int pro = min(a.nst - 1, ntiles);
  for (int t = 0; t < pro; ++t) issue(t);

  const int tb1 = wave & 1, hb1 = wave >> 1;   // this wave's score block (token half, head half)
  bf16x8 qop[KS];
  {
    const __bf16* qrow = a.qt + ((size_t)b * kHeadsPad + hb1 * 16 + li) * a.rk_pad + lg * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qop[ks] = (ks < a.nks) ? *(const bf16x8*)(qrow + ks * 32) : zero_bf16x8();
  }
  LR_WAIT_VM(0);

  float m[2] = {-INFINITY, -INFINITY};
  float lsum[2] = {0.f, 0.f};
  f32x4 acc[2][RB];
#pragma unroll
  for (int hb = 0; hb < 2; ++hb)
#pragma unroll
    for (int j = 0; j < RB; ++j) acc[hb][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int i = 0; i < ntiles; ++i) {
    const int hi = min(i + a.nst - 2, ntiles - 1);
    int younger = 0;
    if (hi > i) younger = (hi - i) * cpw_full + (hi == ntiles - 1 ? cpw_last - cpw_full : 0);
    wait_vmcnt(younger);
    barrier_lds();
    if (i + a.nst - 1 < ntiles) issue(i + a.nst - 1);

    const unsigned char* stg = ring + (i % a.nst) * a.stage_bytes;
    const int nvalid = min(kTileTokens, t_end - (t_begin + i * kTileTokens));

    // ---- scores: this wave's 16 tokens x 16 heads block over the whole rank
    f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
    const unsigned char* krow = stg + (tb1 * 16 + li) * a.row_bytes_k;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks < a.nks) {
        const int k0 = ks * 32 + lg * 8;
        bf16x8 av = k_operand<LT>(krow, k0);
        if (k0 + 8 > a.rk) {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (k0 + e >= a.rk) av[e] = (__bf16)0.f;
        }
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, qop[ks], sacc, 0, 0, 0);
      }
    }
    *(f32x4*)(sx + ((tb1 * 2 + hb1) * 64 + lane) * 4) = sacc;
    barrier_lds();

    // ---- online softmax (base 2; the fold carries log2 e) for both head blocks
    bf16x8 pb[2];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const f32x4 s0 = *(const f32x4*)(sx + ((0 * 2 + hb) * 64 + lane) * 4);
      const f32x4 s1 = *(const f32x4*)(sx + ((1 * 2 + hb) * 64 + lane) * 4);
      float v[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) { v[e] = s0[e]; v[4 + e] = s1[e]; }
      // A NaN score becomes +inf so that it survives the max and poisons exactly this head's
      // sums (fmaxf would drop it and the head would read as empty).
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = (v[e] != v[e]) ? INFINITY : v[e];
      if (nvalid < kTileTokens) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (slot_token(lg, e) >= nvalid) v[e] = -INFINITY;
      }
      float mx = v[0];
#pragma unroll
      for (int e = 1; e < 8; ++e) mx = fmaxf(mx, v[e]);
      mx = wave_max_lg(mx);
      const float mnew = fmaxf(m[hb], mx);
      const bool live = mnew != -INFINITY;
      const float alpha = live ? fast_exp2(m[hb] - mnew) : 1.f;
      m[hb] = mnew;
      float ps = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const __bf16 p = (__bf16)(live ? fast_exp2(v[e] - mnew) : 0.f);
        pb[hb][e] = p;
        ps += (float)p;
      }
      lsum[hb] = lsum[hb] * alpha + ps;
#pragma unroll
      for (int j = 0; j < RB; ++j) acc[hb][j] *= alpha;
    }

    // ---- values: this wave's 16-wide latent blocks, both head blocks
    const unsigned char* sv = stg + a.zv_off;
#pragma unroll
    for (int j = 0; j < RB; ++j) {
      const int rb = wave + 4 * j;
      if (rb < a.nrb) {
        bf16x8 av = v_operand<LT>(sv, a.row_bytes_v, rb * 16 + li, lg);
        if (nvalid < kTileTokens) {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (slot_token(lg, e) >= nvalid) av[e] = (__bf16)0.f;
        }
        acc[0][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, pb[0], acc[0][j], 0, 0, 0);
        acc[1][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, pb[1], acc[1][j], 0, 0, 0);
      }
    }
  }

  // ---- partials of this range
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) lsum[hb] = wave_sum_lg(lsum[hb]);
  const size_t pidx = (size_t)b * a.nsplit + s;
  if (wave == 0 && lg == 0) {
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const int head = hb * 16 + li;
      if (head < a.Hq) {
        a.part_ml[(pidx * a.Hq + head) * 2] = m[hb];
        a.part_ml[(pidx * a.Hq + head) * 2 + 1] = lsum[hb];
      }
    }
  }
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    const int head = hb * 16 + li;
#pragma unroll
    for (int j = 0; j < RB; ++j) {
      const int rb = wave + 4 * j;
      if (rb < a.nrb && head < a.Hq)
        *(f32x4*)(a.part_acc + (pidx * a.Hq + head) * a.rv_pad16 + rb * 16 + 4 * lg) = acc[hb][j];
    }
  }
}

template <int KS, int RB, int LT>
__global__ __launch_bounds__(kDecodeThreads) void lr_decode(DecodeArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  if ((int)blockIdx.x < a.n_win_blocks) {
    window_block<LT>(a, smem);
    return;
  }
  latent_block<KS, RB, LT>(a, smem, (int)blockIdx.x - a.n_win_blocks);
}

// ---------------------------------------------------------------------------------------------
// Fold: qt[b][j][k] = scale * sum_c q[b][j][c] * Bk[k][g(j)*d + c], bf16, zero-padded.
// grid (rk_pad/64, B), 256 threads: thread (slot, k) handles KV heads slot, slot+4, ...
// ---------------------------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ void load8(const T* p, float* out);
template <>
__device__ __forceinline__ void load8<__bf16>(const __bf16* p, float* out) {
  const bf16x8 v = *(const bf16x8*)p;
#pragma unroll
  for (int e = 0; e < 8; ++e) out[e] = (float)v[e];
}
template <>
__device__ __forceinline__ void load8<float>(const float* p, float* out) {
  const f32x4 v0 = *(const f32x4*)p;
  const f32x4 v1 = *(const f32x4*)(p + 4);
#pragma unroll
  for (int e = 0; e < 4; ++e) { out[e] = v0[e]; out[4 + e] = v1[e]; }
}

template <typename T>
__global__ __launch_bounds__(256) void lr_fold(const T* __restrict__ q, const T* __restrict__ bk,
                                               __bf16* __restrict__ qt, int Hq, int Hkv, int d, int D,
                                               int rk, int rk_pad, float scale) {
  extern __shared__ float qs[];
  const int b = blockIdx.y;
  for (int i = threadIdx.x; i < Hq * d; i += 256) qs[i] = to_f32(q[(size_t)b * Hq * d + i]) * scale;
  __syncthreads();
  const int k = blockIdx.x * 64 + (threadIdx.x & 63);
  const int slot = threadIdx.x >> 6;
  if (k >= rk_pad) return;
  const int grp = Hq / Hkv;
  __bf16* out = qt + (size_t)b * kHeadsPad * rk_pad + k;
  for (int g = slot; g < Hkv; g += 4) {
    for (int h0 = 0; h0 < grp; h0 += 8) {
      float acc[8];
#pragma unroll
      for (int hh = 0; hh < 8; ++hh) acc[hh] = 0.f;
      if (k < rk) {
        const T* brow = bk + (size_t)k * D + g * d;
        for (int c = 0; c < d; c += 8) {
          float bv[8];
          load8<T>(brow + c, bv);
#pragma unroll
          for (int hh = 0; hh < 8; ++hh) {
            if (h0 + hh < grp) {
              const float* qj = qs + (g * grp + h0 + hh) * d + c;
#pragma unroll
              for (int e = 0; e < 8; ++e) acc[hh] += qj[e] * bv[e];
            }
          }
        }
      }
#pragma unroll
      for (int hh = 0; hh < 8; ++hh)
        if (h0 + hh < grp) out[(size_t)(g * grp + h0 + hh) * rk_pad] = (__bf16)acc[hh];
    }
  }
  if (slot == 0)
    for (int j = Hq; j < kHeadsPad; ++j) out[(size_t)j * rk_pad] = (__bf16)0.f;
}

// ---------------------------------------------------------------------------------------------
// Combine: one workgroup per (b, j). m* = max over ranges (and window), weights 2^(m_s - m*),
// l* = sum w_s l_s, Ahat = sum w_s A_s, out = (Ahat Bv[:, g] + w_win Aw) / l*.
// ---------------------------------------------------------------------------------------------
struct CombineArgs {
  const float* part_ml;
  const float* part_acc;
  const float* win_part;
  const void* bv;
  void* out;
  int Hq, Hkv, d, D, rv, rv_pad16, nsplit, window;
};

__device__ __forceinline__ float block_reduce(float v, float* red, bool is_max) {
  const int tid = threadIdx.x;
  for (int o = 32; o > 0; o >>= 1) {
    const float w = __shfl_xor(v, o);
    v = is_max ? fmaxf(v, w) : v + w;
  }
  __syncthreads();
  if ((tid & 63) == 0) red[tid >> 6] = v;
  __syncthreads();
  float r = red[0];
  for (int i = 1; i < 4; ++i) r = is_max ? fmaxf(r, red[i]) : r + red[i];
  return r;
}

template <typename BT, typename OT>
__global__ __launch_bounds__(256) void lr_combine(CombineArgs a) {
  extern __shared__ float cs[];
  const int tid = threadIdx.x;
  const int b = blockIdx.x / a.Hq, j = blockIdx.x - b * a.Hq;
  const int g = j / (a.Hq / a.Hkv);
  float* ws = cs;                       // [nsplit]
  float* ahat = ws + a.nsplit;          // [rv]
  float* red = ahat + a.rv_pad16;       // [256]
  const size_t base = (size_t)b * a.nsplit;

  float mloc = -INFINITY;
  for (int s = tid; s < a.nsplit; s += 256) mloc = fmaxf(mloc, a.part_ml[((base + s) * a.Hq + j) * 2]);
  float mw = -INFINITY, lw = 0.f;
  const float* wp = a.win_part + ((size_t)b * a.Hq + j) * (a.d + 2);
  if (a.window) { mw = wp[a.d]; lw = wp[a.d + 1]; }
  const float mstar = block_reduce(fmaxf(mloc, mw), red, true);
  const bool live = mstar != -INFINITY;

  float lloc = 0.f;
  for (int s = tid; s < a.nsplit; s += 256) {
    const float ms = a.part_ml[((base + s) * a.Hq + j) * 2];
    const float w = (live && ms != -INFINITY) ? fast_exp2(ms - mstar) : 0.f;
    ws[s] = w;
    if (w != 0.f) lloc += w * a.part_ml[((base + s) * a.Hq + j) * 2 + 1];
  }
  const float ww = (live && mw != -INFINITY) ? fast_exp2(mw - mstar) : 0.f;
  const float lstar = block_reduce(lloc, red, false) + ww * lw;
  __syncthreads();

  for (int r = tid; r < a.rv; r += 256) {
    float acc = 0.f;
    for (int s = 0; s < a.nsplit; ++s) {
      const float w = ws[s];
      if (w != 0.f) acc += w * a.part_acc[((base + s) * a.Hq + j) * a.rv_pad16 + r];
    }
    ahat[r] = acc;
  }
  __syncthreads();

  const int c = tid & 127, half = tid >> 7;
  const BT* bv = (const BT*)a.bv + g * a.d + c;
  float o = 0.f;
  for (int r = half; r < a.rv; r += 2) o += ahat[r] * to_f32(bv[(size_t)r * a.D]);
  red[tid] = o;
  __syncthreads();
  if (half == 0) {
    o = red[tid] + red[tid + 128];
    if (ww != 0.f) o += ww * wp[c];
    o = (lstar == 0.f) ? 0.f : o / lstar;   // 0 only for a sequence with no tokens; NaN stays NaN
    ((OT*)a.out)[((size_t)b * a.Hq + j) * a.d + c] = from_f32<OT>(o);
  }
}

// ---------------------------------------------------------------------------------------------
// Host launch
// ---------------------------------------------------------------------------------------------
template <int KS, int RB, int LT>
static hipError_t launch_decode_kernel(const DecodeArgs& args, int grid, int lds, hipStream_t st) {
  static bool attr_set[64] = {false};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < 64 && !attr_set[dev]) {
    e = hipFuncSetAttribute((const void*)lr_decode<KS, RB, LT>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            kLdsBytes);
    if (e != hipSuccess) return e;
    attr_set[dev] = true;
  }
  hipLaunchKernelGGL((lr_decode<KS, RB, LT>), dim3(grid), dim3(kDecodeThreads), lds, st, args);
  return hipGetLastError();
}

template <int LT>
static hipError_t dispatch_decode(const DecodePlan& p, const DecodeArgs& args, int grid, hipStream_t st) {
  const int ks = p.nks <= 8 ? 8 : (p.nks <= 12 ? 12 : 16);
  const int rbw = (p.nrb + 3) / 4;
  const int rb = rbw <= 4 ? 4 : (rbw <= 6 ? 6 : 8);
#define LR_CASE(K, R) \
  if (ks == K && rb == R) return launch_decode_kernel<K, R, LT>(args, grid, p.lds_bytes, st);
  LR_CASE(8, 4) LR_CASE(8, 6) LR_CASE(8, 8)
  LR_CASE(12, 4) LR_CASE(12, 6) LR_CASE(12, 8)
  LR_CASE(16, 4) LR_CASE(16, 6) LR_CASE(16, 8)
#undef LR_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodePlan& p, const lr_layer_cache* c, const void* q, void* out,
                         int out_dtype, void* ws, hipStream_t st, hipEvent_t ev_begin, hipEvent_t ev_end) {
  unsigned char* w = (unsigned char*)ws;
  __bf16* qt = (__bf16*)(w + p.off_qt);
  const float scale = p.sm_scale * kLog2e;

  // 1. fold
  {
    dim3 grid((p.rk_pad + 63) / 64, p.B);
    const size_t lds = (size_t)p.Hq * p.d * sizeof(float);
    if (p.latent == LR_F32)
      hipLaunchKernelGGL(lr_fold<float>, grid, dim3(256), lds, st, (const float*)q, (const float*)c->bk, qt,
                         p.Hq, p.Hkv, p.d, p.D, p.rk, p.rk_pad, scale);
    else
      hipLaunchKernelGGL(lr_fold<__bf16>, grid, dim3(256), lds, st, (const __bf16*)q, (const __bf16*)c->bk, qt,
                         p.Hq, p.Hkv, p.d, p.D, p.rk, p.rk_pad, scale);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }

  // 2. latent decode (+ window workgroups)
  DecodeArgs a;
  a.zk = (const unsigned char*)c->zk;
  a.zv = (const unsigned char*)c->zv;
  a.zkq = (const unsigned char*)c->zk_qp;
  a.zvq = (const unsigned char*)c->zv_qp;
  a.qt = qt;
  a.lat_len = c->lat_len;
  a.win_len = c->win_len;
  a.part_ml = (float*)(w + p.off_ml);
  a.part_acc = (float*)(w + p.off_acc);
  a.win_part = (float*)(w + p.off_win);
  a.q = q;
  a.kwin = (const __bf16*)c->kwin;
  a.vwin = (const __bf16*)c->vwin;
  a.t_cap = p.t_cap;
  a.row_bytes_k = p.row_bytes_k;
  a.row_bytes_v = p.row_bytes_v;
  a.qp_bytes_k = p.qp_bytes_k;
  a.qp_bytes_v = p.qp_bytes_v;
  a.rk = p.rk;
  a.rv = p.rv;
  a.rk_pad = p.rk_pad;
  a.nks = p.nks;
  a.nrb = p.nrb;
  a.rv_pad16 = p.rv_pad16;
  a.nsplit = p.nsplit;
  a.split_tokens = p.split_tokens;
  a.max_len = p.max_len;
  a.Hq = p.Hq;
  a.Hkv = p.Hkv;
  a.d = p.d;
  a.D = p.D;
  a.window = p.window;
  a.wscale = scale;
  a.n_win_blocks = p.window > 0 ? p.B : 0;
  a.stage_bytes = p.stage_bytes;
  a.zv_off = p.zv_off;
  a.qpk_off = p.qpk_off;
  a.qpv_off = p.qpv_off;
  a.nst = p.nst;
  const int grid = a.n_win_blocks + p.B * p.nsplit;
  hipError_t e;
  if (ev_begin && (e = hipEventRecord(ev_begin, st)) != hipSuccess) return e;
  if (p.latent == LR_F32) e = dispatch_decode<LT_F32>(p, a, grid, st);
  else e = dispatch_decode<LT_BF16>(p, a, grid, st);
  if (e != hipSuccess) return e;
  if (ev_end && (e = hipEventRecord(ev_end, st)) != hipSuccess) return e;

  // 3. combine + up-projection
  CombineArgs ca;
  ca.part_ml = a.part_ml;
  ca.part_acc = a.part_acc;
  ca.win_part = a.win_part;
  ca.bv = c->bv;
  ca.out = out;
  ca.Hq = p.Hq;
  ca.Hkv = p.Hkv;
  ca.d = p.d;
  ca.D = p.D;
  ca.rv = p.rv;
  ca.rv_pad16 = p.rv_pad16;
  ca.nsplit = p.nsplit;
  ca.window = p.window;
  const size_t lds = (size_t)(p.nsplit + p.rv_pad16 + 256) * sizeof(float);
  const dim3 cgrid(p.B * p.Hq);
  const bool f32b = p.latent == LR_F32;
  const bool f32o = out_dtype == LR_F32;
  if (f32b && f32o) hipLaunchKernelGGL((lr_combine<float, float>), cgrid, dim3(256), lds, st, ca);
  else if (f32b) hipLaunchKernelGGL((lr_combine<float, __bf16>), cgrid, dim3(256), lds, st, ca);
  else if (f32o) hipLaunchKernelGGL((lr_combine<__bf16, float>), cgrid, dim3(256), lds, st, ca);
  else hipLaunchKernelGGL((lr_combine<__bf16, __bf16>), cgrid, dim3(256), lds, st, ca);
  return hipGetLastError();
}

}  // namespace lr
