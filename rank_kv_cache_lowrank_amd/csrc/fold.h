// The fold q~ = (sm_scale * log2 e) q Bk[:, g(j)]^T on the matrix cores (bf16 queries and bases),
// shared by the decode launcher and the decode-step launch that runs it beside the append.
#pragma once

#include "device_common.h"
#include "internal.h"

namespace lr {

__device__ __forceinline__ bf16x8 zero_bf16x8() {
  return __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
}

// Position of latent index k inside an int4 row as the decode kernel dequantises it: within each
// block of 8 indices the order is 0, 4, 1, 5, 2, 6, 3, 7.
__device__ __forceinline__ int i4_pos(int k) { return (k & ~7) | ((k & 3) << 1) | ((k >> 2) & 1); }

constexpr int kFoldD = 128;     // head_dim handled by the fold (validated on the host)

// ---------------------------------------------------------------------------------------------
// Fold on the matrix cores for bf16 q and Bk: one wave per (16-column block of latent indices k,
// KV head g, nq consecutive query sequences; the Bk operand is loaded once for all of them).
// C[h, k] = q[b, g*grp + h, :] . Bk[k, g*d : g*d+d] over d = 128 in four 16x16x32 bf16 steps
// (A = 16 query heads of the group, zero past grp; B = Bk^T; C row h = 4*lg + i, column
// k = lane % 16), scaled by sm_scale * log2 e.
// F32OUT (int4 latents): float32 output at the dequantised tiles' block order; the decode
// kernel picks each head's power-of-two scale and rounds to fp16. Else bf16 output.
// ---------------------------------------------------------------------------------------------
struct FoldArgs {
  const __bf16* q;          // (float32 for the VALU fold)
  const __bf16* bk;
  void* qt;
  int Hq, Hkv, D, rk, rk_pad;
  float scale;
  int nseq, nq;
};

template <bool F32OUT>
__device__ __forceinline__ void fold_body(const FoldArgs& f, int bx, int by, int bz) {
  const __bf16* __restrict__ q = f.q;
  const __bf16* __restrict__ bk = f.bk;
  void* __restrict__ qt = f.qt;
  const int Hq = f.Hq, Hkv = f.Hkv, D = f.D, rk = f.rk, rk_pad = f.rk_pad, nseq = f.nseq, nq = f.nq;
  const float scale = f.scale;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, lg = lane >> 4, li = lane & 15;
  const int blk = bx * 4 + wave;
  const int g = by;
  const int grp = Hq / Hkv;
  if (blk >= (rk_pad >> 4)) return;
  const int k = blk * 16 + li;
  bf16x8 bop[4];
  {
    const __bf16* brow = bk + (size_t)k * D + g * kFoldD + lg * 8;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) bop[ks] = k < rk ? *(const bf16x8*)(brow + ks * 32) : zero_bf16x8();
  }
  const int pos = F32OUT ? i4_pos(k) : k;
  for (int b = bz * nq; b < min(nseq, (bz + 1) * nq); ++b) {
  for (int h0 = 0; h0 < grp; h0 += 16) {
    const int hl = h0 + li;
    const __bf16* qrow = q + ((size_t)b * Hq + g * grp + hl) * kFoldD + lg * 8;
    bf16x8 aop[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) aop[ks] = hl < grp ? *(const bf16x8*)(qrow + ks * 32) : zero_bf16x8();
    f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop[ks], bop[ks], c, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = h0 + 4 * lg + i;
      if (h < grp) {
        const size_t o = ((size_t)b * kHeadsPad + g * grp + h) * rk_pad + pos;
        if constexpr (F32OUT) ((float*)qt)[o] = c[i] * scale;
        else ((__bf16*)qt)[o] = (__bf16)(c[i] * scale);
      }
    }
  }
  if (g == 0) {   // query heads past Hq: zero rows
    for (int h = Hq + lg; h < kHeadsPad; h += 4) {
      const size_t o = ((size_t)b * kHeadsPad + h) * rk_pad + k;
      if constexpr (F32OUT) ((float*)qt)[o] = 0.f;
      else ((__bf16*)qt)[o] = (__bf16)0.f;
    }
  }
  }
}


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

// ---------------------------------------------------------------------------------------------
// Fold with float32 queries and bases (float32 latents), on the VALU:
// qt[b][j][k] = scale * sum_c q[b][j][c] * Bk[k][g(j)*d + c], bf16, zero-padded.
// Workgroup (bx, by = g, bz = b) of rk_pad/64 x Hkv x B, 256 threads: thread (hs, k) computes heads
// hs, hs+4, ... of KV head g for latent index k; its 512-byte slice of Bk row k is loaded with
// independent 16-byte loads.
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ void fold_f32_body(const FoldArgs& f, int bx, int g, int b, float* qs /* [32 x 128] LDS */) {
  const float* __restrict__ q = (const float*)f.q;
  const float* __restrict__ bk = (const float*)f.bk;
  __bf16* __restrict__ qt = (__bf16*)f.qt;
  const int Hq = f.Hq, grp = f.Hq / f.Hkv, D = f.D, rk = f.rk, rk_pad = f.rk_pad;
  const int tid = threadIdx.x;
  for (int i = tid; i < grp * kFoldD; i += 256) qs[i] = q[((size_t)b * Hq + g * grp) * kFoldD + i] * f.scale;
  __syncthreads();
  const int k = bx * 64 + (tid & 63);
  const int hs = tid >> 6;
  if (k >= rk_pad) return;
  __bf16* out = qt + (size_t)b * kHeadsPad * rk_pad + k;
  float bvals[kFoldD];
  if (k < rk) {
    const float* brow = bk + (size_t)k * D + g * kFoldD;
#pragma unroll
    for (int c = 0; c < kFoldD; c += 8) load8<float>(brow + c, bvals + c);
  }
  for (int h = hs; h < grp; h += 4) {
    float acc = 0.f;
    if (k < rk) {
      const float* qh = qs + h * kFoldD;
#pragma unroll
      for (int c = 0; c < kFoldD; ++c) acc += qh[c] * bvals[c];
    }
    out[(size_t)(g * grp + h) * rk_pad] = (__bf16)acc;
  }
  if (g == 0)
    for (int j = Hq + hs; j < kHeadsPad; j += 4) out[(size_t)j * rk_pad] = (__bf16)0.f;
}

// The first launch of a decode call (append.hip): workgroups [0, n_append) append the step's
// token (lowrank_decode_step only), [n_append, n_append + n_fold) fold the query, and the rest
// (W > 0) attend over the exact window, one per (sequence, KV head).
struct FrontPlan {
  int latent;               // lr_dtype of the latents (selects the fold and the append's bases)
  int n_append, nck, ncv;   // append workgroups and their column chunks (0 when no append)
  int n_fold, nfx, nfy;     // fold workgroups and the fold's grid extents (x, y; z follows)
  int n_win;                // window workgroups (B x Hkv, or 0)
  int window;               // W
  long long t_cap;
};
hipError_t launch_front(const FrontPlan& fp, const AppendPlan* ap, const lr_layer_cache* c, const void* k_new,
                        const void* v_new, const FoldArgs& f, float* win_part, float wscale, hipStream_t st);

}  // namespace lr
