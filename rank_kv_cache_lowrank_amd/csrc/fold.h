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
constexpr int kFoldQB = 4;      // query sequences of a fold wave whose loads are in flight together
constexpr int kAppendCols = 32; // latent columns of one append workgroup (one int4 group)

// ---------------------------------------------------------------------------------------------
// Lengths. A standalone append (lowrank_kv_append) counts its workgroups' arrivals in bits 24..30
// of the length word while it runs, so readers mask the length to bits 0..23 (t_cap < 2^24).
// A decode step (lowrank_decode_step) keeps the words as they were before the step until its last
// launch: the front's append and window workgroups and the latent kernel read the old words and
// derive the lengths after the step (step_lens); one combine workgroup per sequence then writes
// the new token into the ring and the new lengths (step_finish), after every reader is done.
// ---------------------------------------------------------------------------------------------
constexpr unsigned kLenMask = 0x00FFFFFFu;

__device__ __forceinline__ int clamp_len(int32_t raw, long long cap) {
  const unsigned v = (unsigned)raw & kLenMask;
  return (int)((long long)v > cap ? cap : (long long)v);
}

// One new token per sequence: L, wl the lengths before the step (latent rows, window slots);
// rows the latent rows it adds (the evicted window token, or with no window the token itself);
// L_new, wl_new the lengths after it. The same rules as a one-token lowrank_kv_append.
struct StepLens {
  int L, wl, rows, L_new, wl_new;
};

__device__ __forceinline__ StepLens step_lens(int32_t raw_len, int32_t raw_win, int W, long long t_cap) {
  StepLens s;
  s.L = clamp_len(raw_len, t_cap);
  s.wl = W > 0 ? (raw_win < 0 ? 0 : (raw_win > W ? W : raw_win)) : 0;
  s.rows = W > 0 ? (s.wl + 1 > W ? s.wl + 1 - W : 0) : 1;
  const long long nl = (long long)s.L + s.rows;
  s.L_new = (int)(nl > t_cap ? t_cap : nl);
  s.wl_new = W > 0 ? (s.wl + 1 > W ? W : s.wl + 1) : 0;
  return s;
}

struct StepFinish {
  const __bf16* k_new;      // [B][D] the step's token
  const __bf16* v_new;
  __bf16* kwin;             // [B][W][D] rings (W > 0)
  __bf16* vwin;
  int32_t* lat_len;         // NULL: not a decode step
  int32_t* win_len;
  long long t_cap;
  int D, window;
};

// Sequence b, by one whole workgroup: the token into ring slot (L + wl) mod W, then the lengths.
__device__ __forceinline__ void step_finish(const StepFinish& f, int b) {
  const StepLens s = step_lens(f.lat_len[b], f.window > 0 ? f.win_len[b] : 0, f.window, f.t_cap);
  if (f.window > 0) {
    const int slot = (s.L + s.wl) % f.window;
    for (int i = threadIdx.x; i < 2 * (f.D / 8); i += blockDim.x) {
      const int kv = i / (f.D / 8), c = i - kv * (f.D / 8);
      const __bf16* src = (kv == 0 ? f.k_new : f.v_new) + (size_t)b * f.D + c * 8;
      __bf16* dst = (kv == 0 ? f.kwin : f.vwin) + ((size_t)b * f.window + slot) * f.D + c * 8;
      *(u32x4*)dst = *(const u32x4*)src;
    }
  }
  __syncthreads();                                   // every thread has read the old lengths
  if (threadIdx.x == 0) {
    if (f.window > 0) f.win_len[b] = s.wl_new;
    f.lat_len[b] = s.L_new;
  }
}

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
  // kFoldQB query sequences at a time: their query loads are all issued before the first product
  const int bend = min(nseq, (bz + 1) * nq);
  for (int b0 = bz * nq; b0 < bend; b0 += kFoldQB) {
    for (int h0 = 0; h0 < grp; h0 += 16) {
      const int hl = h0 + li;
      bf16x8 aop[kFoldQB][4];
#pragma unroll
      for (int u = 0; u < kFoldQB; ++u) {
        const bool ok = hl < grp && b0 + u < bend;
        const __bf16* qrow = q + ((size_t)(ok ? b0 + u : 0) * Hq + g * grp + (ok ? hl : 0)) * kFoldD + lg * 8;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) aop[u][ks] = ok ? *(const bf16x8*)(qrow + ks * 32) : zero_bf16x8();
      }
#pragma unroll
      for (int u = 0; u < kFoldQB; ++u) {
        const int b = b0 + u;
        if (b >= bend) break;
        f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop[u][ks], bop[ks], c, 0, 0, 0);
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
    }
    if (g == 0) {   // query heads past Hq: zero rows
      for (int b = b0; b < min(bend, b0 + kFoldQB); ++b)
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

// Balanced token ranges of a decode call, planned on the device by one workgroup of the first
// launch (the lengths live on the device): every sequence is cut into ranges of the same Q
// tiles, Q the smallest that gives at most nwg ranges in all and at most nslot per sequence;
// sequence b takes n_b = ceil(tiles_b / Q) of them, placed in sequence order. table[4 w ..]:
// (b, slot, first token, end token) of latent workgroup w, b = -1 for a workgroup without a
// range; nrng[b] = n_b. The lengths are those the latent kernel attends (after the step's
// append in a decode step, clamped to max_len).
struct RangeArgs {
  const int32_t* lat_len;
  const int32_t* win_len;
  int* table;               // [nwg][4]
  int* nrng;                // [B]
  long long t_cap;
  int B, nwg, nslot, max_len, window, step;
};

// The first launch of a decode call (append.hip): workgroup 0 plans the balanced ranges (when
// they are on); then [n_win] workgroups attend over the exact window (W > 0), one per (sequence,
// KV head); [n_append] append the step's token (lowrank_decode_step only); the rest fold the
// query. The longest roles are dispatched first.
struct FrontPlan {
  int latent;               // lr_dtype of the latents (selects the fold and the append's bases)
  int n_append, nck, ncv;   // append workgroups and their column chunks (0 when no append)
  int n_fold, nfx, nfy;     // fold workgroups and the fold's grid extents (x, y; z follows)
  int n_win;                // window workgroups (B x Hkv, or 0)
  int window;               // W
  long long t_cap;
  int n_plan;               // 1: the range-planning workgroup runs (rng is filled in)
  RangeArgs rng;
};
hipError_t launch_front(const FrontPlan& fp, const AppendPlan* ap, const lr_layer_cache* c, const void* k_new,
                        const void* v_new, const FoldArgs& f, float* win_part, float wscale, hipStream_t st);

}  // namespace lr
