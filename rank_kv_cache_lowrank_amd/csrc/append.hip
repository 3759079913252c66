// Append path: project new (or evicted) dense K/V rows into the latent space, store them in
// the cache format, and maintain the exact recent window. Also the bulk latent store and the
// dequantisation hook.
//
// iS-KV ("iS-KV: Online Low-Rank KV Cache Compression via Block-Incremental SVD", English
// abstract): the most recent tokens stay exact while older ones are folded into the
// bounded-rank latents. TraceKV ("TraceKV: Policy-Preserving Low-Rank KV Cache Compression for
// Reasoning Vision-Language Models", abstract; ai4snews page, Synopsis): the latents may be
// 4-bit quantised. The workload projects with the caller's pseudo-inverse of the basis.
//
// int4 groups of 32 (one float16 scale and zero per group, from min-max over the group):
//   zero16 = f16(min), scale16 = f16(f32(max - min) / 15), code = clamp(rint((z - zero)/scale))
// every step one IEEE float32/float16 operation, so results are reproducible bit for bit.
#include "device_common.h"
#include "fold.h"
#include "internal.h"

#include <math.h>
#include <string.h>

namespace lr {

// One wave stores one 64-column chunk of one latent row; lane c holds z for column col0 + c.
// latent: LR_F32 / LR_BF16 store elementwise; LR_I4G32 quantises two groups of 32 (lanes 0-31
// and 32-63) and packs two codes per byte (even column in the low nibble).
__device__ __forceinline__ void store_chunk(int latent, float z, int lane, int col0, int r,
                                            unsigned char* row, uint32_t* qp_row) {
#pragma clang fp contract(off)
  const int col = col0 + lane;
  const bool valid = col < r;
  if (latent == LR_F32) {
    if (valid) ((float*)row)[col] = z;
    return;
  }
  if (latent == LR_BF16) {
    if (valid) ((__bf16*)row)[col] = (__bf16)z;
    return;
  }
  float mn = valid ? z : INFINITY;
  float mx = valid ? z : -INFINITY;
#pragma unroll
  for (int o = 1; o < 32; o <<= 1) {
    mn = fminf(mn, __shfl_xor(mn, o));
    mx = fmaxf(mx, __shfl_xor(mx, o));
  }
  const int g = col >> 5;                         // group index (col0 is a multiple of 64)
  const bool group_live = (g * kGroup) < r;       // the group has at least one real element
  unsigned code = 0;
  _Float16 z16 = (_Float16)0.f, s16 = (_Float16)0.f;
  if (group_live) {
    z16 = (_Float16)mn;
    const float range = mx - mn;
    s16 = (_Float16)(range / 15.0f);
    const float z32 = (float)z16;
    const float s32 = (float)s16;
    if (valid && s32 != 0.f) {
      float c = __builtin_rintf((z - z32) / s32);
      c = fminf(fmaxf(c, 0.f), 15.f);
      code = (unsigned)c;
    }
  }
  const unsigned hi = __shfl_xor(code, 1);        // odd neighbour's code
  if (group_live) {
    if ((lane & 1) == 0) row[g * kGroupBytes + ((lane & 31) >> 1)] = (unsigned char)(code | (hi << 4));
    if ((lane & 31) == 0) {
      const unsigned sb = __builtin_bit_cast(unsigned short, s16);
      const unsigned zb = __builtin_bit_cast(unsigned short, z16);
      qp_row[g] = sb | (zb << 16);
    }
  }
}

__device__ __forceinline__ int row_bytes_of(int latent, int r, int ld) {
  if (latent == LR_I4G32) return ((r + kGroup - 1) / kGroup) * kGroupBytes;
  return ld * (latent == LR_F32 ? 4 : 2);
}

struct AppendArgs {
  const __bf16* k_new;
  const __bf16* v_new;
  const void* pk;
  const void* pv;
  unsigned char* zk;
  unsigned char* zv;
  uint32_t* zkq;
  uint32_t* zvq;
  __bf16* kwin;
  __bf16* vwin;
  int32_t* lat_len;
  int32_t* win_len;
  float* z_debug;
  long long t_cap;
  int D, rk, rv, ld_k, ld_v, latent, window, n_new, B;
};

// One launch does the whole append of one token per sequence (a decode step's; more tokens per
// call go through lr_append_rows below): projection, storage, window ring and lengths. The row
// loop below handles any n_new, but the launcher sends only n_new == 1 here.
//
// grid (nck + ncv, ceil(B / 16)): workgroup (x, y) owns latent columns 32c .. 32c + 31 of K
// (x < nck, c = x) or of V (c = x - nck) for sequences 16y .. 16y + 15, and is the only writer
// of them. Per row index e (0 .. n_new - 1): the 16 sequences' source rows (the new token, or
// the window token being evicted) are staged in LDS as the bf16 A operand, and z [16 seq, 32 col]
// = X P runs on the matrix cores (bf16 bases: 16x16x32 with float32 accumulation; wave w owns
// columns 16 (w & 1) .. +15 over half (w >> 1) of each chunk of D, and the two halves' partial
// sums are added in LDS; float32 bases: the VALU, float32 throughout). Each wave then stores the
// rows of sequences 4w .. 4w + 3, two at a time (lanes 0-31 and 32-63; store_chunk: bf16
// rounding, or int4 quantisation of the one group).
//
// The window ring and the lengths may change only after every workgroup of a sequence has read
// them (and the evicted ring slots). Each workgroup, once its reads of a sequence are done, adds
// 1 << 24 to lat_len[b]: the word carries the arrival count in bits 24..30 while L stays in bits
// 0..23 (t_cap < 2^24, so every reader masks it off). The workgroup that sees the count reach
// gx - 1 is the last one: it writes the new tokens into the ring and the final lengths, which
// also clears the count. So a call leaves the lengths clean, and no buffer needs clearing first.
//
// Latency: the lengths go out first, each thread loading those of the sequences it stages, then
// the projection columns, then the source rows (an evicted slot's address needs its lengths; the
// projection's loads stay in flight meanwhile), so the workgroup waits for about one round trip.
constexpr int kAppendSeqs = 16;       // sequences per workgroup (the matrix-core M)
constexpr int kAppendK = 512;         // source-row chunk along D staged at a time
constexpr int kAppendLdsX = kAppendK * 2 + 16;   // LDS row stride of a staged source chunk (bytes)
constexpr unsigned kArrival = 1u << 24;
static_assert(kAppendCols == 32, "one int4 group per workgroup and row");

// readers: the workgroups that read each sequence's lengths and ring (nck + ncv), or 0 inside a
// decode step's front launch, where the lengths and the ring are left as they were and the step's
// last launch finishes them (step_finish).
constexpr int kAppendLds = kAppendSeqs * kAppendLdsX + 2 * kAppendSeqs * kAppendCols * 4 + 4 * kAppendSeqs * 4;

template <bool F32P>
__device__ __forceinline__ void append_body(const AppendArgs& a, int nck, int ncv, int bx, int by, int readers,
                                            unsigned char* smem) {
  unsigned char* xs = smem;                                                   // [16][kAppendLdsX] staged rows
  float (*zt)[kAppendSeqs][kAppendCols] =                                     // [2 halves][16][32] z partials
      (float (*)[kAppendSeqs][kAppendCols])(smem + kAppendSeqs * kAppendLdsX);
  int* s_len = (int*)(smem + kAppendSeqs * kAppendLdsX + 2 * kAppendSeqs * kAppendCols * 4);
  int* s_win = s_len + kAppendSeqs;
  int* s_rows = s_win + kAppendSeqs;
  int* s_last = s_rows + kAppendSeqs;
  const int tid = threadIdx.x, lane = tid & 63, lg = lane >> 4, li = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int cb = wave & 1, kh = wave >> 1;                    // column block, half of the K chunk
  const int kv = bx < nck ? 0 : 1;
  const int col0 = (bx - (kv ? nck : 0)) * kAppendCols;
  const int r = kv == 0 ? a.rk : a.rv;
  const int b0 = by * kAppendSeqs;
  const int nseq = min(kAppendSeqs, a.B - b0);
  const int D = a.D, W = a.window;
  const __bf16* xnew = kv == 0 ? a.k_new : a.v_new;
  const __bf16* win = kv == 0 ? a.kwin : a.vwin;
  unsigned char* zbase = kv == 0 ? a.zk : a.zv;
  uint32_t* qbase = kv == 0 ? a.zkq : a.zvq;
  const int ld = kv == 0 ? a.ld_k : a.ld_v;
  const int rb = row_bytes_of(a.latent, r, ld);
  const int G = (r + kGroup - 1) / kGroup;
  const bool one_chunk = D <= kAppendK;
  constexpr int XV = kAppendSeqs * (kAppendK / 8) / 256;     // staged 16-byte granules per thread
  // with one chunk, staged item i = tid + 256 u is granule c of sequence sq (D / 8 granules a row)
  auto item_seq = [&](int u, int kw) { return (tid + 256 * u) / (kw / 8); };

  // ---- 1. lengths: for the LDS copy, and (W > 0, one chunk) per thread for its staged rows
  int32_t raw_len = 0, raw_win = 0;
  if (tid < nseq) {
    raw_len = a.lat_len[b0 + tid];
    if (W > 0) raw_win = a.win_len[b0 + tid];
  }
  const bool pre_ev = W > 0 && one_chunk;
  int32_t xlen[XV], xwin[XV];
  if (pre_ev) {
#pragma unroll
    for (int u = 0; u < XV; ++u) {
      const int sq = item_seq(u, D);
      xlen[u] = sq < nseq ? a.lat_len[b0 + sq] : 0;
      xwin[u] = sq < nseq ? a.win_len[b0 + sq] : 0;
    }
  }
  // ---- 2. P operand of this wave's 16 columns over its half of one K chunk (bf16 bases). The
  // projection is stored rank-major, pt[i][k] = P[k][i], so lane (li, lg) loads its 8 values
  // pt[col0 + 16 cb + li][k0 + 32 ks + 8 lg .. +7] as one 16-byte load (columns past the rank
  // read as 0). With one chunk (D <= 512) it is loaded once for all row indices.
  const int pcol = col0 + 16 * cb + li;
  bf16x8 pop[F32P ? 1 : kAppendK / 64];
  auto load_pop = [&](int kc, int kw) {
    if constexpr (!F32P) {
      const int nks = kw / 64, k0 = kc + kh * (kw / 2);
      const __bf16* pt = (const __bf16*)(kv == 0 ? a.pk : a.pv) + (size_t)(pcol < r ? pcol : r - 1) * D + k0 + 8 * lg;
#pragma unroll
      for (int ks = 0; ks < kAppendK / 64; ++ks) {
        pop[ks] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
        if (ks < nks && pcol < r) pop[ks] = *(const bf16x8*)(pt + 32 * ks);
      }
    }
  };
  if (one_chunk) load_pop(0, D);
  // ---- 3. source rows of row index e and K chunk kc (zeros for sequences without a row e): the
  // new token's row (W == 0), or the evicted window slot (W > 0), whose slot comes from the
  // lengths (per thread for the first row of one chunk, else from LDS)
  u32x4 xv[XV];
  auto load_x = [&](int e, int kc, int kw, bool per_thread) {
#pragma unroll
    for (int u = 0; u < XV; ++u) {
      const int i = tid + 256 * u;
      const int sq = i / (kw / 8), c = i - sq * (kw / 8);
      xv[u] = u32x4{0u, 0u, 0u, 0u};
      if (sq < nseq) {
        const int b = b0 + sq;
        if (W == 0) {
          if (e < a.n_new) xv[u] = *(const u32x4*)(xnew + ((size_t)b * a.n_new + e) * D + kc + c * 8);
        } else {
          int L, rows;
          if (per_thread) {
            L = clamp_len(xlen[u], a.t_cap);
            const int wl = xwin[u] < 0 ? 0 : (xwin[u] > W ? W : xwin[u]);
            rows = wl + a.n_new - W;
          } else {
            L = s_len[sq];
            rows = s_rows[sq];
          }
          if (e < rows) xv[u] = *(const u32x4*)(win + ((size_t)b * W + (L + e) % W) * D + kc + c * 8);
        }
      }
    }
  };
  const bool pre_x = one_chunk;
  if (pre_x) load_x(0, 0, D, true);
  // the new rows the last workgroup of a sequence writes into the ring (a standalone one-token
  // append with a window)
  const bool pre_new = W > 0 && a.n_new == 1 && one_chunk && readers > 0;
  u32x4 kn[XV], vn[XV];
  if (pre_new) {
#pragma unroll
    for (int u = 0; u < XV; ++u) {
      const int i = tid + 256 * u;
      const int sq = i / (D / 8), c = i - sq * (D / 8);
      if (sq < nseq) {
        kn[u] = *(const u32x4*)(a.k_new + (size_t)(b0 + sq) * D + c * 8);
        vn[u] = *(const u32x4*)(a.v_new + (size_t)(b0 + sq) * D + c * 8);
      }
    }
  }

  if (tid < kAppendSeqs) {
    int L = 0, wl = 0, rows = 0;
    if (tid < nseq) {
      L = clamp_len(raw_len, a.t_cap);
      if (W > 0) {
        wl = raw_win < 0 ? 0 : (raw_win > W ? W : raw_win);
        rows = wl + a.n_new - W;
        rows = rows < 0 ? 0 : rows;
      } else {
        rows = a.n_new;
      }
    }
    s_len[tid] = L;
    s_win[tid] = wl;
    s_rows[tid] = rows;
    s_last[tid] = 0;
  }
  __syncthreads();
  int emax = 0;
#pragma unroll
  for (int sq = 0; sq < kAppendSeqs; ++sq) emax = max(emax, s_rows[sq]);

  for (int e = 0; e < emax; ++e) {
    f32x4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = {0.f, 0.f, 0.f, 0.f};
    float acc[2] = {0.f, 0.f};
    for (int kc = 0; kc < D; kc += kAppendK) {
      const int kw = min(kAppendK, D - kc);                    // a multiple of 128
      if (!(pre_x && e == 0)) load_x(e, kc, kw, false);
#pragma unroll
      for (int u = 0; u < XV; ++u) {
        const int i = tid + 256 * u;
        const int sq = i / (kw / 8), c = i - sq * (kw / 8);
        if (sq < kAppendSeqs) *(u32x4*)(xs + sq * kAppendLdsX + c * 16) = xv[u];
      }
      if (!one_chunk) load_pop(kc, kw);
      __syncthreads();
      if constexpr (!F32P) {
        // C[seq 4 lg + i][col li] of this wave's 16 columns over its K half (two chains)
        const unsigned char* xr = xs + li * kAppendLdsX + kh * kw + lg * 16;
#pragma unroll
        for (int ks = 0; ks < kAppendK / 64; ks += 2) {
          if (ks < kw / 64) {
            c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(const bf16x8*)(xr + ks * 64), pop[ks], c0, 0, 0, 0);
            if (ks + 1 < kw / 64)
              c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(const bf16x8*)(xr + ks * 64 + 64), pop[ks + 1], c1, 0,
                                                           0, 0);
          }
        }
      } else {
        // float32 bases: thread (column lane & 31, sequences 2 (tid >> 5), +1), float32 throughout
        const int cl = tid & 31, s2 = 2 * (tid >> 5);
        const int col = col0 + cl;
        const float* pt = (const float*)(kv == 0 ? a.pk : a.pv) + (size_t)(col < r ? col : r - 1) * D + kc;
        for (int k = 0; k < kw; ++k) {
          const float pv = pt[k];
#pragma unroll
          for (int s1 = 0; s1 < 2; ++s1)
            acc[s1] += (float)*(const __bf16*)(xs + (s2 + s1) * kAppendLdsX + k * 2) * pv;
        }
      }
      __syncthreads();                                         // xs is restaged
    }
    if constexpr (!F32P) {
#pragma unroll
      for (int i = 0; i < 4; ++i) zt[kh][4 * lg + i][16 * cb + li] = c0[i] + c1[i];
    } else {
      const int cl = tid & 31, s2 = 2 * (tid >> 5);
#pragma unroll
      for (int s1 = 0; s1 < 2; ++s1) {
        zt[0][s2 + s1][cl] = col0 + cl < r ? acc[s1] : 0.f;
        zt[1][s2 + s1][cl] = 0.f;
      }
    }
    __syncthreads();
    // store: wave w writes the rows of sequences 4w .. 4w + 3, two per pass (lane = column + 32 x
    // which of the two)
#pragma unroll
    for (int p2 = 0; p2 < 2; ++p2) {
      const int sq = 4 * wave + 2 * p2 + (lane >> 5);
      const int cl = lane & 31;
      if (sq < nseq && e < s_rows[sq]) {                       // uniform over each 32-lane half
        const int b = b0 + sq;
        const float z = zt[0][sq][cl] + zt[1][sq][cl];
        const long long row = (long long)s_len[sq] + e;
        if (a.z_debug && col0 + cl < r)
          a.z_debug[((size_t)b * a.n_new + e) * (a.rk + a.rv) + (kv == 0 ? 0 : a.rk) + col0 + cl] = z;
        if (row < a.t_cap)
          store_chunk(a.latent, z, cl, col0, r, zbase + ((size_t)b * a.t_cap + row) * rb,
                      qbase ? qbase + ((size_t)b * a.t_cap + row) * G : nullptr);
      }
    }
    __syncthreads();                                           // zt is reused
  }

  if (readers == 0) return;
  // arrivals: this workgroup's reads of its sequences are done (the barrier above)
  if (tid < nseq) {
    const unsigned old = atomicAdd((unsigned*)&a.lat_len[b0 + tid], kArrival);
    s_last[tid] = ((old >> 24) & 0x7Fu) == (unsigned)(readers - 1) ? 1 : 0;
  }
  __syncthreads();
  // the last workgroup of a sequence: new tokens into the ring, then the final lengths
  if (W > 0) {
    if (pre_new) {
#pragma unroll
      for (int u = 0; u < XV; ++u) {
        const int i = tid + 256 * u;
        const int sq = i / (D / 8), c = i - sq * (D / 8);
        if (sq < nseq && s_last[sq]) {
          const size_t dst = ((size_t)(b0 + sq) * W + (s_len[sq] + s_win[sq]) % W) * D + c * 8;
          *(u32x4*)(a.kwin + dst) = kn[u];
          *(u32x4*)(a.vwin + dst) = vn[u];
        }
      }
    } else {
      const int vec = D / 8;
      for (int i = tid; i < kAppendSeqs * a.n_new * vec; i += 256) {
        const int sq = i / (a.n_new * vec);
        const int rest = i - sq * a.n_new * vec;
        const int t = rest / vec, c = rest - t * vec;
        if (sq < nseq && s_last[sq]) {
          const int b = b0 + sq;
          const int slot = (s_len[sq] + s_win[sq] + t) % W;
          const size_t dst = ((size_t)b * W + slot) * D + c * 8;
          const size_t src = ((size_t)b * a.n_new + t) * D + c * 8;
          *(u32x4*)(a.kwin + dst) = *(const u32x4*)(a.k_new + src);
          *(u32x4*)(a.vwin + dst) = *(const u32x4*)(a.v_new + src);
        }
      }
    }
  }
  if (tid < nseq && s_last[tid]) {
    const int b = b0 + tid;
    const long long L = s_len[tid];
    if (W > 0) {
      const long long nl = L + s_rows[tid];
      a.win_len[b] = s_win[tid] + a.n_new > W ? W : s_win[tid] + a.n_new;
      a.lat_len[b] = (int)(nl > a.t_cap ? a.t_cap : nl);
    } else {
      const long long nl = L + a.n_new;
      a.lat_len[b] = (int)(nl > a.t_cap ? a.t_cap : nl);
    }
  }
}

template <bool F32P>
__global__ __launch_bounds__(256) void lr_append(AppendArgs a, int nck, int ncv) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  append_body<F32P>(a, nck, ncv, blockIdx.x, blockIdx.y, nck + ncv, smem);
}

// ---------------------------------------------------------------------------------------------
// Bulk append (n_new > 1, e.g. storing a prefill chunk), two launches:
//   lr_append_rows    one matrix-core product over the flattened rows f = b * n_new + e of the
//                     call: workgroup (x, y) owns latent columns 32c .. 32c + 31 of K or V (as
//                     above) for rows 16y .. 16y + 15, whatever sequences they belong to. Row
//                     (b, e) is the e-th token of the stream to leave for the latents: the new
//                     token e (W == 0); with a window, the window token in slot (L + e) mod W
//                     while e < wl, after them (a call of more than W tokens) new token e - wl,
//                     for e < rows_b = wl + n_new - W. It is stored as latent row L + e. The
//                     lengths and the ring are only read.
//   lr_append_finish  one workgroup per sequence, after every read: the last min(n_new, W) new
//                     tokens into the ring (token t in slot (L + wl + t) mod W) and the lengths
//                     after the call.
// The same arithmetic per row as the one-launch path (the same K halves, chains and rounding), so
// the stored rows do not depend on which path stored them.
// ---------------------------------------------------------------------------------------------
template <bool F32P>
__global__ __launch_bounds__(256) void lr_append_rows(AppendArgs a, int nck, int ncv) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  unsigned char* xs = smem;                                                   // [16][kAppendLdsX] staged rows
  float (*zt)[kAppendSeqs][kAppendCols] =                                     // [2 halves][16][32] z partials
      (float (*)[kAppendSeqs][kAppendCols])(smem + kAppendSeqs * kAppendLdsX);
  const int bx = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, lg = lane >> 4, li = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int cb = wave & 1, kh = wave >> 1;
  const int kv = bx < nck ? 0 : 1;
  const int col0 = (bx - (kv ? nck : 0)) * kAppendCols;
  const int r = kv == 0 ? a.rk : a.rv;
  const int D = a.D, W = a.window, n_new = a.n_new;
  const long long nrows = (long long)a.B * n_new;
  const long long f0 = (long long)blockIdx.y * kAppendSeqs;
  const __bf16* xnew = kv == 0 ? a.k_new : a.v_new;
  const __bf16* win = kv == 0 ? a.kwin : a.vwin;
  unsigned char* zbase = kv == 0 ? a.zk : a.zv;
  uint32_t* qbase = kv == 0 ? a.zkq : a.zvq;
  const int ld = kv == 0 ? a.ld_k : a.ld_v;
  const int rb = row_bytes_of(a.latent, r, ld);
  const int G = (r + kGroup - 1) / kGroup;
  // (L, wl, rows) of flattened row f's sequence, and whether the row exists (e < rows)
  auto row_info = [&](long long f, int& b, int& e, int& L, int& wl, bool& live) {
    live = false;
    b = 0;
    e = 0;
    L = 0;
    wl = 0;
    if (f >= nrows) return;
    b = (int)(f / n_new);
    e = (int)(f - (long long)b * n_new);
    L = clamp_len(a.lat_len[b], a.t_cap);
    int rows = n_new;
    if (W > 0) {
      const int raw = a.win_len[b];
      wl = raw < 0 ? 0 : (raw > W ? W : raw);
      rows = wl + n_new - W;
    }
    live = e < rows;
  };
  const int pcol = col0 + 16 * cb + li;
  bf16x8 pop[F32P ? 1 : kAppendK / 64];
  u32x4 xv[4];
  f32x4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = {0.f, 0.f, 0.f, 0.f};
  float acc[2] = {0.f, 0.f};
  for (int kc = 0; kc < D; kc += kAppendK) {
    const int kw = min(kAppendK, D - kc);                      // a multiple of 128
    // lengths of the rows this thread stages first, then P (its loads stay in flight while the
    // lengths give the evicted slots' addresses), then the source rows
    int xb[4], xe[4], xL[4], xw[4];
    bool xlive[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int sq = (tid + 256 * u) / (kw / 8);
      row_info(sq < kAppendSeqs ? f0 + sq : nrows, xb[u], xe[u], xL[u], xw[u], xlive[u]);
    }
    if constexpr (!F32P) {
      const int nks = kw / 64, k0 = kc + kh * (kw / 2);
      const __bf16* pt = (const __bf16*)(kv == 0 ? a.pk : a.pv) + (size_t)(pcol < r ? pcol : r - 1) * D + k0 + 8 * lg;
#pragma unroll
      for (int ks = 0; ks < kAppendK / 64; ++ks) {
        pop[ks] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
        if (ks < nks && pcol < r) pop[ks] = *(const bf16x8*)(pt + 32 * ks);
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = tid + 256 * u;
      const int c = i - (i / (kw / 8)) * (kw / 8);
      xv[u] = u32x4{0u, 0u, 0u, 0u};
      if (xlive[u]) {
        const bool from_ring = W > 0 && xe[u] < xw[u];
        const __bf16* src = from_ring ? win + ((size_t)xb[u] * W + (xL[u] + xe[u]) % W) * D
                                      : xnew + ((size_t)xb[u] * n_new + (xe[u] - xw[u])) * D;
        xv[u] = *(const u32x4*)(src + kc + c * 8);
      }
    }
    if (kc > 0) __syncthreads();                               // xs of the previous chunk consumed
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = tid + 256 * u;
      const int sq = i / (kw / 8), c = i - sq * (kw / 8);
      if (sq < kAppendSeqs) *(u32x4*)(xs + sq * kAppendLdsX + c * 16) = xv[u];
    }
    __syncthreads();
    if constexpr (!F32P) {
      const unsigned char* xr = xs + li * kAppendLdsX + kh * kw + lg * 16;
#pragma unroll
      for (int ks = 0; ks < kAppendK / 64; ks += 2) {
        if (ks < kw / 64) {
          c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(const bf16x8*)(xr + ks * 64), pop[ks], c0, 0, 0, 0);
          if (ks + 1 < kw / 64)
            c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(const bf16x8*)(xr + ks * 64 + 64), pop[ks + 1], c1, 0, 0, 0);
        }
      }
    } else {
      const int cl = tid & 31, s2 = 2 * (tid >> 5);
      const int col = col0 + cl;
      const float* pt = (const float*)(kv == 0 ? a.pk : a.pv) + (size_t)(col < r ? col : r - 1) * D + kc;
      for (int k = 0; k < kw; ++k) {
        const float pv = pt[k];
#pragma unroll
        for (int s1 = 0; s1 < 2; ++s1) acc[s1] += (float)*(const __bf16*)(xs + (s2 + s1) * kAppendLdsX + k * 2) * pv;
      }
    }
  }
  if constexpr (!F32P) {
#pragma unroll
    for (int i = 0; i < 4; ++i) zt[kh][4 * lg + i][16 * cb + li] = c0[i] + c1[i];
  } else {
    const int cl = tid & 31, s2 = 2 * (tid >> 5);
#pragma unroll
    for (int s1 = 0; s1 < 2; ++s1) {
      zt[0][s2 + s1][cl] = col0 + cl < r ? acc[s1] : 0.f;
      zt[1][s2 + s1][cl] = 0.f;
    }
  }
  __syncthreads();
  // store: wave w writes rows 4w .. 4w + 3, two per pass (lane = column + 32 x which of the two)
#pragma unroll
  for (int p2 = 0; p2 < 2; ++p2) {
    const int sq = 4 * wave + 2 * p2 + (lane >> 5);
    const int cl = lane & 31;
    int b, e, L, wl;
    bool live;
    row_info(f0 + sq, b, e, L, wl, live);
    if (live) {                                                // uniform over each 32-lane half
      const float z = zt[0][sq][cl] + zt[1][sq][cl];
      const long long row = (long long)L + e;
      if (a.z_debug && col0 + cl < r)
        a.z_debug[((size_t)b * n_new + e) * (a.rk + a.rv) + (kv == 0 ? 0 : a.rk) + col0 + cl] = z;
      if (row < a.t_cap)
        store_chunk(a.latent, z, cl, col0, r, zbase + ((size_t)b * a.t_cap + row) * rb,
                    qbase ? qbase + ((size_t)b * a.t_cap + row) * G : nullptr);
    }
  }
}

// grid (B): the new tokens of sequence b into the ring, then its lengths (every reader of them,
// the rows launch, has finished).
__global__ __launch_bounds__(256) void lr_append_finish(AppendArgs a) {
  const int b = blockIdx.x, tid = threadIdx.x;
  const int W = a.window, D = a.D, n_new = a.n_new;
  const int L = clamp_len(a.lat_len[b], a.t_cap);
  int wl = 0, rows = n_new;
  if (W > 0) {
    const int raw = a.win_len[b];
    wl = raw < 0 ? 0 : (raw > W ? W : raw);
    rows = wl + n_new - W;
    rows = rows < 0 ? 0 : rows;
    // only the last W tokens stay exact (each slot is written once: no two threads race on it)
    const int t0 = n_new > W ? n_new - W : 0;
    const int vec = D / 8;
    for (int i = tid; i < (n_new - t0) * vec; i += 256) {
      const int t = t0 + i / vec, c = i - (i / vec) * vec;
      const size_t dst = ((size_t)b * W + (L + wl + t) % W) * D + c * 8;
      const size_t src = ((size_t)b * n_new + t) * D + c * 8;
      *(u32x4*)(a.kwin + dst) = *(const u32x4*)(a.k_new + src);
      *(u32x4*)(a.vwin + dst) = *(const u32x4*)(a.v_new + src);
    }
  }
  __syncthreads();                                             // every thread has read the lengths
  if (tid == 0) {
    const long long nl = (long long)L + rows;
    if (W > 0) a.win_len[b] = wl + n_new > W ? W : wl + n_new;
    a.lat_len[b] = (int)(nl > a.t_cap ? a.t_cap : nl);
  }
}

// ---------------------------------------------------------------------------------------------
// Exact window of a decode step (iS-KV abstract: the most recent tokens stay exact), one workgroup
// per (sequence b, KV head g), float32 on the VALU: every head j of the group attends over the live
// window slots with base-2 scores (sm_scale * log2 e folded into the query), and the workgroup
// writes (O unnormalised, m, l) per head for the combine.
// In lowrank_decode_step the window is the one after this step's append, read in the same launch
// as the append: positions L' .. L' + wl' - 1 with L' = L + evicted, wl' = min(wl + 1, W), the
// last being the new token, taken from k_new / v_new; the others are ring slots the append does
// not write. Such a workgroup is one of the sequence's readers in the append's arrival count, and
// if it arrives last it writes the new token into the ring and the final lengths.
// Heads in batches of 8; slots in rounds of 128: thread (u = tid / 2, h = tid % 2) forms half of
// slot u's score (64 dims) for each head, thread (c8 = tid % 16, sg = tid / 16) accumulates
// columns 8 c8 .. +7 over slots 8 sg .. +7 (the value rows are loaded with the key rows, before the
// scores are known); one running max per head.
// ---------------------------------------------------------------------------------------------
struct WinArgs {
  const void* q;            // [B][Hq][d], float32 or bf16
  float* win_part;          // [B][Hq][d + 2]
  int Hq, Hkv;
  float wscale;
  int step;                 // the window after the step's append (lowrank_decode_step): the ring
                            // as it was, without the evicted slot, plus the new token
};

constexpr int kWinHeads = 8;

constexpr int kWinValuLds = (kWinHeads * kFoldD + kWinHeads * 128 + 4 * kWinHeads + 4 * kWinHeads * kFoldD +
                             4 * kWinHeads) * 4 + 16;

template <typename QT>
__device__ void window_body(const WinArgs& w, const AppendArgs& a, int blk, unsigned char* smem) {
  float (*wq)[kFoldD] = (float (*)[kFoldD])smem;                                 // [8][128]
  float (*wsc)[128] = (float (*)[128])(smem + kWinHeads * kFoldD * 4);          // [8][128]
  float (*wmx)[kWinHeads] = (float (*)[kWinHeads])((unsigned char*)wsc + kWinHeads * 128 * 4);   // [4][8]
  float (*wred)[kWinHeads][kFoldD] = (float (*)[kWinHeads][kFoldD])((unsigned char*)wmx + 4 * kWinHeads * 4);
  float (*wl4)[kWinHeads] = (float (*)[kWinHeads])((unsigned char*)wred + 4 * kWinHeads * kFoldD * 4);
  const int grp = w.Hq / w.Hkv, D = a.D, W = a.window;
  const int g = blk % w.Hkv, b = blk / w.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int u = tid >> 1, h2 = tid & 1, c8 = tid & 15, sg = tid >> 4;
  const int L = clamp_len(a.lat_len[b], a.t_cap);
  int wl = a.win_len[b];
  wl = wl < 0 ? 0 : (wl > W ? W : wl);
  int Lw = L, wlw = wl, n_ev = 0;
  if (w.step) {
    n_ev = wl + 1 > W ? wl + 1 - W : 0;
    Lw = L + n_ev;
    wlw = wl + 1 > W ? W : wl + 1;
  }
  // source of window position index t (0 .. wlw - 1) of head g: a ring slot, or the new token
  auto row = [&](const __bf16* ring, const __bf16* xnew, int t) -> const __bf16* {
    if (w.step && t == wlw - 1) return xnew + (size_t)b * D + g * kFoldD;
    return ring + ((size_t)b * W + (Lw + t) % W) * D + g * kFoldD;
  };
  for (int h0 = 0; h0 < grp; h0 += kWinHeads) {
    const int nh = min(kWinHeads, grp - h0);
    __syncthreads();                                  // wq / wred of the previous batch consumed
    for (int i = tid; i < nh * kFoldD; i += 256)
      wq[i / kFoldD][i % kFoldD] =
          to_f32(((const QT*)w.q)[((size_t)b * w.Hq + g * grp + h0) * kFoldD + i]) * w.wscale;
    float m[kWinHeads], lt[kWinHeads], acc[kWinHeads][8];
#pragma unroll
    for (int hh = 0; hh < kWinHeads; ++hh) {
      m[hh] = -INFINITY;
      lt[hh] = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[hh][e] = 0.f;
    }
    for (int c0 = 0; c0 < wlw; c0 += 128) {
      u32x4 kr[8], vr[8];
      const bool kval = c0 + u < wlw;
      const __bf16* kp = row(a.kwin, a.k_new, kval ? c0 + u : 0) + 64 * h2;
#pragma unroll
      for (int i = 0; i < 8; ++i) kr[i] = kval ? *(const u32x4*)(kp + 8 * i) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int t = c0 + 8 * sg + i;
        vr[i] = t < wlw ? *(const u32x4*)(row(a.vwin, a.v_new, t) + 8 * c8) : u32x4{0u, 0u, 0u, 0u};
      }
      __syncthreads();                                // wq visible; the previous round's wsc read
      float sv[kWinHeads];
#pragma unroll
      for (int hh = 0; hh < kWinHeads; ++hh) {
        float part = 0.f;
        if (hh < nh) {
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const bf16x8 k8 = __builtin_bit_cast(bf16x8, kr[i]);
#pragma unroll
            for (int e = 0; e < 8; ++e) part += wq[hh][64 * h2 + 8 * i + e] * (float)k8[e];
          }
        }
        const float sc = part + __shfl_xor(part, 1);
        sv[hh] = kval ? ((sc != sc) ? INFINITY : sc) : -INFINITY;   // NaN: this head only
        if (h2 == 0) wsc[hh][u] = sv[hh];
        float mx = sv[hh];
        for (int o = 2; o < 64; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
        if (lane == 0) wmx[wave][hh] = mx;
      }
      __syncthreads();
#pragma unroll
      for (int hh = 0; hh < kWinHeads; ++hh) {
        const float mx = fmaxf(fmaxf(wmx[0][hh], wmx[1][hh]), fmaxf(wmx[2][hh], wmx[3][hh]));
        const float mnew = fmaxf(m[hh], mx);
        const float alpha = (m[hh] == -INFINITY) ? 0.f : fast_exp2(m[hh] - mnew);
        const bool live = mnew != -INFINITY;
        // running l over this thread's slot (score threads), running O over its 8 slots
        lt[hh] = lt[hh] * alpha + ((h2 == 0 && live) ? fast_exp2(sv[hh] - mnew) : 0.f);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[hh][e] *= alpha;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float p = live ? fast_exp2(wsc[hh][8 * sg + i] - mnew) : 0.f;
          const bf16x8 v8 = __builtin_bit_cast(bf16x8, vr[i]);
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[hh][e] += p * (float)v8[e];
        }
        m[hh] = mnew;
      }
    }
    // reduce: O over the 16 slot groups (4 per wave by shuffles, then the 4 waves through LDS),
    // l over the score threads
#pragma unroll
    for (int hh = 0; hh < kWinHeads; ++hh) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float v = acc[hh][e];
        v += __shfl_xor(v, 16);
        v += __shfl_xor(v, 32);
        if (lane < 16) wred[wave][hh][8 * c8 + e] = v;
      }
      float lv = lt[hh];
      for (int o = 1; o < 64; o <<= 1) lv += __shfl_xor(lv, o);
      if (lane == 0) wl4[wave][hh] = lv;
    }
    __syncthreads();
    for (int i = tid; i < nh * kFoldD; i += 256) {
      const int hh = i / kFoldD, c = i % kFoldD;
      float* wp = w.win_part + ((size_t)b * w.Hq + g * grp + h0 + hh) * (kFoldD + 2);
      wp[c] = ((wred[0][hh][c] + wred[1][hh][c]) + wred[2][hh][c]) + wred[3][hh][c];
      if (c == 0) {
        wp[kFoldD] = m[hh];
        wp[kFoldD + 1] = ((wl4[0][hh] + wl4[1][hh]) + wl4[2][hh]) + wl4[3][hh];
      }
    }
  }
}

// The same on the matrix cores, for bf16 queries and at most 16 heads per KV head: the grp heads
// are the 16 rows of the products (zero past grp). The ring is walked in physical slot order:
// 16-slot tiles of slots 16 t .. 16 t + 15, wave v taking the tiles t = v mod 4 that hold live
// slots, each staged in the wave's own part of LDS: scores from the 16x16x32 bf16 product (16
// slots x 16 heads), a base-2 online softmax, values from the 16x16x16 product through the
// transpose read; the four waves' (O, m, l) are merged through LDS. Slot s holds window position
// (s - Lw) mod W, live when that is below wlw. The order depends only on the window after the
// step, so a decode step (which reads the ring as it was, with the new token in the slot it is
// about to take) and a decode after the append add the same terms in the same order.
// A window of at most 128 slots has at most two tiles per wave: their loads go out with the
// lengths' (every slot of the ring is in bounds), and dead slots are zeroed when staged, so the
// workgroup waits for one round trip. Larger windows load each live tile when it is reached.
constexpr int kWinSlots = 16;
constexpr int kWinMfmaLds = 4 * kWinSlots * kExSK + 4 * kWinSlots * kExSV + 4 * 2 * 16 * 4 + 3 * (kExD / 16) * 64 * 16 + 16;

__device__ void window_mfma_body(const WinArgs& w, const AppendArgs& a, int blk, unsigned char* smem) {
  unsigned char* ktb = smem;                                          // [4][16 * kExSK]
  unsigned char* vtb = ktb + 4 * kWinSlots * kExSK;                   // [4][16 * kExSV]
  float* mrg_ml = (float*)(vtb + 4 * kWinSlots * kExSV);              // [4][2][16]
  f32x4* mrg_o = (f32x4*)(mrg_ml + 4 * 2 * 16);                       // [3][8][64]
  const int grp = w.Hq / w.Hkv, D = a.D, W = a.window;
  const int g = blk % w.Hkv, b = blk / w.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, lg = lane >> 4, li = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool rvalid = li < grp;
  const int ntiles = (W + kWinSlots - 1) / kWinSlots;
  const bool spec = W <= 8 * kWinSlots;                               // at most two tiles per wave
  const int32_t raw_len = a.lat_len[b];
  const int32_t raw_win = a.win_len[b];
  const __bf16* kring = a.kwin + (size_t)b * W * D + g * kExD;
  const __bf16* vring = a.vwin + (size_t)b * W * D + g * kExD;
  // slots 16 t .. 16 t + 15 of head g's slice: 16 rows x 16 granules of 16 bytes, K and V (item
  // i = lane + 64 u is row i >> 4, granule i & 15; slots past W read as 0)
  auto load_tile = [&](int t, u32x4 (&kn)[4], u32x4 (&vn)[4]) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = lane + 64 * u;
      const int s = t * kWinSlots + (i >> 4), gc = i & 15;
      kn[u] = u32x4{0u, 0u, 0u, 0u};
      vn[u] = u32x4{0u, 0u, 0u, 0u};
      if (s < W) {
        kn[u] = *(const u32x4*)(kring + (size_t)s * D + gc * 8);
        vn[u] = *(const u32x4*)(vring + (size_t)s * D + gc * 8);
      }
    }
  };
  u32x4 kA[4], vA[4], kB[4], vB[4];
  if (spec) {
    load_tile(wave, kA, vA);
    load_tile(wave + 4, kB, vB);
  }
  // the step's token, granule lane & 15 of head g's slice (every row item of a lane has that granule)
  u32x4 knew = u32x4{0u, 0u, 0u, 0u}, vnew = u32x4{0u, 0u, 0u, 0u};
  if (w.step) {
    knew = *(const u32x4*)(a.k_new + (size_t)b * D + g * kExD + (lane & 15) * 8);
    vnew = *(const u32x4*)(a.v_new + (size_t)b * D + g * kExD + (lane & 15) * 8);
  }
  // q of this lane's head as the B operand: d indices 32 ks + 8 lg .. +7
  bf16x8 qop[4];
  {
    const __bf16* qr = (const __bf16*)w.q + ((size_t)b * w.Hq + g * grp + (rvalid ? li : 0)) * kExD + lg * 8;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qop[ks] = rvalid ? *(const bf16x8*)(qr + ks * 32) : zero_bf16x8();
  }
  // the window after the step: positions 0 .. wlw - 1 in slots (Lw + t) mod W
  const int L = clamp_len(raw_len, a.t_cap);
  const int wl = raw_win < 0 ? 0 : (raw_win > W ? W : raw_win);
  int Lw = L, wlw = wl;
  if (w.step) {
    Lw = L + (wl + 1 > W ? wl + 1 - W : 0);
    wlw = wl + 1 > W ? W : wl + 1;
  }
  const int s0 = Lw % W;                                              // slot of position 0
  const int new_slot = w.step ? (Lw + wlw - 1) % W : -1;
  auto live_slot = [&](int s) {
    int t = s - s0;
    if (t < 0) t += W;
    return s < W && t < wlw;
  };
  // live tiles: [ta0, tb0] and [ta1, tb1] (empty when a > b), in physical order
  int ta0 = 0, tb0 = -1, ta1 = 0, tb1 = -1;
  if (wlw > 0) {
    const int e = s0 + wlw - 1;                                       // last live slot, unwrapped
    if (e < W) {
      ta0 = s0 / kWinSlots;
      tb0 = e / kWinSlots;
    } else {
      ta0 = 0;
      tb0 = (e - W) / kWinSlots;
      ta1 = s0 / kWinSlots;
      tb1 = ntiles - 1;
      if (ta1 <= tb0 + 1) {                                           // the two runs touch: one
        tb0 = tb1;
        ta1 = 0;
        tb1 = -1;
      }
    }
  }
  auto tile_live = [&](int t) { return (t >= ta0 && t <= tb0) || (t >= ta1 && t <= tb1); };

  float m = -INFINITY, lsum = 0.f;
  f32x4 acc[kExD / 16];
#pragma unroll
  for (int j = 0; j < kExD / 16; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  unsigned char* kw = ktb + wave * kWinSlots * kExSK;
  unsigned char* vw = vtb + wave * kWinSlots * kExSV;
  auto process = [&](int t, const u32x4 (&kn)[4], const u32x4 (&vn)[4]) {
    const int k0 = t * kWinSlots;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = lane + 64 * u;
      const int r = i >> 4, gc = i & 15;
      const int s = k0 + r;
      const bool lv = live_slot(s);
      const u32x4 kx = s == new_slot ? knew : kn[u];
      const u32x4 vx = s == new_slot ? vnew : vn[u];
      *(u32x4*)(kw + r * kExSK + gc * 16) = lv ? kx : u32x4{0u, 0u, 0u, 0u};
      *(u32x4*)(vw + r * kExSV + gc * 16) = lv ? vx : u32x4{0u, 0u, 0u, 0u};
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // the tile is in LDS before it is read
    // scores S^T[slot k0 + 4 lg + i][head li]
    f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
    const unsigned char* krow = kw + li * kExSK + lg * 16;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(const bf16x8*)(krow + ks * 64), qop[ks], sacc, 0, 0, 0);
    float v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float x = sacc[i] * w.wscale;
      v[i] = live_slot(k0 + 4 * lg + i) ? ((x != x) ? INFINITY : x) : -INFINITY;
    }
    const float mx = wave_max_lg(fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])));
    const float mnew = fmaxf(m, mx);
    if (__builtin_amdgcn_ballot_w64(mnew != m) != 0) {
      const float alpha = (m == -INFINITY) ? 0.f : fast_exp2(m - mnew);
      lsum *= alpha;
#pragma unroll
      for (int j = 0; j < kExD / 16; ++j) acc[j] *= alpha;
      m = mnew;
    }
    const bool live = m != -INFINITY;
    bf16x4 pb;
    float ps = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const __bf16 pv = (__bf16)(live ? fast_exp2(v[i] - m) : 0.f);
      pb[i] = pv;
      ps += (float)pv;
    }
    lsum += ps;
    const unsigned char* vbase = vw + (4 * lg + (li >> 2)) * kExSV + (li & 3) * 8;
#pragma unroll
    for (int j = 0; j < kExD / 16; ++j)
      acc[j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(v_operand_tr(vbase + j * 32), pb, acc[j], 0, 0, 0);
  };
  if (spec) {
    if (tile_live(wave)) process(wave, kA, vA);
    if (tile_live(wave + 4)) process(wave + 4, kB, vB);
  } else {
    for (int run = 0; run < 2; ++run) {
      const int ta = run == 0 ? ta0 : ta1, tb = run == 0 ? tb0 : tb1;
      for (int t = ta + ((wave - ta) % 4 + 4) % 4; t <= tb; t += 4) {
        load_tile(t, kA, vA);
        process(t, kA, vA);
      }
    }
  }
  const float l = wave_sum_lg(lsum);
  // merge the four waves' partials into wave 0
  if (lg == 0) {
    mrg_ml[(wave * 2) * 16 + li] = m;
    mrg_ml[(wave * 2 + 1) * 16 + li] = l;
  }
  if (wave > 0) {
#pragma unroll
    for (int j = 0; j < kExD / 16; ++j) mrg_o[((wave - 1) * (kExD / 16) + j) * 64 + lane] = acc[j];
  }
  __syncthreads();
  if (wave == 0 && rvalid) {
    float ms = -INFINITY;
#pragma unroll
    for (int v2 = 0; v2 < 4; ++v2) ms = fmaxf(ms, mrg_ml[(v2 * 2) * 16 + li]);
    float wb[4], lt = 0.f;
#pragma unroll
    for (int v2 = 0; v2 < 4; ++v2) {
      const float mw = mrg_ml[(v2 * 2) * 16 + li];
      wb[v2] = (mw == -INFINITY) ? 0.f : fast_exp2(mw - ms);
      lt += mrg_ml[(v2 * 2 + 1) * 16 + li] * wb[v2];
    }
    float* wp = w.win_part + ((size_t)b * w.Hq + g * grp + li) * (kExD + 2);
#pragma unroll
    for (int j = 0; j < kExD / 16; ++j) {
      f32x4 o = acc[j] * wb[0];
#pragma unroll
      for (int v2 = 1; v2 < 4; ++v2) o += mrg_o[((v2 - 1) * (kExD / 16) + j) * 64 + lane] * wb[v2];
      *(f32x4*)(wp + j * 16 + 4 * lg) = o;
    }
    if (lg == 0) {
      wp[kExD] = ms;
      wp[kExD + 1] = lt;
    }
  }
}

constexpr int kFrontLds = kWinMfmaLds > kAppendLds ? (kWinMfmaLds > kWinValuLds ? kWinMfmaLds : kWinValuLds)
                                                   : (kAppendLds > kWinValuLds ? kAppendLds : kWinValuLds);
static_assert(kFrontLds >= kHeadsPad * kFoldD * 4, "the float32 fold's query tile fits");

// ---------------------------------------------------------------------------------------------
// Range planning of a decode call (one wave of the first launch; RangeArgs in fold.h). Exact
// integer results, the same on every run, and no workgroup barrier: lane l loads sequences l,
// l + 64, ... into LDS; the search for the smallest Q whose ranges fit the grid gives every lane
// its own candidate per round (64 candidates spread over the interval, a ballot picks the first
// that fits, so the interval shrinks 64-fold per round and no cross-lane reduction is chained).
// Totals and prefixes come from broadcast LDS reads, 16 in flight at a time, and each lane
// writes the table entries of its own sequences' ranges.
// ---------------------------------------------------------------------------------------------
constexpr int kPlanLds = 2 * kBalMaxSeqs * 4;
static_assert(kFrontLds >= kPlanLds, "the range plan's tables fit");

// ceil(t / q) for 0 <= t < 2^21, 1 <= q < 2^21: a float quotient (within one of the answer) and
// one exact integer correction each way
__device__ __forceinline__ int plan_cdiv(int t, int q, float rq) {
  const int n = t + q - 1;
  int k = (int)((float)n * rq);
  k -= (k * q > n) ? 1 : 0;
  k += ((k + 1) * q <= n) ? 1 : 0;
  return k;
}

// f(k, tl[k]) for k < B in ascending order, every lane the same: 16-byte broadcast reads, 16 in
// flight per round trip (tl is padded with zeros to a multiple of 64 entries)
template <typename F>
__device__ __forceinline__ void plan_scan(const int* tl, int B, F&& f) {
  for (int k0 = 0; k0 < B; k0 += 64) {
    int4 v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = *(const int4*)(tl + k0 + 4 * i);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int k = k0 + 4 * i;
      if (k < B) {
        f(k, v[i].x);
        f(k + 1, v[i].y);
        f(k + 2, v[i].z);
        f(k + 3, v[i].w);
      }
    }
  }
}

__device__ void range_plan_body(const RangeArgs& r, unsigned char* smem) {
  if (threadIdx.x >= 64) return;
  int* tl = (int*)smem;                  // [B padded to 64] tiles, then ranges, of each sequence
  int* lens = tl + kBalMaxSeqs;          // [B] tokens attended
  const int lane = threadIdx.x, B = r.B;
  const int Bp = (B + 63) & ~63;
  auto attended = [&](int b) {           // tokens the latent kernel attends for sequence b
    int L = r.step ? step_lens(r.lat_len[b], r.window > 0 ? r.win_len[b] : 0, r.window, r.t_cap).L_new
                   : r.lat_len[b];
    return L < 0 ? 0 : (L > r.max_len ? r.max_len : L);
  };
  // the loads of all of a lane's sequences go out together; tiles and tokens into LDS, zeros
  // past B (a sequence with no tiles has no ranges)
  for (int b = lane; b < Bp; b += 64) {
    const int L = b < B ? attended(b) : 0;
    lens[b] = L;
    tl[b] = (L + kTileTokens - 1) / kTileTokens;
  }
  int tmax = 0, tsum = 0;
  plan_scan(tl, B, [&](int, int t) {
    tmax = max(tmax, t);
    tsum += t;
  });
  // the smallest Q in [lo, hi] with sum_b ceil(tiles_b / Q) <= nwg; at Q = tmax the sum is the
  // number of non-empty sequences, at most B <= nwg, so the last lane's candidate always fits
  // and the sum never increases with Q (tiles < 2^20: t_cap < 2^24)
  int lo = max(1, max((tmax + r.nslot - 1) / r.nslot, (tsum + r.nwg - 1) / r.nwg));
  int hi = max(1, tmax);
  if (lo > hi) lo = hi;
  while (lo < hi) {
    const int step = (hi - lo + 64) / 64;
    const int qc = min(lo + (lane + 1) * step - 1, hi);   // lane k covers [lo + k step, qc]
    const float rq = __builtin_amdgcn_rcpf((float)qc);
    int c = 0;
    plan_scan(tl, B, [&](int, int t) { c += plan_cdiv(t, qc, rq); });
    const unsigned long long fits = __ballot(c <= r.nwg);
    const int k = __builtin_ctzll(fits);
    hi = min(lo + (k + 1) * step - 1, hi);
    lo = lo + k * step;
  }
  const int Q = lo;
  const int qt = Q * kTileTokens;
  // ranges per sequence (tl now holds them); each lane's sequences b = lane + 64 i take the
  // workgroups from the exclusive prefix of the ranges before them
  for (int b = lane; b < Bp; b += 64) tl[b] = (tl[b] + Q - 1) / Q;
  int pre[kBalMaxSeqs / 64] = {0}, total = 0;
  plan_scan(tl, B, [&](int k, int t) {
#pragma unroll
    for (int i = 0; i < kBalMaxSeqs / 64; ++i) pre[i] += k < lane + 64 * i ? t : 0;
    total += t;
  });
#pragma unroll
  for (int i = 0; i < kBalMaxSeqs / 64; ++i) {
    const int b = lane + 64 * i;
    if (b < B) {
      const int n = tl[b], L = lens[b];
      r.nrng[b] = n;
      for (int s = 0; s < n; ++s) {
        const int t0 = s * qt;
        *(int4*)(r.table + 4 * (pre[i] + s)) = make_int4(b, s, t0, min(t0 + qt, L));
      }
    }
  }
  for (int w = total + lane; w < r.nwg; w += 64) *(int4*)(r.table + 4 * w) = make_int4(-1, 0, 0, 0);
}

// The first launch of a decode call: [range plan] [window, W > 0] [append (a decode step only)]
// [fold], the longest roles first so that they are dispatched first. Within a decode step none of them writes
// what another reads: the append stores the new latent row at index L (which no role of this
// launch reads), the window reads the ring as it was, and the lengths are left for the step's
// last launch.
template <int LAT>
__global__ __launch_bounds__(256) void lr_front(AppendArgs a, int nck, int ncv, int n_append, FoldArgs f, int nfx,
                                                int nfy, int n_win, WinArgs w, int n_plan, RangeArgs rg) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int x = blockIdx.x - n_plan;
  if (x < 0) {
    range_plan_body(rg, smem);
  } else if (x < n_win) {
    if constexpr (LAT == LR_F32) window_body<float>(w, a, x, smem);
    else if (w.Hq / w.Hkv <= 16) window_mfma_body(w, a, x, smem);
    else window_body<__bf16>(w, a, x, smem);
  } else if (x < n_win + n_append) {
    const int y = x - n_win;
    append_body<LAT == LR_F32>(a, nck, ncv, y % (nck + ncv), y / (nck + ncv), 0, smem);
  } else {
    const int y = x - n_win - n_append;
    if constexpr (LAT == LR_F32) fold_f32_body(f, y % nfx, (y / nfx) % nfy, y / (nfx * nfy), (float*)smem);
    else fold_body<LAT == LR_I4G32>(f, y % nfx, (y / nfx) % nfy, y / (nfx * nfy));
  }
}

// Bulk store: rows [row0, row0 + n_rows) from float32 z.
// grid (ceil(n_rows / 4), 2, B); wave w handles one row, looping over 64-column chunks.
struct StoreArgs {
  const float* zk;
  const float* zv;
  unsigned char* ck;
  unsigned char* cv;
  uint32_t* qk;
  uint32_t* qv;
  long long t_cap, row0, n_rows;
  int rk, rv, ld_k, ld_v, latent;
};

__global__ __launch_bounds__(256) void lr_store(StoreArgs a) {
  const int kv = blockIdx.y, b = blockIdx.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const long long i = (long long)blockIdx.x * 4 + wave;
  if (i >= a.n_rows) return;
  const int r = kv == 0 ? a.rk : a.rv;
  const int ld = kv == 0 ? a.ld_k : a.ld_v;
  const int rb = row_bytes_of(a.latent, r, ld);
  const int G = (r + kGroup - 1) / kGroup;
  const float* src = (kv == 0 ? a.zk : a.zv) + ((size_t)b * a.n_rows + i) * r;
  const long long row = a.row0 + i;
  unsigned char* dst = (kv == 0 ? a.ck : a.cv) + ((size_t)b * a.t_cap + row) * rb;
  uint32_t* q = kv == 0 ? a.qk : a.qv;
  uint32_t* qrow = q ? q + ((size_t)b * a.t_cap + row) * G : nullptr;
  for (int col0 = 0; col0 < r; col0 += 64) {
    const int col = col0 + lane;
    const float z = col < r ? src[col] : 0.f;
    store_chunk(a.latent, z, lane, col0, r, dst, qrow);
  }
}

// Dequantisation hook: float32 values of rows [0, n_rows), the value decode feeds (before its
// bf16 operand rounding). Grid-stride over B * n_rows * r elements.
struct DequantArgs {
  const unsigned char* ck;
  const unsigned char* cv;
  const uint32_t* qk;
  const uint32_t* qv;
  float* ok;
  float* ov;
  long long t_cap, n_rows;
  int B, rk, rv, ld_k, ld_v, latent;
};

__global__ __launch_bounds__(256) void lr_dequant(DequantArgs a) {
  const int kv = blockIdx.y;
  const int r = kv == 0 ? a.rk : a.rv;
  const int ld = kv == 0 ? a.ld_k : a.ld_v;
  const int rb = row_bytes_of(a.latent, r, ld);
  const int G = (r + kGroup - 1) / kGroup;
  const unsigned char* c = kv == 0 ? a.ck : a.cv;
  const uint32_t* q = kv == 0 ? a.qk : a.qv;
  float* o = kv == 0 ? a.ok : a.ov;
  const long long total = (long long)a.B * a.n_rows * r;
  for (long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (long long)gridDim.x * blockDim.x) {
    const long long row_flat = idx / r;
    const int col = (int)(idx - row_flat * r);
    const long long b = row_flat / a.n_rows, t = row_flat - b * a.n_rows;
    const unsigned char* row = c + ((size_t)b * a.t_cap + t) * rb;
    float v;
    if (a.latent == LR_F32) {
      v = ((const float*)row)[col];
    } else if (a.latent == LR_BF16) {
      v = (float)((const __bf16*)row)[col];
    } else {
      const int g = col >> 5, k = col & 31;
      const unsigned byte = row[g * kGroupBytes + (k >> 1)];
      const unsigned code = (k & 1) ? (byte >> 4) : (byte & 15u);
      const uint32_t w = q[((size_t)b * a.t_cap + t) * G + g];
      v = dequant_one(code, half_lo(w), half_hi(w));
    }
    o[idx] = v;
  }
}

static void append_args(const AppendPlan& p, const lr_layer_cache* c, const void* k_new, const void* v_new,
                        float* z_debug, AppendArgs& a) {
  a.k_new = (const __bf16*)k_new;
  a.v_new = (const __bf16*)v_new;
  a.pk = c->pk;
  a.pv = c->pv;
  a.zk = (unsigned char*)c->zk;
  a.zv = (unsigned char*)c->zv;
  a.zkq = (uint32_t*)c->zk_qp;
  a.zvq = (uint32_t*)c->zv_qp;
  a.kwin = (__bf16*)c->kwin;
  a.vwin = (__bf16*)c->vwin;
  a.lat_len = c->lat_len;
  a.win_len = c->win_len;
  a.z_debug = z_debug;
  a.t_cap = p.t_cap;
  a.D = p.D;
  a.rk = p.rk;
  a.rv = p.rv;
  a.ld_k = p.ld_k;
  a.ld_v = p.ld_v;
  a.latent = p.latent;
  a.window = p.window;
  a.n_new = p.n_new;
  a.B = p.B;
}

hipError_t launch_append(const AppendPlan& p, const lr_layer_cache* c, const void* k_new,
                         const void* v_new, float* z_debug, hipStream_t st) {
  AppendArgs a;
  append_args(p, c, k_new, v_new, z_debug, a);
  const int nck = (p.rk + kAppendCols - 1) / kAppendCols, ncv = (p.rv + kAppendCols - 1) / kAppendCols;
  if (p.n_new == 1) {
    const dim3 grid(nck + ncv, (p.B + kAppendSeqs - 1) / kAppendSeqs);
    if (p.latent == LR_F32) hipLaunchKernelGGL(lr_append<true>, grid, dim3(256), kAppendLds, st, a, nck, ncv);
    else hipLaunchKernelGGL(lr_append<false>, grid, dim3(256), kAppendLds, st, a, nck, ncv);
    return hipGetLastError();
  }
  const long long nrows = (long long)p.B * p.n_new;
  const dim3 grid(nck + ncv, (unsigned)((nrows + kAppendSeqs - 1) / kAppendSeqs));
  if (p.latent == LR_F32) hipLaunchKernelGGL(lr_append_rows<true>, grid, dim3(256), kAppendLds, st, a, nck, ncv);
  else hipLaunchKernelGGL(lr_append_rows<false>, grid, dim3(256), kAppendLds, st, a, nck, ncv);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(lr_append_finish, dim3(p.B), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_front(const FrontPlan& fp, const AppendPlan* ap, const lr_layer_cache* c, const void* k_new,
                        const void* v_new, const FoldArgs& f, float* win_part, float wscale, hipStream_t st) {
  AppendArgs a;
  if (ap) {
    append_args(*ap, c, k_new, v_new, nullptr, a);
  } else {      // no append: the window workgroups read only the ring and the lengths
    memset(&a, 0, sizeof(a));
    a.kwin = (__bf16*)c->kwin;
    a.vwin = (__bf16*)c->vwin;
    a.lat_len = c->lat_len;
    a.win_len = c->win_len;
    a.D = f.D;
    a.window = fp.window;
    a.t_cap = fp.t_cap;
  }
  WinArgs w;
  w.q = f.q;
  w.win_part = win_part;
  w.Hq = f.Hq;
  w.Hkv = f.Hkv;
  w.wscale = wscale;
  w.step = ap != nullptr && fp.n_win > 0;
  const dim3 grid(fp.n_plan + fp.n_append + fp.n_fold + fp.n_win);
  if (grid.x == 0) return hipSuccess;
  if (fp.latent == LR_F32)
    hipLaunchKernelGGL(lr_front<LR_F32>, grid, dim3(256), kFrontLds, st, a, fp.nck, fp.ncv, fp.n_append, f, fp.nfx, fp.nfy,
                       fp.n_win, w, fp.n_plan, fp.rng);
  else if (fp.latent == LR_I4G32)
    hipLaunchKernelGGL(lr_front<LR_I4G32>, grid, dim3(256), kFrontLds, st, a, fp.nck, fp.ncv, fp.n_append, f, fp.nfx,
                       fp.nfy, fp.n_win, w, fp.n_plan, fp.rng);
  else
    hipLaunchKernelGGL(lr_front<LR_BF16>, grid, dim3(256), kFrontLds, st, a, fp.nck, fp.ncv, fp.n_append, f, fp.nfx,
                       fp.nfy, fp.n_win, w, fp.n_plan, fp.rng);
  return hipGetLastError();
}

hipError_t launch_store(const AppendPlan& p, const lr_layer_cache* c, int64_t row0, int64_t n_rows,
                        const float* zk, const float* zv, hipStream_t st) {
  if (n_rows == 0) return hipSuccess;
  StoreArgs a;
  a.zk = zk;
  a.zv = zv;
  a.ck = (unsigned char*)c->zk;
  a.cv = (unsigned char*)c->zv;
  a.qk = (uint32_t*)c->zk_qp;
  a.qv = (uint32_t*)c->zv_qp;
  a.t_cap = p.t_cap;
  a.row0 = row0;
  a.n_rows = n_rows;
  a.rk = p.rk;
  a.rv = p.rv;
  a.ld_k = p.ld_k;
  a.ld_v = p.ld_v;
  a.latent = p.latent;
  dim3 grid((unsigned)((n_rows + 3) / 4), 2, p.B);
  hipLaunchKernelGGL(lr_store, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_dequant(const AppendPlan& p, const lr_layer_cache* c, int64_t n_rows, float* zk_out,
                          float* zv_out, hipStream_t st) {
  if (n_rows == 0) return hipSuccess;
  DequantArgs a;
  a.ck = (const unsigned char*)c->zk;
  a.cv = (const unsigned char*)c->zv;
  a.qk = (const uint32_t*)c->zk_qp;
  a.qv = (const uint32_t*)c->zv_qp;
  a.ok = zk_out;
  a.ov = zv_out;
  a.t_cap = p.t_cap;
  a.n_rows = n_rows;
  a.B = p.B;
  a.rk = p.rk;
  a.rv = p.rv;
  a.ld_k = p.ld_k;
  a.ld_v = p.ld_v;
  a.latent = p.latent;
  const long long total = (long long)p.B * n_rows * (p.rk > p.rv ? p.rk : p.rv);
  long long blocks = (total + 255) / 256;
  if (blocks > 65535) blocks = 65535;
  hipLaunchKernelGGL(lr_dequant, dim3((unsigned)blocks, 2), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace lr
