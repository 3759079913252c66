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

// One launch does the whole append: projection, storage, window ring and lengths.
//
// grid (nck + ncv, ceil(B / 16)): workgroup (x, y) owns latent columns 64c .. 64c + 63 of K (x < nck,
// c = x) or of V (c = x - nck) for the 16 sequences 16y .. 16y + 15, and every row this call stores
// for them. Per row index e (0 .. n_new - 1): the 16 sequences' source rows (the new token, or the
// window token being evicted) are staged in LDS as the bf16 A operand, z [16 seq, 64 col] = X P on
// the matrix cores (bf16 bases: 16x16x32 with float32 accumulation, wave w owning columns
// 16w .. 16w + 15; float32 bases: the VALU, float32 throughout), and wave w stores the rows of
// sequences 4w .. 4w + 3 (store_chunk: bf16 rounding, or int4 quantisation of the 2 groups).
//
// The window ring and the lengths may change only after every workgroup of a sequence has read
// them (and the evicted ring slots). Each workgroup, once its reads of a sequence are done, adds
// 1 << 24 to lat_len[b]: the word carries the arrival count in bits 24..30 while L stays in bits
// 0..23 (t_cap < 2^24, so every reader masks it off). The workgroup that sees the count reach
// gx - 1 is the last one: it writes the new tokens into the ring and the final lengths, which
// also clears the count. So a call leaves the lengths clean, and no buffer needs clearing first.
constexpr int kAppendSeqs = 16;       // sequences per workgroup (the matrix-core M)
constexpr int kAppendCols = 64;       // latent columns per workgroup (4 waves x 16; 2 int4 groups)
constexpr int kAppendK = 512;         // source-row chunk along D staged at a time
constexpr int kAppendLdsX = kAppendK * 2 + 16;   // LDS row stride of a staged source chunk (bytes)
constexpr unsigned kLenMask = 0x00FFFFFFu;
constexpr unsigned kArrival = 1u << 24;

__device__ __forceinline__ int clamp_len(int32_t raw, long long cap) {
  const unsigned v = (unsigned)raw & kLenMask;
  return (int)((long long)v > cap ? cap : (long long)v);
}

template <bool F32P>
__device__ __forceinline__ void append_body(const AppendArgs& a, int nck, int ncv, int bx, int by) {
  __shared__ __attribute__((aligned(16))) unsigned char xs[kAppendSeqs * kAppendLdsX];   // staged rows
  __shared__ float zt[kAppendSeqs][kAppendCols];                                         // z tile
  __shared__ int s_len[kAppendSeqs], s_win[kAppendSeqs], s_rows[kAppendSeqs], s_last[kAppendSeqs];
  const int tid = threadIdx.x, lane = tid & 63, lg = lane >> 4, li = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int gx = nck + ncv;
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

  // ---- every load that does not depend on the lengths goes out first, with the lengths' own
  // loads, so that the workgroup waits for one memory round trip instead of several in a row.
  int32_t raw_len = 0, raw_win = 0;
  if (tid < nseq) {
    raw_len = a.lat_len[b0 + tid];
    if (W > 0) raw_win = a.win_len[b0 + tid];
  }
  // P operand of this wave's 16 columns for one K chunk of up to 512 (bf16 bases). The projection
  // is stored rank-major, pt[i][k] = P[k][i], so lane (li, lg) loads its 8 values
  // pt[col0 + 16 wave + li][kc + 32 ks + 8 lg .. +7] as one 16-byte load (columns past the rank
  // read as 0). With one chunk (D <= 512) it is loaded once for all row indices.
  const int pcol = col0 + 16 * wave + li;
  bf16x8 pop[F32P ? 1 : kAppendK / 32];
  auto load_pop = [&](int kc, int nks) {
    if constexpr (!F32P) {
      const __bf16* pt = (const __bf16*)(kv == 0 ? a.pk : a.pv) + (size_t)(pcol < r ? pcol : r - 1) * D + kc + 8 * lg;
#pragma unroll
      for (int ks = 0; ks < kAppendK / 32; ++ks) {
        pop[ks] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
        if (ks < nks && pcol < r) pop[ks] = *(const bf16x8*)(pt + 32 * ks);
      }
    }
  };
  if (one_chunk) load_pop(0, D / 32);
  // Source rows of one row index e and K chunk: item i = tid + 256 u is granule c of sequence sq
  // (zeros for sequences without a row e). The new token's row (W == 0) does not depend on the
  // lengths, the evicted window slot does.
  constexpr int XV = kAppendSeqs * (kAppendK / 8) / 256;
  u32x4 xv[XV];
  auto load_x = [&](int e, int kc, int kw, bool from_new) {
#pragma unroll
    for (int u = 0; u < XV; ++u) {
      const int i = tid + 256 * u;
      const int sq = i / (kw / 8), c = i - sq * (kw / 8);
      xv[u] = u32x4{0u, 0u, 0u, 0u};
      if (sq < nseq) {
        const int b = b0 + sq;
        if (from_new) {
          if (e < a.n_new) xv[u] = *(const u32x4*)(xnew + ((size_t)b * a.n_new + e) * D + kc + c * 8);
        } else if (e < s_rows[sq]) {
          xv[u] = *(const u32x4*)(win + ((size_t)b * W + (s_len[sq] + e) % W) * D + kc + c * 8);
        }
      }
    }
  };
  const bool pre_x = W == 0 && one_chunk;
  if (pre_x) load_x(0, 0, D, true);
  // A decode step (W > 0, one new token): the new rows the last workgroup of a sequence writes into
  // the ring are loaded now too.
  const bool pre_new = W > 0 && a.n_new == 1 && one_chunk;
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
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int kc = 0; kc < D; kc += kAppendK) {
      const int kw = min(kAppendK, D - kc);                    // a multiple of 128
      if (!(pre_x && e == 0)) load_x(e, kc, kw, W == 0);
#pragma unroll
      for (int u = 0; u < XV; ++u) {
        const int i = tid + 256 * u;
        const int sq = i / (kw / 8), c = i - sq * (kw / 8);
        if (sq < kAppendSeqs) *(u32x4*)(xs + sq * kAppendLdsX + c * 16) = xv[u];
      }
      if (!one_chunk) load_pop(kc, kw / 32);
      __syncthreads();
      if constexpr (!F32P) {
        // C[seq 4 lg + i][col li] of this wave's 16 columns (two accumulation chains)
        const unsigned char* xr = xs + li * kAppendLdsX + lg * 16;
#pragma unroll
        for (int ks = 0; ks < kAppendK / 32; ks += 2) {
          if (ks < kw / 32) {
            c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(const bf16x8*)(xr + ks * 64), pop[ks], c0, 0, 0, 0);
            c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(const bf16x8*)(xr + ks * 64 + 64), pop[ks + 1], c1, 0,
                                                         0, 0);
          }
        }
      } else {
        // float32 bases: thread (column lane, sequences 4 wave .. 4 wave + 3), float32 throughout
        const int col = col0 + lane;
        const float* pt = (const float*)(kv == 0 ? a.pk : a.pv) + (size_t)(col < r ? col : r - 1) * D + kc;
        for (int k = 0; k < kw; ++k) {
          const float pv = pt[k];
#pragma unroll
          for (int s4 = 0; s4 < 4; ++s4)
            acc[s4] += (float)*(const __bf16*)(xs + (4 * wave + s4) * kAppendLdsX + k * 2) * pv;
        }
      }
      __syncthreads();                                         // xs is restaged
    }
    if constexpr (!F32P) {
#pragma unroll
      for (int i = 0; i < 4; ++i) zt[4 * lg + i][16 * wave + li] = c0[i] + c1[i];
    } else {
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) zt[4 * wave + s4][lane] = col0 + lane < r ? acc[s4] : 0.f;
    }
    __syncthreads();
    // store: wave w writes the rows of sequences 4w .. 4w + 3 (lane = column)
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      const int sq = 4 * wave + s4;
      if (sq < nseq && e < s_rows[sq]) {                       // wave-uniform
        const int b = b0 + sq;
        const float z = zt[sq][lane];
        const long long row = (long long)s_len[sq] + e;
        if (a.z_debug && col0 + lane < r)
          a.z_debug[((size_t)b * a.n_new + e) * (a.rk + a.rv) + (kv == 0 ? 0 : a.rk) + col0 + lane] = z;
        if (row < a.t_cap)
          store_chunk(a.latent, z, lane, col0, r, zbase + ((size_t)b * a.t_cap + row) * rb,
                      qbase ? qbase + ((size_t)b * a.t_cap + row) * G : nullptr);
      }
    }
    __syncthreads();                                           // zt is reused
  }

  // arrivals: this workgroup's reads of its sequences are done (the barrier above)
  if (tid < nseq) {
    const unsigned old = atomicAdd((unsigned*)&a.lat_len[b0 + tid], kArrival);
    s_last[tid] = ((old >> 24) & 0x7Fu) == (unsigned)(gx - 1) ? 1 : 0;
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
  append_body<F32P>(a, nck, ncv, blockIdx.x, blockIdx.y);
}

// A decode step's first launch: the append's workgroups [0, nck + ncv) x ceil(B / 16) (as lr_append,
// flattened) and the fold's workgroups after them. The fold reads only the query and the key basis,
// so it does not depend on the append (the decode step's window is attended in the combine).
template <bool F32OUT>
__global__ __launch_bounds__(256) void lr_step_front(AppendArgs a, int nck, int ncv, int n_append, FoldArgs f,
                                                     int nfx, int nfy) {
  const int x = blockIdx.x;
  if (x < n_append) {
    append_body<false>(a, nck, ncv, x % (nck + ncv), x / (nck + ncv));
  } else {
    const int y = x - n_append;
    fold_body<F32OUT>(f, y % nfx, (y / nfx) % nfy, y / (nfx * nfy));
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
  const dim3 grid(nck + ncv, (p.B + kAppendSeqs - 1) / kAppendSeqs);
  if (p.latent == LR_F32) hipLaunchKernelGGL(lr_append<true>, grid, dim3(256), 0, st, a, nck, ncv);
  else hipLaunchKernelGGL(lr_append<false>, grid, dim3(256), 0, st, a, nck, ncv);
  return hipGetLastError();
}

hipError_t launch_step_front(const AppendPlan& p, const lr_layer_cache* c, const void* k_new, const void* v_new,
                             const FoldArgs& f, int nfx, int nfy, int nfold, bool i4, hipStream_t st) {
  AppendArgs a;
  append_args(p, c, k_new, v_new, nullptr, a);
  const int nck = (p.rk + kAppendCols - 1) / kAppendCols, ncv = (p.rv + kAppendCols - 1) / kAppendCols;
  const int n_append = (nck + ncv) * ((p.B + kAppendSeqs - 1) / kAppendSeqs);
  const dim3 grid(n_append + nfold);
  if (i4) hipLaunchKernelGGL(lr_step_front<true>, grid, dim3(256), 0, st, a, nck, ncv, n_append, f, nfx, nfy);
  else hipLaunchKernelGGL(lr_step_front<false>, grid, dim3(256), 0, st, a, nck, ncv, n_append, f, nfx, nfy);
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
