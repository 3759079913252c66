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

// Projection + storage of every latent row this call creates.
// grid (column chunks of 64 over max(rk, rv), 2 = {K, V}, B); 512 threads = 8 waves.
// For each row: wave w accumulates z over input dims [w*D/8, (w+1)*D/8) for the chunk's 64
// columns (lane = column; the loads of P are independent and coalesced, 32 in flight per
// lane), the 8 partial sums are added in a fixed order through LDS and wave 0 stores the row.
constexpr int kAppendWaves = 8;

template <typename PT>
__global__ __launch_bounds__(kAppendWaves * 64) void lr_append_project(AppendArgs a) {
  extern __shared__ float xs[];    // [D] source row as float, then [8][64] partial sums
  const int kv = blockIdx.y, b = blockIdx.z;
  const int r = kv == 0 ? a.rk : a.rv;
  const int col0 = blockIdx.x * 64;
  if (col0 >= r) return;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  int L = a.lat_len[b];
  L = L < 0 ? 0 : (L > a.t_cap ? (int)a.t_cap : L);
  int wl = 0, n_rows;
  if (a.window > 0) {
    wl = a.win_len[b];
    wl = wl < 0 ? 0 : (wl > a.window ? a.window : wl);
    n_rows = wl + a.n_new - a.window;
    n_rows = n_rows < 0 ? 0 : n_rows;
  } else {
    n_rows = a.n_new;
  }
  const PT* P = (const PT*)(kv == 0 ? a.pk : a.pv);
  const __bf16* xnew = kv == 0 ? a.k_new : a.v_new;
  const __bf16* win = kv == 0 ? a.kwin : a.vwin;
  unsigned char* zbase = kv == 0 ? a.zk : a.zv;
  uint32_t* qbase = kv == 0 ? a.zkq : a.zvq;
  const int ld = kv == 0 ? a.ld_k : a.ld_v;
  const int rb = row_bytes_of(a.latent, r, ld);
  const int G = (r + kGroup - 1) / kGroup;
  const int col = col0 + lane;
  const int dq = a.D / kAppendWaves;
  float* x = xs;
  float* zpart = xs + a.D;

  for (int e = 0; e < n_rows; ++e) {
    const __bf16* src = (a.window > 0) ? win + ((size_t)b * a.window + (L + e) % a.window) * a.D
                                       : xnew + ((size_t)b * a.n_new + e) * a.D;
    __syncthreads();
    for (int c = tid; c < a.D; c += kAppendWaves * 64) x[c] = (float)src[c];
    __syncthreads();
    float z = 0.f;
    if (col < r) {
      const PT* pc = P + (size_t)(wave * dq) * r + col;
      const float* xw = x + wave * dq;
      int c = 0;
      for (; c + 32 <= dq; c += 32) {
        float pv[32];
#pragma unroll
        for (int u = 0; u < 32; ++u) pv[u] = to_f32(pc[(size_t)(c + u) * r]);
#pragma unroll
        for (int u = 0; u < 32; ++u) z += xw[c + u] * pv[u];
      }
      for (; c < dq; ++c) z += xw[c] * to_f32(pc[(size_t)c * r]);
    }
    zpart[wave * 64 + lane] = z;
    __syncthreads();
    if (wave == 0) {
      z = 0.f;
#pragma unroll
      for (int w = 0; w < kAppendWaves; ++w) z += zpart[w * 64 + lane];
      const long long row = (long long)L + e;
      if (a.z_debug && col < r)
        a.z_debug[((size_t)b * a.n_new + e) * (a.rk + a.rv) + (kv == 0 ? 0 : a.rk) + col] = z;
      if (row < a.t_cap)
        store_chunk(a.latent, z, lane, col0, r, zbase + ((size_t)b * a.t_cap + row) * rb,
                    qbase ? qbase + ((size_t)b * a.t_cap + row) * G : nullptr);
    }
  }
}

// Window ring write and length update; runs after the projection kernel on the same stream.
__global__ __launch_bounds__(256) void lr_append_finish(AppendArgs a) {
  const int b = blockIdx.x;
  int L = a.lat_len[b];
  L = L < 0 ? 0 : (L > a.t_cap ? (int)a.t_cap : L);
  if (a.window > 0) {
    int wl = a.win_len[b];
    wl = wl < 0 ? 0 : (wl > a.window ? a.window : wl);
    const int vec = a.D / 8;
    for (int i = threadIdx.x; i < a.n_new * vec; i += blockDim.x) {
      const int t = i / vec, c = i - t * vec;
      const int slot = (L + wl + t) % a.window;
      const size_t dst = ((size_t)b * a.window + slot) * a.D + c * 8;
      const size_t src = ((size_t)b * a.n_new + t) * a.D + c * 8;
      *(u32x4*)(a.kwin + dst) = *(const u32x4*)(a.k_new + src);
      *(u32x4*)(a.vwin + dst) = *(const u32x4*)(a.v_new + src);
    }
    if (threadIdx.x == 0) {
      int n_ev = wl + a.n_new - a.window;
      n_ev = n_ev < 0 ? 0 : n_ev;
      long long nl = (long long)L + n_ev;
      a.lat_len[b] = (int)(nl > a.t_cap ? a.t_cap : nl);
      a.win_len[b] = wl + a.n_new > a.window ? a.window : wl + a.n_new;
    }
  } else if (threadIdx.x == 0) {
    long long nl = (long long)L + a.n_new;
    a.lat_len[b] = (int)(nl > a.t_cap ? a.t_cap : nl);
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

hipError_t launch_append(const AppendPlan& p, const lr_layer_cache* c, const void* k_new,
                         const void* v_new, float* z_debug, hipStream_t st) {
  AppendArgs a;
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
  const int rmax = p.rk > p.rv ? p.rk : p.rv;
  dim3 grid((rmax + 63) / 64, 2, p.B);
  const size_t lds = (size_t)(p.D + kAppendWaves * 64) * sizeof(float);
  if (p.latent == LR_F32) hipLaunchKernelGGL(lr_append_project<float>, grid, dim3(kAppendWaves * 64), lds, st, a);
  else hipLaunchKernelGGL(lr_append_project<__bf16>, grid, dim3(kAppendWaves * 64), lds, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(lr_append_finish, dim3(p.B), dim3(256), 0, st, a);
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
