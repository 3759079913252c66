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
//   lr_combine  one workgroup per (sequence, head): merges the ranges and the exact-keys partial
//               and up-projects through Bv[:, g(j)].
// int4 latents (groups of 32 with an fp16 scale and zero): the loads bring the codes and the
// scale/zero words into a raw LDS ring, the producer waves dequantise each tile into an fp16
// tile of the same geometry, and the matrix-core products run in fp16 (fp32 accumulate) against
// an fp16 folded query that carries a per-head power-of-two scale.
#include <hip/hip_ext.h>

#include "device_common.h"
#include "fold.h"
#include "internal.h"

#include <math.h>
#include <string.h>

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
  int copy_k, copy_v;       // bytes of each stored row the LDS ring holds
  int nr, raw_stage;        // int4: raw stages in the ring and their size in bytes
  int qpb;                  // query tokens per stored sequence: 1 (decode) or the chunk (prefill);
                            // query sequence sq reads the latents of stored sequence sq / qpb
  const __bf16* kchunk;     // prefill: the chunk's exact rows [B][qpb][D]; NULL for decode
  const __bf16* vchunk;
  int step;                 // a decode step: lat_len / win_len still hold the lengths before the
                            // step's token, and the latent rows attended are step_lens().L_new
  const int* rng;           // balanced ranges (RangeArgs table, written by the first launch) or NULL
};


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
  // row already points at this lane's 8-element slice of K step 0; k0 = 32 * K step
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


// Value operand of the 16x16x16 bf16 product: lane (lg, li) holds latent index rv of tokens
// 4*lg .. 4*lg+3 (K index = token), the rows the score tile's C layout gives this lane.
template <int LT, int SV>
__device__ __forceinline__ bf16x4 v_operand4(const unsigned char* base, int col_bytes) {
  // base = stage value region + 4*lg rows + 2*li (bf16) / 4*li (f32); col_bytes = 32*rb (bf16)
  if constexpr (LT == LT_F32) {
    bf16x4 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = (__bf16)(*(const float*)(base + e * SV + col_bytes));
    return r;
  } else {
    unsigned short h[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) h[e] = *(const unsigned short*)(base + e * SV + col_bytes);
    u32x2 w;
    w[0] = (unsigned)h[0] | ((unsigned)h[1] << 16);
    w[1] = (unsigned)h[2] | ((unsigned)h[3] << 16);
    return __builtin_bit_cast(bf16x4, w);
  }
}

typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __attribute__((__vector_size__(4 * sizeof(_Float16)))) _Float16 f16x4;
typedef __attribute__((__vector_size__(2 * sizeof(_Float16)))) _Float16 f16x2;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;

// Matrix-core products on 16-bit operands held as raw bits: bf16 for float32/bf16 latents,
// fp16 for the dequantised int4 tiles.
template <int LT>
__device__ __forceinline__ f32x4 mfma_k(bf16x8 a, bf16x8 b, f32x4 c) {
  if constexpr (LT == LT_I4)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                  0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
template <int LT>
__device__ __forceinline__ f32x4 mfma_v(bf16x4 a, bf16x4 b, f32x4 c) {
  if constexpr (LT == LT_I4)
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a), __builtin_bit_cast(f16x4, b), c,
                                                 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// Eight int4 codes (w: index i in bits 4i..4i+3) -> eight fp16 values zhat = fma(code, scale,
// zero), one rounding. Output dword i holds indices i and i + 4 (block order 0,4,1,5,2,6,3,7).
// A code lands in the mantissa of an fp16 number whose value is then exactly magic + code: from
// bits 0-3 of a half word under the exponent of 1024 (mantissa unit 1), from bits 4-7 under
// that of 64 (mantissa unit 1/16). So w and w >> 8, each masked twice (one three-operand
// and-or apiece), place all eight codes, and one packed subtraction of the magic recovers them.
// The masks and exponents arrive in registers (0x000F000F, 0x00F000F0, 0x64006400, 0x54005400).
__device__ __forceinline__ u32x4 dequant8_f16(unsigned w, f16x2 s2, f16x2 z2, unsigned m0, unsigned m1,
                                              unsigned e0, unsigned e1) {
  const unsigned w8 = w >> 8;
  const f16x2 k0 = {(_Float16)1024.f, (_Float16)1024.f}, k1 = {(_Float16)64.f, (_Float16)64.f};
  const f16x2 c0 = __builtin_bit_cast(f16x2, (w & m0) | e0) - k0;    // indices 0, 4
  const f16x2 c1 = __builtin_bit_cast(f16x2, (w & m1) | e1) - k1;    // 1, 5
  const f16x2 c2 = __builtin_bit_cast(f16x2, (w8 & m0) | e0) - k0;   // 2, 6
  const f16x2 c3 = __builtin_bit_cast(f16x2, (w8 & m1) | e1) - k1;   // 3, 7
  u32x4 o;
  o[0] = __builtin_bit_cast(unsigned, __builtin_elementwise_fma(c0, s2, z2));
  o[1] = __builtin_bit_cast(unsigned, __builtin_elementwise_fma(c1, s2, z2));
  o[2] = __builtin_bit_cast(unsigned, __builtin_elementwise_fma(c2, s2, z2));
  o[3] = __builtin_bit_cast(unsigned, __builtin_elementwise_fma(c3, s2, z2));
  return o;
}



// ---------------------------------------------------------------------------------------------
// Exact-keys workgroup of query sequence sq: dense attention of every head over the live window
// slots of its stored sequence (iS-KV abstract: the recent window is kept exact) and, in a
// prefill, over the chunk's own rows up to and including its token (causal). Writes (Aw[d], m,
// l) per head, in base-2 softmax units like the latent partials.
// ---------------------------------------------------------------------------------------------
template <int LT, int NTHR>
__device__ void window_block(const DecodeArgs& a, unsigned char* smem) {
  const int sq = blockIdx.x;
  const int b = sq / a.qpb, ci = sq - b * a.qpb;       // stored sequence, token of the chunk
  const int tid = threadIdx.x;
  const int Hq = a.Hq, d = a.d, D = a.D, W = a.window;
  const int grp = Hq / a.Hkv;
  int L = a.lat_len[b];
  L = L < 0 ? 0 : L;
  int wl = W > 0 ? a.win_len[b] : 0;
  wl = wl < 0 ? 0 : (wl > W ? W : wl);
  const int nkeys = wl + (a.kchunk ? ci + 1 : 0);      // window slots, then chunk rows 0 .. ci

  // key rows padded by 16 bytes: the score loop reads 32 rows at once, which would otherwise
  // share one LDS bank (rows 1 KB apart)
  const int KD = D + 8;
  float* qs = (float*)smem;                              // [Hq][d]
  __bf16* kc = (__bf16*)(qs + Hq * d);                   // [32][KD]
  __bf16* vc = kc + 32 * KD;                             // [32][D]
  float* sc = (float*)(vc + 32 * D);                     // [Hq][32]
  float* st = sc + Hq * 32;                              // [Hq][3]: m, l, alpha

  for (int i = tid; i < Hq * d; i += NTHR) {
    float qv;
    if constexpr (LT == LT_F32) qv = ((const float*)a.q)[(size_t)sq * Hq * d + i];
    else qv = (float)((const __bf16*)a.q)[(size_t)sq * Hq * d + i];
    qs[i] = qv * a.wscale;
  }
  for (int j = tid; j < Hq; j += NTHR) { st[j * 3] = -INFINITY; st[j * 3 + 1] = 0.f; }

  constexpr int kMaxAcc = (kHeadsPad * 128 + NTHR - 1) / NTHR;  // Hq*d <= 32*128
  float acc[kMaxAcc];
#pragma unroll
  for (int u = 0; u < kMaxAcc; ++u) acc[u] = 0.f;
  const int nout = Hq * d;

  for (int c0 = 0; c0 < nkeys; c0 += 32) {
    const int n = (nkeys - c0) < 32 ? (nkeys - c0) : 32;
    __syncthreads();
    // stage n exact rows (16 bytes per thread per step)
    const int vec_per_row = D / 8;
    for (int i = tid; i < n * vec_per_row; i += NTHR) {
      const int u = i / vec_per_row, c = i - u * vec_per_row;
      const int e = c0 + u;
      const __bf16 *ks, *vs;
      if (e < wl) {
        const size_t src = ((size_t)b * W + (L + e) % W) * D + c * 8;
        ks = a.kwin + src;
        vs = a.vwin + src;
      } else {
        const size_t src = ((size_t)b * a.qpb + (e - wl)) * D + c * 8;
        ks = a.kchunk + src;
        vs = a.vchunk + src;
      }
      *(u32x4*)(kc + u * KD + c * 8) = *(const u32x4*)ks;
      *(u32x4*)(vc + u * D + c * 8) = *(const u32x4*)vs;
    }
    __syncthreads();
    for (int i = tid; i < Hq * 32; i += NTHR) {
      const int j = i >> 5, u = i & 31;
      float s = -INFINITY;
      if (u < n) {
        const int g = j / grp;
        const float* qj = qs + j * d;
        const __bf16* kr = kc + u * KD + g * d;
        s = 0.f;
        for (int c = 0; c < d; ++c) s += qj[c] * (float)kr[c];
        s = (s != s) ? INFINITY : s;   // NaN propagates to this head only (see latent_block)
      }
      sc[i] = s;
    }
    __syncthreads();
    for (int j = tid; j < Hq; j += NTHR) {
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
      const int o = tid + u * NTHR;
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
  float* wp = a.win_part + (size_t)sq * Hq * (d + 2);
#pragma unroll
  for (int u = 0; u < kMaxAcc; ++u) {
    const int o = tid + u * NTHR;
    if (o < nout) {
      const int j = o / d, c = o - j * d;
      wp[j * (d + 2) + c] = acc[u];
    }
  }
  for (int j = tid; j < Hq; j += NTHR) {
    wp[j * (d + 2) + d] = st[j * 3];
    wp[j * (d + 2) + d + 1] = st[j * 3 + 1];
  }
}

// ---------------------------------------------------------------------------------------------
// Latent workgroup: one (sequence b, token range s): 4 producer waves and G groups of 4 consumer
// waves.
//
// The token range is cut into 16-token tiles that stream through an LDS ring (stage = the 16 Zk
// rows then the 16 Zv rows, each row padded so that the 16 rows a score operand reads fall in
// distinct banks). Each iteration consumes TPI tiles between two workgroup barriers. Consumer
// wave roles (hb = query-head block, heads 16*hb .. 16*hb+15):
//   SP (split): wave (hb, slot) takes tile TPI*it + slot, all value blocks (TPI = 2G);
//   else:       waves (hb, half) of group g share tile G*it + g; value blocks half, half+2, ...
// Per tile a wave computes
//   S^T[16 tokens, 16 heads] = Zk qt^T            (16x16x32, K = rank)
//   online softmax of its 4 scores per lane       (base 2; only cross-lane max)
//   A^T[16 rv, 16 heads] += Zv^T P^T               (16x16x16, K = the 16 tokens)
// so no data crosses waves inside a tile (int4 latents excepted: there the two waves of a tile
// exchange partial scores, see below). At the end the waves holding the same role's partial
// (m, l, A) for different tiles are merged through LDS and written once.
// KS: compile-time bound on K steps of 32; RB: bound on value blocks of a half.
// ---------------------------------------------------------------------------------------------
constexpr int kProducers = 4;           // waves that move data (direct-to-LDS loads; int4: and convert)
constexpr int kMaxChunkPerProducer = 5; // 1 KB DMA chunks per producer per matrix and tile
constexpr float kRescaleSlack = 8.f;    // base-2 headroom before the running reference max moves

// Threads of the decode workgroup for G consumer groups.
constexpr int decode_threads(int G, int LT) { return 64 * (4 * G + kProducers); }

// ---------------------------------------------------------------------------------------------
// int4 latents: 4 consumer waves and 4 loader waves, one workgroup barrier per pair of tiles.
//   loaders    copy a tile's stored bytes (16 rows of codes and of scale/zero words, for Zk then
//              Zv: four contiguous runs in HBM) by 1 KB direct-to-LDS chunks into raw stage
//              t % nr, and turn the value rows of the next iteration's two tiles into fp16
//              stages (t % 4) with the bf16 value-row geometry. In iteration it the raw stages
//              of tiles below 2 it are free (their keys were read in iteration it - 1), so tiles
//              2 it - 2 + nr and 2 it - 1 + nr are issued; tiles 2 it + 2 and 2 it + 3 (landed
//              before the barrier) are dequantised; then the wave waits for tiles up to 2 it + 5.
//   consumers  wave (slot, hb) takes tile 2 it + slot for head block hb. The tile's two waves
//              split its key side: each dequantises half of every key group's codes from the
//              raw stage straight into matrix-core operands, computes the partial scores of
//              both head blocks (one tile ahead), and passes the other head block's half to its
//              partner through LDS. Values come from the fp16 stage through the transpose read.
// Each stored byte thus crosses LDS once as raw bytes, each key code is read and dequantised
// once, and only the value rows are written back, as fp16. Before any copy the consumers issue
// their query loads (a barrier orders the two), so that those do not queue behind the copies.
// ---------------------------------------------------------------------------------------------
struct I4Raw {      // byte offsets of the four runs inside a raw stage, and the stage size
  int cbk, qbk, cbv, qbv, o_qk, o_cv, o_qv, rs;
  __device__ I4Raw(const DecodeArgs& a)
      : cbk(a.row_bytes_k), qbk(a.qp_bytes_k), cbv(a.row_bytes_v), qbv(a.qp_bytes_v),
        o_qk(kTileTokens * a.row_bytes_k), o_cv(o_qk + kTileTokens * a.qp_bytes_k),
        o_qv(o_cv + kTileTokens * a.row_bytes_v), rs(a.raw_stage) {}
};

// fp16 pairs (x, x) of the low and of the high half of a scale/zero word
__device__ __forceinline__ f16x2 bcast_lo16(unsigned w) {
  return __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(w, w, 0x01000100u));
}
__device__ __forceinline__ f16x2 bcast_hi16(unsigned w) {
  return __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(w, w, 0x03020302u));
}

// 1 KB chunks a loader wave copies per tile: a full tile's four runs hold at most 10 chunks
// (rank 512: 4 + 1 + 4 + 1), numbered across the runs and dealt round-robin to the 4 waves.
// (All four waves copy: measured, one wave copying for all is slower, since a wave's copies
// stall in issue once the memory pipeline holds enough of them.)
constexpr int kI4ChunksPerWave = 3;

template <int RB>
__device__ __forceinline__ void i4_loader(const DecodeArgs& a, unsigned char* smem, int b, int t_begin, int t_end,
                                          int ntiles, int pw) {
  constexpr int SV = lds_stride_v(RB, 2);
  constexpr int VSTAGE = i4_vstage(RB);
  constexpr int NI = RB / 4;          // value dwords (8 codes each) per loader lane and tile
  const int lane = threadIdx.x & 63;
  unsigned char* raw = smem + kI4VStages * VSTAGE;
  const I4Raw R(a);
  const int NR = a.nr;
  const size_t row0 = (size_t)b * a.t_cap + t_begin;

  // This wave's chunks of a tile (the numbering of a full tile; a final partial tile copies the
  // chunks that start inside its shorter runs): run, start byte inside the run, LDS offset.
  const unsigned char* c_src[kI4ChunksPerWave];
  int c_rb[kI4ChunksPerWave], c_start[kI4ChunksPerWave], c_dst[kI4ChunksPerWave];
  int nchw = 0;
  {
    const unsigned char* rsrc[4] = {a.zk + row0 * R.cbk, a.zkq + row0 * R.qbk, a.zv + row0 * R.cbv,
                                    a.zvq + row0 * R.qbv};
    const int rrb[4] = {R.cbk, R.qbk, R.cbv, R.qbv};
    const int rdst[4] = {0, R.o_qk, R.o_cv, R.o_qv};
    int gc = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int n = (kTileTokens * rrb[r] + 1023) >> 10;
      for (int c = 0; c < n; ++c, ++gc) {
        if ((gc & 3) == pw && nchw < kI4ChunksPerWave) {
          c_src[nchw] = rsrc[r];
          c_rb[nchw] = rrb[r];
          c_start[nchw] = c * 1024;
          c_dst[nchw] = rdst[r] + c * 1024;
          ++nchw;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kI4ChunksPerWave; ++u)
      if (u >= nchw) { c_src[u] = rsrc[0]; c_rb[u] = 0; c_start[u] = 0; c_dst[u] = 0; }
  }
  auto tile_loads = [&](int rows) {                  // chunks this wave copies for a tile
    int n = 0;
#pragma unroll
    for (int u = 0; u < kI4ChunksPerWave; ++u) n += (u < nchw && c_start[u] < rows * c_rb[u]) ? 1 : 0;
    return n;
  };
  const int rows_last = ntiles > 0 ? t_end - (t_begin + (ntiles - 1) * kTileTokens) : 0;
  const int cnt_full = tile_loads(kTileTokens);
  const int cnt_last = ntiles > 0 ? tile_loads(rows_last) : 0;
  auto count = [&](int lo, int hi) {     // this wave's loads for tiles (lo, hi]
    if (hi <= lo) return 0;
    return (hi - lo) * cnt_full + (hi == ntiles - 1 ? cnt_last - cnt_full : 0);
  };
  // whether this lane copies 16 bytes of copy u of a full tile (16 rows), computed once
  bool fu[kI4ChunksPerWave];
#pragma unroll
  for (int u = 0; u < kI4ChunksPerWave; ++u) fu[u] = u < nchw && c_start[u] + lane * 16 < kTileTokens * c_rb[u];
  int issue_stage = 0;                   // raw stage of the next tile issued (tiles go in order)
  auto issue = [&](int t) {
    unsigned char* st = raw + issue_stage * R.rs;
    issue_stage = issue_stage + 1 == NR ? 0 : issue_stage + 1;
    const int t0 = t * kTileTokens;
    const int rows = min(kTileTokens, t_end - t_begin - t0);
    if (rows == kTileTokens) {
#pragma unroll
      for (int u = 0; u < kI4ChunksPerWave; ++u)
        if (fu[u]) dma16(c_src[u] + (size_t)t0 * c_rb[u] + c_start[u] + lane * 16, st + c_dst[u]);
      return;
    }
#pragma unroll
    for (int u = 0; u < kI4ChunksPerWave; ++u) {
      const int lim = rows * c_rb[u];
      if (u < nchw && c_start[u] < lim) {
        const int off = c_start[u] + lane * 16;
        if (off < lim) dma16(c_src[u] + (size_t)t0 * c_rb[u] + off, st + c_dst[u]);
      }
    }
  };

  // Value item i (one dword of codes of one row) of a tile, i = lane + 256 u over the loader
  // waves; its offsets are the same for every tile, so they are computed once. Every item of
  // the tile's 16 rows is converted, also for a final partial tile (its stale rows are masked
  // by the consumers); items past the row's groups read row 0 and write into the never-read
  // 32-byte pad of row 0. So the conversion has no branch, and two tiles' reads are all issued
  // before the first conversion.
  const int dv = R.cbv >> 2;                         // code dwords per value row
  const int nitems = kTileTokens * dv;
  int i_src[NI], i_qp[NI], i_dst[NI];
#pragma unroll
  for (int u = 0; u < NI; ++u) {
    const int i = pw * 64 + lane + u * kProducers * 64;
    i_src[u] = R.o_cv;
    i_qp[u] = R.o_qv;
    i_dst[u] = SV - 16;
    if (i < nitems) {
      const int row = i / dv, word = i - row * dv;  // word = 4 * group + quarter
      i_src[u] = R.o_cv + row * R.cbv + word * 4;
      i_qp[u] = R.o_qv + row * R.qbv + (word >> 2) * 4;
      i_dst[u] = row * SV + word * 16;
    }
  }
  unsigned kM0 = 0x000F000Fu, kM1 = 0x00F000F0u, kE0 = 0x64006400u, kE1 = 0x54005400u;
  asm volatile("" : "+v"(kM0), "+v"(kM1), "+v"(kE0), "+v"(kE1));
  // Dequantise tiles t and t + 1 (raw stages rs0, rs1) into fp16 value stages t % 4, (t+1) % 4;
  // tile t + 1 only if two (wave-uniform).
  auto dequant2 = [&](int t, int rs0, int rs1, bool two) {
    const unsigned char* s0 = raw + rs0 * R.rs;
    const unsigned char* s1 = raw + rs1 * R.rs;
    unsigned w0[NI], q0[NI], w1[NI], q1[NI];
#pragma unroll
    for (int u = 0; u < NI; ++u) {
      w0[u] = *(const unsigned*)(s0 + i_src[u]);
      q0[u] = *(const unsigned*)(s0 + i_qp[u]);
    }
    if (two) {
#pragma unroll
      for (int u = 0; u < NI; ++u) {
        w1[u] = *(const unsigned*)(s1 + i_src[u]);
        q1[u] = *(const unsigned*)(s1 + i_qp[u]);
      }
    }
    unsigned char* d0 = smem + (t & 3) * VSTAGE;
#pragma unroll
    for (int u = 0; u < NI; ++u)
      *(u32x4*)(d0 + i_dst[u]) = dequant8_f16(w0[u], bcast_lo16(q0[u]), bcast_hi16(q0[u]), kM0, kM1, kE0, kE1);
    if (two) {
      unsigned char* d1 = smem + ((t + 1) & 3) * VSTAGE;
#pragma unroll
      for (int u = 0; u < NI; ++u)
        *(u32x4*)(d1 + i_dst[u]) = dequant8_f16(w1[u], bcast_lo16(q1[u]), bcast_hi16(q1[u]), kM0, kM1, kE0, kE1);
    }
  };

  // the two halves of dequant2 for one tile: its raw words into registers, then its fp16 stage
  auto raw_read = [&](int rs, unsigned (&w)[NI], unsigned (&q)[NI]) {
    const unsigned char* s0 = raw + rs * R.rs;
#pragma unroll
    for (int u = 0; u < NI; ++u) {
      w[u] = *(const unsigned*)(s0 + i_src[u]);
      q[u] = *(const unsigned*)(s0 + i_qp[u]);
    }
  };
  auto stage_write = [&](int t, const unsigned (&w)[NI], const unsigned (&q)[NI]) {
    unsigned char* d0 = smem + (t & 3) * VSTAGE;
#pragma unroll
    for (int u = 0; u < NI; ++u)
      *(u32x4*)(d0 + i_dst[u]) = dequant8_f16(w[u], bcast_lo16(q[u]), bcast_hi16(q[u]), kM0, kM1, kE0, kE1);
  };

  // The consumers' query loads go first (the copies would queue ahead of them in the memory
  // pipeline); then tiles 0-3 are copied, 0 and 1 converted, and the rest of the ring filled.
  barrier_lds();                                     // the consumers' query loads are issued
  const int pro = min(NR, ntiles), pro0 = min(4, pro);
  for (int t = 0; t < pro0; ++t) issue(t);
  wait_vmcnt(count(1, pro0 - 1));                    // tiles 0 and 1 landed
  barrier_lds();                                     // ... and visible to every loader
  if (ntiles > 0) dequant2(0, 0, 1 % NR, ntiles > 1);
  for (int t = pro0; t < pro; ++t) issue(t);
  wait_vmcnt(count(3, pro - 1));                     // tiles 2 and 3 landed
  const int niter = (ntiles + 1) / 2;
  int dq_stage = 2 % NR;                             // raw stage of tile 2 it + 2
  for (int it = 0; it < niter; ++it) {
    barrier_lds();                                   // fp16 values of 2it, 2it+1 visible
    // copies as early as their stages are free (measured: converting both tiles first and
    // copying after is slower)
    // one tile's copies, one tile's conversion, then the other's: spread out, the copies stall
    // less on the memory pipeline's backlog (measured: 53.1 against 54.1 us at T = 16K)
    // Both tiles' raw words are read first (their stages landed before the barrier; the copies
    // issued below go to stages of tiles 2it - 2 and 2it - 1, as the ring holds at least 6), so
    // the second tile's LDS round trip overlaps the first one's conversion.
    const int dq1 = dq_stage + 1 == NR ? 0 : dq_stage + 1;
    const bool ha = 2 * it + 2 < ntiles, hb = 2 * it + 3 < ntiles;   // wave-uniform
    unsigned wa[NI], qa[NI], wb[NI], qb[NI];
    if (ha) raw_read(dq_stage, wa, qa);
    if (hb) raw_read(dq1, wb, qb);
    if (it > 0 && 2 * it - 2 + NR < ntiles) issue(2 * it - 2 + NR);
    if (ha) stage_write(2 * it + 2, wa, qa);
    if (it > 0 && 2 * it - 1 + NR < ntiles) issue(2 * it - 1 + NR);
    if (hb) stage_write(2 * it + 3, wb, qb);
    dq_stage = dq1 + 1 == NR ? 0 : dq1 + 1;
    wait_vmcnt(count(2 * it + 5, min(2 * it - 1 + NR, ntiles - 1)));
  }
}

template <int KS, int RB, int LT, int G, bool SP>
__device__ __forceinline__ void latent_block(const DecodeArgs& a, unsigned char* smem, int wg) {
  constexpr int NTHR = decode_threads(G, LT);
  constexpr bool I4 = LT == LT_I4;
  constexpr int ES = LT == LT_F32 ? 4 : 2;             // bytes per latent element in the LDS tile
  constexpr int SK = lds_stride_k(KS, ES);             // LDS row strides (bytes)
  constexpr int SV = lds_stride_v(RB, ES);
  // value rows' offset inside a stage, stage bytes, stages (int4: the fp16 value stages; the
  // raw ring follows them)
  constexpr int ZV = I4 ? 0 : kTileTokens * SK;
  constexpr int STAGE = I4 ? i4_vstage(RB) : lds_stage(KS, RB, ES);
  constexpr int NST = I4 ? kI4VStages : lds_nst(KS, RB, ES);
  constexpr int TPI = SP ? 2 * G : G;                  // tiles per iteration
  constexpr int NVB = SP ? 2 * RB : RB;                // value blocks per consumer wave
  static_assert(NST % TPI == 0 && NST / TPI >= 2, "LDS ring must hold two iterations of tiles");
  static_assert(!I4 || (G == 1 && SP && KS % 4 == 0), "int4: one split group, key groups in fours");
  static_assert(I4 || ((kTileTokens * SK + 1023) / 1024 <= kProducers * kMaxChunkPerProducer &&
                       (kTileTokens * SV + 1023) / 1024 <= kProducers * kMaxChunkPerProducer), "DMA chunks");

  const int tid = threadIdx.x, lane = tid & 63, lg = lane >> 4, li = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const bool producer = wave >= 4 * G;
  int sq, s, t_begin, t_end;
  if (a.rng) {                                       // balanced: this workgroup's table entry
    const int* e = a.rng + 4 * wg;
    sq = e[0];
    s = e[1];
    t_begin = e[2];
    t_end = e[3];
    if (sq < 0) {                                    // no range: an empty pass, nothing written
      sq = 0;
      s = -1;
      t_begin = t_end = 0;
    }
  } else {
    sq = wg / a.nsplit;                              // query sequence (token of a chunk)
    s = wg - sq * a.nsplit;
    const int b0 = sq / a.qpb;
    int L = a.step ? step_lens(a.lat_len[b0], a.window > 0 ? a.win_len[b0] : 0, a.window, a.t_cap).L_new
                   : a.lat_len[b0];
    L = L < 0 ? 0 : (L > a.max_len ? a.max_len : L);
    t_begin = s * a.split_tokens;
    t_end = min(t_begin + a.split_tokens, L);
  }
  const int b = sq / a.qpb;                          // stored sequence whose latents it reads
  const int ntiles = t_end > t_begin ? (t_end - t_begin + kTileTokens - 1) / kTileTokens : 0;
  const int niter = (ntiles + TPI - 1) / TPI;

  unsigned char* ring = smem;
  // Zero, once, the LDS columns of every stage row that no copy (or dequantisation) writes: the
  // K steps and value blocks past the rank then read as exact zeros for the whole workgroup.
  // These bytes are disjoint from everything the producers write, so no barrier is needed here:
  // the first loop barrier orders them before any consumer read.
  {
    constexpr int KB = KS * 32 * ES, VB = RB * 32 * ES;        // bytes of a row the operands read
    const int ck = I4 ? a.nks * 64 : a.copy_k;                  // bytes written per K / V row
    const int cv = I4 ? ((a.rv + 31) / 32) * 64 : a.copy_v;
    const int npk = I4 ? 0 : (KB - ck) >> 4, npv = (VB - cv) >> 4;   // 16-byte granules to clear
    const int per_stage = kTileTokens * (npk + npv);
    for (int i = tid; i < NST * per_stage; i += NTHR) {
      const int st = i / per_stage, j = i - st * per_stage;
      unsigned char* p;
      if (j < kTileTokens * npk) {
        const int row = j / (npk > 0 ? npk : 1), gk = j - row * npk;
        p = ring + st * STAGE + row * SK + ck + gk * 16;
      } else {
        const int jj = j - kTileTokens * npk;
        const int row = jj / npv, gv = jj - row * npv;
        p = ring + st * STAGE + ZV + row * SV + cv + gv * 16;
      }
      *(u32x4*)p = u32x4{0u, 0u, 0u, 0u};
    }
  }

  float m = -INFINITY, lsum = 0.f;
  f32x4 acc[NVB];
#pragma unroll
  for (int j = 0; j < NVB; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (I4 && producer) {
    i4_loader<RB>(a, smem, b, t_begin, t_end, ntiles, wave - 4 * G);
  } else if (producer) {
    // ---------------- producer waves: keep the ring full ----------------
    const int pw = wave - 4 * G;
    const unsigned char* gk = a.zk + ((size_t)b * a.t_cap + t_begin) * a.row_bytes_k;
    const unsigned char* gv = a.zv + ((size_t)b * a.t_cap + t_begin) * a.row_bytes_v;
    // Source offset, inside a tile's stored rows, of the 16 bytes this lane lands at LDS
    // position c*1024 + 16*lane of a stage region (c = pw + kProducers*u); -1 = not copied.
    int offk[kMaxChunkPerProducer], offv[kMaxChunkPerProducer];
#pragma unroll
    for (int u = 0; u < kMaxChunkPerProducer; ++u) {
      const int o = (pw + kProducers * u) * 1024 + lane * 16;
      int row = o / SK, col = o - row * SK;
      offk[u] = (col < a.copy_k) ? row * a.row_bytes_k + col : -1;
      row = o / SV;
      col = o - row * SV;
      offv[u] = (col < a.copy_v) ? row * a.row_bytes_v + col : -1;
    }
    // chunks holding at least one needed byte of a tile with `rows` rows
    auto nchunks = [](int rows, int stride, int cp) { return ((rows - 1) * stride + cp + 1023) >> 10; };
    auto pcnt = [&](int nch) { return nch > pw ? (nch - pw + kProducers - 1) / kProducers : 0; };
    auto tile_cnt = [&](int rows) {
      return pcnt(nchunks(rows, SK, a.copy_k)) + pcnt(nchunks(rows, SV, a.copy_v));
    };
    const int rows_last = ntiles > 0 ? t_end - (t_begin + (ntiles - 1) * kTileTokens) : 0;
    const int cnt_full = tile_cnt(kTileTokens);
    const int cnt_last = ntiles > 0 ? tile_cnt(rows_last) : 0;
    // loads issued for tiles (lo, hi] (hi <= ntiles - 1)
    auto count = [&](int lo, int hi) {
      if (hi <= lo) return 0;
      return (hi - lo) * cnt_full + (hi == ntiles - 1 ? cnt_last - cnt_full : 0);
    };
    // whether this lane copies 16 bytes of chunk u of a full tile (16 rows): fixed for the range,
    // so a full tile's loads test one precomputed lane flag each (the general per-lane
    // conditions cost a compare chain and an exec-mask round trip per load)
    const int nck16 = nchunks(kTileTokens, SK, a.copy_k), ncv16 = nchunks(kTileTokens, SV, a.copy_v);
    bool fk[kMaxChunkPerProducer], fv[kMaxChunkPerProducer];
#pragma unroll
    for (int u = 0; u < kMaxChunkPerProducer; ++u) {
      const int c = pw + kProducers * u;
      fk[u] = c < nck16 && offk[u] >= 0 && offk[u] < kTileTokens * a.row_bytes_k;
      fv[u] = c < ncv16 && offv[u] >= 0 && offv[u] < kTileTokens * a.row_bytes_v;
    }
    auto issue = [&](int t) {
      unsigned char* stg = ring + (t % NST) * STAGE;
      const int t0 = t * kTileTokens;
      const int rows = min(kTileTokens, t_end - t_begin - t0);
      const unsigned char* srck = gk + (size_t)t0 * a.row_bytes_k;
      const unsigned char* srcv = gv + (size_t)t0 * a.row_bytes_v;
      if (rows == kTileTokens) {
#pragma unroll
        for (int u = 0; u < kMaxChunkPerProducer; ++u)
          if (fk[u]) dma16(srck + offk[u], stg + (pw + kProducers * u) * 1024);
#pragma unroll
        for (int u = 0; u < kMaxChunkPerProducer; ++u)
          if (fv[u]) dma16(srcv + offv[u], stg + ZV + (pw + kProducers * u) * 1024);
        return;
      }
      const int nck = nchunks(rows, SK, a.copy_k);
      const int ncv = nchunks(rows, SV, a.copy_v);
      const int limk = rows * a.row_bytes_k, limv = rows * a.row_bytes_v;
#pragma unroll
      for (int u = 0; u < kMaxChunkPerProducer; ++u) {
        const int c = pw + kProducers * u;
        if (c < nck && offk[u] >= 0 && offk[u] < limk) dma16(srck + offk[u], stg + c * 1024);
      }
#pragma unroll
      for (int u = 0; u < kMaxChunkPerProducer; ++u) {
        const int c = pw + kProducers * u;
        if (c < ncv && offv[u] >= 0 && offv[u] < limv) dma16(srcv + offv[u], stg + ZV + c * 1024);
      }
    };
    const int pro = min(NST - TPI, ntiles);
    for (int t = 0; t < pro; ++t) issue(t);
    wait_vmcnt(count(TPI - 1, pro - 1));               // iteration 0's tiles landed
    for (int it = 0; it < niter; ++it) {
      barrier_lds();                                   // iteration it visible; it-1's stages free
#pragma unroll
      for (int j = 0; j < TPI; ++j)
        if (TPI * it + NST - TPI + j < ntiles) issue(TPI * it + NST - TPI + j);
      const int hi = min(TPI * it + NST - 1, ntiles - 1);
      wait_vmcnt(count(TPI * it + 2 * TPI - 1, hi));   // iteration it+1's tiles landed
    }
  } else {
    // ---------------- consumer waves: scores, online softmax, values ----------------
    const int slot = SP ? (wave >> 1) : (wave >> 2);   // tile of the iteration this wave takes
    const int hb = wave & 1;
    const int half = SP ? 0 : (wave >> 1) & 1;
    // int4: the two waves of a tile split the keys' K steps, each computing partial scores of
    // both head blocks; qop[h2 * KS/2 + 2*kq + jj] is head block h2's operand of K step
    // (kq, 2*hb + jj).
    constexpr int KH = KS / 2;
    bf16x8 qop[KS];
    float qxh[2] = {1.f, 1.f};  // int4: per head block, the power of two its fp16 operands were divided by
    if constexpr (I4) {
      // The folded query arrives in float32. For each head block, the largest magnitude of the
      // wave's half of a head's row is brought into [2^14, 2^15) by a power of two so that the
      // fp16 operands cannot overflow; the partial scores are multiplied back by that power
      // before the two waves add them. The 4 lane groups holding a head share its scale.
      // K step (kq, j) of lane group lg holds quarter j (8 indices) of key group 4*kq + lg, the
      // order in which the key operands are dequantised; groups past the rank are 0.
      const float* qb = (const float*)a.qt + (size_t)sq * kHeadsPad * a.rk_pad;
      float qf[2][KH][8];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const float* qrow = qb + (size_t)(h2 * 16 + li) * a.rk_pad;
#pragma unroll
        for (int kq = 0; kq < KS / 4; ++kq) {
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            const int g = 4 * kq + lg;
            if (g < a.nks) {
              const float* p = qrow + g * 32 + (2 * hb + jj) * 8;
              const f32x4 x0 = *(const f32x4*)p;
              const f32x4 x1 = *(const f32x4*)(p + 4);
#pragma unroll
              for (int e = 0; e < 4; ++e) { qf[h2][2 * kq + jj][e] = x0[e]; qf[h2][2 * kq + jj][4 + e] = x1[e]; }
            } else {
#pragma unroll
              for (int e = 0; e < 8; ++e) qf[h2][2 * kq + jj][e] = 0.f;
            }
          }
        }
      }
      // the loaders start their copies after this barrier: the query loads, issued above, are
      // ahead of them in the memory pipeline
      barrier_lds();
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        float mxq = 0.f;
#pragma unroll
        for (int k = 0; k < KH; ++k)
#pragma unroll
          for (int e = 0; e < 8; ++e) mxq = fmaxf(mxq, fabsf(qf[h2][k][e]));
        mxq = wave_max_lg(mxq);
        int ex = 0;
        if (mxq > 0.f && mxq <= 3.4e38f) {
          ex = ilogbf(mxq) - 14;
          ex = ex < -100 ? -100 : (ex > 100 ? 100 : ex);
        }
        const float fac = ldexpf(1.f, -ex);
        qxh[h2] = ldexpf(1.f, ex);
#pragma unroll
        for (int k = 0; k < KH; ++k) {
          f16x8 h;
#pragma unroll
          for (int e = 0; e < 8; ++e) h[e] = (_Float16)(qf[h2][k][e] * fac);
          qop[h2 * KH + k] = __builtin_bit_cast(bf16x8, h);
        }
      }
    } else {
      const __bf16* qrow = a.qt + ((size_t)sq * kHeadsPad + hb * 16 + li) * a.rk_pad + lg * 8;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        qop[ks] = (ks < a.nks) ? *(const bf16x8*)(qrow + ks * 32) : zero_bf16x8();
    }
    LR_WAIT_VM(0);
    if constexpr (I4) barrier_lds();                 // pairs with the loaders' second barrier
    unsigned kM0 = 0x000F000Fu, kM1 = 0x00F000F0u, kE0 = 0x64006400u, kE1 = 0x54005400u;
    if constexpr (I4) asm volatile("" : "+v"(kM0), "+v"(kM1), "+v"(kE0), "+v"(kE1));
    // AND-mask for the last K step: latent indices >= rk read as 0 (the copied granule may
    // hold pad columns, and they may hold anything, including NaN patterns). int4 keys need
    // none: a pad index of a stored group dequantises, like the group's own indices, to
    // code * scale + zero with a 4-bit code, and its query entry is 0.
    u32x4 tailmask;
    {
      const int k0 = (a.nks - 1) * 32 + lg * 8;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        tailmask[i] = (k0 + 2 * i < a.rk ? 0x0000FFFFu : 0u) | (k0 + 2 * i + 1 < a.rk ? 0xFFFF0000u : 0u);
    }
    const bool ktail = !I4 && (a.rk & 7) != 0;
    // value block j of this wave covers latent indices 16*rb .. 16*rb+15 with rb = j (split) or
    // half + 2j (blocks past the rank read the zero-filled tail of the rows, never stored)
    const int krow_off = li * SK + lg * 8 * ES;
    const int vrow_off = (LT == LT_F32) ? ZV + 4 * lg * SV + li * ES + half * 16 * ES
                                        : ZV + (4 * lg + (li >> 2)) * SV + (li & 3) * 8 + half * 32;

    // int4 keys straight from the raw stage: lane (li, lg) reads quarters 2*hb and 2*hb + 1 of
    // key group 4*kq + lg of token li (8 code bytes) and the group's scale/zero word, and
    // dequantises them into the operands of K steps (kq, 2*hb) and (kq, 2*hb + 1), each shared
    // by the products of both head blocks. Groups past the rank read as zero codes with a zero
    // scale/zero word (their query entries are 0 as well).
    const I4Raw R(a);
    auto i4_scores = [&](int rstage, f32x4& c0, f32x4& c1) {
      const unsigned char* rst = smem + NST * STAGE + rstage * R.rs;
      u32x2 cw[KS / 4];
      unsigned qw[KS / 4];
#pragma unroll
      for (int kq = 0; kq < KS / 4; ++kq) {
        const int g = 4 * kq + lg;
        const int ge = g < a.nks ? g : 0;
        cw[kq] = *(const u32x2*)(rst + li * R.cbk + ge * 16 + hb * 8);
        qw[kq] = *(const unsigned*)(rst + R.o_qk + li * R.qbk + ge * 4);
        if (g >= a.nks) {
          cw[kq] = u32x2{0u, 0u};
          qw[kq] = 0u;
        }
      }
      c0 = f32x4{0.f, 0.f, 0.f, 0.f};
      c1 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kq = 0; kq < KS / 4; ++kq) {
        if (4 * kq < a.nks) {                          // wave-uniform
          const f16x2 s2 = bcast_lo16(qw[kq]), z2 = bcast_hi16(qw[kq]);
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            const bf16x8 op = __builtin_bit_cast(bf16x8, dequant8_f16(cw[kq][jj], s2, z2, kM0, kM1, kE0, kE1));
            c0 = mfma_k<LT>(op, qop[2 * kq + jj], c0);
            c1 = mfma_k<LT>(op, qop[KH + 2 * kq + jj], c1);
          }
        }
      }
      c0 *= qxh[0];
      c1 *= qxh[1];
    };
    // int4: this wave's partial scores of its tile of the next iteration (its raw tile landed
    // before this iteration's barrier) go through LDS to the partner wave: the half for the
    // partner's head block is written to xch[parity][slot][other hb], and after the next barrier
    // each wave adds the partner's half to its own. Parity = the iteration that wrote it.
    f32x4 s_own = {0.f, 0.f, 0.f, 0.f};
    int rs_next = 0;
    f32x4* xch = (f32x4*)(smem + NST * STAGE + a.nr * R.rs);
    auto xslot = [&](int par, int h) { return xch + ((par * 2 + slot) * 2 + h) * 64 + lane; };
    auto next_scores = [&](int par) {
      f32x4 c0, c1;
      i4_scores(rs_next, c0, c1);
      s_own = hb ? c1 : c0;
      *xslot(par, 1 - hb) = hb ? c0 : c1;
      rs_next = rs_next + TPI >= a.nr ? rs_next + TPI - a.nr : rs_next + TPI;
    };
    if constexpr (I4) {
      rs_next = slot % a.nr;
      if (slot < ntiles) next_scores(1);
    }

    for (int it = 0; it < niter; ++it) {
      barrier_lds();
      const int t = TPI * it + slot;
      if (t < ntiles) {
        const unsigned char* stg = ring + (t % NST) * STAGE;
        const int nvalid = min(kTileTokens, t_end - t_begin - t * kTileTokens);

        // ---- scores of this wave's head block: S^T[token 4*lg+i][head li]
        const unsigned char* krow = stg + krow_off;
        // two independent accumulation chains (even / odd K steps) halve the dependent latency
        // (one chain where the registers of two consumer groups with wide value blocks are tight)
        constexpr int NCH = (G == 2 && NVB > 8) ? 1 : 2;
        f32x4 sacc2[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
        if constexpr (I4) {
          sacc2[0] = s_own + *xslot((it + 1) & 1, hb);  // computed one iteration ahead
        } else {
#pragma unroll
        for (int ks0 = 0; ks0 < KS; ks0 += 4) {      // 4 K steps of reads in flight, then 4 products
          bf16x8 av[4];
#pragma unroll
          for (int u = 0; u < 4; ++u)
            if (ks0 + u < KS) av[u] = k_operand<LT>(krow, (ks0 + u) * 32);
          if (ktail) {
#pragma unroll
            for (int u = 0; u < 4; ++u)
              if (ks0 + u < KS && ks0 + u == a.nks - 1)
                av[u] = __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, av[u]) & tailmask);
          }
#pragma unroll
          for (int u = 0; u < 4; ++u)
            if (ks0 + u < KS) sacc2[u % NCH] = mfma_k<LT>(av[u], qop[ks0 + u], sacc2[u % NCH]);
        }
        }
        const f32x4 sacc = NCH == 2 ? sacc2[0] + sacc2[1] : sacc2[0];

        // ---- value operands: read in chunks of VC blocks; the first chunk's reads are issued
        // before the softmax so that its LDS latency hides under it
        // (6 for more than 16 blocks: with 8, the rank-358 bf16 wave needed 256 registers and
        // spilled q operands; their reloads from scratch queue behind the producers' loads in the
        // compute unit's memory pipeline)
        constexpr int VC = NVB < 8 ? NVB : (NVB > 16 ? 6 : 8);
        const unsigned char* vbase = stg + vrow_off;
        auto vread = [&](int j) -> bf16x4 {
          if constexpr (LT == LT_F32) return v_operand4<LT, SV>(vbase, j * (SP ? 16 : 32) * ES);
          else return v_operand_tr(vbase + j * (SP ? 32 : 64));
        };
        bf16x4 vop[VC];
#pragma unroll
        for (int u = 0; u < VC; ++u) vop[u] = vread(u);
        // the next tile's scores interleave with this tile's softmax and values (a stage past
        // the last tile holds stale bytes: its scores are never used)
        if constexpr (I4) next_scores(it & 1);

        // ---- online softmax over the tile's 16 tokens (4 per lane, 4 lane groups)
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[i] = sacc[i];
          v[i] = (v[i] != v[i]) ? INFINITY : v[i];   // NaN survives the max, poisons only this head
        }
        // rows past the range's end: score -inf, value operand 0 (the stage may hold stale rows)
        u32x2 tm = {0xFFFFFFFFu, 0xFFFFFFFFu};
        const bool partial = nvalid < kTileTokens;
        if (partial) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (4 * lg + i >= nvalid) v[i] = -INFINITY;
          tm[0] = (4 * lg < nvalid ? 0x0000FFFFu : 0u) | (4 * lg + 1 < nvalid ? 0xFFFF0000u : 0u);
          tm[1] = (4 * lg + 2 < nvalid ? 0x0000FFFFu : 0u) | (4 * lg + 3 < nvalid ? 0xFFFF0000u : 0u);
        }
        float mx = fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3]));
        mx = wave_max_lg(mx);
        // m is a reference max: scores are exponentiated against it and it only moves when a
        // tile's max exceeds it by more than kRescaleSlack, so most tiles skip the rescale.
        const bool move = mx > m + kRescaleSlack;     // false when the tile is empty (mx = -inf)
        if (__builtin_amdgcn_ballot_w64(move) != 0) {
          const float mnew = move ? mx : m;
          const float alpha = (m == -INFINITY) ? 0.f : fast_exp2(m - mnew);
          m = mnew;
          lsum *= alpha;
#pragma unroll
          for (int j = 0; j < NVB; ++j) acc[j] *= alpha;
        }
        const bool live = m != -INFINITY;
        bf16x4 pb;
        float ps = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float pf = live ? fast_exp2(v[i] - m) : 0.f;
          if constexpr (I4) {
            const _Float16 p = (_Float16)pf;
            pb[i] = __builtin_bit_cast(__bf16, p);
            ps += (float)p;
          } else {
            const __bf16 p = (__bf16)pf;
            pb[i] = p;
            ps += (float)p;
          }
        }
        lsum += ps;

        // ---- values: A^T[rv][head li] over this wave's value blocks
#pragma unroll
        for (int j0 = 0; j0 < NVB; j0 += VC) {
          if (j0 > 0) {
#pragma unroll
            for (int u = 0; u < VC; ++u)
              if (j0 + u < NVB) vop[u] = vread(j0 + u);
          }
          if (partial) {
#pragma unroll
            for (int u = 0; u < VC; ++u)
              vop[u] = __builtin_bit_cast(bf16x4, __builtin_bit_cast(u32x2, vop[u]) & tm);
          }
#pragma unroll
          for (int u = 0; u < VC; ++u)
            if (j0 + u < NVB) acc[j0 + u] = mfma_v<LT>(vop[u], pb, acc[j0 + u]);
        }
      }
    }
    lsum = wave_sum_lg(lsum);
  }

  // ---- merge the consumer waves' partials per role, write this range's partial
  // Roles: hb (split) or (hb, half). The main wave of a role (slot 0) absorbs the NX extra
  // waves of its role through LDS: m [NX][64], l [NX][64], A [NX][NVB][64] f32x4.
  constexpr int NROLE = SP ? 2 : 4;
  constexpr int NX = 4 * G - NROLE;
  barrier_lds();                                   // the ring is no longer read
  float* mbuf = (float*)smem;
  float* lbuf = mbuf + 64 * (NX > 0 ? NX : 1);
  f32x4* abuf = (f32x4*)(smem + 512 * (NX > 0 ? NX : 1));
  const int role = wave % NROLE;
  const int wslot = wave / NROLE;                  // 0 = the role's main wave
  if constexpr (NX > 0) {
    if (!producer && wslot > 0) {
      const int x = (wslot - 1) * NROLE + role;
      mbuf[x * 64 + lane] = m;
      lbuf[x * 64 + lane] = lsum;
#pragma unroll
      for (int j = 0; j < NVB; ++j) abuf[(x * NVB + j) * 64 + lane] = acc[j];
    }
  }
  barrier_lds();
  if (!producer && wslot == 0) {
    const int hb = wave & 1;
    const int half = SP ? 0 : (wave >> 1) & 1;
    float ms = m;
#pragma unroll
    for (int w2 = 1; w2 <= NX / NROLE; ++w2) ms = fmaxf(ms, mbuf[((w2 - 1) * NROLE + role) * 64 + lane]);
    const float wa = (m == -INFINITY) ? 0.f : fast_exp2(m - ms);
    float lt = lsum * wa;
#pragma unroll
    for (int j = 0; j < NVB; ++j) acc[j] *= wa;
#pragma unroll
    for (int w2 = 1; w2 <= NX / NROLE; ++w2) {
      const int x = (w2 - 1) * NROLE + role;
      const float mo = mbuf[x * 64 + lane];
      const float wb = (mo == -INFINITY) ? 0.f : fast_exp2(mo - ms);
      lt += lbuf[x * 64 + lane] * wb;
#pragma unroll
      for (int j = 0; j < NVB; ++j) acc[j] += abuf[(x * NVB + j) * 64 + lane] * wb;
    }
    const size_t pidx = (size_t)sq * a.nsplit + (s < 0 ? 0 : s);
    const int head = s < 0 ? a.Hq : hb * 16 + li;    // a workgroup without a range writes nothing
    // The range's value partial. float32 latents: float32. bf16 and int4 latents: fp16 with a
    // power of two per (range, head) folded into (m, l): the head's largest |A| is brought into
    // [2^14, 2^15) by A' = A 2^-e, and (m', l') = (m + e, l 2^-e), so 2^(m' - m*) A' = 2^(m - m*) A
    // for any reference m* of the combine. One rounding to 11 significant bits: at most 2^-12 of
    // the head's largest value per element, under a tenth of the bf16 latents' 5e-3 budget,
    // while the bytes written here and read by the combine halve. (bf16 partials, at 2^-9, took
    // the rank-1 bf16 case to 96% of that budget.)
    float psc = 1.f;
    if constexpr (LT != LT_F32) {
      float mxa = 0.f;
#pragma unroll
      for (int j = 0; j < NVB; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) mxa = fmaxf(mxa, fabsf(acc[j][e]));
      mxa = wave_max_lg(mxa);                        // the head's 4 lane groups
      if constexpr (!SP) {                           // halves: the head's other half (role ^ 2)
        float* xm = (float*)(smem + 512 * (NX > 0 ? NX : 1) + NX * NVB * 1024);   // past the merge buffers
        xm[role * 64 + lane] = mxa;
        barrier_lds();                               // every other wave: the barrier below
        mxa = fmaxf(mxa, xm[(role ^ 2) * 64 + lane]);
      }
      int ex = 0;
      if (mxa > 0.f && mxa <= 3.4e38f) {             // 0, inf and NaN keep e = 0
        ex = ilogbf(mxa) - 14;
        ex = ex < -100 ? -100 : (ex > 100 ? 100 : ex);
      }
      psc = ldexpf(1.f, -ex);
      if (ms != -INFINITY) ms += (float)ex;
      lt *= psc;
    } else if constexpr (!SP) {
      barrier_lds();                                 // pairs with the exchange barrier above
    }
    if (half == 0 && lg == 0 && head < a.Hq) {
      a.part_ml[(pidx * a.Hq + head) * 2] = ms;
      a.part_ml[(pidx * a.Hq + head) * 2 + 1] = lt;
    }
#pragma unroll
    for (int j = 0; j < NVB; ++j) {
      const int rb = SP ? j : half + 2 * j;
      const size_t o = (pidx * a.Hq + head) * a.rv_pad16 + rb * 16 + 4 * lg;
      if (rb < a.nrb && head < a.Hq) {
        if constexpr (LT == LT_F32) {
          *(f32x4*)(a.part_acc + o) = acc[j];
        } else {
          f16x4 h;
#pragma unroll
          for (int e = 0; e < 4; ++e) h[e] = (_Float16)(acc[j][e] * psc);
          *(f16x4*)((_Float16*)a.part_acc + o) = h;
        }
      }
    }
  } else if constexpr (!SP) {
    barrier_lds();                                   // pairs with the main waves' exchange barrier
  }
}

template <int KS, int RB, int LT, int G, bool SP>
__global__ __launch_bounds__(decode_threads(G, LT)) void lr_decode(DecodeArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  if ((int)blockIdx.x < a.n_win_blocks) {
    window_block<LT, decode_threads(G, LT)>(a, smem);
    return;
  }
  latent_block<KS, RB, LT, G, SP>(a, smem, (int)blockIdx.x - a.n_win_blocks);
}

template <typename T>
__global__ __launch_bounds__(256) void lr_fold(const T* __restrict__ q, const T* __restrict__ bk,
                                               __bf16* __restrict__ qt, int Hq, int Hkv, int D,
                                               int rk, int rk_pad, float scale) {
  FoldArgs f;
  f.q = (const __bf16*)q;
  f.bk = (const __bf16*)bk;
  f.qt = qt;
  f.Hq = Hq;
  f.Hkv = Hkv;
  f.D = D;
  f.rk = rk;
  f.rk_pad = rk_pad;
  f.scale = scale;
  __shared__ float qs[kHeadsPad * kFoldD];
  fold_f32_body(f, blockIdx.x, blockIdx.y, blockIdx.z, qs);
}

template <bool F32OUT>
__global__ __launch_bounds__(256) void lr_fold_mfma(FoldArgs f) {
  fold_body<F32OUT>(f, blockIdx.x, blockIdx.y, blockIdx.z);
}

// ---------------------------------------------------------------------------------------------
// Combine: one workgroup per (b, j). m* = max over ranges (and window), weights 2^(m_s - m*),
// l* = sum w_s l_s, Ahat = sum w_s A_s, out = (Ahat Bv[:, g] + w_win Aw) / l*.
// ---------------------------------------------------------------------------------------------
struct CombineArgs {
  const float* part_ml;
  const float* part_acc;    // [B][nsplit][Hq][rv_pad16]: float32 (float32 latents), else fp16
                            // values scaled by 2^-e, e folded into part_ml
  const float* win_part;
  const void* bv;
  void* out;
  int Hq, Hkv, d, D, rv, rv_pad16, nsplit;
  int exact;                // exact-keys partials present in win_part (window, prefill chunk)
  int i4_order;             // partials are in the dequantised int4 tiles' block order
  StepFinish fin;           // a decode step (fin.lat_len != NULL): workgroup (b, head 0) also
                            // writes sequence b's new token into the ring and its new lengths
  const int* nrng;          // balanced ranges: ranges (partial slots in use) per sequence, or NULL
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


template <typename T>
__device__ __forceinline__ void load8f(const T* p, float* out) { load8<T>(p, out); }

// Layout: phase 1 (weights): threads over ranges. Phase 2 (merge): thread (sg, r4) sums ranges
// s = sg, sg+4, ... over 4 consecutive latent indices with 16-byte loads. Phase 3 (up-project):
// thread (rg, cg) accumulates 8 output columns over latent rows rg, rg+16, ... with 16-byte
// loads of Bv; the 16 row groups are reduced through LDS.
template <typename BT, typename OT, bool PB>
__global__ __launch_bounds__(256) void lr_combine(CombineArgs a) {
  extern __shared__ float cs[];
  const int tid = threadIdx.x;
  const int b = blockIdx.x / a.Hq, j = blockIdx.x - b * a.Hq;
  const int g = j / (a.Hq / a.Hkv);
  const int pw = a.rv_pad16 > 512 ? a.rv_pad16 : 512;
  float* part = cs;                       // [4][pw] merge partials, reused as [16][128]
  float* ahat = part + 4 * pw;            // [rv_pad16]
  float* ws = ahat + a.rv_pad16;          // [nsplit]
  float* red = ws + a.nsplit;             // [8]
  const size_t base = (size_t)b * a.nsplit;
  const int ns = a.nrng ? a.nrng[b] : a.nsplit;  // slots of this sequence in use
  // no reader of the ring or the lengths is left in the step (this launch reads neither)
  if (a.fin.lat_len != nullptr && j == 0) step_finish(a.fin, b);

  float mw = -INFINITY, lw = 0.f;
  const float* wp = a.win_part + ((size_t)b * a.Hq + j) * (a.d + 2);
  if (a.exact) {
    mw = wp[a.d];
    lw = wp[a.d + 1];
  }
  float mloc = -INFINITY;
  // the slot loads do not wait for ns: slots past it are loaded and then ignored. Up to 256 slots
  // (one per thread) the slot's (m, l) come in one load and stay in registers for the weights.
  const bool one = a.nsplit <= 256;
  f32x2 ml_own = {-INFINITY, 0.f};
  if (one) {
    if (tid < a.nsplit) ml_own = *(const f32x2*)(a.part_ml + ((base + tid) * a.Hq + j) * 2);
    if (tid < ns) mloc = ml_own[0];
  } else {
    for (int s = tid; s < a.nsplit; s += 256) {
      const float mv = a.part_ml[((base + s) * a.Hq + j) * 2];
      if (s < ns) mloc = fmaxf(mloc, mv);
    }
  }
  const float mstar = block_reduce(fmaxf(mloc, mw), red, true);
  const bool live = mstar != -INFINITY;

  float lloc = 0.f;
  if (one) {
    if (tid < ns) {
      const float w = (live && ml_own[0] != -INFINITY) ? fast_exp2(ml_own[0] - mstar) : 0.f;
      ws[tid] = w;
      if (w != 0.f) lloc += w * ml_own[1];
    }
  } else {
    for (int s = tid; s < ns; s += 256) {
      const float ms = a.part_ml[((base + s) * a.Hq + j) * 2];
      const float w = (live && ms != -INFINITY) ? fast_exp2(ms - mstar) : 0.f;
      ws[s] = w;
      if (w != 0.f) lloc += w * a.part_ml[((base + s) * a.Hq + j) * 2 + 1];
    }
  }
  const float ww = (live && mw != -INFINITY) ? fast_exp2(mw - mstar) : 0.f;
  const float lstar = block_reduce(lloc, red, false) + ww * lw;
  __syncthreads();

  // merge the ranges: Ahat[r] = sum_s w_s A_s[r], thread (sg, r4) over slots s = sg, sg + 4, ...
  // in ascending order; the loads of up to 8 slots go out together (slot indices clamped to the
  // last one in use, with weight 0 past it), so a sequence with more ranges costs no extra round
  // trip until it has more than 32
  {
    constexpr int U = 8;
    const int sg = tid >> 6, r4 = (tid & 63) * 4;
    for (int r0 = 0; r0 < a.rv_pad16; r0 += 256) {
      const int r = r0 + r4;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      if (r < a.rv_pad16) {
        for (int s0 = sg; s0 < ns; s0 += 4 * U) {
          f32x4 v[U];
          float w[U];
#pragma unroll
          for (int u = 0; u < U; ++u) {
            const int s = s0 + 4 * u;
            const int sc = s < ns ? s : ns - 1;
            w[u] = s < ns ? ws[sc] : 0.f;
            const size_t o = ((base + sc) * a.Hq + j) * a.rv_pad16 + r;
            if constexpr (PB) {                   // fp16 partials (bf16 and int4 latents)
              const f16x4 h = *(const f16x4*)((const _Float16*)a.part_acc + o);
              v[u] = f32x4{(float)h[0], (float)h[1], (float)h[2], (float)h[3]};
            } else {
              v[u] = *(const f32x4*)(a.part_acc + o);
            }
          }
#pragma unroll
          for (int u = 0; u < U; ++u)
            if (w[u] != 0.f) acc += w[u] * v[u];
        }
        *(f32x4*)(part + sg * pw + r) = acc;
      }
    }
  }
  __syncthreads();
  for (int r = tid; r < a.rv_pad16; r += 256) {
    const int p = a.i4_order ? i4_pos(r) : r;
    ahat[r] = r < a.rv ? part[p] + part[pw + p] + part[2 * pw + p] + part[3 * pw + p] : 0.f;
  }
  __syncthreads();

  // up-project: o[c] = sum_r ahat[r] Bv[r][g*d + c]
  {
    const int cg = tid & 15, rg = tid >> 4;
    const BT* bv = (const BT*)a.bv + g * a.d + cg * 8;
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = 0.f;
    // 8 rows per round, every load issued: rows past rv read row rv - 1 (finite) against a zero
    // weight, so the rows still add in ascending order and a rank that is not a multiple of
    // 128 costs no extra one-load rounds
    constexpr int U = 8;
    for (int r = rg; r < a.rv; r += 16 * U) {
      float v[U][8];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int row = r + 16 * u;
        load8f<BT>(bv + (size_t)(row < a.rv ? row : a.rv - 1) * a.D, v[u]);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int row = r + 16 * u;
        const float h = row < a.rv ? ahat[row] : 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] += h * v[u][e];
      }
    }
    float* ored = part;     // [16][128]
#pragma unroll
    for (int e = 0; e < 8; ++e) ored[rg * 128 + cg * 8 + e] = o[e];
  }
  __syncthreads();
  if (tid < 128) {
    float o = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) o += part[i * 128 + tid];
    if (ww != 0.f) o += ww * wp[tid];
    o = (lstar == 0.f) ? 0.f : o / lstar;   // 0 only for a sequence with no tokens; NaN stays NaN
    ((OT*)a.out)[((size_t)b * a.Hq + j) * a.d + tid] = from_f32<OT>(o);
  }
}


// ---------------------------------------------------------------------------------------------
// Host launch
// ---------------------------------------------------------------------------------------------
// ev_begin/ev_end (optional) are attached to the kernel's own dispatch (hipExtLaunchKernel),
// so no separate marker packets enter the stream.
template <int KS, int RB, int LT, int G, bool SP>
static hipError_t launch_decode_kernel(const DecodeArgs& args, int grid, int lds, hipStream_t st,
                                       hipEvent_t ev_begin, hipEvent_t ev_end) {
  static bool attr_set[64] = {false};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < 64 && !attr_set[dev]) {
    e = hipFuncSetAttribute((const void*)lr_decode<KS, RB, LT, G, SP>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
    if (e != hipSuccess) return e;
    attr_set[dev] = true;
  }
  if (ev_begin || ev_end)
    hipExtLaunchKernelGGL((lr_decode<KS, RB, LT, G, SP>), dim3(grid), dim3(decode_threads(G, LT)), lds, st, ev_begin,
                          ev_end, 0, args);
  else
    hipLaunchKernelGGL((lr_decode<KS, RB, LT, G, SP>), dim3(grid), dim3(decode_threads(G, LT)), lds, st, args);
  return hipGetLastError();
}

// One instantiation per (KS, RB) bound of the latent dtype; the consumer layout and group count
// follow from the bounds (decode_split / decode_groups).
template <int LT>
static hipError_t dispatch_decode(const DecodePlan& p, const DecodeArgs& args, int grid, hipStream_t st,
                                  hipEvent_t ev_begin, hipEvent_t ev_end) {
  constexpr int LAT = LT == LT_I4 ? LR_I4G32 : (LT == LT_F32 ? LR_F32 : LR_BF16);
  const int ks = decode_ks(p.nks);
  const int rb = decode_rb(p.nrb);
#define LR_CASE(K, R)                                                                                     \
  if (ks == K && rb == R)                                                                                \
    return launch_decode_kernel<K, R, LT, decode_groups(LAT, K, R), decode_split(LAT, K, R)>(           \
        args, grid, p.lds_bytes, st, ev_begin, ev_end);
  LR_CASE(8, 8) LR_CASE(8, 12) LR_CASE(8, 16)
  LR_CASE(12, 8) LR_CASE(12, 12) LR_CASE(12, 16)
  LR_CASE(16, 8) LR_CASE(16, 12) LR_CASE(16, 16)
#undef LR_CASE
  return hipErrorInvalidValue;
}

// Arguments of the matrix-core fold (bf16 queries) for plan p; *nfold = its workgroups.
static void fold_args(const DecodePlan& p, const lr_layer_cache* c, const void* q, void* qt, float scale, FoldArgs* f,
                      int* nfold) {
  // query sequences per wave: 4 (the loads of kFoldQB sequences go out together, and a decode
  // batch of 16 takes a quarter of the workgroups), 16 for the many tokens of a prefill chunk
  const int nq = p.B >= 512 ? 16 : (p.B >= 4 ? 4 : 1);
  f->q = (const __bf16*)q;
  f->bk = (const __bf16*)c->bk;
  f->qt = qt;
  f->Hq = p.Hq;
  f->Hkv = p.Hkv;
  f->D = p.D;
  f->rk = p.rk;
  f->rk_pad = p.rk_pad;
  f->scale = scale;
  f->nseq = p.B;
  f->nq = nq;
  *nfold = ((p.rk_pad / 16 + 3) / 4) * p.Hkv * ((p.B + nq - 1) / nq);
}

// The first launch of a decode call: the fold, the exact window (W > 0) and, for a decode step,
// the append of the step's token.
static hipError_t decode_front(const DecodePlan& p, const AppendPlan* ap, const lr_layer_cache* c, const void* q,
                               const void* k_new, const void* v_new, void* ws, hipStream_t st) {
  unsigned char* w = (unsigned char*)ws;
  const float scale = p.sm_scale * kLog2e;
  FoldArgs f;
  int nfold = 0;
  fold_args(p, c, q, w + p.off_qt, scale, &f, &nfold);
  FrontPlan fp;
  fp.latent = p.latent;
  fp.nck = ap ? (ap->rk + kAppendCols - 1) / kAppendCols : 0;
  fp.ncv = ap ? (ap->rv + kAppendCols - 1) / kAppendCols : 0;
  fp.n_append = ap ? (fp.nck + fp.ncv) * ((ap->B + 15) / 16) : 0;
  if (p.latent == LR_F32) {
    fp.nfx = (p.rk_pad + 63) / 64;
    fp.nfy = p.Hkv;
    fp.n_fold = fp.nfx * fp.nfy * p.B;
  } else {
    fp.nfx = (p.rk_pad / 16 + 3) / 4;
    fp.nfy = p.Hkv;
    fp.n_fold = nfold;
  }
  fp.n_win = p.window > 0 ? p.B * p.Hkv : 0;
  fp.window = p.window;
  fp.t_cap = p.t_cap;
  memset(&fp.rng, 0, sizeof(fp.rng));
  fp.n_plan = p.bal ? 1 : 0;
  if (p.bal) {
    fp.rng.lat_len = c->lat_len;
    fp.rng.win_len = c->win_len;
    fp.rng.table = (int*)(w + p.off_rng);
    fp.rng.nrng = (int*)(w + p.off_rng) + 4 * p.nwg;
    fp.rng.t_cap = p.t_cap;
    fp.rng.B = p.B;
    fp.rng.nwg = p.nwg;
    fp.rng.nslot = p.nsplit;
    fp.rng.max_len = p.max_len;
    fp.rng.window = p.window;
    fp.rng.step = ap != nullptr;
  }
  return launch_front(fp, ap, c, k_new, v_new, f, (float*)(w + p.off_win), scale, st);
}

hipError_t launch_decode_step(const AppendPlan& ap, const DecodePlan& p, const lr_layer_cache* c, const void* k_new,
                              const void* v_new, const void* q, void* out, int out_dtype, void* ws, hipStream_t st,
                              hipEvent_t ev_begin, hipEvent_t ev_end) {
  const hipError_t e = decode_front(p, &ap, c, q, k_new, v_new, ws, st);
  if (e != hipSuccess) return e;
  return launch_decode(p, c, q, out, out_dtype, ws, st, ev_begin, ev_end, nullptr, nullptr, k_new, v_new);
}

hipError_t launch_decode(const DecodePlan& p, const lr_layer_cache* c, const void* q, void* out,
                         int out_dtype, void* ws, hipStream_t st, hipEvent_t ev_begin, hipEvent_t ev_end,
                         const void* k_chunk, const void* v_chunk, const void* step_k_new,
                         const void* step_v_new) {
  unsigned char* w = (unsigned char*)ws;
  __bf16* qt = (__bf16*)(w + p.off_qt);
  const float scale = p.sm_scale * kLog2e;

  // Exact keys. A decode step (no chunk rows): the window workgroups of the first launch. A prefill
  // chunk (the window and the chunk's own rows, causally): for bf16 queries the matrix-core
  // exact-keys kernel runs before the latent kernel, for float32 queries B extra workgroups of the
  // decode kernel (window_block); each leaves a partial the combine merges.
  const bool decode_step = k_chunk == nullptr;
  const bool exact_mfma = !decode_step && p.exact && p.latent != LR_F32;
  const bool step = step_k_new != nullptr;            // lowrank_decode_step: the front already ran

  // 1. fold (+ the window of a decode step), unless a decode step's first launch already ran it
  if (!step) {
    hipError_t e;
    if (decode_step) {
      e = decode_front(p, nullptr, c, q, nullptr, nullptr, ws, st);
    } else if (p.latent == LR_F32) {
      hipLaunchKernelGGL(lr_fold<float>, dim3((p.rk_pad + 63) / 64, p.Hkv, p.B), dim3(256), 0, st, (const float*)q,
                         (const float*)c->bk, qt, p.Hq, p.Hkv, p.D, p.rk, p.rk_pad, scale);
      e = hipGetLastError();
    } else {
      FoldArgs f;
      int nfold = 0;
      fold_args(p, c, q, qt, scale, &f, &nfold);
      const dim3 fgrid((p.rk_pad / 16 + 3) / 4, p.Hkv, (p.B + f.nq - 1) / f.nq);
      if (p.latent == LR_I4G32) hipLaunchKernelGGL(lr_fold_mfma<true>, fgrid, dim3(256), 0, st, f);
      else hipLaunchKernelGGL(lr_fold_mfma<false>, fgrid, dim3(256), 0, st, f);
      e = hipGetLastError();
    }
    if (e != hipSuccess) return e;
  }

  // 2. latent decode (+ exact-keys workgroups: window, prefill chunk)
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
  a.n_win_blocks = (!decode_step && p.exact && !exact_mfma) ? p.B : 0;
  a.qpb = p.qpb;
  a.kchunk = (const __bf16*)k_chunk;
  a.vchunk = (const __bf16*)v_chunk;
  a.stage_bytes = p.stage_bytes;
  a.zv_off = p.zv_off;
  a.qpk_off = p.qpk_off;
  a.qpv_off = p.qpv_off;
  a.nst = p.nst;
  a.copy_k = p.copy_k;
  a.copy_v = p.copy_v;
  a.nr = p.nr;
  a.raw_stage = p.raw_stage;
  a.step = step;
  a.rng = p.bal ? (const int*)(w + p.off_rng) : nullptr;
  hipError_t e;
  if (p.pf) {
    // prefill over bf16 latents: the dedicated exact-keys kernel (window slots and the chunk's
    // causal rows) and latent kernel
    e = launch_prefill_exact(p, c, q, k_chunk, v_chunk, a.win_part, st);
    if (e != hipSuccess) return e;
    e = launch_prefill_latent(p, c, qt, a.part_ml, a.part_acc, st, ev_begin, ev_end);
  } else {
    if (exact_mfma) {
      e = launch_prefill_exact(p, c, q, k_chunk, v_chunk, a.win_part, st);
      if (e != hipSuccess) return e;
    }
    const int grid = a.n_win_blocks + p.nwg;
    if (p.latent == LR_F32) e = launch_decode_kernel<8, 8, LT_F32, 2, false>(a, grid, p.lds_bytes, st, ev_begin, ev_end);
    else if (p.latent == LR_I4G32) e = dispatch_decode<LT_I4>(p, a, grid, st, ev_begin, ev_end);
    else e = dispatch_decode<LT_BF16>(p, a, grid, st, ev_begin, ev_end);
  }
  if (e != hipSuccess) return e;

  // 3. combine + up-projection
  if (p.pf) return launch_prefill_combine(p, c, a.part_ml, a.part_acc, a.win_part, out, out_dtype, st);
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
  ca.exact = p.exact;
  ca.i4_order = p.latent == LR_I4G32;
  ca.nrng = p.bal ? (const int*)(w + p.off_rng) + 4 * p.nwg : nullptr;
  memset(&ca.fin, 0, sizeof(ca.fin));
  if (step) {
    ca.fin.k_new = (const __bf16*)step_k_new;
    ca.fin.v_new = (const __bf16*)step_v_new;
    ca.fin.kwin = (__bf16*)c->kwin;
    ca.fin.vwin = (__bf16*)c->vwin;
    ca.fin.lat_len = c->lat_len;
    ca.fin.win_len = c->win_len;
    ca.fin.t_cap = p.t_cap;
    ca.fin.D = p.D;
    ca.fin.window = p.window;
  }
  const size_t lds = (size_t)(p.nsplit + p.rv_pad16 + 4 * (p.rv_pad16 > 512 ? p.rv_pad16 : 512) + 8) * sizeof(float);
  const dim3 cgrid(p.B * p.Hq);
  const bool f32b = p.latent == LR_F32;
  const bool f32o = out_dtype == LR_F32;
  if (f32b && f32o) hipLaunchKernelGGL((lr_combine<float, float, false>), cgrid, dim3(256), lds, st, ca);
  else if (f32b) hipLaunchKernelGGL((lr_combine<float, __bf16, false>), cgrid, dim3(256), lds, st, ca);
  else if (f32o) hipLaunchKernelGGL((lr_combine<__bf16, float, true>), cgrid, dim3(256), lds, st, ca);
  else hipLaunchKernelGGL((lr_combine<__bf16, __bf16, true>), cgrid, dim3(256), lds, st, ca);
  return hipGetLastError();
}

}  // namespace lr
