// Chunked prefill over a low-rank latent cache: the latent part as one dense product per token
// group (TraceKV, "TraceKV: Policy-Preserving Low-Rank KV Cache Compression for Reasoning
// Vision-Language Models", abstract: attention runs on the low-dimensional latents; iS-KV,
// "iS-KV: Online Low-Rank KV Cache Compression via Block-Incremental SVD", abstract: the recent
// tokens stay exact).
//
// Every token of a prefill chunk attends to the same latent prefix [0, lat_len) of its sequence
// without a mask (the chunk's own rows and the window are exact keys, handled by the decode
// kernel's exact-keys workgroups), so the latent part is a plain dense attention of the chunk's
// C x 32 folded query rows against the latent rows. lr_prefill_latent gives each wave one chunk
// token's 16-row head blocks (one or both) of the folded query (heads padded from the query heads
// to 32) for the whole latent range, so every latent byte brought into LDS feeds all of a
// workgroup's four tokens and both head blocks:
//
//   S^T[16 tokens, 16 heads] = Zk qt^T           16x16x32 bf16, K = rank (A = latent rows)
//   online softmax in base 2                      (reference max with slack, as in decode)
//   A^T[16 rv, 16 heads] += Zv^T P^T              16x16x32 bf16, K = a pair of tiles' 32 tokens
//
// Workgroup = 4 chunk tokens, as 8 waves of one (token, head block) each (two waves per SIMD: the
// accumulators of one head block over the full value rank fit half the register file) or 4 waves
// of one token with both head blocks (one wave per SIMD; ~430 registers), chosen by the length of
// the token range (launch_prefill_latent). All waves load the LDS ring with 16-byte
// direct-to-LDS loads, cached (the token groups of a range share its rows through L2), each wave
// waiting for exactly its own loads, one barrier per pair of 16-token tiles (per tile when the
// ring holds only 4 stages); the value products contract a pair of tiles at once (K = 32
// tokens). The partials (m, l, A) per
// (query token, token range), A in fp16, have the decode layout; lr_prefill_combine merges them
// with the exact-keys partials and up-projects.
#include <hip/hip_ext.h>

#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace lr {

namespace {

typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 pf_bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short pf_s16x4;
typedef __attribute__((__vector_size__(4 * sizeof(_Float16)))) _Float16 pf_f16x4;

constexpr float kPfMaxLead = 64.f;       // base-2 lead of a score over the reference max that
                                         // pass 0 tolerates (p <= 2^64: finite in bf16 and f32)
constexpr int kPfTokens = 4;             // chunk tokens per workgroup
// NHB = head blocks per wave: 2 (4 waves, one chunk token each) or 1 (8 waves, one (token, head
// block) each); waves, threads and 1 KB direct-to-LDS chunks per wave per matrix and tile
constexpr int pf_waves(int nhb) { return nhb == 2 ? 4 : 8; }
constexpr int pf_threads(int nhb) { return 64 * pf_waves(nhb); }
constexpr int pf_max_chunks(int nhb) { return nhb == 2 ? 5 : 3; }

// 16 bytes per lane straight into LDS, cached: the token groups of a range read the same rows
// through their XCD's L2
__device__ __forceinline__ void pf_dma16(const void* g, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(g, LR_LDS(lds_wave_base), 16, 0, 0);
}

// Value operand of the 16x16x16 product (A = Zv^T, K = token) through the gfx950 transpose
// read: in each 16-lane group g, lane j's element e comes from the address of lane 16g + 4e +
// j/4 at element offset j%4, so lane 16g + 4e + q points at row 4g + e, column 4q of the block.
__device__ __forceinline__ pf_bf16x4 pf_vread(const unsigned char* p) {
  return __builtin_bit_cast(pf_bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                           (__attribute__((address_space(3))) pf_s16x4*)(p)));
}

__device__ __forceinline__ bf16x8 pf_zero8() { return __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u}); }

}  // namespace

struct PrefillArgs {
  const unsigned char* zk;
  const unsigned char* zv;
  const __bf16* qt;          // [query sequences][32][rk_pad] folded queries (bf16)
  const int32_t* lat_len;
  float* part_ml;            // [query sequence][nsplit][Hq][2]
  float* part_acc;           // [query sequence][nsplit][Hq][rv_pad16] as fp16
  long long t_cap;
  int row_bytes_k, row_bytes_v, copy_k, copy_v;
  int rk, rk_pad, nks, nrb, rv_pad16;
  int nsplit, split_tokens, max_len;
  int Hq, C;                 // query heads; query tokens per stored sequence (the chunk)
  int ntg, nunits, nst;      // token groups per sequence, units (sequence x range), ring stages
};

// KS: bound on K steps of 32 (nks <= KS); NV: bound on value blocks of 16 (nrb <= NV); NHB: head
// blocks per wave.
template <int KS, int NV, int NHB>
__global__ __launch_bounds__(pf_threads(NHB)) void lr_prefill_latent(PrefillArgs a) {
  constexpr int kPfWaves = pf_waves(NHB), kPfThreads = pf_threads(NHB), kPfMaxChunks = pf_max_chunks(NHB);
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  constexpr int SK = lds_stride_k(KS, 2);              // LDS row strides (bytes), as in decode
  constexpr int SV = lds_stride_v(NV / 2, 2);
  constexpr int ZV = kTileTokens * SK;
  constexpr int STAGE = kTileTokens * (SK + SV);
  static_assert((kTileTokens * SK + 1023) / 1024 <= kPfWaves * kPfMaxChunks &&
                (kTileTokens * SV + 1023) / 1024 <= kPfWaves * kPfMaxChunks, "DMA chunks");
  const int NST = a.nst;

  // workgroup -> (unit u = sequence x token range, token group tg). The token groups of a unit
  // take workgroup indices of one residue mod 8, so they run on one XCD and share its L2.
  const int wgi = blockIdx.x;
  const int tg = (wgi >> 3) % a.ntg;
  const int u = ((wgi >> 3) / a.ntg) * 8 + (wgi & 7);
  if (u >= a.nunits) return;                           // whole workgroup, before any barrier
  const int b = u / a.nsplit, s = u - b * a.nsplit;
  const int tid = threadIdx.x, lane = tid & 63, lg = lane >> 4, li = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tok = tg * kPfTokens + (NHB == 2 ? wave : wave >> 1);   // chunk token of this wave
  const int hb0 = NHB == 2 ? 0 : wave & 1;             // its first head block (heads 16 hb0 ..)
  const bool active = tok < a.C;                       // idle waves still load and meet barriers
  const int sq = b * a.C + tok;

  int L = a.lat_len[b];
  L = L < 0 ? 0 : (L > a.max_len ? a.max_len : L);
  const int t_begin = s * a.split_tokens;
  const int t_end = min(t_begin + a.split_tokens, L);
  const int ntiles = t_end > t_begin ? (t_end - t_begin + kTileTokens - 1) / kTileTokens : 0;

  // Zero, once, the LDS columns of every stage row that no load writes (K steps and value
  // blocks past the rank read as exact zeros). Disjoint from every loaded byte; the first
  // barrier orders them before any read.
  {
    constexpr int KB = KS * 64, VB = NV * 32;
    const int npk = (KB - a.copy_k) >> 4, npv = (VB - a.copy_v) >> 4;
    const int per_stage = kTileTokens * (npk + npv);
    for (int i = tid; i < NST * per_stage; i += kPfThreads) {
      const int st = i / per_stage, j = i - st * per_stage;
      unsigned char* p;
      if (j < kTileTokens * npk) {
        const int row = j / npk, gk = j - row * npk;
        p = smem + st * STAGE + row * SK + a.copy_k + gk * 16;
      } else {
        const int jj = j - kTileTokens * npk;
        const int row = jj / npv, gv = jj - row * npv;
        p = smem + st * STAGE + ZV + row * SV + a.copy_v + gv * 16;
      }
      *(u32x4*)p = u32x4{0u, 0u, 0u, 0u};
    }
  }

  // ---- direct-to-LDS loads: chunk c (1 KB of a stage's K or V region) belongs to wave c % 4;
  // lane l of the chunk lands at c*1024 + 16*l, i.e. at (row, col) of the region's row stride.
  const unsigned char* gk = a.zk + ((size_t)b * a.t_cap + t_begin) * a.row_bytes_k;
  const unsigned char* gv = a.zv + ((size_t)b * a.t_cap + t_begin) * a.row_bytes_v;
  int offk[kPfMaxChunks], offv[kPfMaxChunks];
#pragma unroll
  for (int k = 0; k < kPfMaxChunks; ++k) {
    const int o = (wave + kPfWaves * k) * 1024 + lane * 16;
    int row = o / SK, col = o - row * SK;
    offk[k] = (col < a.copy_k) ? row * a.row_bytes_k + col : -1;
    row = o / SV;
    col = o - row * SV;
    offv[k] = (col < a.copy_v) ? row * a.row_bytes_v + col : -1;
  }
  // chunks holding at least one loaded byte of a tile with `rows` rows (each such chunk is one
  // load instruction of its wave: at least one lane is active in it)
  auto nchunks = [](int rows, int stride, int cp) { return ((rows - 1) * stride + cp + 1023) >> 10; };
  auto pcnt = [&](int nch) { return nch > wave ? (nch - wave + kPfWaves - 1) / kPfWaves : 0; };
  auto tile_cnt = [&](int rows) { return pcnt(nchunks(rows, SK, a.copy_k)) + pcnt(nchunks(rows, SV, a.copy_v)); };
  const int rows_last = ntiles > 0 ? t_end - (t_begin + (ntiles - 1) * kTileTokens) : 0;
  const int cnt_full = tile_cnt(kTileTokens);
  const int cnt_last = ntiles > 0 ? tile_cnt(rows_last) : 0;
  auto count = [&](int lo, int hi) {     // this wave's loads for tiles lo+1 .. hi (hi <= ntiles - 1)
    if (hi <= lo) return 0;
    return (hi - lo) * cnt_full + (hi == ntiles - 1 ? cnt_last - cnt_full : 0);
  };
  // whether this lane loads 16 bytes of chunk k of a full tile (16 rows), and whether they are the
  // key granule holding latent index rk: fixed for the whole range, so a full tile's loads test
  // one precomputed lane flag each (the partial last tile takes the general conditions)
  const int nck16 = nchunks(kTileTokens, SK, a.copy_k), ncv16 = nchunks(kTileTokens, SV, a.copy_v);
  bool fk[kPfMaxChunks], fv[kPfMaxChunks], ft[kPfMaxChunks];
#pragma unroll
  for (int k = 0; k < kPfMaxChunks; ++k) {
    const int c = wave + kPfWaves * k;
    fk[k] = c < nck16 && offk[k] >= 0 && offk[k] < kTileTokens * a.row_bytes_k;
    fv[k] = c < ncv16 && offv[k] >= 0 && offv[k] < kTileTokens * a.row_bytes_v;
    ft[k] = fk[k] && (c * 1024 + lane * 16) % SK == a.copy_k - 16;
  }
  // tile t into stage stg (the callers track stages incrementally)
  auto issue = [&](int t, unsigned char* stg) {
    const int t0 = t * kTileTokens;
    const int rows = min(kTileTokens, t_end - t_begin - t0);
    const unsigned char* srck = gk + (size_t)t0 * a.row_bytes_k;
    const unsigned char* srcv = gv + (size_t)t0 * a.row_bytes_v;
    if (rows == kTileTokens) {
#pragma unroll
      for (int k = 0; k < kPfMaxChunks; ++k)
        if (fk[k]) pf_dma16(srck + offk[k], stg + (wave + kPfWaves * k) * 1024);
#pragma unroll
      for (int k = 0; k < kPfMaxChunks; ++k)
        if (fv[k]) pf_dma16(srcv + offv[k], stg + ZV + (wave + kPfWaves * k) * 1024);
      return;
    }
    {
      // the stage's value rows past the range end still hold an older tile (possibly NaN
      // patterns): zero them, so that P = 0 meets 0 there (plain LDS stores, published by the
      // barrier that precedes the tile's use)
      const int ng = (kTileTokens - rows) * (NV * 2);          // 16-byte granules (NV*32 bytes a row)
      for (int g = wave * 64 + lane; g < ng; g += kPfThreads) {
        const int row = rows + g / (NV * 2), col = (g % (NV * 2)) * 16;
        *(u32x4*)(stg + ZV + row * SV + col) = u32x4{0u, 0u, 0u, 0u};
      }
    }
    const int nck = nchunks(rows, SK, a.copy_k), ncv = nchunks(rows, SV, a.copy_v);
    const int limk = rows * a.row_bytes_k, limv = rows * a.row_bytes_v;
#pragma unroll
    for (int k = 0; k < kPfMaxChunks; ++k) {
      const int c = wave + kPfWaves * k;
      if (c < nck && offk[k] >= 0 && offk[k] < limk) pf_dma16(srck + offk[k], stg + c * 1024);
    }
#pragma unroll
    for (int k = 0; k < kPfMaxChunks; ++k) {
      const int c = wave + kPfWaves * k;
      if (c < ncv && offv[k] >= 0 && offv[k] < limv) pf_dma16(srcv + offv[k], stg + ZV + c * 1024);
    }
  };

  // The key granule that holds latent index rk (when rk is not a multiple of 8) also holds
  // pad columns of the stored row, which may hold anything: the lane that loaded it clears
  // them in LDS once its load has landed (before the barrier that publishes the tile), so the
  // score products see exact zeros there.
  u32x4 gmask;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = (a.rk & 7);
    gmask[i] = (2 * i < e ? 0x0000FFFFu : 0u) | (2 * i + 1 < e ? 0xFFFF0000u : 0u);
  }
  const bool ktail = (a.rk & 7) != 0;
  auto fix_tail = [&](int t, unsigned char* stg) {
    if (!ktail) return;
    const int rows = min(kTileTokens, t_end - t_begin - t * kTileTokens);
    if (rows == kTileTokens) {
#pragma unroll
      for (int k = 0; k < kPfMaxChunks; ++k) {
        if (ft[k]) {
          u32x4* p = (u32x4*)(stg + (wave + kPfWaves * k) * 1024 + lane * 16);
          *p = *p & gmask;
        }
      }
      return;
    }
    const int nck = nchunks(rows, SK, a.copy_k), limk = rows * a.row_bytes_k;
#pragma unroll
    for (int k = 0; k < kPfMaxChunks; ++k) {
      const int c = wave + kPfWaves * k;
      const int o = c * 1024 + lane * 16;
      if (c < nck && offk[k] >= 0 && offk[k] < limk && o % SK == a.copy_k - 16) {
        u32x4* p = (u32x4*)(stg + o);
        *p = *p & gmask;
      }
    }
  };

  // ---- this wave's folded query (its head blocks) as B operands: lane (lg, li) holds head
  // 16*(hb0+h) + li, latent indices 32*ks + 8*lg .. +7
  bf16x8 qop[NHB][KS];
  {
    const __bf16* qrow = a.qt + ((size_t)(active ? sq : 0) * kHeadsPad + hb0 * 16 + li) * a.rk_pad + lg * 8;
#pragma unroll
    for (int h = 0; h < NHB; ++h)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        qop[h][ks] = (active && ks < a.nks) ? *(const bf16x8*)(qrow + (size_t)h * 16 * a.rk_pad + ks * 32)
                                            : pf_zero8();
  }
  const int krow_off = li * SK + lg * 16;
  const int vrow_off = ZV + (4 * lg + (li >> 2)) * SV + (li & 3) * 8;

  // Rescale-free online softmax. The accumulators live in the accumulation registers, which
  // vector ALU instructions cannot touch, so no pass ever rescales them:
  //   pass 0: each head's reference max mref is its first tile's max; scores exponentiate
  //           against it (p <= 2^kPfMaxLead keeps P, l and A finite); a tile whose max leads
  //           mref by more than kPfMaxLead marks the workgroup;
  //   pass 1 (marked workgroups only): the exact max of every head over the range (scores only);
  //   pass 2 (marked only): pass 0 with mref fixed to that max, which no score exceeds.
  // Each pass is its own loop, so the accumulators' loop-carried values never merge with a
  // path that skips the products.

  // streams the range's tiles through the ring, calling body(stage, valid rows) per tile (the
  // exact-max pass; the full passes use the pipelined stream_full below)
  // stage of the tile after the one in stage p
  auto next_stage = [&](unsigned char* p) { return p + STAGE == smem + NST * STAGE ? smem : p + STAGE; };
  auto stream = [&](auto&& body) {
    const int pro = min(NST - 1, ntiles);
    for (int t = 0; t < pro; ++t) issue(t, smem + t * STAGE);
    wait_vmcnt(count(0, pro - 1));                     // tile 0 landed (this wave's part)
    if (ntiles > 0) fix_tail(0, smem);
    barrier_lds();
    unsigned char* s_cur = smem;                       // stage of tile it
    unsigned char* s_iss = smem + (NST - 1) * STAGE;   // stage of tile it + NST - 1
    for (int it = 0; it < ntiles; ++it) {
      // stage of tile it - 1: every wave finished reading it before the last barrier
      if (it + NST - 1 < ntiles) issue(it + NST - 1, s_iss);
      body(s_cur, min(kTileTokens, t_end - t_begin - it * kTileTokens));
      wait_vmcnt(count(it + 1, min(it + NST - 1, ntiles - 1)));   // tile it + 1 landed
      s_cur = next_stage(s_cur);
      s_iss = next_stage(s_iss);
      if (it + 1 < ntiles) fix_tail(it + 1, s_cur);
      barrier_lds();
    }
  };
  // raw score products of this wave's head blocks for one tile: sacc[h][i] = S^T[token 4*lg+i]
  // [head 16*(hb0+h)+li] (waves without a token compute on a zero query); with one head block,
  // two accumulation chains (even and odd K steps)
  auto products = [&](const unsigned char* stg, f32x4 (&sacc)[NHB]) {
    const unsigned char* krow = stg + krow_off;
    f32x4 s2[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int ks0 = 0; ks0 < KS; ks0 += 4) {
      bf16x8 av[4];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (ks0 + k < KS) av[k] = *(const bf16x8*)(krow + (ks0 + k) * 64);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if (ks0 + k < KS) {
          if constexpr (NHB == 2) {
            s2[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[k], qop[0][ks0 + k], s2[0], 0, 0, 0);
            s2[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[k], qop[1][ks0 + k], s2[1], 0, 0, 0);
          } else {
            s2[k & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[k], qop[0][ks0 + k], s2[k & 1], 0, 0, 0);
          }
        }
      }
    }
    if constexpr (NHB == 2) {
      sacc[0] = s2[0];
      sacc[1] = s2[1];
    } else {
      sacc[0] = s2[0] + s2[1];
    }
  };
  // masked base-2 scores from the raw products (rows past the range end -inf; NaN -> +inf so
  // that it survives the max and poisons only its head) and the tile's max per head
  auto masked = [&](const f32x4 (&sacc)[NHB], int nvalid, float (&v)[NHB][4], float (&mx)[NHB]) {
#pragma unroll
    for (int h = 0; h < NHB; ++h) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x = sacc[h][i];
        v[h][i] = (4 * lg + i < nvalid) ? ((x != x) ? INFINITY : x) : -INFINITY;
      }
      mx[h] = wave_max_lg(fmaxf(fmaxf(v[h][0], v[h][1]), fmaxf(v[h][2], v[h][3])));
    }
  };
  auto scores = [&](const unsigned char* stg, int nvalid, float (&v)[NHB][4], float (&mx)[NHB]) {
    f32x4 sacc[NHB];
    products(stg, sacc);
    masked(sacc, nvalid, v, mx);
  };

  float mref[NHB], lsum[NHB];
  f32x4 acc[NHB][NV];
#pragma unroll
  for (int h = 0; h < NHB; ++h) {
    mref[h] = -INFINITY;
    lsum[h] = 0.f;
#pragma unroll
    for (int j = 0; j < NV; ++j) acc[h][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  bool bad = false;
  // Softmax of one tile, then its value products. The 16x16x16 products take as long per
  // instruction as the 16x16x32 ones (measured on gfx950: 1.2 against 2.3 PFLOP/s), so tiles go
  // in pairs: mode 0 keeps the first tile's P in registers (pdef) and does no products; mode 1
  // contracts both tiles at once, K = 32 tokens: slots 0-3 of lane group lg hold tokens 4 lg ..
  // 4 lg + 3 of the first tile and slots 4-7 the same tokens of the second, which is how the two
  // score tiles and the two transpose reads land (no shuffle); mode 2 is a lone last tile, K = 16.
  // No pass rescales, so a deferred P stays valid.
  pf_bf16x4 pdef[NHB];
  auto finish = [&](auto mode_c, const unsigned char* stg, const unsigned char* sprev, int nvalid,
                    const f32x4 (&sacc)[NHB]) {
    constexpr int MODE = decltype(mode_c)::value;
    float v[NHB][4], mx[NHB];
    masked(sacc, nvalid, v, mx);
    // first value operands in flight under the softmax (a pair reads two per block: 4 blocks in
    // flight past 24 blocks, where 8 would spill)
    constexpr int VC = (MODE == 1 && NV > 24) ? 4 : 8;
    const unsigned char* vbase = stg + vrow_off;
    const unsigned char* pbase = sprev + vrow_off;
    pf_bf16x4 vop[VC], vpr[VC];
    if constexpr (MODE != 0) {
#pragma unroll
      for (int k = 0; k < VC; ++k) vop[k] = pf_vread(vbase + k * 32);
    }
    if constexpr (MODE == 1) {
#pragma unroll
      for (int k = 0; k < VC; ++k) vpr[k] = pf_vread(pbase + k * 32);
    }
    pf_bf16x4 pb[NHB];
#pragma unroll
    for (int h = 0; h < NHB; ++h) {
      // a head without a reference yet takes this tile's max: its A and l are still 0
      if (mref[h] == -INFINITY) mref[h] = mx[h];
      bad = bad || (mx[h] > mref[h] + kPfMaxLead);
      const bool live = mref[h] != -INFINITY;
      float ps = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const __bf16 pv = (__bf16)(live ? fast_exp2(v[h][i] - mref[h]) : 0.f);
        pb[h][i] = pv;
        ps += (float)pv;
      }
      lsum[h] += ps;
    }
    if constexpr (MODE == 0) {
#pragma unroll
      for (int h = 0; h < NHB; ++h) pdef[h] = pb[h];
      return;
    }
    bf16x8 pb8[NHB];
#pragma unroll
    for (int h = 0; h < NHB; ++h) pb8[h] = __builtin_shufflevector(pdef[h], pb[h], 0, 1, 2, 3, 4, 5, 6, 7);
    // values: A^T[rv][head li] of the wave's head blocks, one operand read per block and tile
#pragma unroll
    for (int j0 = 0; j0 < NV; j0 += VC) {
      if (j0 > 0) {
#pragma unroll
        for (int k = 0; k < VC; ++k) {
          if (j0 + k < NV) {
            vop[k] = pf_vread(vbase + (j0 + k) * 32);
            if constexpr (MODE == 1) vpr[k] = pf_vread(pbase + (j0 + k) * 32);
          }
        }
      }
#pragma unroll
      for (int k = 0; k < VC; ++k)
        if (j0 + k < NV)
#pragma unroll
          for (int h = 0; h < NHB; ++h) {
            if constexpr (MODE == 1)
              acc[h][j0 + k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  __builtin_shufflevector(vpr[k], vop[k], 0, 1, 2, 3, 4, 5, 6, 7), pb8[h], acc[h][j0 + k], 0, 0, 0);
            else
              acc[h][j0 + k] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vop[k], pb[h], acc[h][j0 + k], 0, 0, 0);
          }
    }
  };

  // The full passes, software-pipelined by one tile: step it issues tile it + 1's score products
  // before tile it's softmax and value products, so the matrix cores work on the former while the
  // latter's ALU work runs. A pair's value products run in the step of its second tile, so tile
  // it - 1 is still read in step it. Each loop iteration takes one pair of tiles in two
  // straight-line steps, so the accumulators' loop-carried values never merge with a path that
  // skips the products.
  // Publication: with at least 5 stages, only the first step of a pair meets the workgroup
  // barrier: it publishes tiles it + 1 and it + 2 (the next step's score products need the
  // latter) and refills the stages of tiles it - 2 and it - 1 (the pair before, finished before
  // that barrier) with tiles it + NST - 2 and it + NST - 1. With 4 stages every step meets the
  // barrier, publishes tile it + 1 and refills the stage of tile it - 2 with tile it + NST - 2.
  // Either way tile t lives in stage t mod NST, and before step it tiles up to it + NST - 3 are
  // issued.
  auto stream_full = [&]() {
    const bool pairb = NST >= 5;
    const int pro = min(NST - 2, ntiles);                // tiles 0 .. NST - 3
    for (int t = 0; t < pro; ++t) issue(t, smem + t * STAGE);
    wait_vmcnt(count(0, pro - 1));                     // tile 0 landed (this wave's part)
    if (ntiles > 0) fix_tail(0, smem);
    barrier_lds();
    unsigned char* s_prv = smem;                       // stage of tile it - 1
    unsigned char* s_cur = smem;                       // stage of tile it
    unsigned char* s_nxt = next_stage(smem);           // stage of tile it + 1
    unsigned char* s_iss = smem + (NST - 2) * STAGE;   // stage of tile it + NST - 2 (= it - 2)
    f32x4 cur[NHB];
    if (ntiles > 0) products(smem, cur);
    auto step = [&](int it, auto mode_c) {
      constexpr int MODE = decltype(mode_c)::value;
      if (!pairb || MODE != 1) {
        const int last = min(it + (pairb ? 2 : 1), ntiles - 1);   // last tile this step publishes
        if (it + 1 < ntiles) {
          wait_vmcnt(count(last, min(it + NST - 3, ntiles - 1)));
          fix_tail(it + 1, s_nxt);
          if (last > it + 1) fix_tail(last, next_stage(s_nxt));
        }
        barrier_lds();
        if (it + NST - 2 < ntiles) issue(it + NST - 2, s_iss);
        if (pairb && it + NST - 1 < ntiles) issue(it + NST - 1, next_stage(s_iss));
      }
      f32x4 nxt[NHB];
      products(s_nxt, nxt);                            // (last step: a stale stage, unused)
      finish(mode_c, s_cur, s_prv, min(kTileTokens, t_end - t_begin - it * kTileTokens), cur);
      s_prv = s_cur;
      s_cur = s_nxt;
      s_nxt = next_stage(s_nxt);
      s_iss = next_stage(s_iss);
#pragma unroll
      for (int h = 0; h < NHB; ++h) cur[h] = nxt[h];
      // interleave the next tile's score products with this tile's softmax: one matrix-core
      // instruction, then three vector ALU instructions, once per score product
#pragma unroll
      for (int k = 0; k < NHB * KS; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
      }
    };
    for (int it = 0; it + 1 < ntiles; it += 2) {
      step(it, std::integral_constant<int, 0>{});
      step(it + 1, std::integral_constant<int, 1>{});
    }
    if (ntiles & 1) step(ntiles - 1, std::integral_constant<int, 2>{});
  };
  int* flag = (int*)(smem + NST * STAGE + 64);         // in the slack after the ring
  if (tid == 0) *flag = 0;                             // ordered by the first barrier of the stream
  stream_full();                                       // pass 0
  // any wave with a lead beyond kPfMaxLead sends the whole workgroup through passes 1-2
  if (__builtin_amdgcn_ballot_w64(bad) != 0 && lane == 0) *flag = 1;
  barrier_lds();
  if (*flag != 0) {
    float mexact[NHB];
#pragma unroll
    for (int h = 0; h < NHB; ++h) mexact[h] = -INFINITY;
    stream([&](const unsigned char* stg, int nvalid) {   // pass 1
      float v[NHB][4], mx[NHB];
      scores(stg, nvalid, v, mx);
#pragma unroll
      for (int h = 0; h < NHB; ++h) mexact[h] = fmaxf(mexact[h], mx[h]);
    });
#pragma unroll
    for (int h = 0; h < NHB; ++h) {
      mref[h] = mexact[h];
      lsum[h] = 0.f;
#pragma unroll
      for (int j = 0; j < NV; ++j) acc[h][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    stream_full();                                     // pass 2
  }

  if (!active) return;
  // The partial (m, l, A) of each (chunk token, range, head), A in fp16 with a power of two per
  // row folded into (m, l): the head's largest |A| is brought into [2^14, 2^15) by A' = A 2^-e,
  // and (m', l') = (m + e, l 2^-e), so 2^(m' - m*) A' = 2^(m - m*) A for any reference m* of the
  // combine. One rounding to 11 significant bits (at most 2^-12 of the row's largest value per
  // element), and half the bytes written here and read by the combine.
  const size_t pidx = (size_t)sq * a.nsplit + s;
#pragma unroll
  for (int h = 0; h < NHB; ++h) {
    float l = wave_sum_lg(lsum[h]);
    float mxa = 0.f;
#pragma unroll
    for (int j = 0; j < NV; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) mxa = fmaxf(mxa, fabsf(acc[h][j][e]));
    mxa = wave_max_lg(mxa);                          // the head's 4 lane groups
    int ex = 0;
    if (mxa > 0.f && mxa <= 3.4e38f) {               // 0, inf and NaN keep e = 0
      ex = ilogbf(mxa) - 14;
      ex = ex < -100 ? -100 : (ex > 100 ? 100 : ex);
    }
    const float psc = ldexpf(1.f, -ex);
    const float mw = mref[h] == -INFINITY ? mref[h] : mref[h] + (float)ex;
    l *= psc;
    const int head = (hb0 + h) * 16 + li;
    if (head >= a.Hq) continue;
    if (lg == 0) {
      a.part_ml[(pidx * a.Hq + head) * 2] = mw;
      a.part_ml[(pidx * a.Hq + head) * 2 + 1] = l;
    }
    _Float16* pa = (_Float16*)a.part_acc + (pidx * a.Hq + head) * a.rv_pad16 + 4 * lg;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      if (j < a.nrb) {
        pf_f16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (_Float16)(acc[h][j][e] * psc);
        *(pf_f16x4*)(pa + j * 16) = v;
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Exact keys of a prefill chunk (iS-KV abstract: the recent tokens stay exact): the live window
// slots, then the chunk's own rows, causally. Workgroup = (stored sequence b, KV head g, 64 of
// the C * grp query rows of that head's group; row = token c * grp + head h), one 16-row block
// per wave. Keys are staged 32 at a time in LDS (the head's 128-wide slice of K and V) and shared
// by the workgroup's rows:
//   S^T[16 keys, 16 rows] = K q^T          16x16x32 bf16 (fp32 sum), times sm_scale * log2 e
//   online softmax in base 2 (key j is visible to row (c, h) when j < live window + c + 1)
//   O^T[16 d, 16 rows] += V^T P^T           16x16x16 bf16 through the transpose read
// The partial (O, m, l) per (query token, head) has the layout of the decode kernel's
// exact-keys partial, so the combine merges it unchanged.
// ---------------------------------------------------------------------------------------------
constexpr int kExKeys = 32;               // keys per staged tile

__global__ __launch_bounds__(256) void lr_prefill_exact(ExactArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char kt[kExKeys * kExSK];
  __shared__ __attribute__((aligned(16))) unsigned char vt[kExKeys * kExSV];
  const int grp = a.Hq / a.Hkv;
  const int rb = blockIdx.x % a.nrb;
  const int g = (blockIdx.x / a.nrb) % a.Hkv;
  const int b = blockIdx.x / (a.nrb * a.Hkv);
  const int tid = threadIdx.x, lane = tid & 63, lg = lane >> 4, li = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nrows = a.C * grp;
  const int row0 = rb * 64 + wave * 16;              // first row of this wave's block
  const int row = row0 + li;                         // this lane's row (as B-operand column)
  const bool rvalid = row < nrows;
  const int c = rvalid ? row / grp : 0, h = rvalid ? row - c * grp : 0;
  int L = a.lat_len[b];
  L = L < 0 ? 0 : L;
  int wl = a.W > 0 ? a.win_len[b] : 0;
  wl = wl < 0 ? 0 : (wl > a.W ? a.W : wl);
  // chunk rows as keys (causal): the prefill's own rows; none for a decode step, whose new token
  // is already a window slot
  const bool chunk_keys = a.kchunk != nullptr;
  const int nkeys = wl + (chunk_keys ? a.C : 0);
  // keys this wave's rows can see: up to the last valid row's token
  const int c_hi = min(row0 + 15, nrows - 1) / grp;
  const int wave_keys = row0 < nrows ? wl + (chunk_keys ? c_hi + 1 : 0) : 0;
  const int my_keys = rvalid ? wl + (chunk_keys ? c + 1 : 0) : 0;

  // q of this lane's row as the B operand: d indices 32 ks + 8 lg .. +7
  bf16x8 qop[4];
  {
    const __bf16* qr = a.q + (((size_t)b * a.C + c) * a.Hq + g * grp + h) * kExD + lg * 8;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qop[ks] = rvalid ? *(const bf16x8*)(qr + ks * 32) : pf_zero8();
  }
  float m = -INFINITY, lsum = 0.f;
  f32x4 acc[kExD / 16];
#pragma unroll
  for (int j = 0; j < kExD / 16; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int t0 = 0; t0 < nkeys; t0 += kExKeys) {
    __syncthreads();                                 // the previous tile is no longer read
    // stage keys t0 .. t0+31 (head g's slice): 16 granules of 16 bytes per row and matrix
    for (int i = tid; i < kExKeys * 16; i += 256) {
      const int r = i >> 4, gc = i & 15;
      const int j = t0 + r;
      u32x4 kv = u32x4{0u, 0u, 0u, 0u}, vv = u32x4{0u, 0u, 0u, 0u};
      if (j < nkeys) {
        const __bf16 *ks, *vs;
        if (j < wl) {
          const size_t src = ((size_t)b * a.W + (L + j) % a.W) * a.D + g * kExD + gc * 8;
          ks = a.kwin + src;
          vs = a.vwin + src;
        } else {
          const size_t src = ((size_t)b * a.C + (j - wl)) * a.D + g * kExD + gc * 8;
          ks = a.kchunk + src;
          vs = a.vchunk + src;
        }
        kv = *(const u32x4*)ks;
        vv = *(const u32x4*)vs;
      }
      *(u32x4*)(kt + r * kExSK + gc * 16) = kv;
      *(u32x4*)(vt + r * kExSV + gc * 16) = vv;
    }
    __syncthreads();
    if (t0 >= wave_keys) continue;                   // nothing this wave's rows can see
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int k0 = t0 + half * 16;
      if (k0 >= wave_keys) break;
      // scores S^T[key k0 + 4 lg + i][row li]
      f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
      const unsigned char* krow = kt + (half * 16 + li) * kExSK + lg * 16;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(const bf16x8*)(krow + ks * 64), qop[ks], sacc, 0, 0, 0);
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x = sacc[i] * a.wscale;
        v[i] = (k0 + 4 * lg + i < my_keys) ? ((x != x) ? INFINITY : x) : -INFINITY;
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
      pf_bf16x4 pb;
      float ps = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const __bf16 pv = (__bf16)(live ? fast_exp2(v[i] - m) : 0.f);
        pb[i] = pv;
        ps += (float)pv;
      }
      lsum += ps;
      const unsigned char* vbase = vt + (half * 16 + 4 * lg + (li >> 2)) * kExSV + (li & 3) * 8;
#pragma unroll
      for (int j = 0; j < kExD / 16; ++j)
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pf_vread(vbase + j * 32), pb, acc[j], 0, 0, 0);
    }
  }
  const float l = wave_sum_lg(lsum);
  if (!rvalid) return;
  float* wp = a.win_part + (((size_t)b * a.C + c) * a.Hq + g * grp + h) * (kExD + 2);
#pragma unroll
  for (int j = 0; j < kExD / 16; ++j) *(f32x4*)(wp + j * 16 + 4 * lg) = acc[j];
  if (lg == 0) {
    wp[kExD] = m;
    wp[kExD + 1] = l;
  }
}

hipError_t launch_prefill_exact(const DecodePlan& p, const lr_layer_cache* c, const void* q, const void* k_chunk,
                                const void* v_chunk, float* win_part, hipStream_t st) {
  ExactArgs a;
  a.q = (const __bf16*)q;
  a.kwin = (const __bf16*)c->kwin;
  a.vwin = (const __bf16*)c->vwin;
  a.kchunk = (const __bf16*)k_chunk;
  a.vchunk = (const __bf16*)v_chunk;
  a.lat_len = c->lat_len;
  a.win_len = c->win_len;
  a.win_part = win_part;
  a.C = p.qpb;
  a.Hq = p.Hq;
  a.Hkv = p.Hkv;
  a.D = p.D;
  a.W = p.window;
  a.wscale = p.sm_scale * kLog2e;
  a.nrb = (p.qpb * (p.Hq / p.Hkv) + 63) / 64;
  const int grid = (p.B / p.qpb) * p.Hkv * a.nrb;
  hipLaunchKernelGGL(lr_prefill_exact, dim3(grid), dim3(256), 0, st, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Combine of a prefill: for each (query token, head) merge the latent partials of the token
// ranges and the exact-keys partial (m* = max of the m's, weights 2^(m_s - m*), l* = sum w_s l_s,
// Ahat = sum w_s A_s, in float32) and up-project, out = (Ahat Bv[:, g] + w_x Ax) / l*.
// Workgroup = (stored sequence b, KV head g, up to 4 chunk tokens): its rows (token, head of the
// group) share Bv[:, g]. The up-projection runs on the matrix cores: Ahat is split into
// bf16 hi + lo (hi = bf16(a), lo = bf16(a - hi): a to about 2^-16 relative), Bv is bf16
// already, so O = hi Bv + lo Bv in two 16x16x32 products with float32 sums; Bv is staged 64
// rows at a time and read with the transpose read (K = its rows).
// ---------------------------------------------------------------------------------------------
constexpr int kCbMaxTokens = 4;                // chunk tokens per workgroup: 4, 2 or 1
constexpr int kCbChunk = 64;                   // rows of Bv staged at a time
constexpr int kCbBvStride = 128 * 2 + 32;      // LDS row stride (bytes) of the staged Bv rows

struct PfCombineArgs {
  const float* part_ml;     // [query sequence][nsplit][Hq][2]: (m, l), the row's 2^e folded in
  const float* part_acc;    // [query sequence][nsplit][Hq][rv_pad16] fp16 values scaled by 2^-e
  const float* win_part;
  const __bf16* bv;        // [rv][D]
  void* out;               // [B * C][Hq][d]
  int out_f32;
  int C, Hq, Hkv, D, rv, rv_pad16, nsplit, ntg;
  int tpw;                 // chunk tokens per workgroup
  int rows_alloc;          // tpw * (heads per group), rounded up to 16
  int kp;                  // rv rounded up to 64 (Ahat columns, zero past rv)
};

// B operand (K = 32 staged Bv rows from row k0, N = 16 columns from c0) by the transpose read:
// lane (g, j) receives column c0 + j of rows 8g .. 8g + 7 (lane 16g + 4e + q addresses row
// 8g + e, columns c0 + 4q .. +3; the second read the rows 4 further down).
__device__ __forceinline__ bf16x8 cb_bv_operand(const unsigned char* tile, int k0, int c0, int lane) {
  const int g = lane >> 4, e = (lane >> 2) & 3, q = lane & 3;
  const unsigned char* p = tile + (k0 + 8 * g + e) * kCbBvStride + (c0 + 4 * q) * 2;
  const pf_bf16x4 lo = pf_vread(p), hi = pf_vread(p + 4 * kCbBvStride);
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r[i] = lo[i];
    r[4 + i] = hi[i];
  }
  return r;
}

__global__ __launch_bounds__(256) void lr_prefill_combine(PfCombineArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char cmem[];
  const int grp = a.Hq / a.Hkv;
  const int tg = blockIdx.x % a.ntg;
  const int g = (blockIdx.x / a.ntg) % a.Hkv;
  const int b = blockIdx.x / (a.ntg * a.Hkv);
  const int c0 = tg * a.tpw;
  const int ntok = min(a.tpw, a.C - c0);
  const int R = ntok * grp;                      // rows: (token c0 + i / grp, head g*grp + i % grp)
  const int tid = threadIdx.x, lane = tid & 63, lg = lane >> 4, li = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ahs = a.kp + 4;                      // Ahat row stride (floats): rows spread over banks
  float* ahat = (float*)cmem;                    // [rows_alloc][ahs]
  float* rowx = ahat + a.rows_alloc * ahs;       // [rows_alloc][2]: weight of the exact-keys partial, l*
  float* rowm = rowx + 2 * a.rows_alloc;         // [rows_alloc]: m*
  unsigned char* bvs = (unsigned char*)(rowm + a.rows_alloc);   // [kCbChunk][kCbBvStride]

  // Bv rows r0 .. r0+63 of head g, four 16-byte granules per thread (zero past rv): loaded into
  // registers a chunk ahead (the first one before the merge), stored to LDS when it is consumed
  u32x4 pre[kCbChunk * 16 / 256];
  auto bv_load = [&](int r0) {
#pragma unroll
    for (int k = 0; k < kCbChunk * 16 / 256; ++k) {
      const int i = tid + 256 * k, r = i >> 4, q = i & 15;
      pre[k] = (r0 + r < a.rv) ? *(const u32x4*)(a.bv + (size_t)(r0 + r) * a.D + g * 128 + q * 8)
                               : u32x4{0u, 0u, 0u, 0u};
    }
  };
  bv_load(0);

  // ---- per row: m* (over the ranges and the exact-keys partial), its weight, l*
  if (tid < R) {
    const int rr = tid;
    const int sq = b * a.C + c0 + rr / grp, head = g * grp + rr % grp;
    const float* ml = a.part_ml + ((size_t)sq * a.nsplit * a.Hq + head) * 2;   // range s at + s*Hq*2
    const float* wp = a.win_part + ((size_t)sq * a.Hq + head) * 130;
    const float mw = wp[128], lw = wp[129];
    // ranges 8 at a time: their loads go out together (indices clamped, extra ones ignored)
    float mstar = mw;
    for (int s0 = 0; s0 < a.nsplit; s0 += 8) {
      float mv[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) mv[k] = ml[(size_t)min(s0 + k, a.nsplit - 1) * a.Hq * 2];
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (s0 + k < a.nsplit) mstar = fmaxf(mstar, mv[k]);
    }
    const bool live = mstar != -INFINITY;
    float l = 0.f;
    for (int s0 = 0; s0 < a.nsplit; s0 += 8) {
      float mv[8], lv[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const size_t o = (size_t)min(s0 + k, a.nsplit - 1) * a.Hq * 2;
        mv[k] = ml[o];
        lv[k] = ml[o + 1];
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float w = (s0 + k < a.nsplit && live && mv[k] != -INFINITY) ? fast_exp2(mv[k] - mstar) : 0.f;
        if (w != 0.f) l += w * lv[k];
      }
    }
    const float ww = (live && mw != -INFINITY) ? fast_exp2(mw - mstar) : 0.f;
    rowm[rr] = mstar;
    rowx[rr * 2] = ww;
    rowx[rr * 2 + 1] = l + ww * lw;
  }
  __syncthreads();
  // ---- Ahat: items (row, 4 consecutive latent indices) over rows_alloc x kp, zero past R and rv;
  // four independent items per thread at a time so that their loads are in flight together
  {
    const int nq4 = a.kp >> 2;
    const int nitems = a.rows_alloc * nq4;
    for (int i0 = tid; i0 < nitems; i0 += 4 * 256) {
      f32x4 acc[4];
      size_t rowoff[4];
      float mst[4];
      bool use[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int idx = min(i0 + 256 * u, nitems - 1);
        const int rr = idx / nq4, r = 4 * (idx - rr * nq4);
        use[u] = i0 + 256 * u < nitems && rr < R && r < a.rv;
        const int rs = rr < R ? rr : 0;
        const int sq = b * a.C + c0 + rs / grp, head = g * grp + rs % grp;
        rowoff[u] = (size_t)sq * a.nsplit * a.Hq + head;   // + s * Hq selects range s
        mst[u] = rowm[rs];
      }
      // 4 ranges x 4 items of loads in flight together (range indices clamped; the ranges are
      // still added in ascending order)
      int r4s[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) r4s[u] = min(i0 + 256 * u, nitems - 1) % nq4;
      for (int s0 = 0; s0 < a.nsplit; s0 += 4) {
        float msv[4][4];
        f32x4 xv[4][4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const size_t row = rowoff[u] + (size_t)min(s0 + k, a.nsplit - 1) * a.Hq;
            msv[u][k] = a.part_ml[row * 2];
            const pf_f16x4 h = *(const pf_f16x4*)((const _Float16*)a.part_acc + row * a.rv_pad16 + 4 * r4s[u]);
            xv[u][k] = f32x4{(float)h[0], (float)h[1], (float)h[2], (float)h[3]};
          }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const float ms = msv[u][k];
            const float w = (use[u] && s0 + k < a.nsplit && mst[u] != -INFINITY && ms != -INFINITY)
                                ? fast_exp2(ms - mst[u]) : 0.f;
            if (w != 0.f) acc[u] += w * xv[u][k];
          }
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int idx = i0 + 256 * u;
        if (idx < nitems) {
          const int rr = idx / nq4, r = 4 * (idx - rr * nq4);
          f32x4 v = acc[u];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = (r + e < a.rv) ? v[e] : 0.f;   // pad indices: not merged
          *(f32x4*)(ahat + rr * ahs + r) = v;
        }
      }
    }
  }

  // ---- up-project: wave w takes output column blocks 2w, 2w+1 for every 16-row block
  const int nrbk = a.rows_alloc >> 4;            // <= 4
  f32x4 oacc[4][2];
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int j = 0; j < 2; ++j) oacc[rb][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int r0 = 0; r0 < a.kp; r0 += kCbChunk) {
    __syncthreads();                             // Ahat complete / previous chunk no longer read
#pragma unroll
    for (int k = 0; k < kCbChunk * 16 / 256; ++k) {
      const int i = tid + 256 * k, r = i >> 4, q = i & 15;
      *(u32x4*)(bvs + r * kCbBvStride + q * 16) = pre[k];
    }
    __syncthreads();
    if (r0 + kCbChunk < a.kp) bv_load(r0 + kCbChunk);
#pragma unroll
    for (int ks = 0; ks < kCbChunk / 32; ++ks) {
      const bf16x8 b0 = cb_bv_operand(bvs, ks * 32, (2 * wave) * 16, lane);
      const bf16x8 b1 = cb_bv_operand(bvs, ks * 32, (2 * wave + 1) * 16, lane);
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        if (rb < nrbk) {
          const float* ar = ahat + (rb * 16 + li) * ahs + r0 + ks * 32 + lg * 8;
          const f32x4 x0 = *(const f32x4*)ar, x1 = *(const f32x4*)(ar + 4);
          bf16x8 hi, lo;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            hi[e] = (__bf16)x0[e];
            hi[4 + e] = (__bf16)x1[e];
            lo[e] = (__bf16)(x0[e] - (float)hi[e]);
            lo[4 + e] = (__bf16)(x1[e] - (float)hi[4 + e]);
          }
          oacc[rb][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi, b0, oacc[rb][0], 0, 0, 0);
          oacc[rb][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo, b0, oacc[rb][0], 0, 0, 0);
          oacc[rb][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi, b1, oacc[rb][1], 0, 0, 0);
          oacc[rb][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo, b1, oacc[rb][1], 0, 0, 0);
        }
      }
    }
  }
  // ---- out[row 16 rb + 4 lg + i][column 16 cb + li] = (O + w_x Ax) / l*
#pragma unroll
  for (int rb = 0; rb < 4; ++rb) {
    if (rb >= nrbk) break;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = (2 * wave + j) * 16 + li;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rr = rb * 16 + 4 * lg + i;
        if (rr >= R) continue;
        const int sq = b * a.C + c0 + rr / grp, head = g * grp + rr % grp;
        const float ww = rowx[rr * 2], lstar = rowx[rr * 2 + 1];
        float v = oacc[rb][j][i];
        if (ww != 0.f) v += ww * a.win_part[((size_t)sq * a.Hq + head) * 130 + col];
        v = (lstar == 0.f) ? 0.f : v / lstar;    // 0 only for a row with no keys; NaN stays NaN
        const size_t o = ((size_t)sq * a.Hq + head) * 128 + col;
        if (a.out_f32) ((float*)a.out)[o] = v;
        else ((__bf16*)a.out)[o] = (__bf16)v;
      }
    }
  }
}

hipError_t launch_prefill_combine(const DecodePlan& p, const lr_layer_cache* c, const float* part_ml,
                                  const float* part_acc, const float* win_part, void* out, int out_dtype,
                                  hipStream_t st) {
  PfCombineArgs a;
  a.part_ml = part_ml;
  a.part_acc = part_acc;
  a.win_part = win_part;
  a.bv = (const __bf16*)c->bv;
  a.out = out;
  a.out_f32 = out_dtype == LR_F32;
  a.C = p.qpb;
  a.Hq = p.Hq;
  a.Hkv = p.Hkv;
  a.D = p.D;
  a.rv = p.rv;
  a.rv_pad16 = p.rv_pad16;
  a.nsplit = p.nsplit;
  // tokens per workgroup: 4 where that still gives >= 512 workgroups, else fewer
  const int nbg = (p.B / p.qpb) * p.Hkv;
  a.tpw = kCbMaxTokens;
  while (a.tpw > 1 && nbg * ((p.qpb + a.tpw - 1) / a.tpw) < 512) a.tpw >>= 1;
  a.ntg = (p.qpb + a.tpw - 1) / a.tpw;
  a.rows_alloc = (a.tpw * (p.Hq / p.Hkv) + 15) / 16 * 16;
  a.kp = (p.rv + 63) / 64 * 64;
  const int grid = (p.B / p.qpb) * p.Hkv * a.ntg;
  const size_t lds = (size_t)a.rows_alloc * (a.kp + 4) * 4 + 3 * a.rows_alloc * 4 + kCbChunk * kCbBvStride;
  static bool attr_set[64] = {false};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < 64 && !attr_set[dev]) {
    e = hipFuncSetAttribute((const void*)lr_prefill_combine, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
    if (e != hipSuccess) return e;
    attr_set[dev] = true;
  }
  hipLaunchKernelGGL(lr_prefill_combine, dim3(grid), dim3(256), lds, st, a);
  return hipGetLastError();
}

template <int KS, int NV, int NHB>
static hipError_t launch_pf(const PrefillArgs& args, int grid, int lds, hipStream_t st, hipEvent_t ev_begin,
                            hipEvent_t ev_end) {
  static bool attr_set[64] = {false};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < 64 && !attr_set[dev]) {
    e = hipFuncSetAttribute((const void*)lr_prefill_latent<KS, NV, NHB>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            kLdsBytes);
    if (e != hipSuccess) return e;
    attr_set[dev] = true;
  }
  if (ev_begin || ev_end)
    hipExtLaunchKernelGGL((lr_prefill_latent<KS, NV, NHB>), dim3(grid), dim3(pf_threads(NHB)), lds, st, ev_begin,
                          ev_end, 0, args);
  else
    hipLaunchKernelGGL((lr_prefill_latent<KS, NV, NHB>), dim3(grid), dim3(pf_threads(NHB)), lds, st, args);
  return hipGetLastError();
}

// Head blocks per wave of the latent kernel. Measured over whole prefill calls at B = 16: token
// ranges of up to 4096 tokens run faster with one head block per wave (eight waves; T = 4K: 302
// against 334 us at rank 358 and C = 32, 227 against 252 us at rank 256), longer ranges with two
// (four waves; T = 32K, rank 256, C = 16: 790 against 841 us; T = 16K, rank 512, C = 32: 1086
// against 1251 us).
static int pf_heads_per_wave(const DecodePlan& p) { return p.split_tokens <= 4096 ? 1 : 2; }

hipError_t launch_prefill_latent(const DecodePlan& p, const lr_layer_cache* c, const __bf16* qt, float* part_ml,
                                 float* part_acc, hipStream_t st, hipEvent_t ev_begin, hipEvent_t ev_end) {
  PrefillArgs a;
  a.zk = (const unsigned char*)c->zk;
  a.zv = (const unsigned char*)c->zv;
  a.qt = qt;
  a.lat_len = c->lat_len;
  a.part_ml = part_ml;
  a.part_acc = part_acc;
  a.t_cap = p.t_cap;
  a.row_bytes_k = p.row_bytes_k;
  a.row_bytes_v = p.row_bytes_v;
  a.copy_k = p.copy_k;
  a.copy_v = p.copy_v;
  a.rk = p.rk;
  a.rk_pad = p.rk_pad;
  a.nks = p.nks;
  a.nrb = p.nrb;
  a.rv_pad16 = p.rv_pad16;
  a.nsplit = p.nsplit;
  a.split_tokens = p.split_tokens;
  a.max_len = p.max_len;
  a.Hq = p.Hq;
  a.C = p.qpb;
  a.ntg = p.pf_ntg;
  a.nunits = (p.B / p.qpb) * p.nsplit;
  a.nst = p.pf_nst;
  const int grid = ((a.nunits + 7) / 8) * 8 * a.ntg;
  const int ks = decode_ks(p.nks), nv = prefill_nv(p.nrb);
  const int nhb = pf_heads_per_wave(p);
#define LR_CASE(K, V)                                                                          \
  if (ks == K && nv == V)                                                                      \
    return nhb == 2 ? launch_pf<K, V, 2>(a, grid, p.pf_lds, st, ev_begin, ev_end)              \
                    : launch_pf<K, V, 1>(a, grid, p.pf_lds, st, ev_begin, ev_end);
  LR_CASE(8, 16) LR_CASE(8, 24) LR_CASE(8, 32)
  LR_CASE(12, 16) LR_CASE(12, 24) LR_CASE(12, 32)
  LR_CASE(16, 16) LR_CASE(16, 24) LR_CASE(16, 32)
#undef LR_CASE
  return hipErrorInvalidValue;
}

}  // namespace lr
