// Host-side plans shared by the C ABI (abi.cpp) and the kernel launchers (*.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "lowrank_attn.h"

namespace lr {

constexpr int kTileTokens = 16;     // tokens per decode tile
constexpr int kHeadsPad = 32;       // query heads padded for the 16x16 matrix-core tiles
constexpr int kLdsBytes = 160 * 1024;
constexpr int kLdsPad = 128;        // slack after the ring for operand over-reads
constexpr int kMaxSplit = 4096;     // token ranges per sequence (bounds the combine's LDS)
// Latent rows per sequence: lengths stay below 2^24, so append can carry an arrival count in the
// high bits of the length words while it runs.
constexpr int64_t kMaxTCap = ((int64_t)1 << 24) - 1;

// Compile-time bounds the decode kernel is instantiated for: KS K steps of 32 latent indices
// for the keys, RB value blocks of 16 per wave (two waves share the value blocks, so
// 32*RB value indices).
inline int decode_ks(int nks) { return nks <= 8 ? 8 : (nks <= 12 ? 12 : 16); }
inline int decode_rb(int nrb) {
  const int w = (nrb + 1) / 2;
  return w <= 8 ? 8 : (w <= 12 ? 12 : 16);
}
// LDS ring geometry for given bounds and element size (bytes): each stage holds 16 key rows of
// KS*32 elements then 16 value rows of RB*32 elements. Row padding keeps the operand reads free
// of bank conflicts: key rows are read 16 B per lane down 16 rows (stride = 4 dwords mod 64),
// value rows by the transpose read, 8 B per lane over 4 rows x 4 chunks (stride = 8 dwords
// mod 16, so the 4 rows land on disjoint 8-bank groups).
constexpr int lds_stride_k(int KS, int es) { return KS * 32 * es + 16; }
constexpr int lds_stride_v(int RB, int es) { return RB * 32 * es + 32; }
constexpr int lds_stage(int KS, int RB, int es) {
  return kTileTokens * (lds_stride_k(KS, es) + lds_stride_v(RB, es));
}
// Consumer layout of the decode workgroup (beside the 4 producer waves), chosen where the
// registers fit:
//   split: each consumer wave owns one 16-head block for every other tile of its group and
//          accumulates all value blocks (bf16 latents, value rank <= 384);
//   half:  the two waves of a head block share each tile and split the value blocks.
// (split needs up to 256 registers per consumer wave, so one group: 8 waves. Measured at rank
// 256, T = 32K: split is ~5% faster than two groups of halves, 12 waves. fp32 latents keep the
// two groups of halves.)
//   int4 latents always split.
constexpr bool decode_split(int latent, int KS, int RB) {
  return latent == LR_I4G32 ||
         (latent == LR_BF16 && ((KS <= 12 && RB <= 12) || (KS == 16 && RB == 8)));
}
constexpr int decode_groups(int latent, int KS, int RB) {
  return latent == LR_I4G32 ? 1
       : latent == LR_F32   ? 2
       : 1;
}
// Tiles each iteration of the decode loop consumes (one workgroup barrier per iteration).
constexpr int decode_tpi(int latent, int KS, int RB) {
  return decode_groups(latent, KS, RB) * (decode_split(latent, KS, RB) ? 2 : 1);
}
// Prefill latent kernel (bf16 latents): bound on the value blocks of 16 one wave accumulates
// for both of its head blocks (0 = unsupported).
inline int prefill_nv(int nrb) { return nrb <= 16 ? 16 : (nrb <= 24 ? 24 : (nrb <= 32 ? 32 : 0)); }
constexpr int kPrefillTokensPerWg = 4;   // chunk tokens per prefill workgroup
// int4 latents: raw stages (16 rows of codes and scale/zero words, as stored) for the
// direct-to-LDS loads; the value rows are dequantised into four fp16 stages of 16 value rows
// (two iterations of two tiles), the key rows are read raw by the consumers.
constexpr int kI4VStages = 4;
constexpr int kI4MaxRawStages = 16;
constexpr int kI4MinRawStages = 6;   // tiles of iterations it (keys) and it + 1 (values) + 2 in flight
constexpr int i4_vstage(int RB) { return kTileTokens * lds_stride_v(RB, 2); }
// int4: the consumers' partial-score exchange (2 iterations x 2 tiles x 2 head blocks x 1 KB)
constexpr int kI4XchBytes = 8 * 1024;
constexpr int i4_raw_stage(int gk, int gv) { return kTileTokens * 20 * (gk + gv); }
constexpr int lds_nst(int KS, int RB, int es) {   // stages in the ring: even, at most 8
  return ((kLdsBytes - kLdsPad) / lds_stage(KS, RB, es) > 8 ? 8
                                                             : (kLdsBytes - kLdsPad) / lds_stage(KS, RB, es)) & ~1;
}

// Exact keys (window slots and, in a prefill, the chunk's own rows): dense attention of each head
// on the matrix cores, written as an (O, m, l) partial the combine merges.
constexpr int kExD = 128;                 // head dim (the fold requires it too)
constexpr int kExSK = kExD * 2 + 16;      // LDS row strides (bytes): key rows for the A operand,
constexpr int kExSV = kExD * 2 + 32;      // value rows for the transpose read

struct ExactArgs {
  const __bf16* q;           // [B * C][Hq][d]
  const __bf16* kwin;        // [B][W][D] ring (slot of window entry e: (lat_len + e) % W)
  const __bf16* vwin;
  const __bf16* kchunk;      // [B][C][D], or NULL: no chunk rows among the keys (decode)
  const __bf16* vchunk;
  const int32_t* lat_len;
  const int32_t* win_len;
  float* win_part;           // [B * C][Hq][d + 2]: O (unnormalised), m, l
  int C, Hq, Hkv, D, W;
  float wscale;              // sm_scale * log2 e
  int nrb;                   // 64-row blocks per (b, g)
};

struct DecodePlan {
  int B;               // query sequences: stored sequences x qpb
  int qpb;             // query tokens per stored sequence (1 = decode, the chunk = prefill)
  int exact;           // exact-keys workgroups run (window > 0, or a prefill chunk)
  int Hq, Hkv, d, D;
  int rk, rv;
  int rk_pad;          // rk rounded up to 32 (matrix-core K steps)
  int rv_pad16;        // rv rounded up to 16 (matrix-core M blocks)
  int nks, nrb;        // K steps of 32, value blocks of 16
  int latent;          // lr_dtype
  float sm_scale;
  int window;
  int max_len, nsplit, split_tokens;  // nsplit: partial slots per sequence
  int bal;             // decode with ranges balanced over the sequences' lengths (range table)
  int nwg;             // latent workgroups of the grid (B x nsplit when not balanced)
  int64_t t_cap;
  int row_bytes_k, row_bytes_v;     // bytes of one stored latent row (codes for int4)
  int qp_bytes_k, qp_bytes_v;       // int4: bytes of one row's scale/zero words, else 0
  int stage_bytes, zv_off, qpk_off, qpv_off, nst;  // LDS ring layout
  int copy_k, copy_v;               // bytes of each stored row the ring holds
  int nr, raw_stage;                // int4: raw (codes + scale/zero) stages and their bytes
  int lds_bytes;                    // dynamic LDS of the decode kernel
  int pf;                           // prefill with the dedicated latent kernel (bf16 latents)
  int pf_ntg, pf_nst, pf_lds;       // its token groups per sequence, ring stages, dynamic LDS
  size_t off_qt, off_ml, off_acc, off_win, off_rng, ws_bytes;
};

// Balanced token ranges (decode, automatic split, 2 <= B <= kBalMaxSeqs): the grid keeps about
// one latent workgroup per compute unit, and each sequence gets up to twice as many partial
// slots, so that longer sequences can take more ranges.
constexpr int kBalMaxSeqs = 256;

// Fills *p; returns LR_OK or an error code with a message in *msg. n_q query tokens per stored
// sequence; prefill: the queries are a chunk whose own rows are exact keys (causal).
int plan_attention(const lr_model_desc* m, int layer, int batch, int n_q, bool prefill, int max_len,
                   const lr_decode_opts* o, DecodePlan* p, const char** msg);
inline int plan_decode(const lr_model_desc* m, int layer, int batch, int max_len, const lr_decode_opts* o,
                       DecodePlan* p, const char** msg) {
  return plan_attention(m, layer, batch, 1, false, max_len, o, p, msg);
}

hipError_t launch_decode(const DecodePlan& p, const lr_layer_cache* c, const void* q, void* out,
                         int out_dtype, void* ws, hipStream_t st, hipEvent_t ev_begin, hipEvent_t ev_end,
                         const void* k_chunk = nullptr, const void* v_chunk = nullptr,
                         const void* step_k_new = nullptr, const void* step_v_new = nullptr);

// The latent part of a prefill (p.pf): partials per (query token, token range) in the decode
// layout, for the decode combine.
hipError_t launch_prefill_latent(const DecodePlan& p, const lr_layer_cache* c, const __bf16* qt, float* part_ml,
                                 float* part_acc, hipStream_t st, hipEvent_t ev_begin, hipEvent_t ev_end);

// The exact keys of a prefill with the dedicated kernels (p.pf): window slots and the chunk's
// rows, causally; partials in the decode kernel's exact-keys layout.
hipError_t launch_prefill_exact(const DecodePlan& p, const lr_layer_cache* c, const void* q, const void* k_chunk,
                                const void* v_chunk, float* win_part, hipStream_t st);

// The combine of a prefill with the dedicated kernels (p.pf): rows of one KV head's group share
// the up-projection's Bv slice.
hipError_t launch_prefill_combine(const DecodePlan& p, const lr_layer_cache* c, const float* part_ml,
                                  const float* part_acc, const float* win_part, void* out, int out_dtype,
                                  hipStream_t st);

struct AppendPlan {
  int B, D, rk, rv, latent, window, n_new;
  int64_t t_cap;
  int ld_k, ld_v;
};

// One decode step: the append of one new token per sequence, then decode, in three launches: the
// append, the fold and the window in the first; the latent kernel; the combine, which also writes
// the new token into the ring and the lengths after the step (step_k_new / step_v_new non-NULL in
// launch_decode: the first launch already ran, and the lengths are still those before the step).
struct DecodePlan;
hipError_t launch_decode_step(const AppendPlan& ap, const DecodePlan& p, const lr_layer_cache* c, const void* k_new,
                              const void* v_new, const void* q, void* out, int out_dtype, void* ws, hipStream_t st,
                              hipEvent_t ev_begin, hipEvent_t ev_end);

hipError_t launch_append(const AppendPlan& p, const lr_layer_cache* c, const void* k_new,
                         const void* v_new, float* z_debug, hipStream_t st);

hipError_t launch_store(const AppendPlan& p, const lr_layer_cache* c, int64_t row0, int64_t n_rows,
                        const float* zk, const float* zv, hipStream_t st);

hipError_t launch_dequant(const AppendPlan& p, const lr_layer_cache* c, int64_t n_rows, float* zk_out,
                          float* zv_out, hipStream_t st);

struct RebasePlan {
  int B, rk, rv, rk_new, rv_new, latent, max_len;
};

hipError_t launch_rebase(const RebasePlan& p, const lr_layer_cache* src, const lr_layer_cache* dst,
                         const void* wk, const void* wv, hipStream_t st);
size_t svd_workspace_bytes(int n, int D);
size_t svd_workspace_stride(int n, int D);   // per matrix of a batch (256-byte multiple)
hipError_t launch_sens_svd(const void* x, const float* w, int n_mat, int n, int D, int rank, int sweeps, void* basis,
                           int basis_f32, float* sigma, void* ws, hipStream_t st);

size_t basis_update_workspace_bytes(int r, int n, int D);
hipError_t launch_basis_update(const void* basis, int f32, const float* sigma, int r, const void* rows, int n, int D,
                               int r_new, int sweeps, void* basis_new, float* sigma_new, void* w, void* ws,
                               hipStream_t st);

hipError_t launch_rank_allocate(const float* sigma, int n_mat, int sigma_ld, long long n_take, int r_min,
                                int g, int nb, int32_t* ranks, void* ws, hipStream_t st);

// Host plans of the rebase and weighted-SVD kernels (plans.cpp), shared with their launchers.
constexpr int kRbConsumers = 4;     // rebase: waves that hold W blocks and multiply (one per SIMD)
constexpr int kRbAllWaves = 8;      // rebase, all-waves form: every wave loads and multiplies
constexpr int kJb = 16;             // weighted SVD: Jacobi block size
constexpr int kJs = 2 * kJb;        // its pair subproblem size (32)
constexpr int kRqRows = 64;         // rows of G0 per workgroup of the Rayleigh quotients
int svd_nsplit(int n);              // sample ranges of the Gram

struct RebaseShape {
  int nks_t, nb, col_chunk, nchunk;
  int all;             // the all-waves form (kRbAllWaves waves of nb blocks each)
};
// bf16 kernel shape of one matrix; it can be rebased in place only when nchunk is 1.
void rebase_shape(int r_old, int r_new, RebaseShape* s);   // new coordinates per workgroup chunk (bf16)

int device_cu_count();

// Allocation-free decode: the workspace is a device array of the library (noalloc.hip).
constexpr size_t kNoAllocScratchBytes = (size_t)32 << 20;
constexpr int kMaxDevices = 64;
hipError_t noalloc_scratch(void** ptr);

}  // namespace lr
