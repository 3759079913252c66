// Host-side plans shared by the C ABI (abi.cpp) and the kernel launchers (*.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "lowrank_attn.h"

namespace lr {

constexpr int kTileTokens = 32;     // tokens per decode tile
constexpr int kHeadsPad = 32;       // query heads padded for the 16x16x32 matrix-core tiles
constexpr int kDecodeThreads = 256; // 4 waves
constexpr int kLdsBytes = 160 * 1024;
constexpr int kExchangeBytes = 4 * 64 * 16;   // score exchange between the 4 waves
constexpr int kLdsPad = 128;                  // slack after the ring for operand over-reads

struct DecodePlan {
  int B, Hq, Hkv, d, D;
  int rk, rv;
  int rk_pad;          // rk rounded up to 32 (matrix-core K steps)
  int rv_pad16;        // rv rounded up to 16 (matrix-core M blocks)
  int nks, nrb;        // K steps of 32, value blocks of 16
  int latent;          // lr_dtype
  float sm_scale;
  int window;
  int max_len, nsplit, split_tokens;
  int64_t t_cap;
  int row_bytes_k, row_bytes_v;     // bytes of one stored latent row (codes for int4)
  int qp_bytes_k, qp_bytes_v;       // int4: bytes of one row's scale/zero words, else 0
  int stage_bytes, zv_off, qpk_off, qpv_off, nst;  // LDS ring layout
  int lds_bytes;                    // dynamic LDS of the decode kernel
  size_t off_qt, off_ml, off_acc, off_win, ws_bytes;
};

// Fills *p; returns LR_OK or an error code with a message in *msg.
int plan_decode(const lr_model_desc* m, int layer, int batch, int max_len, const lr_decode_opts* o,
                DecodePlan* p, const char** msg);

hipError_t launch_decode(const DecodePlan& p, const lr_layer_cache* c, const void* q, void* out,
                         int out_dtype, void* ws, hipStream_t st, hipEvent_t ev_begin, hipEvent_t ev_end);

struct AppendPlan {
  int B, D, rk, rv, latent, window, n_new;
  int64_t t_cap;
  int ld_k, ld_v;
};

hipError_t launch_append(const AppendPlan& p, const lr_layer_cache* c, const void* k_new,
                         const void* v_new, float* z_debug, hipStream_t st);

hipError_t launch_store(const AppendPlan& p, const lr_layer_cache* c, int64_t row0, int64_t n_rows,
                        const float* zk, const float* zv, hipStream_t st);

hipError_t launch_dequant(const AppendPlan& p, const lr_layer_cache* c, int64_t n_rows, float* zk_out,
                          float* zv_out, hipStream_t st);

int device_cu_count();

}  // namespace lr
