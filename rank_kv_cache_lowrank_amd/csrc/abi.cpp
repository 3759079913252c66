// C ABI: argument validation, launch planning and the exported entry points.
// Every host-checkable precondition is checked before any launch; no exception crosses the ABI.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <exception>
#include <string>

#include "internal.h"
#include "lowrank_attn.h"

namespace lr {

static thread_local std::string g_last_error;

static int fail(int code, const char* msg) {
  g_last_error = msg;
  return code;
}

int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

static inline int round_up(int x, int m) { return (x + m - 1) / m * m; }
static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
static inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

static int check_model(const lr_model_desc* m, int layer, int* rk, int* rv, const char** msg) {
  if (!m) return *msg = "model descriptor is NULL", LR_EINVAL;
  if (m->n_layers < 1) return *msg = "n_layers must be >= 1", LR_EINVAL;
  if (layer < 0 || layer >= m->n_layers) return *msg = "layer out of range", LR_EINVAL;
  if (!m->rank_k || !m->rank_v) return *msg = "rank tables must not be NULL", LR_EINVAL;
  if (m->n_q_heads < 1 || m->n_kv_heads < 1) return *msg = "head counts must be >= 1", LR_EINVAL;
  if (m->n_q_heads % m->n_kv_heads != 0) return *msg = "n_q_heads must be a multiple of n_kv_heads", LR_EINVAL;
  if (m->n_q_heads > kHeadsPad) return *msg = "more than 32 query heads is not supported", LR_EUNSUPPORTED;
  if (m->head_dim != 128) return *msg = "head_dim must be 128", LR_EUNSUPPORTED;
  if (m->latent_dtype != LR_F32 && m->latent_dtype != LR_BF16 && m->latent_dtype != LR_I4G32)
    return *msg = "unknown latent dtype", LR_EINVAL;
  if (!(isfinite(m->sm_scale))) return *msg = "sm_scale must be finite", LR_EINVAL;
  if (m->window < 0 || m->window > 65536) return *msg = "window must be in 0..65536", LR_EINVAL;
  *rk = m->rank_k[layer];
  *rv = m->rank_v[layer];
  if (*rk < 1 || *rk > 512 || *rv < 1 || *rv > 512) return *msg = "ranks must be in 1..512", LR_EINVAL;
  return LR_OK;
}

static int row_bytes(int latent, int r, int ld) {
  if (latent == LR_I4G32) return (r + 31) / 32 * 16;
  return ld * (latent == LR_F32 ? 4 : 2);
}

// Workspace layout (independent of the cache strides).
static void layout_workspace(DecodePlan* p) {
  size_t off = 0;
  p->off_qt = off;   // folded query: bf16, or float32 for int4 latents
  off = align256(off + (size_t)p->B * kHeadsPad * p->rk_pad * (p->latent == LR_I4G32 ? 4 : 2));
  p->off_ml = off;
  off = align256(off + (size_t)p->B * p->nsplit * p->Hq * 2 * 4);
  p->off_acc = off;
  // value partials: fp16 for bf16 and int4 latents (the decode and the prefill latent kernels),
  // float32 for float32 latents
  const int acc_bytes = p->latent != LR_F32 ? 2 : 4;
  off = align256(off + (size_t)p->B * p->nsplit * p->Hq * p->rv_pad16 * acc_bytes);
  p->off_win = off;
  if (p->exact) off = align256(off + (size_t)p->B * p->Hq * (p->d + 2) * 4);
  p->off_rng = off;   // range table: [nwg] int4 (sequence, slot, first token, end token), [B] int
  if (p->bal) off = align256(off + (size_t)p->nwg * 16 + (size_t)p->B * 4);
  p->ws_bytes = off > 0 ? off : 256;
}

int plan_attention(const lr_model_desc* m, int layer, int batch, int n_q, bool prefill, int max_len,
                   const lr_decode_opts* o, DecodePlan* p, const char** msg) {
  int rk = 0, rv = 0;
  int st = check_model(m, layer, &rk, &rv, msg);
  if (st != LR_OK) return st;
  if (batch < 0) return *msg = "batch must be >= 0", LR_EINVAL;
  if (max_len < 0) return *msg = "max_lat_len must be >= 0", LR_EINVAL;
  if (o) {
    bool bad = o->reserved0 != 0;
    for (int i = 0; i < 4; ++i) bad = bad || o->reserved[i] != 0;
    if (bad) return *msg = "lr_decode_opts reserved fields must be zero", LR_EINVAL;
    if (o->nsplit < 0) return *msg = "nsplit must be >= 0", LR_EINVAL;
  }
  if (n_q < 1 || n_q > 65536) return *msg = "tokens per sequence must be in 1..65536", LR_EINVAL;
  if ((int64_t)batch * n_q > 65535) return *msg = "batch x query tokens must be <= 65535", LR_EINVAL;
  memset(p, 0, sizeof(*p));
  p->B = batch * n_q;
  p->qpb = n_q;
  p->exact = (m->window > 0 || prefill) ? 1 : 0;
  p->Hq = m->n_q_heads;
  p->Hkv = m->n_kv_heads;
  p->d = m->head_dim;
  p->D = m->n_kv_heads * m->head_dim;
  p->rk = rk;
  p->rv = rv;
  p->rk_pad = round_up(rk, 32);
  p->rv_pad16 = round_up(rv, 16);
  p->nks = p->rk_pad / 32;
  p->nrb = p->rv_pad16 / 16;
  p->latent = m->latent_dtype;
  p->sm_scale = m->sm_scale;
  p->window = m->window;
  p->max_len = max_len;

  // prefill over bf16 latents: the dedicated latent kernel, one workgroup per group of
  // kPrefillTokensPerWg chunk tokens and token range
  p->pf = (prefill && p->latent == LR_BF16 && p->Hq / p->Hkv <= 16) ? 1 : 0;
  p->pf_ntg = p->pf ? (n_q + kPrefillTokensPerWg - 1) / kPrefillTokensPerWg : 0;

  // token ranges: about one workgroup per compute unit over the batch unless overridden
  const int max_split = max_len > 0 ? (max_len + kTileTokens - 1) / kTileTokens : 1;
  const int nb = p->pf ? (batch * p->pf_ntg > 0 ? batch * p->pf_ntg : 1) : (p->B > 0 ? p->B : 1);
  int target = (o && o->nsplit > 0) ? o->nsplit : (device_cu_count() + nb - 1) / nb;
  if (target < 1) target = 1;
  if (target > kMaxSplit) target = kMaxSplit;
  if (target > max_split) target = max_split;
  if (max_len == 0) {
    p->split_tokens = kTileTokens;
    p->nsplit = 1;
  } else {
    p->split_tokens = round_up((max_len + target - 1) / target, kTileTokens);
    p->nsplit = (max_len + p->split_tokens - 1) / p->split_tokens;
  }
  p->nwg = p->B * p->nsplit;
  // ragged lengths: the same grid, ranges balanced over the sequences on the device (the front
  // launch writes the range table), up to twice the slots per sequence
  if (!prefill && n_q == 1 && !(o && o->nsplit > 0) && p->B >= 2 && p->B <= kBalMaxSeqs && max_len > 0) {
    int slots = 2 * p->nsplit;
    if (slots > max_split) slots = max_split;
    if (slots > kMaxSplit) slots = kMaxSplit;
    if (slots > p->nsplit) {
      p->bal = 1;
      p->nsplit = slots;
    }
  }

  layout_workspace(p);
  return LR_OK;
}

// End-of-range merge of the consumer waves' partials: (m, l, value blocks) per extra wave.
static int merge_lds(int latent, int KS, int RB) {
  const int G = decode_groups(latent, KS, RB);
  const bool split = decode_split(latent, KS, RB);
  const int extra = split ? 4 * G - 2 : 4 * (G - 1);
  const int nvb = split ? 2 * RB : RB;
  return extra * (512 + nvb * 1024);
}

// LDS ring for the cache's row strides (the geometry itself is fixed by the kernel's bounds).
static int plan_lds(DecodePlan* p, int ld_k, int ld_v, const char** msg) {
  p->row_bytes_k = row_bytes(p->latent, p->rk, ld_k);
  p->row_bytes_v = row_bytes(p->latent, p->rv, ld_v);
  const int es = p->latent == LR_F32 ? 4 : 2;
  const int KS = decode_ks(p->nks), RB = decode_rb(p->nrb);
  int window_lds = 0;
  if (p->exact)
    window_lds = p->Hq * p->d * 4 + 2 * 32 * p->D * 2 + 32 * 16 + p->Hq * 32 * 4 + p->Hq * 3 * 4;
  if (p->latent == LR_I4G32) {
    const int gk = (p->rk + 31) / 32, gv = (p->rv + 31) / 32;
    p->qp_bytes_k = gk * 4;
    p->qp_bytes_v = gv * 4;
    p->stage_bytes = i4_vstage(RB);
    p->zv_off = 0;
    p->nst = kI4VStages;
    p->raw_stage = i4_raw_stage(gk, gv);
    int nr = (kLdsBytes - kLdsPad - kI4VStages * p->stage_bytes - kI4XchBytes) / p->raw_stage;
    if (nr > kI4MaxRawStages) nr = kI4MaxRawStages;
    if (nr < kI4MinRawStages) return *msg = "latent rows too wide for the LDS ring", LR_EUNSUPPORTED;
    p->nr = nr;
    int lds = kI4VStages * p->stage_bytes + nr * p->raw_stage + kI4XchBytes + kLdsPad;
    const int merge = merge_lds(p->latent, KS, RB);
    if (merge > lds) lds = merge;
    if (window_lds > lds) lds = window_lds;
    if (lds > kLdsBytes) return *msg = "decode staging exceeds LDS", LR_EUNSUPPORTED;
    p->lds_bytes = lds;
    return LR_OK;
  }
  if (p->latent == LR_F32 && (KS > 8 || RB > 8))
    return *msg = "float32 latents support ranks up to 256", LR_EUNSUPPORTED;
  const int sk = lds_stride_k(KS, es), sv = lds_stride_v(RB, es);
  // copy the 16-byte granules that hold the rank's elements; the rest of the LDS row is zero
  p->copy_k = (p->rk * es + 15) / 16 * 16;
  p->copy_v = (p->rv * es + 15) / 16 * 16;
  if (p->pf) {
    const int nv = prefill_nv(p->nrb);
    const int pstage = kTileTokens * (lds_stride_k(KS, 2) + lds_stride_v(nv / 2, 2));
    int nst = (kLdsBytes - kLdsPad) / pstage;
    nst = nst > 8 ? 8 : nst;
    if (nv == 0 || nst < 4 || p->copy_k > KS * 64 || p->copy_v > nv * 32)
      return *msg = "latent rows too wide for the prefill kernel", LR_EUNSUPPORTED;
    p->pf_nst = nst;
    p->pf_lds = nst * pstage + kLdsPad;
  }
  if (p->copy_k > sk - 16 || p->copy_v > sv - 32) return *msg = "rank exceeds the kernel bounds", LR_EINVAL;
  p->stage_bytes = lds_stage(KS, RB, es);
  p->zv_off = kTileTokens * sk;
  p->nst = lds_nst(KS, RB, es);
  const int tpi = decode_tpi(p->latent, KS, RB);
  if (p->nst < 2 * tpi || p->nst % tpi != 0)
    return *msg = "latent rows too wide for the LDS ring", LR_EUNSUPPORTED;
  int lds = p->nst * p->stage_bytes + kLdsPad;
  const int merge = merge_lds(p->latent, KS, RB);
  if (merge > lds) lds = merge;
  if (window_lds > lds) lds = window_lds;
  if (lds > kLdsBytes) return *msg = "decode staging exceeds LDS", LR_EUNSUPPORTED;
  p->lds_bytes = lds;
  return LR_OK;
}

static int check_cache_common(const lr_model_desc* m, const lr_layer_cache* c, int rk, int rv,
                              const char** msg) {
  if (!c) return *msg = "cache is NULL", LR_EINVAL;
  if (!c->zk || !c->zv) return *msg = "latent buffers zk/zv must not be NULL", LR_EINVAL;
  if (!c->lat_len) return *msg = "lat_len must not be NULL", LR_EINVAL;
  if (c->t_cap < 1 || c->t_cap > kMaxTCap) return *msg = "t_cap must be in 1..2^24-1", LR_EINVAL;
  if (!aligned(c->zk, 16) || !aligned(c->zv, 16)) return *msg = "latent buffers must be 16-byte aligned", LR_EINVAL;
  if (m->latent_dtype == LR_I4G32) {
    if (!c->zk_qp || !c->zv_qp) return *msg = "int4 caches need zk_qp/zv_qp", LR_EINVAL;
    if (!aligned(c->zk_qp, 4) || !aligned(c->zv_qp, 4)) return *msg = "scale/zero buffers must be 4-byte aligned", LR_EINVAL;
  } else {
    if (c->ld_k < rk || c->ld_v < rv) return *msg = "ld must be >= rank", LR_EINVAL;
    if (c->ld_k % 8 != 0 || c->ld_v % 8 != 0) return *msg = "ld must be a multiple of 8", LR_EINVAL;
    if (c->ld_k > 4096 || c->ld_v > 4096) return *msg = "ld must be <= 4096", LR_EINVAL;
  }
  if (m->window > 0) {
    if (!c->kwin || !c->vwin || !c->win_len) return *msg = "window buffers and win_len are required when window > 0", LR_EINVAL;
    if (!aligned(c->kwin, 16) || !aligned(c->vwin, 16)) return *msg = "window rings must be 16-byte aligned", LR_EINVAL;
  }
  return LR_OK;
}

}  // namespace lr

using namespace lr;

#define LR_GUARD_BEGIN try {
#define LR_GUARD_END                                              \
  }                                                               \
  catch (const std::exception& ex) {                              \
    return fail(LR_EINVAL, ex.what());                            \
  }                                                               \
  catch (...) {                                                   \
    return fail(LR_EINVAL, "unexpected internal error");          \
  }

extern "C" {

size_t lowrank_attn_decode_workspace_size(const lr_model_desc* model, int32_t layer, int32_t batch,
                                          int32_t max_lat_len, const lr_decode_opts* opts) {
  try {
    DecodePlan p;
    const char* msg = "";
    if (plan_decode(model, layer, batch, max_lat_len, opts, &p, &msg) != LR_OK) return 0;
    return p.ws_bytes;
  } catch (...) {
    return 0;
  }
}

// Everything lowrank_attn_decode checks before its workspace: the plan, the cache, the query and
// output buffers, the LDS layout.
static int plan_decode_call(const lr_model_desc* model, int32_t layer, const lr_layer_cache* cache, int32_t batch,
                            int32_t max_lat_len, const void* q, const void* out, int32_t out_dtype,
                            const lr_decode_opts* opts, DecodePlan* p, const char** msg) {
  int st = plan_decode(model, layer, batch, max_lat_len, opts, p, msg);
  if (st != LR_OK) return st;
  st = check_cache_common(model, cache, p->rk, p->rv, msg);
  if (st != LR_OK) return st;
  if ((int64_t)max_lat_len > cache->t_cap) return *msg = "max_lat_len must be <= t_cap", LR_EINVAL;
  if (!q || !out) return *msg = "q and out must not be NULL", LR_EINVAL;
  if (!cache->bk || !cache->bv) return *msg = "bases bk/bv must not be NULL", LR_EINVAL;
  if (!aligned(cache->bk, 16) || !aligned(cache->bv, 16) || !aligned(q, 16))
    return *msg = "q and the bases must be 16-byte aligned", LR_EINVAL;
  if (out_dtype != LR_F32 && out_dtype != LR_BF16) return *msg = "out_dtype must be LR_F32 or LR_BF16", LR_EINVAL;
  if (p->latent == LR_I4G32 && (!aligned(cache->zk_qp, 16) || !aligned(cache->zv_qp, 16)))
    return *msg = "int4 decode needs 16-byte aligned scale/zero buffers", LR_EINVAL;
  st = plan_lds(p, cache->ld_k, cache->ld_v, msg);
  if (st != LR_OK) return st;
  p->t_cap = cache->t_cap;
  return LR_OK;
}

int lowrank_attn_decode(const lr_model_desc* model, int32_t layer, const lr_layer_cache* cache,
                        int32_t batch, int32_t max_lat_len, const void* q, void* out, int32_t out_dtype,
                        void* workspace, size_t workspace_bytes, const lr_decode_opts* opts, void* stream) {
  LR_GUARD_BEGIN
  DecodePlan p;
  const char* msg = "";
  int st = plan_decode_call(model, layer, cache, batch, max_lat_len, q, out, out_dtype, opts, &p, &msg);
  if (st != LR_OK) return fail(st, msg);
  if (!workspace) return fail(LR_EINVAL, "workspace must not be NULL");
  if (!aligned(workspace, 256)) return fail(LR_EINVAL, "workspace must be 256-byte aligned");
  if (workspace_bytes < p.ws_bytes) return fail(LR_EWORKSPACE, "workspace too small");
  if (batch == 0) return LR_OK;
  hipError_t e = launch_decode(p, cache, q, out, out_dtype, workspace, (hipStream_t)stream,
                               opts ? (hipEvent_t)opts->event_begin : nullptr,
                               opts ? (hipEvent_t)opts->event_end : nullptr);
  if (e != hipSuccess) return fail(LR_EHIP, hipGetErrorString(e));
  return LR_OK;
  LR_GUARD_END
}

int lowrank_attn_decode_noalloc(const lr_model_desc* model, int32_t layer, const lr_layer_cache* cache,
                                int32_t batch, int32_t max_lat_len, const void* q, void* out, int32_t out_dtype,
                                const lr_decode_opts* opts, void* stream) {
  LR_GUARD_BEGIN
  DecodePlan p;
  const char* msg = "";
  int st = plan_decode_call(model, layer, cache, batch, max_lat_len, q, out, out_dtype, opts, &p, &msg);
  if (st != LR_OK) return fail(st, msg);
  if (p.ws_bytes > kNoAllocScratchBytes)
    return fail(LR_EWORKSPACE, "this decode needs more workspace than the library's scratch array holds "
                               "(LOWRANK_NOALLOC_SCRATCH_BYTES); use lowrank_attn_decode with a caller workspace");
  if (batch == 0) return LR_OK;
  void* ws = nullptr;
  hipError_t e = noalloc_scratch(&ws);
  if (e != hipSuccess) return fail(LR_EHIP, hipGetErrorString(e));
  e = launch_decode(p, cache, q, out, out_dtype, ws, (hipStream_t)stream,
                    opts ? (hipEvent_t)opts->event_begin : nullptr, opts ? (hipEvent_t)opts->event_end : nullptr);
  if (e != hipSuccess) return fail(LR_EHIP, hipGetErrorString(e));
  return LR_OK;
  LR_GUARD_END
}

size_t lowrank_attn_prefill_workspace_size(const lr_model_desc* model, int32_t layer, int32_t batch,
                                           int32_t n_new, int32_t max_lat_len, const lr_decode_opts* opts) {
  try {
    DecodePlan p;
    const char* msg = "";
    if (plan_attention(model, layer, batch, n_new, true, max_lat_len, opts, &p, &msg) != LR_OK) return 0;
    return p.ws_bytes;
  } catch (...) {
    return 0;
  }
}

int lowrank_attn_prefill(const lr_model_desc* model, int32_t layer, const lr_layer_cache* cache,
                         int32_t batch, int32_t n_new, int32_t max_lat_len, const void* q,
                         const void* k_new, const void* v_new, void* out, int32_t out_dtype,
                         void* workspace, size_t workspace_bytes, const lr_decode_opts* opts, void* stream) {
  LR_GUARD_BEGIN
  DecodePlan p;
  const char* msg = "";
  int st = plan_attention(model, layer, batch, n_new, true, max_lat_len, opts, &p, &msg);
  if (st != LR_OK) return fail(st, msg);
  st = check_cache_common(model, cache, p.rk, p.rv, &msg);
  if (st != LR_OK) return fail(st, msg);
  if ((int64_t)max_lat_len > cache->t_cap) return fail(LR_EINVAL, "max_lat_len must be <= t_cap");
  if (!q || !out || !k_new || !v_new) return fail(LR_EINVAL, "q, k_new, v_new and out must not be NULL");
  if (!cache->bk || !cache->bv) return fail(LR_EINVAL, "bases bk/bv must not be NULL");
  if (!aligned(cache->bk, 16) || !aligned(cache->bv, 16) || !aligned(q, 16) || !aligned(k_new, 16) ||
      !aligned(v_new, 16))
    return fail(LR_EINVAL, "q, k_new, v_new and the bases must be 16-byte aligned");
  if (out_dtype != LR_F32 && out_dtype != LR_BF16) return fail(LR_EINVAL, "out_dtype must be LR_F32 or LR_BF16");
  if (p.latent == LR_I4G32 && (!aligned(cache->zk_qp, 16) || !aligned(cache->zv_qp, 16)))
    return fail(LR_EINVAL, "int4 needs 16-byte aligned scale/zero buffers");
  st = plan_lds(&p, cache->ld_k, cache->ld_v, &msg);
  if (st != LR_OK) return fail(st, msg);
  if (!workspace) return fail(LR_EINVAL, "workspace must not be NULL");
  if (!aligned(workspace, 256)) return fail(LR_EINVAL, "workspace must be 256-byte aligned");
  if (workspace_bytes < p.ws_bytes) return fail(LR_EWORKSPACE, "workspace too small");
  if (batch == 0) return LR_OK;
  p.t_cap = cache->t_cap;
  hipError_t e = launch_decode(p, cache, q, out, out_dtype, workspace, (hipStream_t)stream,
                               opts ? (hipEvent_t)opts->event_begin : nullptr,
                               opts ? (hipEvent_t)opts->event_end : nullptr, k_new, v_new);
  if (e != hipSuccess) return fail(LR_EHIP, hipGetErrorString(e));
  return LR_OK;
  LR_GUARD_END
}

static int plan_append(const lr_model_desc* model, int layer, const lr_layer_cache* cache, int batch,
                       AppendPlan* p, const char** msg) {
  int rk = 0, rv = 0;
  int st = check_model(model, layer, &rk, &rv, msg);
  if (st != LR_OK) return st;
  st = check_cache_common(model, cache, rk, rv, msg);
  if (st != LR_OK) return st;
  if (batch < 0) return *msg = "batch must be >= 0", LR_EINVAL;
  p->B = batch;
  p->D = model->n_kv_heads * model->head_dim;
  p->rk = rk;
  p->rv = rv;
  p->latent = model->latent_dtype;
  p->window = model->window;
  p->t_cap = cache->t_cap;
  p->ld_k = cache->ld_k;
  p->ld_v = cache->ld_v;
  p->n_new = 0;
  return LR_OK;
}

int lowrank_kv_append(const lr_model_desc* model, int32_t layer, const lr_layer_cache* cache, int32_t batch,
                      int32_t n_new, const void* k_new, const void* v_new, float* z_debug, void* stream) {
  LR_GUARD_BEGIN
  AppendPlan p;
  const char* msg = "";
  int st = plan_append(model, layer, cache, batch, &p, &msg);
  if (st != LR_OK) return fail(st, msg);
  if (n_new < 0) return fail(LR_EINVAL, "n_new must be >= 0");
  if (n_new > 0 && (!k_new || !v_new)) return fail(LR_EINVAL, "k_new/v_new must not be NULL");
  if (!cache->pk || !cache->pv) return fail(LR_EINVAL, "append needs the down-projections pk/pv");
  if (!aligned(cache->pk, 16) || !aligned(cache->pv, 16)) return fail(LR_EINVAL, "pk/pv must be 16-byte aligned");
  if ((k_new && !aligned(k_new, 16)) || (v_new && !aligned(v_new, 16)))
    return fail(LR_EINVAL, "k_new/v_new must be 16-byte aligned");
  if (batch == 0 || n_new == 0) return LR_OK;
  p.n_new = n_new;
  hipError_t e = launch_append(p, cache, k_new, v_new, z_debug, (hipStream_t)stream);
  if (e != hipSuccess) return fail(LR_EHIP, hipGetErrorString(e));
  return LR_OK;
  LR_GUARD_END
}

int lowrank_decode_step(const lr_model_desc* model, int32_t layer, const lr_layer_cache* cache, int32_t batch,
                        const void* k_new, const void* v_new, const void* q, void* out, int32_t out_dtype,
                        int32_t max_lat_len, void* workspace, size_t workspace_bytes, const lr_decode_opts* opts,
                        void* stream) {
  LR_GUARD_BEGIN
  DecodePlan p;
  const char* msg = "";
  int st = plan_decode_call(model, layer, cache, batch, max_lat_len, q, out, out_dtype, opts, &p, &msg);
  if (st != LR_OK) return fail(st, msg);
  AppendPlan ap;
  st = plan_append(model, layer, cache, batch, &ap, &msg);
  if (st != LR_OK) return fail(st, msg);
  if (!k_new || !v_new) return fail(LR_EINVAL, "k_new/v_new must not be NULL");
  if (!aligned(k_new, 16) || !aligned(v_new, 16)) return fail(LR_EINVAL, "k_new/v_new must be 16-byte aligned");
  if (!cache->pk || !cache->pv) return fail(LR_EINVAL, "append needs the down-projections pk/pv");
  if (!aligned(cache->pk, 16) || !aligned(cache->pv, 16)) return fail(LR_EINVAL, "pk/pv must be 16-byte aligned");
  if (!workspace) return fail(LR_EINVAL, "workspace must not be NULL");
  if (!aligned(workspace, 256)) return fail(LR_EINVAL, "workspace must be 256-byte aligned");
  if (workspace_bytes < p.ws_bytes) return fail(LR_EWORKSPACE, "workspace too small");
  if (batch == 0) return LR_OK;
  ap.n_new = 1;
  hipError_t e = launch_decode_step(ap, p, cache, k_new, v_new, q, out, out_dtype, workspace, (hipStream_t)stream,
                                    opts ? (hipEvent_t)opts->event_begin : nullptr,
                                    opts ? (hipEvent_t)opts->event_end : nullptr);
  if (e != hipSuccess) return fail(LR_EHIP, hipGetErrorString(e));
  return LR_OK;
  LR_GUARD_END
}

int lowrank_kv_store(const lr_model_desc* model, int32_t layer, const lr_layer_cache* cache, int32_t batch,
                     int64_t row0, int64_t n_rows, const float* zk_rows, const float* zv_rows, void* stream) {
  LR_GUARD_BEGIN
  AppendPlan p;
  const char* msg = "";
  int st = plan_append(model, layer, cache, batch, &p, &msg);
  if (st != LR_OK) return fail(st, msg);
  if (row0 < 0 || n_rows < 0 || row0 + n_rows > cache->t_cap) return fail(LR_EINVAL, "rows out of range");
  if (n_rows > 0 && batch > 0 && (!zk_rows || !zv_rows)) return fail(LR_EINVAL, "zk_rows/zv_rows must not be NULL");
  if (batch == 0 || n_rows == 0) return LR_OK;
  if (n_rows > (int64_t)4 * 65535 * 16384) return fail(LR_EINVAL, "too many rows for one call");
  hipError_t e = launch_store(p, cache, row0, n_rows, zk_rows, zv_rows, (hipStream_t)stream);
  if (e != hipSuccess) return fail(LR_EHIP, hipGetErrorString(e));
  return LR_OK;
  LR_GUARD_END
}

int lowrank_kv_dequant(const lr_model_desc* model, int32_t layer, const lr_layer_cache* cache, int32_t batch,
                       int64_t n_rows, float* zk_out, float* zv_out, void* stream) {
  LR_GUARD_BEGIN
  AppendPlan p;
  const char* msg = "";
  int st = plan_append(model, layer, cache, batch, &p, &msg);
  if (st != LR_OK) return fail(st, msg);
  if (n_rows < 0 || n_rows > cache->t_cap) return fail(LR_EINVAL, "n_rows must be in 0..t_cap");
  if (n_rows > 0 && batch > 0 && (!zk_out || !zv_out)) return fail(LR_EINVAL, "outputs must not be NULL");
  if (batch == 0 || n_rows == 0) return LR_OK;
  hipError_t e = launch_dequant(p, cache, n_rows, zk_out, zv_out, (hipStream_t)stream);
  if (e != hipSuccess) return fail(LR_EHIP, hipGetErrorString(e));
  return LR_OK;
  LR_GUARD_END
}

int lowrank_kv_rebase(const lr_model_desc* model, int32_t layer, const lr_layer_cache* src,
                      const lr_layer_cache* dst, int32_t batch, int32_t max_lat_len, int32_t rank_k_new,
                      int32_t rank_v_new, const void* wk, const void* wv, void* stream) {
  LR_GUARD_BEGIN
  int rk = 0, rv = 0;
  const char* msg = "";
  int st = check_model(model, layer, &rk, &rv, &msg);
  if (st != LR_OK) return fail(st, msg);
  if (model->latent_dtype == LR_I4G32) return fail(LR_EUNSUPPORTED, "rebase supports float32 and bf16 latents");
  if (batch < 0) return fail(LR_EINVAL, "batch must be >= 0");
  if (max_lat_len < 0) return fail(LR_EINVAL, "max_lat_len must be >= 0");
  if (rank_k_new < 1 || rank_k_new > 512 || rank_v_new < 1 || rank_v_new > 512)
    return fail(LR_EINVAL, "new ranks must be in 1..512");
  // only the latent rows, their strides, t_cap and (src) lat_len take part
  if (!src || !dst) return fail(LR_EINVAL, "src/dst is NULL");
  if (!src->zk || !src->zv || !dst->zk || !dst->zv) return fail(LR_EINVAL, "latent buffers zk/zv must not be NULL");
  if (!src->lat_len) return fail(LR_EINVAL, "src lat_len must not be NULL");
  if (src->t_cap < 1 || src->t_cap > kMaxTCap || dst->t_cap < 1 || dst->t_cap > kMaxTCap)
    return fail(LR_EINVAL, "t_cap must be in 1..2^24-1");
  if (!aligned(src->zk, 16) || !aligned(src->zv, 16) || !aligned(dst->zk, 16) || !aligned(dst->zv, 16))
    return fail(LR_EINVAL, "latent buffers must be 16-byte aligned");
  if (src->ld_k < rk || src->ld_v < rv) return fail(LR_EINVAL, "src ld must be >= the current rank");
  if (src->ld_k % 8 != 0 || src->ld_v % 8 != 0 || src->ld_k > 4096 || src->ld_v > 4096)
    return fail(LR_EINVAL, "src ld must be a multiple of 8, at most 4096");
  if (dst->ld_k < rank_k_new || dst->ld_v < rank_v_new) return fail(LR_EINVAL, "dst ld must be >= the new rank");
  if (dst->ld_k % 8 != 0 || dst->ld_v % 8 != 0 || dst->ld_k > 4096 || dst->ld_v > 4096)
    return fail(LR_EINVAL, "dst ld must be a multiple of 8, at most 4096");
  if ((int64_t)max_lat_len > src->t_cap || (int64_t)max_lat_len > dst->t_cap)
    return fail(LR_EINVAL, "max_lat_len must be <= the t_cap of src and dst");
  if (!wk || !wv) return fail(LR_EINVAL, "wk/wv must not be NULL");
  if (!aligned(wk, 16) || !aligned(wv, 16)) return fail(LR_EINVAL, "wk/wv must be 16-byte aligned");
  // in place: same rows and strides, and each row handled by one workgroup (one W chunk)
  const bool inplace_k = dst->zk == src->zk, inplace_v = dst->zv == src->zv;
  if ((inplace_k && (dst->ld_k != src->ld_k || dst->t_cap != src->t_cap)) ||
      (inplace_v && (dst->ld_v != src->ld_v || dst->t_cap != src->t_cap)))
    return fail(LR_EINVAL, "in-place rebase needs the same row stride and t_cap");
  RebasePlan p;
  p.B = batch;
  p.rk = rk;
  p.rv = rv;
  p.rk_new = rank_k_new;
  p.rv_new = rank_v_new;
  p.latent = model->latent_dtype;
  p.max_len = max_lat_len;
  if (model->latent_dtype == LR_BF16 && (inplace_k || inplace_v)) {
    RebaseShape sk, sv;
    rebase_shape(rk, rank_k_new, &sk);
    rebase_shape(rv, rank_v_new, &sv);
    if ((inplace_k && sk.nchunk > 1) || (inplace_v && sv.nchunk > 1))
      return fail(LR_EUNSUPPORTED, "these ranks need a separate dst (the new coordinates of a row span two workgroups)");
  }
  if (batch == 0 || max_lat_len == 0) return LR_OK;
  hipError_t e = launch_rebase(p, src, dst, wk, wv, (hipStream_t)stream);
  if (e != hipSuccess) return fail(LR_EHIP, hipGetErrorString(e));
  return LR_OK;
  LR_GUARD_END
}

static int check_rank_args(int32_t n_mat, int32_t n_sigma, int32_t sigma_ld, int32_t r_min, int32_t r_max,
                           int32_t granule, const char** msg) {
  if (n_mat < 1) return *msg = "n_mat must be >= 1", LR_EINVAL;
  if (granule < 1) return *msg = "granule must be >= 1", LR_EINVAL;
  if (r_min < 1 || r_max < r_min || r_max > n_sigma) return *msg = "need 1 <= r_min <= r_max <= n_sigma", LR_EINVAL;
  if (sigma_ld < n_sigma) return *msg = "sigma_ld must be >= n_sigma", LR_EINVAL;
  if ((r_max - r_min) % granule != 0) return *msg = "r_max - r_min must be a multiple of granule", LR_EINVAL;
  const int64_t N = (int64_t)n_mat * ((r_max - r_min) / granule);
  if (N > 65536 || n_mat > 65536) return *msg = "at most 65536 granules and 65536 matrices", LR_EINVAL;
  return LR_OK;
}

size_t lowrank_rank_allocate_workspace_size(int32_t n_mat, int32_t r_min, int32_t r_max, int32_t granule) {
  const char* msg = "";
  if (check_rank_args(n_mat, r_max, r_max, r_min, r_max, granule, &msg) != LR_OK) return 0;
  const int64_t N = (int64_t)n_mat * ((r_max - r_min) / granule);
  return align256((size_t)(N > n_mat ? N : n_mat) * 12);   // keys (8 bytes) and counts (4) per granule
}

int lowrank_rank_allocate(const float* sigma, int32_t n_mat, int32_t n_sigma, int32_t sigma_ld, int64_t budget,
                          int32_t r_min, int32_t r_max, int32_t granule, int32_t* ranks, void* workspace,
                          size_t workspace_bytes, void* stream) {
  LR_GUARD_BEGIN
  const char* msg = "";
  int st = check_rank_args(n_mat, n_sigma, sigma_ld, r_min, r_max, granule, &msg);
  if (st != LR_OK) return fail(st, msg);
  if (!sigma || !ranks || !workspace) return fail(LR_EINVAL, "sigma, ranks and workspace must not be NULL");
  if (!aligned(sigma, 4) || !aligned(ranks, 4) || !aligned(workspace, 256))
    return fail(LR_EINVAL, "sigma and ranks must be 4-byte aligned, workspace 256-byte aligned");
  if (budget < (int64_t)n_mat * r_min) return fail(LR_EINVAL, "budget must be >= n_mat * r_min");
  if (workspace_bytes < lowrank_rank_allocate_workspace_size(n_mat, r_min, r_max, granule))
    return fail(LR_EWORKSPACE, "workspace too small");
  const int nb = (r_max - r_min) / granule;
  int64_t n_take = (budget - (int64_t)n_mat * r_min) / granule;
  if (n_take > (int64_t)n_mat * nb) n_take = (int64_t)n_mat * nb;
  hipError_t e = launch_rank_allocate(sigma, n_mat, sigma_ld, (long long)n_take, r_min, granule, nb, ranks,
                                      workspace, (hipStream_t)stream);
  if (e != hipSuccess) return fail(LR_EHIP, hipGetErrorString(e));
  return LR_OK;
  LR_GUARD_END
}

size_t lowrank_sens_svd_workspace_size(int32_t n_samples, int32_t dim) {
  if (n_samples < 0 || dim < 64 || dim > 512 || dim % 64 != 0) return 0;
  return align256(svd_workspace_bytes(n_samples, dim));
}

int lowrank_sens_svd(const void* x, const float* w, int32_t n_samples, int32_t dim, int32_t rank,
                     int32_t sweeps, void* basis, int32_t basis_dtype, float* sigma, void* workspace,
                     size_t workspace_bytes, void* stream) {
  LR_GUARD_BEGIN
  if (n_samples < 0) return fail(LR_EINVAL, "n_samples must be >= 0");
  if (dim < 64 || dim > 512 || dim % 64 != 0) return fail(LR_EUNSUPPORTED, "dim must be a multiple of 64 in 64..512");
  if (rank < 1 || rank > dim) return fail(LR_EINVAL, "rank must be in 1..dim");
  if (sweeps < 0 || sweeps > 64) return fail(LR_EINVAL, "sweeps must be in 0..64 (0 = default 10)");
  if (basis_dtype != LR_F32 && basis_dtype != LR_BF16) return fail(LR_EINVAL, "basis_dtype must be LR_F32 or LR_BF16");
  if ((n_samples > 0 && (!x || !w)) || !basis || !sigma || !workspace)
    return fail(LR_EINVAL, "x, w, basis, sigma and workspace must not be NULL");
  if (!aligned(x, 16) || !aligned(w, 4) || !aligned(basis, 4) || !aligned(sigma, 4) || !aligned(workspace, 256))
    return fail(LR_EINVAL, "x must be 16-byte aligned, workspace 256-byte aligned");
  if (workspace_bytes < lowrank_sens_svd_workspace_size(n_samples, dim))
    return fail(LR_EWORKSPACE, "workspace too small");
  hipError_t e = launch_sens_svd(x, w, 1, n_samples, dim, rank, sweeps == 0 ? 10 : sweeps, basis,
                                 basis_dtype == LR_F32, sigma, workspace, (hipStream_t)stream);
  if (e != hipSuccess) return fail(LR_EHIP, hipGetErrorString(e));
  return LR_OK;
  LR_GUARD_END
}

size_t lowrank_sens_svd_batched_workspace_size(int32_t n_mat, int32_t n_samples, int32_t dim) {
  if (n_mat < 1 || n_mat > 65535 || n_samples < 0 || dim < 64 || dim > 512 || dim % 64 != 0) return 0;
  return (size_t)n_mat * svd_workspace_stride(n_samples, dim);
}

int lowrank_sens_svd_batched(const void* x, const float* w, int32_t n_mat, int32_t n_samples, int32_t dim,
                             int32_t rank, int32_t sweeps, void* basis, int32_t basis_dtype, float* sigma,
                             void* workspace, size_t workspace_bytes, void* stream) {
  LR_GUARD_BEGIN
  if (n_mat < 1 || n_mat > 65535) return fail(LR_EINVAL, "n_mat must be in 1..65535");
  if (n_samples < 0) return fail(LR_EINVAL, "n_samples must be >= 0");
  if (dim < 64 || dim > 512 || dim % 64 != 0) return fail(LR_EUNSUPPORTED, "dim must be a multiple of 64 in 64..512");
  if (rank < 1 || rank > dim) return fail(LR_EINVAL, "rank must be in 1..dim");
  if (sweeps < 0 || sweeps > 64) return fail(LR_EINVAL, "sweeps must be in 0..64 (0 = default 10)");
  if (basis_dtype != LR_F32 && basis_dtype != LR_BF16) return fail(LR_EINVAL, "basis_dtype must be LR_F32 or LR_BF16");
  if ((n_samples > 0 && (!x || !w)) || !basis || !sigma || !workspace)
    return fail(LR_EINVAL, "x, w, basis, sigma and workspace must not be NULL");
  if (!aligned(x, 16) || !aligned(w, 4) || !aligned(basis, 4) || !aligned(sigma, 4) || !aligned(workspace, 256))
    return fail(LR_EINVAL, "x must be 16-byte aligned, workspace 256-byte aligned");
  if (workspace_bytes < lowrank_sens_svd_batched_workspace_size(n_mat, n_samples, dim))
    return fail(LR_EWORKSPACE, "workspace too small");
  hipError_t e = launch_sens_svd(x, w, n_mat, n_samples, dim, rank, sweeps == 0 ? 10 : sweeps, basis,
                                 basis_dtype == LR_F32, sigma, workspace, (hipStream_t)stream);
  if (e != hipSuccess) return fail(LR_EHIP, hipGetErrorString(e));
  return LR_OK;
  LR_GUARD_END
}

static int check_basis_update_args(int32_t rank, int32_t n_rows, int32_t dim, int32_t rank_new, const char** msg) {
  if (dim < 64 || dim > 512 || dim % 64 != 0) return *msg = "dim must be a multiple of 64 in 64..512", LR_EUNSUPPORTED;
  if (rank < 1 || rank > dim) return *msg = "rank must be in 1..dim", LR_EINVAL;
  if (n_rows < 0 || n_rows > 65536) return *msg = "n_rows must be in 0..65536", LR_EINVAL;
  const int cap = rank + n_rows < dim ? rank + n_rows : dim;
  if (rank_new < 1 || rank_new > cap) return *msg = "rank_new must be in 1..min(dim, rank + n_rows)", LR_EINVAL;
  return LR_OK;
}

size_t lowrank_basis_update_workspace_size(int32_t rank, int32_t n_rows, int32_t dim) {
  const char* msg = "";
  if (check_basis_update_args(rank, n_rows, dim, 1, &msg) != LR_OK) return 0;
  return align256(basis_update_workspace_bytes(rank, n_rows, dim));
}

int lowrank_basis_update(const void* basis, int32_t basis_dtype, const float* sigma, int32_t rank, const void* rows,
                         int32_t n_rows, int32_t dim, int32_t rank_new, int32_t sweeps, void* basis_new,
                         float* sigma_new, void* w, void* workspace, size_t workspace_bytes, void* stream) {
  LR_GUARD_BEGIN
  const char* msg = "";
  int st = check_basis_update_args(rank, n_rows, dim, rank_new, &msg);
  if (st != LR_OK) return fail(st, msg);
  if (basis_dtype != LR_F32 && basis_dtype != LR_BF16) return fail(LR_EINVAL, "basis_dtype must be LR_F32 or LR_BF16");
  if (sweeps < 0 || sweeps > 64) return fail(LR_EINVAL, "sweeps must be in 0..64 (0 = default 10)");
  if (!basis || !sigma || (n_rows > 0 && !rows) || !basis_new || !sigma_new || !w || !workspace)
    return fail(LR_EINVAL, "basis, sigma, rows, basis_new, sigma_new, w and workspace must not be NULL");
  if (!aligned(basis, 4) || !aligned(sigma, 4) || (rows && !aligned(rows, 2)) || !aligned(basis_new, 4) ||
      !aligned(sigma_new, 4) || !aligned(w, 4) || !aligned(workspace, 256))
    return fail(LR_EINVAL, "buffers must be 4-byte aligned (rows 2-byte), workspace 256-byte aligned");
  if (workspace_bytes < lowrank_basis_update_workspace_size(rank, n_rows, dim))
    return fail(LR_EWORKSPACE, "workspace too small");
  hipError_t e = launch_basis_update(basis, basis_dtype == LR_F32, sigma, rank, rows, n_rows, dim, rank_new,
                                     sweeps == 0 ? 10 : sweeps, basis_new, sigma_new, w, workspace,
                                     (hipStream_t)stream);
  if (e != hipSuccess) return fail(LR_EHIP, hipGetErrorString(e));
  return LR_OK;
  LR_GUARD_END
}

const char* lowrank_last_error(void) { return g_last_error.c_str(); }

int lowrank_abi_version(void) { return LOWRANK_ABI_VERSION; }

}  // extern "C"
