/*
 * lowrank_attn.h -- C ABI of the MI355X (gfx950) low-rank KV-cache decode-attention library.
 *
 * The method: the KV cache stores low-dimensional latents of the key and value states,
 * optionally quantised, and decode attention is computed from those latents (TraceKV,
 * "TraceKV: Policy-Preserving Low-Rank KV Cache Compression for Reasoning Vision-Language
 * Models", abstract; ai4snews page on TraceKV, Synopsis: 70% rank ratio with 4-bit
 * quantisation). An exact window of the most recent tokens can sit beside the latent history,
 * older tokens being folded into the latents (iS-KV, "iS-KV: Online Low-Rank KV Cache
 * Compression via Block-Incremental SVD", English abstract). Ranks may differ per layer
 * (TraceKV abstract and ai4snews Interpretation: global rank allocation).
 *
 * One layer l of a model with Hq query heads, Hkv KV heads and head dimension d (D = Hkv*d):
 *   K = Zk Bk,  V = Zv Bv           Zk [T, rank_k[l]], Bk [rank_k[l], D]  (same for V)
 *   head j uses KV head g = j / (Hq/Hkv), columns g*d .. g*d+d-1 of K and V
 *   out_j = softmax_t(sm_scale * q_j . K[t, g]) V[t, g]  over latent and window tokens
 * The library never reconstructs K or V: it folds q_j into the latent space
 * (qt_j = q_j Bk[:, g]^T), scores the latent keys, runs an online softmax split over token
 * ranges, accumulates the probability-weighted latent values and up-projects once through Bv.
 *
 * Conventions (all entry points)
 *   - Every pointer not marked "host" is HIP device memory owned by the caller. The library
 *     allocates nothing, keeps no pointer after a call returns and holds no state (apart from
 *     the per-GPU device scratch array behind lowrank_attn_decode_noalloc).
 *   - All device work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *     nothing synchronises with the host. Buffers must stay alive until the stream reaches
 *     the work.
 *   - Every precondition the host can check is checked before any launch. On failure the
 *     call returns LR_EINVAL or LR_EUNSUPPORTED, launches nothing and records a message for
 *     lowrank_last_error(). A launch failure returns LR_EHIP. No exception crosses the ABI
 *     and nothing is printed. Outputs are undefined after an error.
 *   - Device-side lengths (lat_len, win_len) cannot be checked without a sync; kernels clamp
 *     them to [0, t_cap] and [0, window] (and decode to max_lat_len), so no access is ever out
 *     of bounds, but the result for an out-of-range length is unspecified.
 *   - Calls on the same stream are ordered; calls that share an output or workspace buffer on
 *     different streams race.
 */
#ifndef LOWRANK_ATTN_H
#define LOWRANK_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LOWRANK_ABI_VERSION 2

typedef enum {
  LR_OK = 0,
  LR_EINVAL = -1,        /* a null pointer, a size out of range, an inconsistent layout */
  LR_EUNSUPPORTED = -2,  /* valid but not implemented (e.g. head_dim != 128, > 32 q heads) */
  LR_EWORKSPACE = -3,    /* workspace smaller than lowrank_attn_decode_workspace_size() */
  LR_EHIP = -4           /* a HIP launch or runtime call failed */
} lr_status;

typedef enum {
  LR_F32 = 0,    /* float32 */
  LR_BF16 = 1,   /* bfloat16 */
  LR_I4G32 = 2   /* int4 codes in groups of 32 along the rank, float16 scale and zero per group */
} lr_dtype;

/* Static description of a model; host memory. */
typedef struct {
  int32_t n_layers;        /* >= 1 */
  int32_t n_q_heads;       /* Hq, 1..32 */
  int32_t n_kv_heads;      /* Hkv, divides Hq */
  int32_t head_dim;        /* d; must be 128 */
  const int32_t* rank_k;   /* host [n_layers]: the per-layer key rank table, each in 1..512 */
  const int32_t* rank_v;   /* host [n_layers]: the per-layer value rank table, each in 1..512 */
  float sm_scale;          /* softmax scale, normally 1/sqrt(d) */
  int32_t window;          /* W: exact recent tokens kept dense per sequence; 0 = none */
  int32_t latent_dtype;    /* lr_dtype of the stored latents: LR_F32, LR_BF16 or LR_I4G32 */
} lr_model_desc;

/*
 * One layer's cache. B sequences, each with t_cap latent rows allocated.
 *
 * Latent storage, per sequence b and row t (row = absolute token position t < lat_len[b]):
 *   LR_F32 / LR_BF16: zk [B][t_cap][ld_k], zv [B][t_cap][ld_v] elements of that dtype.
 *                     Elements rank..ld-1 of a row are never read into a result.
 *   LR_I4G32:         zk [B][t_cap][ceil(rank_k/32)*16] bytes of packed codes: group g of a
 *                     row is 16 bytes, code i of the group in byte i/2, even i in the low
 *                     nibble; unused nibbles of a partial last group are 0.
 *                     zk_qp [B][t_cap][ceil(rank_k/32)] uint32: float16 scale in the low half,
 *                     float16 zero in the high half. Element value = code * scale + zero,
 *                     evaluated as one float32 fused multiply-add. ld_k, ld_v are ignored.
 *                     Decode needs zk, zv, zk_qp and zv_qp 16-byte aligned; it evaluates the
 *                     element as one float16 fused multiply-add (the float16 matrix-core
 *                     operand), so groups whose values lie below float16's normal range
 *                     (|value| < 2^-14) lose relative precision there.
 *   Quantisation of a row z (float32), per group of 32 indices (the last may be partial; its
 *   min/max run over its real elements): zero = f16(min), scale = f16(f32(max-min)/15),
 *   code = clamp(rint((z - zero)/scale), 0, 15) in float32, all codes 0 if scale == 0.
 * Bases (row-major): bk [rank_k][D], bv [rank_v][D]; float32 if latent_dtype == LR_F32, else
 *   bfloat16. Down-projections pk [rank_k][D], pv [rank_v][D], rank-major: row i holds the
 *   weights that give latent coordinate i of a dense row x, z_i = x . pk[i] (the caller's
 *   pseudo-inverse P = pinv(B) [D][rank], stored transposed; for orthonormal bases pk = bk). Same
 *   dtype as the bases, 16-byte aligned; used by append only, may be NULL for decode.
 * Exact window (window W > 0): kwin, vwin [B][W][D] bfloat16 rings; the token at absolute
 *   position p sits in slot p mod W. Sequence b holds win_len[b] window tokens at positions
 *   lat_len[b] .. lat_len[b]+win_len[b]-1. NULL when W == 0.
 * Lengths: lat_len, win_len [B] int32 device arrays; decode reads them, append advances them.
 *   win_len may be NULL when W == 0.
 */
typedef struct {
  void* zk;
  void* zv;
  void* zk_qp;
  void* zv_qp;
  const void* bk;
  const void* bv;
  const void* pk;
  const void* pv;
  void* kwin;
  void* vwin;
  int32_t* lat_len;
  int32_t* win_len;
  int32_t ld_k;            /* latent row stride in elements (F32/BF16): >= rank_k, multiple of 8 */
  int32_t ld_v;            /* >= rank_v, multiple of 8 */
  int64_t t_cap;           /* latent rows allocated per sequence, 1 .. 2^24 - 1 */
} lr_layer_cache;

/* Optional decode tuning and timing hooks. */
typedef struct {
  int32_t nsplit;          /* token ranges per sequence; 0 = automatic */
  int32_t reserved0;       /* must be 0 */
  void* event_begin;       /* NULL, or a hipEvent_t stamped when the latent decode kernel (the
                              one that streams the cache) starts; it is attached to that
                              kernel's dispatch, so the pair times exactly its execution */
  void* event_end;         /* NULL, or a hipEvent_t stamped when that kernel ends */
  int32_t reserved[4];     /* must be 0 */
} lr_decode_opts;

/*
 * Bytes of device workspace lowrank_attn_decode needs for this layer, batch and length bound
 * (256-byte aligned base required). Returns 0 if the arguments are invalid.
 */
size_t lowrank_attn_decode_workspace_size(const lr_model_desc* model, int32_t layer, int32_t batch,
                                          int32_t max_lat_len, const lr_decode_opts* opts);

/*
 * Decode attention for one new query token per sequence, layer `layer`.
 *   q   [B][Hq][d]: float32 if latent_dtype == LR_F32, else bfloat16.
 *   out [B][Hq][d]: out_dtype LR_F32 or LR_BF16. Sequences with no token give 0.
 *   max_lat_len: host upper bound on lat_len[b] (sizes the grid); 0 <= max_lat_len <= t_cap.
 *   workspace: >= lowrank_attn_decode_workspace_size(...) bytes, 256-byte aligned; its
 *   contents on entry do not matter.
 * Writes only `out` and `workspace`. opts may be NULL.
 */
int lowrank_attn_decode(const lr_model_desc* model, int32_t layer, const lr_layer_cache* cache,
                        int32_t batch, int32_t max_lat_len, const void* q, void* out,
                        int32_t out_dtype, void* workspace, size_t workspace_bytes,
                        const lr_decode_opts* opts, void* stream);

/*
 * lowrank_attn_decode without a caller workspace, for callers that cannot allocate device memory
 * (code under graph capture, tight serving loops, harnesses that forbid hipMalloc). The workspace
 * is a device array inside the library, LOWRANK_NOALLOC_SCRATCH_BYTES long, one per GPU, held from
 * the first call on that GPU until the process ends; the call allocates nothing. Arguments,
 * results and errors are those of lowrank_attn_decode (same kernels, same output bit for bit), and
 * a call whose lowrank_attn_decode_workspace_size(...) exceeds the array returns LR_EWORKSPACE
 * before any launch. All calls on one GPU share the array: calls that overlap in time on one GPU
 * (different streams, or host threads) race and must be serialised by the caller.
 */
#define LOWRANK_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int lowrank_attn_decode_noalloc(const lr_model_desc* model, int32_t layer, const lr_layer_cache* cache,
                                int32_t batch, int32_t max_lat_len, const void* q, void* out,
                                int32_t out_dtype, const lr_decode_opts* opts, void* stream);

/*
 * Bytes of device workspace lowrank_attn_prefill needs (256-byte aligned base required);
 * 0 if the arguments are invalid.
 */
size_t lowrank_attn_prefill_workspace_size(const lr_model_desc* model, int32_t layer, int32_t batch,
                                           int32_t n_new, int32_t max_lat_len,
                                           const lr_decode_opts* opts);

/*
 * Chunked prefill attention (TraceKV abstract: the latents hold the KV states of large
 * multimodal contexts; the pages describe decode, and this is the same attention for a chunk of
 * n_new new tokens per sequence). Query token c of sequence b attends, causally, to the latent
 * history rows [0, lat_len[b]), the win_len[b] exact window slots (W > 0), and the chunk's own
 * exact rows 0 .. c:
 *   q     [B][n_new][Hq][d]: float32 if latent_dtype == LR_F32, else bfloat16.
 *   k_new, v_new [B][n_new][D] bfloat16: the chunk's dense key and value rows.
 *   out   [B][n_new][Hq][d]: out_dtype LR_F32 or LR_BF16.
 *   max_lat_len, workspace, opts: as for decode (workspace from
 *   lowrank_attn_prefill_workspace_size; opts->nsplit splits each query token's latent range).
 * 1 <= n_new and batch * n_new <= 65535. The cache is not modified: store the chunk afterwards
 * with lowrank_kv_append(..., n_new, k_new, v_new, ...), which projects, quantises and evicts
 * exactly as for decode. Every chunk token reads the whole latent stream (the latent part is
 * decode's kernel over batch * n_new query sequences that share their stored sequence's rows).
 * Writes only `out` and `workspace`.
 */
int lowrank_attn_prefill(const lr_model_desc* model, int32_t layer, const lr_layer_cache* cache,
                         int32_t batch, int32_t n_new, int32_t max_lat_len, const void* q,
                         const void* k_new, const void* v_new, void* out, int32_t out_dtype,
                         void* workspace, size_t workspace_bytes, const lr_decode_opts* opts,
                         void* stream);

/*
 * Append n_new tokens per sequence (iS-KV abstract: keep the recent window exact, fold older
 * tokens into the latent history; TraceKV abstract: latents optionally quantised).
 *   k_new, v_new [B][n_new][D] bfloat16 dense rows, in arrival order.
 * W == 0: token i of sequence b becomes latent row lat_len[b] + i, z = x P (float32
 *   accumulation), stored in the cache dtype (bf16: round to nearest even; int4: quantised
 *   as described above).
 * W > 0: tokens enter the window ring; whenever the window is full the oldest window token
 *   (absolute position lat_len[b]) is projected and stored as latent row lat_len[b], and
 *   lat_len[b] grows by one. The result is that of appending the tokens one at a time, for any
 *   n_new: a call of more than W tokens leaves only its last W in the window, and the ones
 *   before them go to the latent rows after the window tokens they push out.
 * Requires lat_len[b] + (number of new latent rows) <= t_cap (clamped otherwise: rows past
 * t_cap are dropped and lengths stop at t_cap).
 * n_new == 1 is one launch: while it runs, bits 24..30 of each lat_len word count the workgroups
 * that have read that sequence's inputs (the length itself stays in bits 0..23); the last one
 * writes the final lengths, so after the call the words hold plain lengths again. n_new > 1 is
 * two launches: one matrix-core product over all B * n_new rows, then one that writes the ring
 * and the lengths. Either way nothing may read or write the lengths on another stream during
 * the call.
 * z_debug: NULL, or [B][n_new][rank_k + rank_v] float32 receiving, for each latent row this
 *   call writes (the i-th such row of sequence b at index i), its z before storage rounding.
 * Writes latent rows, window slots and the two length arrays, nothing else.
 */
int lowrank_kv_append(const lr_model_desc* model, int32_t layer, const lr_layer_cache* cache,
                      int32_t batch, int32_t n_new, const void* k_new, const void* v_new,
                      float* z_debug, void* stream);

/*
 * One decode step of one layer: lowrank_kv_append of one new token per sequence (k_new, v_new
 * [B][1][D] bfloat16, no z_debug) followed by lowrank_attn_decode for the query q, with the same
 * results as those two calls in that order. max_lat_len bounds lat_len[b] after the append;
 * workspace as for lowrank_attn_decode. Three launches: the append, the query fold and the
 * exact window in the first (the window is read as it was, with the new token in the slot it
 * takes), the latent kernel, then the combine, which also writes the new token into the ring
 * and the new lengths; until then lat_len and win_len hold their values from before the call.
 * Errors: those of both calls, checked before any launch.
 */
int lowrank_decode_step(const lr_model_desc* model, int32_t layer, const lr_layer_cache* cache,
                        int32_t batch, const void* k_new, const void* v_new, const void* q, void* out,
                        int32_t out_dtype, int32_t max_lat_len, void* workspace, size_t workspace_bytes,
                        const lr_decode_opts* opts, void* stream);

/*
 * Bulk store of given latent rows (e.g. a prompt compressed elsewhere): rows
 * [row0, row0 + n_rows) of every sequence receive zk_rows [B][n_rows][rank_k] and zv_rows
 * [B][n_rows][rank_v] (float32), converted to the cache dtype exactly as append stores z.
 * Lengths are not touched. Requires 0 <= row0 and row0 + n_rows <= t_cap.
 */
int lowrank_kv_store(const lr_model_desc* model, int32_t layer, const lr_layer_cache* cache,
                     int32_t batch, int64_t row0, int64_t n_rows, const float* zk_rows,
                     const float* zv_rows, void* stream);

/*
 * Dequantise (or widen) stored latent rows [0, n_rows) of every sequence to float32:
 * zk_out [B][n_rows][rank_k], zv_out [B][n_rows][rank_v]: the stored value itself (float32,
 * bfloat16 widened exactly, int4 as the float32 fused multiply-add above). Decode rounds this
 * value once to its 16-bit matrix-core operand (bfloat16 for float32/bf16 caches, float16 for
 * int4). Requires n_rows <= t_cap.
 */
int lowrank_kv_dequant(const lr_model_desc* model, int32_t layer, const lr_layer_cache* cache,
                       int32_t batch, int64_t n_rows, float* zk_out, float* zv_out, void* stream);

/*
 * Historical-coordinate sync after a basis update (iS-KV, English abstract and method summary:
 * as the low-rank basis evolves, the stored coordinates are synchronised with it, otherwise the
 * history drifts). Every stored latent row z of rows [0, lat_len[b]) of src becomes its
 * least-squares coordinates in the new basis B',
 *     z' = z B pinv(B') = z W^T,
 * written to the same row of dst in the cache dtype (bf16: round to nearest even).
 *   wk [rank_k_new][round_up(rank_k, 8)], wv [rank_v_new][round_up(rank_v, 8)]: W = the
 *     caller's (B pinv(B'))^T in the base dtype (float32 caches: float32, else bfloat16),
 *     16-byte aligned; pad columns are ignored.
 *   src: the cache with the current ranks (model->rank_k/rank_v[layer]); only zk, zv, ld_k,
 *     ld_v, t_cap and lat_len (device, [batch]) are used, with the layout rules of decode.
 *     dst: latent buffers for the new ranks (ld >= new rank, a multiple of 8, <= 4096;
 *     t_cap >= max_lat_len); only zk, zv, ld_k, ld_v and t_cap are used.
 *     dst may be src itself (same buffers, strides and t_cap): always for float32; for bf16
 *     when one workgroup produces all new coordinates of a row, i.e. new rank <= 512 / 256 /
 *     192 / 128 for a current rank <= 128 / 256 / 384 / 512 (LR_EUNSUPPORTED otherwise).
 *     Partially overlapping buffers are not allowed.
 *   max_lat_len: host upper bound on lat_len[b] (sizes the grid); rows past it are not
 *     touched even where lat_len[b] is larger.
 *   stream: hipStream_t (NULL = default stream); the call only enqueues work and returns
 *     LR_EHIP if a launch fails. All buffers are the caller's and stay so.
 * Rows past lat_len[b] and columns past the new rank of dst are not written. Lengths, window
 * and bases are untouched: the caller switches the model to the new ranks and bases.
 * int4 caches: LR_EUNSUPPORTED.
 */
int lowrank_kv_rebase(const lr_model_desc* model, int32_t layer, const lr_layer_cache* src,
                      const lr_layer_cache* dst, int32_t batch, int32_t max_lat_len,
                      int32_t rank_k_new, int32_t rank_v_new, const void* wk, const void* wv,
                      void* stream);

/*
 * Sensitivity-weighted SVD basis construction (TraceKV abstract; ai4snews Synopsis and
 * Interpretation: KV states are weighted by their sensitivity before the SVD). For samples
 * x [n_samples][dim] bfloat16 (one KV matrix's rows, e.g. calibration tokens) and sensitivities
 * w [n_samples] float32 (finite, >= 0), with y_n = bf16(sqrt(w_n) * x_n) (float32 product, one
 * rounding):
 *   basis [rank][dim] (basis_dtype LR_F32 or LR_BF16): the top-rank right singular vectors of
 *     Y as rows, each with its largest-magnitude component positive (ready as bk or bv);
 *   sigma [dim] float32: all singular values of Y, descending (the spectrum for
 *     lowrank_rank_allocate).
 * Method: float32 Gram G = Y^T Y on the matrix cores, then block Jacobi on G (`sweeps` sweeps,
 * 0 = 10; each sweep is dim/16 - 1 rounds of two launches). dim must be a multiple of 64 in
 * 64..512. workspace: lowrank_sens_svd_workspace_size() bytes, 256-byte aligned.
 */
size_t lowrank_sens_svd_workspace_size(int32_t n_samples, int32_t dim);
int lowrank_sens_svd(const void* x, const float* w, int32_t n_samples, int32_t dim, int32_t rank,
                     int32_t sweeps, void* basis, int32_t basis_dtype, float* sigma,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * lowrank_sens_svd for n_mat matrices of one shape in one call (e.g. the K and V matrices of
 * every layer of a model): x [n_mat][n_samples][dim] bfloat16, w [n_mat][n_samples] float32,
 * basis [n_mat][rank][dim], sigma [n_mat][dim], contiguous; matrix m's results equal those of
 * lowrank_sens_svd on its slices (the same kernels, with the matrix index as a grid dimension,
 * so the Jacobi rounds of all matrices run together). 1 <= n_mat <= 65535; the other arguments
 * and errors as for lowrank_sens_svd. workspace: lowrank_sens_svd_batched_workspace_size()
 * bytes (n_mat times the single-matrix size), 256-byte aligned.
 */
size_t lowrank_sens_svd_batched_workspace_size(int32_t n_mat, int32_t n_samples, int32_t dim);
int lowrank_sens_svd_batched(const void* x, const float* w, int32_t n_mat, int32_t n_samples, int32_t dim,
                             int32_t rank, int32_t sweeps, void* basis, int32_t basis_dtype, float* sigma,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * Global rank allocation (TraceKV abstract; ai4snews Synopsis and Interpretation: the rank
 * budget is allocated globally across the KV states). Rule (the pages do not give one): every
 * matrix m (K or V of a layer) starts at r_min and grows by granules of `granule` up to r_max;
 * while the budget allows, the granule with the largest energy gain
 * sum_{k=r}^{r+granule-1} sigma_m[k]^2 is added (float64, index order; equal gains: lower m
 * first). Equivalently the best min(floor((budget - n_mat*r_min)/granule), all) granules of
 * the model are taken.
 *   sigma [n_mat][sigma_ld] float32: each matrix's spectrum (its sensitivity-weighted singular
 *     values), non-increasing and finite, n_sigma >= r_max entries used. With a spectrum that
 *     increases somewhere the result is the best-granules rule, not the greedy one.
 *   ranks [n_mat] int32 (output): r_min + granule * (granules given to m).
 *   Requires 1 <= r_min <= r_max <= n_sigma, (r_max - r_min) % granule == 0,
 *   budget >= n_mat * r_min, n_mat * (r_max - r_min) / granule <= 65536.
 *   workspace: lowrank_rank_allocate_workspace_size() bytes, 256-byte aligned.
 */
size_t lowrank_rank_allocate_workspace_size(int32_t n_mat, int32_t r_min, int32_t r_max, int32_t granule);
int lowrank_rank_allocate(const float* sigma, int32_t n_mat, int32_t n_sigma, int32_t sigma_ld,
                          int64_t budget, int32_t r_min, int32_t r_max, int32_t granule,
                          int32_t* ranks, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Block-incremental basis update of one KV matrix (iS-KV, "iS-KV: Online Low-Rank KV Cache
 * Compression via Block-Incremental SVD", English abstract and method summary: the low-rank basis
 * evolves incrementally while older states are folded, block by block, into the bounded-rank
 * history, and the historical coordinates are synchronised with the updated basis; the pages name
 * block-incremental SVD without its equations, read here as the textbook incremental SVD).
 * The history is held as U diag(sigma) B; folding the block of dense rows Y gives the new basis
 * and spectrum as the top rank_new right singular vectors and values of M = [diag(sigma) B ; Y].
 *   basis   [rank][dim] (basis_dtype LR_F32 or LR_BF16): the current basis, orthonormal rows
 *   sigma   [rank] float32 >= 0: its singular values (e.g. from lowrank_sens_svd or an earlier
 *           update)
 *   rows    [n_rows][dim] bfloat16: the block of dense K (or V) rows being folded in, e.g. the
 *           tokens leaving the exact window (may be NULL when n_rows == 0)
 *   basis_new [rank_new][dim] (basis_dtype, output): the new basis, each row with its
 *           largest-magnitude component positive
 *   sigma_new [rank_new] float32 (output): the new singular values, descending
 *   w       [rank_new][round_up(rank, 8)] (basis_dtype, output; pad columns 0): W = B' B^T, the
 *           sync weights lowrank_kv_rebase takes (z' = z W^T; B' has orthonormal rows, so this is
 *           z B pinv(B'))
 * Computed on the rows [bf16(sigma_i * B_i) (float32 product, one rounding) ; Y] with the weighted
 * SVD of lowrank_sens_svd (unit weights; `sweeps` Jacobi sweeps, 0 = 10): the exact SVD of those
 * rows to the Jacobi's float32 accuracy. Requires dim a multiple of 64 in 64..512,
 * 1 <= rank <= dim, 0 <= n_rows <= 65536, 1 <= rank_new <= min(dim, rank + n_rows). workspace:
 * lowrank_basis_update_workspace_size() bytes, 256-byte aligned. The inputs are only read; the
 * outputs must not overlap them.
 */
size_t lowrank_basis_update_workspace_size(int32_t rank, int32_t n_rows, int32_t dim);
int lowrank_basis_update(const void* basis, int32_t basis_dtype, const float* sigma, int32_t rank,
                         const void* rows, int32_t n_rows, int32_t dim, int32_t rank_new, int32_t sweeps,
                         void* basis_new, float* sigma_new, void* w, void* workspace,
                         size_t workspace_bytes, void* stream);

/* Message for the last non-OK status returned on this host thread ("" if none). */
const char* lowrank_last_error(void);

/* LOWRANK_ABI_VERSION of the library. */
int lowrank_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LOWRANK_ATTN_H */
