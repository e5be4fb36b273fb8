/*
 * cacheblend.h - C ABI of the MI355X (gfx950) library for CacheBlend's per-layer
 * KV fusion step (selective KV recompute).
 *
 * What the calls compute (from the pages):
 *   - CacheBlend explainer (0h-n0.github.io), "HKVD token selection": the KV
 *     deviation of token j at layer i is the L2 norm of cached minus recomputed KV.
 *   - same page, "Gradual filtering": each layer recomputes the tokens kept by the
 *     previous layer and narrows them to the r% of largest deviation.
 *   - same page, "Position encoding update": a cached K is moved to its position
 *     in the fused prompt by the rotation K_new = R(dp) K_cached.
 *   - same page, "vLLM integration": the three calls fetch_kv(text, layer),
 *     prefill_layer(input, KVCache) and synchronize().
 *   - CacheBlend review (jaehun.me), section on which tokens are recomputed: per
 *     layer, Q/K/V of the selected tokens are computed from their inputs, the other
 *     tokens keep their cached K/V, the selected queries attend under the causal
 *     mask to all available K/V, and the output goes to the next layer; section on
 *     overlapping loading and recompute: T_layer ~ max(T_load, T_recompute).
 *
 * Conventions shared by every call:
 *   - Layers are numbered 0 .. n_layers-1.
 *   - Positions: the fused prompt is chunk 0, chunk 1, ..., then the query rows.
 *     Row p of a fused K/V buffer holds the token at absolute position p.
 *     chunk_offsets[c] is the first row of chunk c, chunk_offsets[n_chunks] is the
 *     context length N_ctx; query rows are N_ctx .. N_ctx + n_query - 1.
 *     Every chunk cache was computed alone at positions 0.. (offset 0).
 *   - K/V layout: token-major [rows][n_kv_heads][head_dim], element type = dtype.
 *     The K/V heads of a row are contiguous.
 *   - Weights: row-major nn.Linear layout [out][in], element type = dtype,
 *     RMSNorm gains fp32.  The residual stream (hidden rows) is always fp32.
 *   - Every device pointer is caller-owned device memory (HBM) and must stay valid
 *     until the work enqueued on the compute stream has finished.  The library
 *     allocates only its context, its events and a RoPE table at cb_create.
 *   - Every call is asynchronous: it validates its arguments on the host, returns
 *     a non-OK status without enqueuing anything if they are wrong, and otherwise
 *     enqueues kernels on the compute stream (copies on the copy stream).  Faults in
 *     enqueued work surface at the caller's next synchronisation of that stream.
 *   - Device-side index arrays (sel_idx ...) cannot be checked on the host; kernels
 *     skip any out-of-range row instead of touching memory outside the buffers.
 *   - One context per host thread.  cb_last_error() describes the last non-OK
 *     status returned on the calling thread.
 */
#ifndef CACHEBLEND_H_
#define CACHEBLEND_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CB_OK = 0,
  CB_EINVAL = -1,        /* a NULL pointer, a negative size, a non-monotone offset list */
  CB_ESHAPE = -2,        /* sizes inconsistent with each other or with the model */
  CB_ESTATE = -3,        /* call order violated (e.g. blend before synchronize) */
  CB_EHIP = -4,          /* a HIP runtime call or kernel launch failed */
  CB_ENOMEM = -5,        /* workspace smaller than cb_workspace_size asks for */
  CB_EUNSUPPORTED = -6   /* a shape the kernels do not implement */
} cb_status;

typedef enum {
  CB_F32 = 0,   /* fp32 weights, K/V, Q and attention output */
  CB_BF16 = 1   /* bfloat16 storage, fp32 accumulation and softmax */
} cb_dtype;

/* Model shape.  Requirements: n_q_heads % n_kv_heads == 0; head_dim 64 or 128
 * (bf16: 128); d_model, n_q_heads*head_dim and ffn_dim multiples of 64;
 * max_tokens >= the longest fused prompt the context will see. */
typedef struct {
  int32_t n_layers, d_model, n_q_heads, n_kv_heads, head_dim, ffn_dim, vocab_size, max_tokens;
  float rope_base;  /* RoPE angle of pair i at position p: p * rope_base^(-2i/head_dim) */
  float rms_eps;    /* RMSNorm epsilon inside the square root */
  int32_t dtype;    /* cb_dtype */
} cb_model_desc;

/* Device pointers of one decoder layer (retained, not copied). */
typedef struct {
  const void* w_qkv;      /* [(n_q_heads + 2 n_kv_heads) * head_dim][d_model]: Q rows, K rows, V rows */
  const void* w_o;        /* [d_model][n_q_heads * head_dim] */
  const void* w_gate_up;  /* [2 ffn_dim][d_model]: gate rows, then up rows */
  const void* w_down;     /* [d_model][ffn_dim] */
  const float* g_attn;    /* [d_model] gain of the pre-attention RMSNorm */
  const float* g_ffn;     /* [d_model] gain of the pre-FFN RMSNorm */
} cb_layer_weights;

typedef struct cb_ctx cb_ctx;

/* Create a context on HIP device `device`.  compute_stream / copy_stream are
 * hipStream_t handles owned by the caller (NULL = the null stream; copy_stream NULL
 * means copies go to the compute stream and nothing overlaps).  Builds the RoPE
 * cos/sin table for positions 0 .. max_tokens-1 in double precision (stored fp32). */
cb_status cb_create(const cb_model_desc* desc, int32_t device, void* compute_stream,
                    void* copy_stream, cb_ctx** out);
/* Synchronize the context's streams, then free its events and tables and the context itself,
 * whatever fails along the way; CB_EHIP reports the first HIP error met (a stream that could
 * not be synchronized, e.g. after a device fault).  NULL is a no-op. */
cb_status cb_destroy(cb_ctx* ctx);

/* Register the weights of `layer`.  Must precede cb_blend_layer / cb_layer_rest on it. */
cb_status cb_set_layer_weights(cb_ctx* ctx, int32_t layer, const cb_layer_weights* w);

/* The int8-weight variant of a layer (bf16 contexts only): every linear weight as int8 q with
 * one fp32 scale per output channel (row), the layer's products computing
 * sum_k bf16(x_k) * q[n][k] in fp32 (exact products, |q| <= 127) times s[n].  Same shapes and
 * row orders as cb_layer_weights; the scales are fp32 device arrays of one entry per weight
 * row (s_qkv [(n_q_heads + 2 n_kv_heads) * head_dim], s_o [d_model], s_gate_up [2 ffn_dim],
 * s_down [d_model]).  Row strides (d_model, n_q_heads * head_dim, ffn_dim) must be multiples
 * of 16 bytes.  Replaces any weights set before for the layer.  CB_EUNSUPPORTED on an fp32
 * context; CB_EINVAL for NULL pointers. */
typedef struct {
  const int8_t* w_qkv;
  const int8_t* w_o;
  const int8_t* w_gate_up;
  const int8_t* w_down;
  const float* s_qkv;
  const float* s_o;
  const float* s_gate_up;
  const float* s_down;
  const float* g_attn;
  const float* g_ffn;
} cb_layer_weights_i8;
cb_status cb_set_layer_weights_i8(cb_ctx* ctx, int32_t layer, const cb_layer_weights_i8* w);

/* Bytes of workspace that cb_blend_layer and cb_layer_rest need for fused prompts of at
 * most n_tokens rows and selected sets of at most n_sel_max rows. */
cb_status cb_workspace_size(const cb_ctx* ctx, int32_t n_tokens, int32_t n_sel_max, size_t* bytes);

/* hidden_out[i][:] = table[tokens[i]][:] as fp32.  tokens: device int32 [n];
 * table: device [vocab_size][d_model] of dtype; hidden_out: device fp32 [n][d_model].
 * Token ids outside [0, vocab_size) give zero rows. */
cb_status cb_embed(cb_ctx* ctx, const int32_t* tokens, int32_t n, const void* table, float* hidden_out);

/* Layer-pipelined load (explainer, "Pipelined design"; fetch_kv) with the position update
 * (explainer, "Position encoding update": K_new = R(delta p) K_cached).  Enqueues on the copy
 * stream, once the compute stream is done with the last cb_blend_layer of this layer
 * enqueued before the call (its fused rows are then free):
 *   1. host-to-device copies of layer `layer`'s cached K and V of every chunk: host_k[c],
 *      host_v[c] point to pinned host memory holding [len_c][n_kv_heads][head_dim]
 *      (len_c = chunk_offsets_host[c+1] - chunk_offsets_host[c]) and land in rows
 *      [chunk_offsets_host[c], chunk_offsets_host[c+1]) of fused_k / fused_v;
 *   2. the position update of those rows in place: row j of chunk c gets K[j] <- R(o_c) K[j];
 * and records the layer's event.  The rows then hold the re-rotated cache: pass
 * kv_cached_k = kv_cached_v = NULL to cb_blend_layer.  chunk_offsets_dev: the same offsets
 * on the device.  CB_ESTATE if the layer already has a fetch that no cb_synchronize has
 * consumed. */
/* How cb_fetch_layer moves the rows.  CB_FETCH_KERNEL: when every chunk pointer is page-locked
 * host memory that kernels can read at the same address (hipHostMalloc, torch's pinned
 * tensors), one kernel on the copy stream reads the rows over PCIe, rotates K and writes K and
 * V into the fused buffers (one pass, no per-chunk copy commands); other pointers fall back to
 * the copy engine.  CB_FETCH_COPY: always the copy engine, then the rotation in place; chunks
 * whose host rows follow one another (host_k[c + 1] starts where chunk c's K rows end, and the
 * same for V) go as one hipMemcpyAsync per run of such chunks.  CB_FETCH_AUTO (default): the
 * copy engine when those copies average at least 1 MiB, else as CB_FETCH_KERNEL.  The fetch
 * kernel loads faster when the per-copy cost of the copy engine dominates (small chunks: a
 * load-bound layer), but it holds CUs that the compute stream's kernels then lack; large copies
 * amortize that cost, and the copy engine leaves every CU to compute (measured on MI355X: 256
 * KiB chunks load at about 16 GB/s through the copy engine against 31 GB/s with the kernel;
 * with 1 MiB chunks of a compute-bound layer the prefill ran 2% faster through the copy
 * engine).  Results are identical.  CB_EINVAL for another mode. */
typedef enum { CB_FETCH_COPY = 0, CB_FETCH_KERNEL = 1, CB_FETCH_AUTO = 2 } cb_fetch_mode;
cb_status cb_set_fetch_mode(cb_ctx* ctx, int32_t mode);

/* Launch shape of the CB_FETCH_KERNEL path: `blocks` workgroups of `threads` threads (a
 * multiple of 64, at most 1024), each thread keeping `unroll` (1, 2 or 4) row pieces of 16
 * bytes of K and V in flight.  The reads cross PCIe, so a few requests in flight already reach
 * the link's rate; more only queue in the memory system that the compute stream's kernels
 * share.  Results do not depend on the shape.  (0, 0, 0) restores the library's default
 * shape.  CB_EINVAL outside these ranges. */
cb_status cb_set_fetch_launch(cb_ctx* ctx, int32_t blocks, int32_t threads, int32_t unroll);

cb_status cb_fetch_layer(cb_ctx* ctx, int32_t layer, const void* const* host_k,
                         const void* const* host_v, const int32_t* chunk_offsets_host,
                         int32_t n_chunks, const int32_t* chunk_offsets_dev, void* fused_k,
                         void* fused_v);

/* The same from a cache already in device memory: cache_k / cache_v are
 * [N_ctx][n_kv_heads][head_dim] offset-0 chunk caches in prompt order; on the copy stream,
 * fused K rows get R(o_c) K_cache and fused V rows a copy of V_cache (in place when the cache
 * aliases the fused buffers), then the layer's event is recorded.  This moves the position
 * update off the compute stream, where it would otherwise run inside cb_blend_layer. */
cb_status cb_fetch_layer_device(cb_ctx* ctx, int32_t layer, const void* cache_k, const void* cache_v,
                                const int32_t* chunk_offsets_host, int32_t n_chunks,
                                const int32_t* chunk_offsets_dev, void* fused_k, void* fused_v);

/* The position update of several layers at once, for caches already in device memory
 * (explainer, "Position encoding update"): on the compute stream, one launch (per 64 layers)
 * writes, for every layer l in [first_layer, first_layer + n_layers) and every context row j
 * of chunk c, fused_k[i][j] <- R(o_c) cache_k[i][j] and fused_v[i][j] <- cache_v[i][j]
 * (i = l - first_layer; in place when a layer's cache aliases its fused buffers, which must
 * then hold for K and V and for every layer).  Arrays of n_layers device pointers, in host
 * memory; layouts as for cb_fetch_layer_device.  The fused rows then hold the re-rotated cache:
 * pass kv_cached_k = kv_cached_v = NULL to cb_blend_layer.  With the whole cache resident in
 * HBM there is no load to hide behind the layers, and one launch replaces one per layer.
 * CB_EINVAL for a layer range outside the model or NULL pointers, CB_ESTATE if a layer has a
 * pending fetch. */
cb_status cb_rotate_layers(cb_ctx* ctx, int32_t first_layer, int32_t n_layers, const void* const* cache_k,
                           const void* const* cache_v, const int32_t* chunk_offsets_host, int32_t n_chunks,
                           const int32_t* chunk_offsets_dev, void* const* fused_k, void* const* fused_v);

/* synchronize(): make the compute stream wait for layer `layer`'s fetch event.  Does not
 * block the host.  A no-op for a layer that was never fetched.  (The fetch calls order the
 * copy stream after earlier steps through events recorded outside any capture, so a HIP-graph
 * capture should contain the compute-stream calls with kv_cached given to cb_blend_layer,
 * not the fetch calls.) */
cb_status cb_synchronize(cb_ctx* ctx, int32_t layer);

/* One layer of the fusion step (prefill_layer on the selected rows).  Enqueues:
 *  1. position update: every context row j of chunk c gets K[j] <- R(o_c) K_cached[j],
 *     V[j] <- V_cached[j] in kv_fused (skipped when kv_cached_k is NULL: the fused
 *     buffer then already holds the re-rotated cache; in place when kv_cached_* ==
 *     kv_fused_*);
 *  2. x = RMSNorm(hidden_sel) (or x_sel when given) and fresh K, V of the rows of
 *     S_l = sel_idx (RoPE at their absolute positions);
 *  3. deviation d_i = ||K_new - K_fused||^2 + ||V_new - V_fused||^2 (fp32) of the
 *     context rows of S_l against the re-rotated cache, before it is overwritten;
 *  4. k = floor(ratio * N_ctx + 0.5) (ratio as given, product in double) clamped to
 *     [0, n_sel - n_query]; the kept set is the k context rows of largest d (ties to
 *     the lower position) plus every query row, ascending;
 *  5. fused rows sel_idx <- fresh K, V (every recomputed row);
 *  6. Q of the kept rows (RoPE at their positions) and causal GQA attention of each
 *     kept row over fused rows 0 .. its position.
 * Arguments:
 *   hidden_sel       device fp32 [n_sel][d_model]: residual-stream rows of S_l
 *   x_sel            device [n_sel][d_model] (dtype) or NULL: RMSNorm(hidden_sel) with this
 *                    layer's attention gain, already computed (cb_layer_rest's x_next of the
 *                    previous layer); NULL computes it here (for up to 4 rows in bf16
 *                    the Q/K/V products form it from hidden_sel as they load it)
 *   kv_cached_k/_v   device [N_ctx][n_kv_heads][head_dim]: offset-0 chunk caches in
 *                    prompt order, or NULL (see 1.)
 *   kv_fused_k/_v    device [N_ctx + n_query][n_kv_heads][head_dim]: the layer's fused K/V
 *   chunk_offsets_dev / _host  the same [n_chunks + 1] offsets on device and host (the device
 *                    copy is read only by the position update, so it may be NULL when
 *                    kv_cached_k is NULL);
 *                    n_chunks may be 0 (no context: every row is a query row, which is
 *                    how a chunk's own cache is built)
 *   sel_idx          device int32 [n_sel] strictly ascending positions; its last n_query
 *                    entries must be the query rows
 *   new_sel_idx      device int32 [k + n_query] out: kept positions, ascending
 *   new_sel_local    device int32 [k + n_query] out: index of each kept row within sel_idx
 *   n_new            host out: k + n_query, set before the call returns
 *   out_sel          device [k + n_query][n_q_heads * head_dim] out (dtype): attention
 *                    output of the kept rows (before the o-projection)
 *   deviation        device fp32 [n_sel] out or NULL: entries 0 .. n_sel-n_query-1 get d;
 *                    with NULL, a layer that keeps every candidate (k = n_sel - n_query,
 *                    whose selection d does not decide) skips step 3 and, in bf16, writes
 *                    the fresh K/V rows of step 5 from the K/V product itself
 *   workspace        device scratch of at least cb_workspace_size(N, n_sel) bytes
 * CB_ESTATE if the layer was fetched and not yet synchronized. */
cb_status cb_blend_layer(cb_ctx* ctx, int32_t layer, const float* hidden_sel, const void* x_sel,
                         const void* kv_cached_k, const void* kv_cached_v,
                         void* kv_fused_k, void* kv_fused_v,
                         const int32_t* chunk_offsets_dev, const int32_t* chunk_offsets_host,
                         int32_t n_chunks, const int32_t* sel_idx, int32_t n_sel, int32_t n_query,
                         float ratio, int32_t* new_sel_idx, int32_t* new_sel_local, int32_t* n_new,
                         void* out_sel, float* deviation, void* workspace, size_t workspace_bytes);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): cb_blend_layer with the library's own static
 * workspace instead of a workspace argument; every other argument as in cb_blend_layer.  The
 * workspace is one file-scope device array of 128 MiB per device (held from the library's
 * load until the process ends).  A call whose cb_workspace_size(N, n_sel) exceeds 128 MiB
 * returns CB_ENOMEM before anything is enqueued.  Nothing is allocated.  The array keeps the
 * last call's contents and is shared by every call on that device: calls that overlap on one
 * device (other streams, other threads, other contexts) race on it, so callers serialize them. */
cb_status cb_blend_layer_static(cb_ctx* ctx, int32_t layer, const float* hidden_sel, const void* x_sel,
                                const void* kv_cached_k, const void* kv_cached_v,
                                void* kv_fused_k, void* kv_fused_v,
                                const int32_t* chunk_offsets_dev, const int32_t* chunk_offsets_host,
                                int32_t n_chunks, const int32_t* sel_idx, int32_t n_sel, int32_t n_query,
                                float ratio, int32_t* new_sel_idx, int32_t* new_sel_local, int32_t* n_new,
                                void* out_sel, float* deviation);

/* Generation with the fused KV (CacheBlend review: the answer is generated with the fused KV
 * cache).  One layer of a decode step for n_new new tokens at positions n_past .. n_past +
 * n_new - 1: fresh Q/K/V of the new rows (RoPE at their positions) from hidden_new (device fp32
 * [n_new][d_model]; or x_new, its RMSNorm, as in cb_blend_layer), their K/V written to rows
 * n_past .. of kv_fused (which must hold the fused rows 0 .. n_past - 1 and have room), and
 * their causal attention over fused rows 0 .. position into out_sel [n_new][n_q_heads *
 * head_dim].  pos_dev: device int32 [n_new] holding n_past, n_past + 1, ... (kernels bound
 * positions by n_past + n_new).  Then cb_layer_rest on the same rows with new_sel_local =
 * 0 .. n_new - 1.  The workspace is cb_workspace_size(n_past + n_new, n_new).  It is
 * cb_blend_layer with the past rows as one already-fused context span and the new rows as
 * query rows.  Up to 4 new rows whose count (taken as 1, 2 or 4) times the GQA group is at
 * most 8 run a few-row attention on the vector ALUs over 64-key ranges (at most 64 ranges) and
 * a combine of the ranges; other counts take the prefill attention with 256-key ranges. */
cb_status cb_decode_layer(cb_ctx* ctx, int32_t layer, const float* hidden_new, const void* x_new,
                          void* kv_fused_k, void* kv_fused_v, int32_t n_past, int32_t n_new,
                          const int32_t* pos_dev, void* out_sel, void* workspace, size_t workspace_bytes);

/* Rest of the layer on the kept rows (the output passed to the next layer):
 *   h1 = hidden_sel[new_sel_local] + out_sel W_o^T
 *   hidden_next = h1 + W_down( silu(W_gate m) * (W_up m) ),  m = RMSNorm(h1)
 * hidden_sel: device fp32 [n_sel][d]; new_sel_local / out_sel as returned by
 * cb_blend_layer; hidden_next: device fp32 [n_new][d] (must not alias hidden_sel).
 * x_next: device [n_new][d] (dtype) or NULL: if given, also RMSNorm(hidden_next) with the
 * attention gain of layer + 1 (which must exist and have its weights set), the x_sel of the
 * next cb_blend_layer; it is fused with the down-projection's reduction.  For up to 4 rows
 * in bf16, m is formed by the gate/up product from h1 as it loads it (no launch of its own);
 * a decode step that passes no x_next lets the next layer do the same for its x. */
cb_status cb_layer_rest(cb_ctx* ctx, int32_t layer, const float* hidden_sel, int32_t n_sel,
                        const int32_t* new_sel_local, int32_t n_new, const void* out_sel,
                        float* hidden_next, void* x_next, void* workspace, size_t workspace_bytes);

/* Where the calls leave intermediates in the caller's workspace, for checking a layer piece by
 * piece (host only; nothing is enqueued):
 *   q_offset, q_ld  after cb_blend_layer(..., n_sel, ...) has run: Q of the kept rows after
 *                   RoPE (model dtype; row j = the j-th kept row, rows q_ld elements apart),
 *                   until cb_layer_rest reuses the workspace.  all_kept != 0 when that call kept
 *                   every candidate (n_new == n_sel), which places Q in the joint Q|K|V product.
 *   h1_offset       after cb_layer_rest(..., n_sel, ...) has run: h1 (fp32 [n_new][d]);
 *   act_offset      then also the SwiGLU product silu(W_gate m) * (W_up m) (model dtype
 *                   [n_new][ffn_dim]), both until the next call that uses the workspace.
 * CB_EINVAL for a NULL pointer or a negative n_sel. */
typedef struct {
  size_t q_offset;
  int32_t q_ld;
  size_t h1_offset, act_offset;
} cb_ws_views;
cb_status cb_workspace_views(const cb_ctx* ctx, int32_t n_sel, int32_t all_kept, cb_ws_views* out);

/* Selection variants (KVBoost page, section on seam repair).
 *
 * Deviation score of cb_blend_layer on this context (default CB_SCORE_L2):
 *   CB_SCORE_L2      d = ||K_new - K_fused||^2 + ||V_new - V_fused||^2 (CacheBlend explainer,
 *                    "HKVD token selection");
 *   CB_SCORE_COSINE  d = 1 - <a, b> / (|a| |b|) with a, b the row's fresh and fused K|V over
 *                    all KV heads (the deviation-guided repair's token-wise cosine deviation;
 *                    0 when both rows are zero, 1 when only one is).
 * Ranking, ties and k are the same for both.  CB_EINVAL for another mode. */
typedef enum { CB_SCORE_L2 = 0, CB_SCORE_COSINE = 1 } cb_score_mode;
cb_status cb_set_score_mode(cb_ctx* ctx, int32_t mode);

/* The spatial repair set: the `window` positions just before every chunk boundary (the page's
 * default is 16; a window longer than its chunk covers the chunk), then the n_query query
 * rows, ascending, written to out (host int32, capacity entries).  *n_out is the set size; if
 * it exceeds capacity nothing is written and CB_ESHAPE is returned.  Recomputing exactly this
 * set at every layer is cb_blend_layer with sel_idx = this set and a ratio >= 1.  Host-only,
 * needs no context. */
cb_status cb_seam_select(const int32_t* chunk_offsets_host, int32_t n_chunks, int32_t n_query,
                         int32_t window, int32_t* out, int32_t capacity, int32_t* n_out);

/* Loading controller (CacheBlend explainer, "Pipelined design" and the section on tuning the
 * ratio to the storage; CacheBlend review, overlapping loading and recompute; LMCache blog,
 * section 5, break-even).  Host-only, needs no context.  Per layer:
 *   T_load      = n_ctx * kv_bytes_per_token_layer / bandwidth + latency_layer_s
 *   T_prefill_l = n_ctx * prefill_s_per_token / n_layers   (full prefill of one layer)
 *   break-even  = kv_bytes_per_token_layer * n_layers / prefill_s_per_token  (bytes/s)
 * At or below break-even the plan is load = 0, ratio = 1 (recompute every row: loading
 * cannot win).  Above it, ratio = T_load / T_prefill_l clamped to [r_min, r_max]: the largest
 * recompute that still hides under the load, T_recompute = ratio * T_prefill_l, and
 * T_layer = max(T_load, T_recompute), t_total = n_layers * T_layer (pipeline fill and drain
 * left aside).  CB_EINVAL for non-positive sizes, bandwidth or prefill time, or ratios outside
 * 0 <= r_min <= r_max <= 1. */
typedef struct {
  int32_t load;
  float ratio;
  double t_load_layer, t_recompute_layer, t_layer, t_total, break_even_bandwidth;
} cb_ratio_plan;
cb_status cb_plan_ratio(int32_t n_ctx, int32_t n_layers, double kv_bytes_per_token_layer, double bandwidth,
                        double prefill_s_per_token, double latency_layer_s, float r_min, float r_max,
                        cb_ratio_plan* out);

/* The same policy with a layer's recompute time measured on this GPU (seconds) instead of an
 * even split of the full prefill: T_recompute(r) = t_fixed_layer + r * (t_full_layer -
 * t_fixed_layer), where t_full_layer is a layer recomputing every row and t_fixed_layer a layer
 * recomputing none (query rows, attention over the cache, fixed kernel costs); t_fixed_layer = 0
 * is the explainer's linear model.  Per layer T_load = kv_bytes_layer / bandwidth +
 * latency_layer_s.  The fetch and the compute running side by side slow each other: the
 * longer of the two is stretched by `contention` seconds per second of overlap with the other
 * (measured; 0 is the review's max(T_load, T_recompute)): T_layer(r) = max(T_load,
 * T_recompute(r)) + contention * min(T_load, T_recompute(r)).  Loading pays when
 * T_layer(r_min) < t_full_layer; then ratio = (T_load - t_fixed_layer) / (t_full_layer -
 * t_fixed_layer) clamped to [r_min, r_max] (the recompute the load hides) and T_layer =
 * T_layer(ratio); otherwise load = 0,
 * ratio = 1, T_layer = t_full_layer, t_load_layer = 0.  The first layer recomputes every row in
 * either case; when loading, the next layer, the first to filter (it scores every context row),
 * adds t_select_layer over a later layer: t_total = t_first_layer + t_select_layer + (n_layers -
 * 1) * T_layer (t_first_layer + (n_layers - 1) * t_full_layer when not loading).
 * break_even_bandwidth = kv_bytes_layer / t_full_layer.  CB_EINVAL for non-positive sizes,
 * bandwidth or t_full_layer, negative latency, t_first_layer, t_select_layer or contention,
 * t_fixed_layer outside [0, t_full_layer], or ratios outside 0 <= r_min <= r_max <= 1. */
cb_status cb_plan_ratio_measured(int32_t n_layers, double kv_bytes_layer, double bandwidth, double latency_layer_s,
                                 double t_first_layer, double t_select_layer, double t_full_layer,
                                 double t_fixed_layer, double contention, float r_min, float r_max,
                                 cb_ratio_plan* out);

/* ---------------------------------------------------------------- chunk KV store
 * The offline side of the path: every chunk is prefilled alone at positions 0.. (CacheBlend
 * explainer, background: documents' KV precomputed independently) and its per-layer K and V
 * kept in host memory, found again through a hash table in CPU memory (explainer, integration
 * with vLLM: about 16 MB per million chunks).  Host-only except cb_store_put_layer.  Every
 * store call is thread-safe (one lock per store). */

/* FIPS 180-4 SHA-256 of n bytes into digest[32]. */
cb_status cb_sha256(const void* data, size_t n, uint8_t* digest);

/* 64-bit chunk key (KVBoost article, dual hash keys; the explainer's RAG example keeps the first
 * 64 bits of a SHA-256 digest): the first 8 digest bytes, read big-endian, of SHA-256 over
 * n_prior earlier keys (8 bytes big-endian each) followed by the n token ids (int32,
 * little-endian).  n_prior = 0 gives the content key (position-free); the content keys of
 * every earlier chunk of the prompt as prior give the prefix key.  CB_EINVAL for negative
 * lengths or NULL arrays of non-zero length. */
cb_status cb_chunk_key(const int32_t* tokens, int32_t n, const uint64_t* prior, int32_t n_prior, uint64_t* key);

typedef struct cb_store cb_store;

/* A store of n_slots chunks of at most max_chunk_tokens tokens for the model desc (its
 * n_layers, n_kv_heads, head_dim, dtype).  One slot holds, per layer, K and V, each
 * [max_chunk_tokens][n_kv_heads][head_dim] of dtype.  The arena is layer-major: for each layer,
 * the K rows of slots 0 .. n_slots - 1 back to back, then their V rows, so that full-length
 * entries in consecutive slots (a producer's chunks, filled in order) are one contiguous range
 * per layer, which cb_fetch_layer moves in one copy.  It is allocated once, pinned
 * (hipHostMalloc, pinned != 0; the form cb_fetch_layer copies from without a staging copy) or
 * pageable (malloc).  The index is open addressing with linear probing over
 * n_slots * 5/4 + 1 buckets of 16 bytes (key, slot), kept at most 80% full; deletion moves
 * later buckets back (no tombstones).  CB_EINVAL for non-positive sizes, CB_ENOMEM when the
 * arena cannot be allocated. */
cb_status cb_store_create(const cb_model_desc* desc, int32_t max_chunk_tokens, int32_t n_slots, int32_t pinned,
                          cb_store** out);
/* Frees the arena and the store.  Copies into or out of it must have completed.  CB_EHIP if
 * freeing the pinned arena fails (the store is released all the same). */
cb_status cb_store_destroy(cb_store* store);

/* Slot of the committed entry whose tokens and prior keys equal these (key match verified
 * against the stored tokens), else -1 (counted as a miss).  A hit makes the entry the most
 * recently used; pin != 0 also holds it (not evictable) until cb_store_release. */
cb_status cb_store_lookup(cb_store* store, const int32_t* tokens, int32_t n, const uint64_t* prior,
                          int32_t n_prior, int32_t pin, int32_t* slot);

/* Find or make the entry of this chunk (1 <= n <= max_chunk_tokens, else CB_ESHAPE).  Already
 * present (committed or not): made most recent, *is_new = 0.  Otherwise the lowest free slot,
 * or else the least recently used entry that nobody holds is evicted (*evicted = its slot,
 * else -1), and the new entry is uncommitted, *is_new = 1: the caller fills its layers
 * (cb_store_put_layer, or writes through cb_store_layer) and then calls cb_store_commit;
 * lookups miss it until then.  pin != 0 holds the entry.  CB_ESTATE when every entry is
 * held (nothing is changed). */
cb_status cb_store_insert(cb_store* store, const int32_t* tokens, int32_t n, const uint64_t* prior,
                          int32_t n_prior, int32_t pin, int32_t* slot, int32_t* is_new, int32_t* evicted);

/* Mark the entry's data complete (after the stream that filled it has been synchronized). */
cb_status cb_store_commit(cb_store* store, int32_t slot);

/* Drop one hold of the entry (CB_ESTATE if it has none). */
cb_status cb_store_release(cb_store* store, int32_t slot);

/* Host addresses of layer `layer`'s K and V rows of the entry in `slot`, and its token count.
 * The rows are [n_tokens][n_kv_heads][head_dim], K at positions 0.. (offset-0 cache): the
 * host_k[c] / host_v[c] that cb_fetch_layer takes.  Valid while the entry is not evicted. */
cb_status cb_store_layer(cb_store* store, int32_t slot, int32_t layer, void** host_k, void** host_v,
                         int32_t* n_tokens);

/* Producer: enqueue on the context's compute stream the device-to-host copies of the entry's
 * n_tokens rows of layer `layer` from dev_k / dev_v (device [n_tokens][n_kv_heads][head_dim],
 * the K/V a prefill of the chunk alone at positions 0.. wrote for that layer).  CB_ESHAPE
 * when the store was made for another model. */
cb_status cb_store_put_layer(cb_ctx* ctx, cb_store* store, int32_t slot, int32_t layer, const void* dev_k,
                             const void* dev_v);

typedef struct {
  int64_t hits, misses, evictions;
  int32_t entries, capacity;
  size_t index_bytes, arena_bytes, slot_bytes;
} cb_store_stats;
cb_status cb_store_get_stats(cb_store* store, cb_store_stats* out);

/* Thread-local description of the last non-OK status ("" if none). */
const char* cb_last_error(void);

/* Per-kernel timing with HIP events recorded on the compute stream around each launch.
 * Ids of the timed operations: */
typedef enum {
  CB_K_EMBED = 0, CB_K_ROPE = 1, CB_K_RMSNORM = 2, CB_K_GEMM_KV = 3, CB_K_DEV_SCATTER = 4,
  CB_K_TOPK = 5, CB_K_GEMM_Q = 6, CB_K_ATTN = 7, CB_K_GEMM_O = 8, CB_K_GEMM_GATE_UP = 9,
  CB_K_GEMM_DOWN = 10, CB_K_FETCH = 11, CB_K_COUNT = 12
} cb_kernel_id;
/* Start (on != 0) or stop recording; starting clears earlier records.  At most 16384 timed
 * launches are kept; later ones are not timed. */
cb_status cb_profile_enable(cb_ctx* ctx, int32_t on);
/* Wait for the recorded events and report, for one id: total ms, number of launches, and
 * the algorithmic work of those launches (flops for GEMM and attention, bytes moved for
 * the others, for CB_K_FETCH the cached K and V bytes read from host memory) as computed
 * from their shapes.  Launches on the copy stream (fetches and their position updates) are
 * timed on that stream. */
cb_status cb_profile_read(cb_ctx* ctx, int32_t kernel_id, double* total_ms, int64_t* launches,
                          double* work);

#ifdef __cplusplus
}
#endif
#endif /* CACHEBLEND_H_ */
