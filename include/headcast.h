/*
 * headcast.h - C ABI of the MI355X (gfx950) head-routed attention library.
 *
 * Method: "HeadCast: Casting Attention Heads for Efficient Autoregressive Video
 * Generation" (arXiv 2607.20125). After a warm-up, a one-time classifier labels every
 * attention head Sink, Dummy, Spatial or Global (Sec. 4.2, Eqs. 2-5); the monolithic
 * sliding-window KV cache is split into compact per-head buffers (Sec. 4.3); every
 * later attention call routes each head through its own path and concatenates the
 * results along heads (Sec. 4.4).
 *
 * Conventions shared by every call:
 *  - Tokens are frame-major, then row-major inside a frame:
 *    token = frame * S + row * frame_w + col, S = frame_h * frame_w.
 *  - Q, K, V and outputs are [tokens][num_heads][head_dim], dtype per hc_layer_desc
 *    (bf16 = raw 16-bit bfloat16, or fp32), 16-byte aligned device pointers.
 *  - The window is F = window_frames frames: the sink block (the first C =
 *    chunk_frames frames), rolling blocks, and the current block (the last C frames).
 *    "History" is every window frame before the current block (F - C frames).
 *  - Key sets: Sink = sink block + current block; Dummy = current block; Spatial =
 *    current block + the grid_h x grid_w window around the query's (row, col) in
 *    every history frame, origin clamp(row - grid/2, 0, frame - grid), never cut;
 *    Global = the whole window. Attention is softmax(q k^T * softmax_scale) v.
 *  - Device memory is always owned by the caller; the library never allocates device
 *    memory. Host handles (hc_head_buffers) are allocated by the library and released
 *    with hc_free_head_buffers.
 *  - Calls are asynchronous on `stream` (a hipStream_t passed as void*, NULL = the
 *    default stream) unless stated otherwise.
 *  - Every argument is validated on the host before any HIP call; on failure nothing
 *    is launched and the call returns a status != HC_OK, with a message available
 *    from hc_last_error() (per thread).
 */
#ifndef HEADCAST_H
#define HEADCAST_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { HC_SINK = 0, HC_DUMMY = 1, HC_SPATIAL = 2, HC_GLOBAL = 3 } hc_class;

typedef enum {
  HC_OK = 0,
  HC_ERR_NULL = 1,       /* a required pointer is NULL */
  HC_ERR_SHAPE = 2,      /* sizes inconsistent or out of the supported range */
  HC_ERR_DTYPE = 3,      /* unknown dtype */
  HC_ERR_LABEL = 4,      /* a head label outside 0..3 */
  HC_ERR_WORKSPACE = 5,  /* caller memory smaller than required */
  HC_ERR_ALIGN = 6,      /* a device pointer not 16-byte aligned */
  HC_ERR_DEVICE = 7,     /* no HIP device, or the current device is not gfx950 */
  HC_ERR_HIP = 8,        /* a HIP runtime call or kernel launch failed */
  HC_ERR_STATE = 9       /* the call does not fit the buffers' state */
} hc_status;

typedef enum { HC_BF16 = 0, HC_F32 = 1 } hc_dtype;

/* Path variants (hc_layer_desc.variant, a bit set). The default (0) follows the
 * classifier's proxies: Dummy = current block; Spatial = current block + the sliding
 * grid_h x grid_w window in every history frame. The pages' deployed forms:
 *  HC_VARIANT_DUMMY_PREVIOUS: Dummy heads also attend the window's most recent history
 *    block (appendix B cost model; Sec. 4.4's fused Sink/Dummy launch over one block);
 *    Dummy heads then keep a one-block buffer.
 *  HC_VARIANT_SPATIAL_CELLS: Spatial heads attend only the keys of their own
 *    non-overlapping grid_h x grid_w cell (cells tile the frame from (0,0); the last
 *    row/column of cells keeps the remainder) in every window frame, the current block
 *    included (Sec. 4.4, Fig. 3; Sec. 5.1 uses 10 x 10 cells).
 * A launch option (results equal up to rounding order, within the bf16 tolerance):
 *  HC_VARIANT_SPATIAL_OWN_LAUNCH: the Spatial heads' history part runs as its own
 *    kernel after the dense launch. Without it, for bf16 with head_dim 128, sliding
 *    windows and at most 16 Spatial heads, the routed call runs the Spatial tiles as the
 *    last items of the dense launch, where they fill the workgroup slots the dense
 *    items leave idle at the end, and merges their partials afterwards (one more
 *    partial slot per Spatial head in the workspace). */
typedef enum {
  HC_VARIANT_DUMMY_PREVIOUS = 1,
  HC_VARIANT_SPATIAL_CELLS = 2,
  HC_VARIANT_SPATIAL_OWN_LAUNCH = 4
} hc_variant;

typedef struct {
  int32_t num_heads;      /* H, 1..64 */
  int32_t head_dim;       /* d, 64 or 128 */
  int32_t frame_h;        /* latent frame rows */
  int32_t frame_w;        /* latent frame columns */
  int32_t chunk_frames;   /* C: frames per AR block (the current block) */
  int32_t window_frames;  /* F: window frames incl. sink and current block; F % C == 0, F >= C;
                             one window tensor, F*S*H*d elements, stays under 4 GiB */
  int32_t grid_h;         /* Spatial path window rows (>= 1; >= frame_h means whole frame) */
  int32_t grid_w;         /* Spatial path window columns */
  float softmax_scale;    /* usually 1/sqrt(d) */
  int32_t dtype;          /* hc_dtype */
  int32_t variant;        /* hc_variant bits, 0 = proxy-consistent paths */
} hc_layer_desc;

/* Classifier parameters (Sec. 4.2 Eq. 5 thresholds; Eq. 4 gamma and percentile). */
typedef struct {
  float theta_sink, theta_dummy, theta_spatial; /* cosine thresholds (pages: 0.95) */
  float theta_score;                            /* Spatial score threshold (pages: 0.755) */
  float gamma;                                  /* MSE weight in the Spatial score (pages: 5) */
  float percentile;                             /* token-cosine percentile (pages: 5) */
  int32_t proxy_grid_h, proxy_grid_w;           /* Spatial proxy window (0 = the desc grid) */
  int32_t sink_proxy_includes_current;          /* 0: Sink proxy = first block only */
} hc_classify_params;

typedef struct hc_head_buffers hc_head_buffers; /* opaque host handle */

const char* hc_status_string(int status);
const char* hc_last_error(void);

/* Fills the pages' defaults: thresholds 0.95, score threshold 0.755, gamma 5,
 * 5th percentile, proxy grid = desc grid, Sink proxy without the current block. */
hc_status hc_default_classify_params(hc_classify_params* params);

/* ---------------------------------------------------------------- buffers (Sec. 4.3)
 * Per-head compact KV buffers split out of the monolithic cache: a Sink head keeps
 * the frozen first block (C*S rows); a Dummy head keeps nothing (with
 * HC_VARIANT_DUMMY_PREVIOUS: the window's latest history block, C*S rows); Spatial and Global
 * heads keep the sink block plus R = F/C - 2 rolling blocks ((F - C)*S rows), the
 * block with absolute index b >= 1 living at block position 1 + (b - 1) mod R.
 */

/* Bytes of caller device memory the per-head buffers need (K and V regions). */
hc_status hc_head_buffers_bytes(const hc_layer_desc* desc, const int32_t* labels /* host [H] */,
                                size_t* bytes);

/* Builds the per-head buffers from the monolithic history K/V [n_hist_frames*S][H][d]
 * (logical frame order: sink block first; n_hist_frames % C == 0, <= F - C) into
 * `buffer_mem` (device, >= hc_head_buffers_bytes). The copy is stream-ordered; the
 * returned host handle refers to buffer_mem, which must outlive it. The next append
 * stores absolute block n_hist_frames / C. */
hc_status hc_build_head_buffers(const hc_layer_desc* desc, const int32_t* labels,
                                const void* k_hist, const void* v_hist, int32_t n_hist_frames,
                                void* buffer_mem, size_t buffer_bytes, hc_head_buffers** out,
                                void* stream);

/* Builds the buffers of a rollout resumed at any point (Sec. 4.3 rolling overwrite):
 * next_block is the absolute index of the block the next hc_append_chunk stores, and
 * k_hist / v_hist hold the window's history in logical order, [n_hist_frames*S][H][d]:
 * the sink block, then the window's rolling blocks oldest first (blocks
 * max(1, next_block - R) .. next_block - 1). n_hist_frames must equal C times the number
 * of those blocks (0 for next_block 0; C*(1 + min(next_block - 1, R)) otherwise), else
 * HC_ERR_SHAPE. Each block lands at its ring position, so the handle's slot table,
 * buffer contents and later appends are those of a handle that stored every block in
 * turn. hc_build_head_buffers is this call with next_block = n_hist_frames / C. */
hc_status hc_build_head_buffers_at(const hc_layer_desc* desc, const int32_t* labels, const void* k_hist,
                                   const void* v_hist, int32_t n_hist_frames, int64_t next_block,
                                   void* buffer_mem, size_t buffer_bytes, hc_head_buffers** out,
                                   void* stream);

/* Host-only planning handle: the same layout, ring state (next_block) and routed
 * plan as a built handle, without device memory. Only the size, state and index
 * queries accept it; append and routed calls return HC_ERR_STATE. */
hc_status hc_plan_head_buffers(const hc_layer_desc* desc, const int32_t* labels, int64_t next_block,
                               hc_head_buffers** out);

/* Stores a finished block's K/V [C*S][H][d] (Sec. 4.3 rolling overwrite): block 0
 * goes to the sink position of every head with a buffer; a later block overwrites
 * rolling position 1 + (b - 1) mod R of the Spatial and Global heads. */
hc_status hc_append_chunk(hc_head_buffers* buffers, const void* k_chunk, const void* v_chunk,
                          void* stream);

/* Absolute index of the block the next hc_append_chunk stores. */
hc_status hc_buffers_state(const hc_head_buffers* buffers, int64_t* next_block);

hc_status hc_free_head_buffers(hc_head_buffers* buffers); /* host handle only */

/* ---------------------------------------------------------------- routed step (Sec. 4.4)
 * out = every head's attention over its own key set, for the current block's queries
 * q [C*S][H][d] with the current block's k_cur / v_cur [C*S][H][d]. `workspace`
 * (device, >= hc_routed_workspace_bytes) holds fp32 partial results (split key ranges,
 * the Spatial heads' current-block part and history frame parts); its contents need no
 * initialisation. The size covers every fill state of the handle's window. Output
 * dtype = input dtype. Calls on one handle are ordered by their streams; calls that
 * share a workspace must not overlap. (The workspace argument is this library's
 * addition to the step's inputs: the library allocates no device memory.) */
hc_status hc_routed_workspace_bytes(const hc_head_buffers* buffers, size_t* bytes);
hc_status hc_routed_attention(const hc_head_buffers* buffers, const void* q, const void* k_cur,
                              const void* v_cur, void* out, void* workspace, size_t ws_bytes,
                              void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation): the routed step of
 * hc_routed_attention with its partial results in a scratch array that the library
 * keeps on every device it runs on (HC_NOALLOC_SCRATCH_BYTES, held until the process
 * ends) instead of a caller workspace. It calls no allocation routine. On a handle's
 * first such call the library plans its launches within the scratch (fewer key splits
 * than hc_routed_attention may use when they do not fit; same outputs up to rounding
 * order); HC_ERR_WORKSPACE if the Spatial heads' partials alone exceed the scratch.
 * All calls on one device share the scratch: calls that overlap in time on one device
 * (several streams or host threads) race and must be ordered by the caller. Contents
 * need no initialisation. */
#define HC_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
hc_status hc_routed_attention_noalloc(hc_head_buffers* buffers, const void* q, const void* k_cur,
                                      const void* v_cur, void* out, void* stream);

/* ---------------------------------------------------------------- classification (Sec. 4.2)
 * One-time classification over the full window: the reference output (Eq. 2) and the
 * Sink / Dummy / Spatial proxy outputs in fp32, per-token cosines against the
 * reference, their means (Eq. 3), the Spatial score P_pct(cos) - gamma * MSE (Eq. 4)
 * and the decision of Eq. 5. Requires n_hist_frames >= C (the sink block present).
 * Synchronises `stream`. labels_out: host [H]; stats_out (nullable): host [H][6] =
 * {cos_sink, cos_dummy, cos_spatial, p_pct, mse, score}, in double because the host
 * reduces the per-token values in fp64; the percentile and MSE are returned beside the
 * score so that each part of Eq. 4 can be checked. n_hist_frames: the frames the history
 * tensors hold (classification may run before the window is full). */
hc_status hc_classify_workspace_bytes(const hc_layer_desc* desc, const hc_classify_params* params,
                                      int32_t n_hist_frames, size_t* bytes);
hc_status hc_classify_heads(const hc_layer_desc* desc, const hc_classify_params* params,
                            const void* q, const void* k_hist, const void* v_hist,
                            int32_t n_hist_frames, const void* k_cur, const void* v_cur,
                            void* workspace, size_t ws_bytes, int32_t* labels_out,
                            double* stats_out, void* stream);

/* Host-only pieces of the classifier, exposed for checking without a GPU.
 * hc_reduce_statistics: from per-token values [lq][4] = {cos_sink, cos_dummy,
 * cos_spatial, squared error summed over d} computes stats_out[6] as above.
 * hc_decide: Eq. 5 with >= and the order Sink, Dummy, Spatial, else Global. */
hc_status hc_reduce_statistics(const float* per_token, int64_t lq, int32_t head_dim, double gamma,
                               double percentile, double* stats_out);
int32_t hc_decide(double cos_sink, double cos_dummy, double cos_spatial, double score,
                  const hc_classify_params* params);

/* ---------------------------------------------------------------- index exports
 * hc_debug_slot_table: absolute frame held at each of the F - C history positions of
 * every head, -1 when empty (host [H][F - C]); pure host.
 * hc_debug_head_region: byte offsets of head h's K and V rows inside buffer_mem and
 * its row capacity (-1 / 0 for a head without buffer); pure host.
 * hc_debug_gather_origins: device int32 [S][2] = Spatial window origin (row, col) of
 * every position for a grid_h x grid_w window (the classifier's proxy window may differ
 * from the routing grid), computed on `stream` by the device code the Spatial kernel uses.
 * hc_debug_routed_plan: the dense work entries of a routed call, host
 * [n][8] = {head, hist_rows, cur_rows, nsplit, split_len, slot, item_begin, queries per item}.
 * hc_debug_dense_queues: the XCD queues of the routed call's (first) dense launch: host
 * runs [8][16][2] = {first item, items} (-1 / 0 past n_runs[x]), n_runs [8], and the
 * longest queue; workgroup i runs on XCD i % 8, taking position i / 8 of its queue.
 * With the Spatial tiles in the launch, items from the dense item count on (see
 * hc_debug_routed_plan) are the tiles: Spatial head by head in increasing head order,
 * each head's tile_r x tile_c position tiles row-major (frame part by frame part).
 * hc_debug_spatial_plan: the Spatial launch of a routed call, host [5] = {tile rows,
 * tile columns, frame parts, partial slots of the whole call, 1 if the Spatial tiles
 * run as the last items of the dense launch}; zeros without Spatial heads (the slot
 * count excepted). Pure host. */
hc_status hc_debug_slot_table(const hc_head_buffers* buffers, int32_t* frames);
hc_status hc_debug_head_region(const hc_head_buffers* buffers, int32_t head, int64_t* k_offset,
                               int64_t* v_offset, int64_t* rows);
hc_status hc_debug_gather_origins(const hc_layer_desc* desc, int32_t grid_h, int32_t grid_w,
                                  void* r0c0, void* stream);
hc_status hc_debug_routed_plan(const hc_head_buffers* buffers, int32_t* entries, int32_t max_entries,
                               int32_t* n_entries, int32_t* n_items);
hc_status hc_debug_dense_queues(const hc_head_buffers* buffers, int32_t* runs, int32_t* n_runs,
                                int32_t* queue_len);
hc_status hc_debug_spatial_plan(const hc_head_buffers* buffers, int32_t* plan);

/* ---------------------------------------------------------------- timing
 * When enabled, every kernel the library launches is bracketed by HIP events on its
 * stream. hc_timing_read synchronises those events, returns per-kernel-kind totals
 * (ms_out, counts_out: [6] = dense, merge, spatial, copy, stats, fp32) and clears. */
hc_status hc_timing_enable(int32_t enable);
hc_status hc_timing_read(double* ms_out, int64_t* counts_out);

#ifdef __cplusplus
}
#endif

#endif /* HEADCAST_H */
