/*
 * wf.h -- C ABI of libwf, the MI355X (gfx950) hot path of one Wave Forcing
 * round: chunk-wise causal attention over a ring-buffer history cache.
 *
 * What a round is. Wave Forcing denoises several video chunks at staggered
 * noise levels at once and re-runs a finished chunk to refresh the history
 * cache, one output chunk per round (Wave Forcing paper pages, Abstract:
 * the 1F1C schedule finishes one chunk per concurrent forward). The in-flight
 * chunks of a round (refresh chunk first, then the denoising chunks from
 * cleanest to noisiest; README usage on the airadar.tv summaries: wp-size =
 * step count + 1) form one query block. A chunk attends to the cached
 * history, to every earlier (cleaner) in-flight chunk and to itself, never to
 * a later one (Abstract: chunk-wise causal attention reads earlier, cleaner
 * chunks while their denoising is still under way).
 *
 * Conventions shared by every call
 *  - Pointers named k, v, q, x, out, workspace, lse, k_pool, v_pool are DEVICE
 *    pointers; slots / out_slot / n are HOST pointers. The caller owns all
 *    device memory. The library allocates only the small host cache handle;
 *    no call allocates or frees device memory or synchronizes the device.
 *  - stream is a hipStream_t passed as void* (NULL = the null stream). Every
 *    device-side effect is enqueued on it; ordering is the stream's.
 *  - Element types: WF_F32 (float) or WF_BF16 (bfloat16 stored as uint16).
 *    Token-major layout [tokens][n_heads][head_dim], contiguous.
 *  - Return value: WF_OK (0) or a negative WF_E_* code. On error nothing was
 *    enqueued and the cache table is unchanged; wf_last_error() describes the
 *    failure (thread-local). Device faults are asynchronous and surface at the
 *    caller's next synchronization.
 *  - A cache handle is not thread-safe.
 */
#ifndef WF_H
#define WF_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---- */
#define WF_OK 0
#define WF_E_NULL (-1)        /* a required pointer is NULL                       */
#define WF_E_SHAPE (-2)       /* a size is out of range or inconsistent           */
#define WF_E_DTYPE (-3)       /* unknown element type, or not valid for the call  */
#define WF_E_SLOT (-4)        /* slot / logical index out of range or duplicated  */
#define WF_E_FULL (-5)        /* no free slot, or the table is at WF_MAX_TABLE    */
#define WF_E_EMPTY (-6)       /* fewer table entries than the call needs          */
#define WF_E_UNSUPPORTED (-7) /* head_dim not 64/128, or another unsupported mode */
#define WF_E_HIP (-8)         /* a kernel launch was rejected by the HIP runtime  */

/* ---- element types ---- */
#define WF_F32 0
#define WF_BF16 1
#define WF_I32 2 /* raw int32 accumulators (wf_gemm_w8a8 output only) */

/* Largest number of table entries (history + in-flight chunks) and slots. */
#define WF_MAX_TABLE 64

/* wf_kv_cache_create flags */
#define WF_KV_ADOPT 0     /* take the pools as they are (padding already zero) */
#define WF_KV_ZERO_FILL 1 /* enqueue a zero fill of both pools on the stream   */

typedef struct wf_kv_cache wf_kv_cache;

/* ------------------------------------------------------------------------
 * History cache (Abstract: a history cache that later chunks read, and a
 * cache-refresh stage that rewrites a finished chunk's K/V).
 *
 * Storage: two caller-owned device pools of n_slots chunk slots each.
 * A slot holds one chunk of chunk_tokens tokens for all heads, padded to
 * S_pad = chunk_tokens rounded up to a multiple of 128 tokens, as images of
 * 64-key tiles that the attention kernel copies byte for byte into LDS.
 * With E = 16 / sizeof(element) (8 for bf16, 4 for fp32):
 *   K pool: [n_slots][n_heads][S_pad/64 tiles][head_dim/E][64 keys][E]
 *           (16-byte pieces of head_dim, key-major inside a piece)
 *   V pool: [n_slots][n_heads][S_pad/64 tiles][64/E][head_dim][E]
 *           (16-byte runs of E consecutive keys, one run per head_dim row)
 * Element (key t, dim d) of head h in slot s therefore sits at K index
 *   ((s*n_heads + h)*S_pad/64 + t/64)*64*head_dim + (d/E)*64*E + (t%64)*E + d%E
 * and V index
 *   ((s*n_heads + h)*S_pad/64 + t/64)*64*head_dim + ((t%64)/E)*head_dim*E + d*E + t%E.
 * Padding is zero and stays zero. A host-side table lists the slots of the
 * cache's chunks in logical order, oldest first; at attention time the last
 * n_inflight entries are the in-flight chunks (refresh chunk first) and the
 * entries before them are the history.
 * ------------------------------------------------------------------------ */

/* Bytes of ONE pool (K or V) for the given shape, padding included; 0 if the
 * shape is invalid. */
size_t wf_kv_pool_bytes(int n_slots, int chunk_tokens, int n_heads, int head_dim, int dtype);

/* Creates a cache over k_pool and v_pool (each wf_kv_pool_bytes() bytes,
 * 256-byte aligned). With WF_KV_ZERO_FILL both pools are zeroed on stream;
 * with WF_KV_ADOPT nothing is enqueued and the caller guarantees that the
 * padding is zero (pools that a cache already used, e.g. to re-attach a
 * snapshot with wf_kv_set_table). The table starts empty and every slot is
 * free. *out receives the handle.
 * Limits: 1 <= n_slots <= WF_MAX_TABLE, 1 <= chunk_tokens <= 2^20,
 * 1 <= n_heads <= 1024, head_dim in {64, 128}, dtype WF_F32 or WF_BF16. */
int wf_kv_cache_create(wf_kv_cache** out, void* k_pool, void* v_pool, int n_slots,
                       int chunk_tokens, int n_heads, int head_dim, int dtype, int flags,
                       void* stream);

/* Frees the host handle only (the pools stay the caller's). NULL is accepted. */
int wf_kv_cache_destroy(wf_kv_cache* kv);

/* Appends a chunk: takes the oldest free slot, enqueues the copy of k and v
 * (each [chunk_tokens][n_heads][head_dim] in the cache's dtype, 16-byte
 * aligned) into it and
 * pushes the slot onto the end of the table. *out_slot (may be NULL) receives
 * the physical slot. WF_E_FULL when no slot is free. */
int wf_kv_append(wf_kv_cache* kv, const void* k, const void* v, void* stream, int* out_slot);

/* Refresh: overwrites, in place, the slot of table entry logical_idx
 * (0 = oldest) with k and v (same layout as append). Attention launched later
 * on the same stream reads the new values. */
int wf_kv_refresh(wf_kv_cache* kv, int logical_idx, const void* k, const void* v, void* stream);

/* Pops the n_oldest oldest table entries; their slots become free (appended to
 * the free list in table order). Host-only; work already enqueued keeps the
 * table it was launched with. */
int wf_kv_evict(wf_kv_cache* kv, int n_oldest);

/* Replaces the table with slots[0..n-1] (distinct, each in [0, n_slots)); all
 * other slots become free in increasing order. Contents are not touched. Used
 * for non-contiguous layouts and to restore a snapshot. */
int wf_kv_set_table(wf_kv_cache* kv, const int* slots, int n);

/* Copies up to cap table entries into slots and the table length into *n. */
int wf_kv_get_table(const wf_kv_cache* kv, int* slots, int cap, int* n);

/* ------------------------------------------------------------------------
 * 3D rotary embedding, in place on x [n_tokens][n_heads][head_dim] (dtype).
 * The pages do not describe positional encoding; this call serves the
 * long-rollout workload and follows one stated convention:
 *   head_dim = d_t + d_h + d_w (all even); inside each axis segment of width
 *   d_a the pair (x[o+2i], x[o+2i+1]) rotates by pos_a * theta^(-2i/d_a);
 *   token u of chunk g (u in frame-major, then row, then column order) sits
 *   at (frames_per_chunk*g + frame, row, col); chunk g of the block is
 *   first_global_chunk + token / chunk_tokens, where
 *   chunk_tokens = frames_per_chunk * grid_h * grid_w.
 * Angles are fp32 products pos * inv_freq (inv_freq rounded once to fp32);
 * arithmetic is fp32; bf16 results are rounded to nearest even.
 * n_tokens must be a multiple of chunk_tokens and at most 2^27.
 * ------------------------------------------------------------------------ */
int wf_rope3d(void* x, int n_tokens, int n_heads, int head_dim, int dtype, int first_global_chunk,
              int frames_per_chunk, int grid_h, int grid_w, int d_t, int d_h, int d_w, float theta,
              void* stream);

/* ------------------------------------------------------------------------
 * Cache writes with RoPE on K (fused producer). They write the same slot
 * contents as wf_rope3d applied to a copy of k (chunk index global_chunk,
 * the convention above) followed by wf_kv_append / wf_kv_refresh, bit for bit,
 * but K is rotated on its way into the slot: rotated K is never stored
 * token-major, which saves one write and one read of K per chunk. k and v are
 * not modified; V is written unrotated.
 * ------------------------------------------------------------------------ */

/* Sets the RoPE geometry of the cache (frames_per_chunk * grid_h * grid_w must
 * equal chunk_tokens; split and theta as for wf_rope3d). Host-only; may be
 * called again to change it. */
int wf_kv_set_rope(wf_kv_cache* kv, int frames_per_chunk, int grid_h, int grid_w, int d_t, int d_h, int d_w,
                   float theta);

/* wf_kv_append with K rotated at the positions of global chunk global_chunk
 * (>= 0). WF_E_UNSUPPORTED when no geometry was set. */
int wf_kv_append_rope(wf_kv_cache* kv, const void* k, const void* v, int global_chunk, void* stream,
                      int* out_slot);

/* wf_kv_refresh with K rotated at the positions of global chunk global_chunk. */
int wf_kv_refresh_rope(wf_kv_cache* kv, int logical_idx, const void* k, const void* v, int global_chunk,
                       void* stream);

/* ------------------------------------------------------------------------
 * Chunk-wise causal attention of one round (the round's hot loop).
 * q, out: [n_inflight*chunk_tokens][n_heads][head_dim] in the cache dtype;
 * query chunk j (0 = refresh chunk) reads the first n_hist + j + 1 table
 * entries, n_hist = table length - n_inflight:
 *   out[i,h] = sum_k exp(s_ik) v_kh / sum_k exp(s_ik),  s_ik = scale <q_ih, k_kh>
 *   lse[h][i] = ln sum_k exp(s_ik)          (fp32, layout [n_heads][n_q]; may be NULL)
 * Accumulation is fp32; for WF_BF16 the softmax weights are rounded to bf16
 * before the weighted sum of values, and out is rounded to nearest even.
 * Results are deterministic: bitwise identical run to run, for any physical
 * slot placement, and unaffected by the contents of later chunks.
 * Requires 1 <= n_inflight <= table length, scale > 0, q and out 16-byte
 * aligned, and a round that fits one launch:
 * 2 (n_inflight + 1) n_heads (chunk_tokens + 255) < 2^32 and
 * 64 chunk_tokens n_heads < 2^32 (WF_E_SHAPE otherwise).
 * ------------------------------------------------------------------------ */
int wf_chunk_causal_attn_fwd(const void* q, const wf_kv_cache* kv, int n_inflight, float scale,
                             void* out, float* lse, void* stream);

/* Same operation with a caller-owned workspace that lets a bf16 round run
 * in-flight chunk 0 (the chunk that sees the fewest keys) as two halves of
 * its key range, whose partial softmax sums a second kernel merges: the
 * shortest work items are halved so they pack into the end of the grid.
 * Used when workspace != NULL, n_inflight >= 2 and chunk 0 sees at least two
 * 64-key tiles; otherwise this is wf_chunk_causal_attn_fwd. The merge changes
 * the summation order of chunk 0's rows only (results stay deterministic and
 * within the same tolerance of the exact values; other chunks' rows are
 * bitwise those of wf_chunk_causal_attn_fwd).
 * workspace: NULL, or device memory of wf_attn_fwd_workspace_bytes(kv) bytes,
 * 256-byte aligned, caller-owned, not overlapping q/out/lse, overwritten by
 * every call (one buffer serves every round of a cache); after a split call
 * it holds f32 [2][H][C][D] unnormalized halves, then at the next multiple of
 * 256 bytes f32 [2][H][C][2] their log2-domain row max and weight sum.
 * Calls that share a workspace must be ordered on one stream.
 * Errors: those of wf_chunk_causal_attn_fwd; WF_E_SHAPE for a misaligned
 * workspace or one that overlaps q, out, lse or a cache pool. */
size_t wf_attn_fwd_workspace_bytes(const wf_kv_cache* kv); /* 0 for fp32 caches */

int wf_chunk_causal_attn_fwd_ws(const void* q, const wf_kv_cache* kv, int n_inflight, float scale,
                                void* workspace, void* out, float* lse, void* stream);

/* Allocation-free form of wf_chunk_causal_attn_fwd_ws, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the key-split partials live in a static
 * device array of WF_STATIC_SCRATCH_BYTES bytes inside the library instead of
 * a caller's workspace. Same result, bitwise, as wf_chunk_causal_attn_fwd_ws
 * with a workspace. The caller still passes q, out and lse; the call itself
 * allocates nothing (no hipMalloc, no hipFree). Each GPU the library runs on
 * holds its own copy of the array until the process ends. Every call on one
 * GPU shares that GPU's copy: calls that overlap on one GPU (concurrent
 * streams, or host threads without ordering) race on it and must be ordered
 * on one stream. Nothing in it needs to start at zero (each call writes all it
 * reads) and it keeps the last call's partials.
 * Errors: those of wf_chunk_causal_attn_fwd; WF_E_SHAPE when the cache's
 * partials (wf_attn_fwd_workspace_bytes, about 8 n_heads chunk_tokens
 * (head_dim + 2) bytes) exceed WF_STATIC_SCRATCH_BYTES (64 MiB): 4680-token
 * chunks of head_dim 128 fit up to 13 heads, 14 heads do not. fp32 caches
 * never split and use no scratch. */
#define WF_STATIC_SCRATCH_BYTES (64ull << 20)
int wf_chunk_causal_attn_fwd_static(const void* q, const wf_kv_cache* kv, int n_inflight, float scale,
                                    void* out, float* lse, void* stream);

/* ------------------------------------------------------------------------
 * int8-QK variant (bf16 caches, head_dim 128). The pages name a
 * quantized-QK attention backend (SageAttention) in their DiT-only tests
 * (Abstract) without its internals; this call implements one scheme:
 *   mean_h = per-(head, channel) mean of the keys every query chunk sees:
 *   the n_hist history chunks and in-flight chunk 0 (fp64 sum, rounded once
 *   to fp32). No later in-flight chunk enters it, so chunk j's output depends
 *   on chunks 0..n_hist+j only (chunk-wise causal attention, Abstract; K/V
 *   handed one way from earlier to later chunks, airadar.tv summaries);
 *   Q and K - mean are quantized per head in blocks of 128 tokens that start
 *   at every chunk start: s = amax/127 (1 if amax = 0), code =
 *   clamp(round_half_even(x/s), -127, 127), all decisions in fp32;
 *   S = int32 dot products of the codes times s_q * s_k * scale (the
 *   kernel's log2-domain factor s_q * s_k * scale * log2(e) keeps 21
 *   significant bits); softmax fp32; P rounded to bf16; P.V in bf16 with
 *   fp32 accumulation; the softmax denominator sums the fp32 weights.
 * The mean shift changes no softmax row; lse refers to the unshifted keys
 * (the kernel adds scale * <q^_i, mean_h>, q^ the dequantized query).
 * workspace: device memory of wf_attn_i8qk_workspace_bytes() bytes, 256-byte
 * aligned, caller-owned, not overlapping q, out, lse or a cache pool
 * (WF_E_SHAPE), overwritten by every call. After a call it holds,
 * each array starting at the next multiple of 256 bytes, in this order
 * (n_tab = table length, N = n_inflight, C = chunk_tokens, nb = ceil(C/128)):
 *   f64 [n_hist+1][4][H][128]  key sums of each quarter of the 64-key tiles
 *       of history chunk c (c < n_hist) or in-flight chunk 0 (c = n_hist)
 *       (tiles [g*T/4, (g+1)*T/4), T = ceil(C/64))   f32 [H][128] key mean
 *   i8  [n_tab][H][S_pad/64][8][64][16]  K - mean codes as 64-key tile images
 *       (16-dim pieces, key-major), in table order, zero past each chunk end
 *   f32 [H][n_tab][nb] K block scales   i8 [N*C][H][128] Q codes
 *   f32 [H][N][nb] Q block scales       f32 [H][N*C] <q^_i, mean_h>
 * Limit: the K scales of all table entries (n_tab * nb floats) must fit in
 * 64 KB of LDS beside the tile stages, i.e. n_tab * nb <= 16384; larger
 * rounds return WF_E_SHAPE.
 * ------------------------------------------------------------------------ */
size_t wf_attn_i8qk_workspace_bytes(const wf_kv_cache* kv, int n_inflight);

int wf_chunk_causal_attn_fwd_i8qk(const void* q, const wf_kv_cache* kv, int n_inflight,
                                  float scale, void* workspace, void* out, float* lse,
                                  void* stream);

/* ------------------------------------------------------------------------
 * W8A8 linear (the int8 linears around attention). The pages name a W8A8
 * backend for the DiT linears in their DiT-only tests (Abstract) without its
 * internals; this is one concrete scheme:
 *   per row (token of X, output channel of W): s = amax/127 (1 if amax = 0),
 *   code = clamp(round_half_even(x/s), -127, 127), all decisions in fp32;
 *   acc[m][n] = sum_k Xq[m][k] Wq[n][k] exactly in int32;
 *   y[m][n] = bf16( fma((float)acc, s_x[m] * s_w[n], bias[n]) ).
 * ------------------------------------------------------------------------ */

/* Quantizes rows x[rows][cols] (WF_BF16, device, 16-byte aligned; cols a
 * multiple of 8; rows <= 2^24) into caller-owned codes int8 [rows][cols]
 * (8-byte aligned) and scales fp32 [rows], enqueued on the stream.
 * Errors: WF_E_NULL, WF_E_DTYPE (x not WF_BF16), WF_E_SHAPE (sizes or
 * alignment), WF_E_HIP (launch); nothing is enqueued on an argument error. */
int wf_quant_rows_i8(const void* x, int rows, int cols, int dtype, void* codes, float* scales, void* stream);

/* Y = W8A8 linear of xq int8 [M][K] (scales sx [M]) with wq int8 [N][K]
 * (output features x input features, scales sw [N]) and optional bias
 * (WF_BF16 [N], may be NULL). out_dtype WF_BF16 gives y bf16 [M][N];
 * WF_I32 gives the raw int32 accumulators (sx, sw, bias ignored).
 * Requires N a multiple of 8, K a multiple of 64 (<= 131072, so |acc| < 2^31),
 * at most 2^22 output tiles of 256 x 256, xq, wq, y 16-byte aligned. All
 * pointers are caller-owned device pointers; y is written, nothing else.
 * Errors: WF_E_NULL (xq, wq, y, or sx/sw for WF_BF16 output), WF_E_DTYPE,
 * WF_E_SHAPE, WF_E_HIP; M = 0 is a no-op. */
int wf_gemm_w8a8(const void* xq, const float* sx, const void* wq, const float* sw, const void* bias, int M, int N,
                 int K, int out_dtype, void* y, void* stream);

/* ------------------------------------------------------------------------
 * 1F1C rollout: the round structure around the attention path.
 * The pages stagger the denoising stages and the cache-refresh stage so that
 * they run concurrently, and after the pipeline fills every forward round
 * outputs one chunk (Abstract); the run holds wp-size = steps + 1 stages
 * (airadar.tv summaries, usage section). Reading used here:
 *   stage s of chunk c runs in round c + s; s = 0 .. n_steps-1 are the
 *   denoising steps (0 = noisiest), s = n_steps is the refresh pass that
 *   writes the finished chunk's clean K/V for later chunks;
 *   round r's query block lists its chunks cleanest first (ascending chunk);
 *   the chunk at stage n_steps-1 is the round's output, so rounds
 *   0 .. n_steps-2 output nothing (pipeline fill);
 *   the last chunk has no refresh pass: n_chunks chunks take
 *   n_chunks + n_steps - 1 rounds;
 *   history in round r: the newest hist_window chunks whose refresh pass
 *   ran in an earlier round.
 * ------------------------------------------------------------------------ */
typedef struct wf_round_plan {
  int round;
  int n_inflight;                   /* chunks in this round's query block, 1 .. n_steps + 1 */
  int inflight_chunk[WF_MAX_TABLE]; /* their chunk ids, cleanest first                     */
  int inflight_stage[WF_MAX_TABLE]; /* their stages; n_steps = the refresh pass            */
  int n_hist;                       /* history chunks visible this round                   */
  int hist_chunk[WF_MAX_TABLE];     /* their chunk ids, oldest first                       */
  int new_chunk;                    /* chunk entering at stage 0 (appended), or -1         */
  int output_chunk;                 /* chunk finishing its last denoising stage, or -1     */
  int evict_after;                  /* oldest entries to evict after attention             */
} wf_round_plan;

/* Rounds of a rollout: n_chunks + n_steps - 1, or a negative status for
 * n_steps < 1, n_chunks < 1 or n_steps + 1 > WF_MAX_TABLE. */
int wf_1f1c_rounds(int n_steps, int n_chunks);

/* Fills *plan for round `round` (0 .. rounds-1). Needs hist_window >= 0 and
 * hist_window + n_steps + 1 <= WF_MAX_TABLE. Host only; no device work. */
int wf_1f1c_plan(int n_steps, int n_chunks, int hist_window, int round, wf_round_plan* plan);

/* Enqueues one round on the stream, in this order: append the new chunk's
 * K/V (k[n_inflight-1], v[n_inflight-1]) when plan->new_chunk >= 0; refresh
 * every other in-flight entry i with k[i], v[i] (this round's K/V of that
 * chunk, [chunk_tokens][n_heads][head_dim] each, 16-byte aligned); run
 * wf_chunk_causal_attn_fwd_ws over the n_inflight chunks (q, out: the round's
 * query block [n_inflight*chunk_tokens][n_heads][head_dim]; lse optional;
 * workspace NULL or of wf_attn_fwd_workspace_bytes(kv) bytes, 256-aligned,
 * disjoint from q, out, lse and the cache pools);
 * evict plan->evict_after oldest entries. The cache table must hold the
 * previous round's state: n_hist + n_inflight entries, less one when a chunk
 * is appended. k and v are host arrays of n_inflight device pointers.
 * With a RoPE geometry on the cache (wf_kv_set_rope), the query block is
 * first rotated in place (chunk ids inflight_chunk[0] .. as global chunk
 * indices, which must be consecutive) and K is rotated inside the cache
 * writes (wf_kv_append_rope / wf_kv_refresh_rope); V is written as is.
 * Every argument is checked before anything is enqueued (WF_E_NULL,
 * WF_E_SHAPE, WF_E_FULL; the cache is unchanged on these); WF_E_HIP means a
 * launch was rejected after earlier steps of the round were enqueued. */
int wf_1f1c_run_round(wf_kv_cache* kv, const wf_round_plan* plan, void* q, const void* const* k,
                      const void* const* v, float scale, void* workspace, void* out, float* lse,
                      void* stream);

/* ---- diagnostics ---- */
const char* wf_status_str(int status); /* static string for a status code      */
const char* wf_last_error(void);      /* thread-local text of the last failure */
int wf_version(void);                 /* major*10000 + minor*100 + patch       */
/* Compute units and peak shader clock (kHz) of a device, as the runtime reports
 * them: the dense bf16 MFMA peak is n_cu x 4096 flop/clk x clock. Host only,
 * no device work; WF_E_NULL, or WF_E_HIP for an invalid device. */
int wf_device_peak_info(int device, int* n_cu, int* peak_clock_khz);

#ifdef __cplusplus
}
#endif

#endif /* WF_H */
