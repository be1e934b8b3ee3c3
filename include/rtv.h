/*
 * rtv.h — C ABI of the KV-cache upkeep + chunk-attention library for MI355X (gfx950).
 *
 * What the library does, as the pages describe the serving path of an
 * autoregressive video diffusion transformer at batch size one:
 *   - each new four-frame chunk's K/V enter a per-layer cache ONCE, with RoPE
 *     and FP8 quantization applied at that moment, into a circular buffer that
 *     advances by moving a head index rather than by copying
 *     [page "Runway explains how it serves a 57B video model in real time"
 *      (aidose.in), fourth paragraph; page "Runway: Πώς ένα AI 57 δισ.
 *      παραμέτρων παράγει βίντεο στα 24 fps" (pttl.gr), section "Από οκτώ H100
 *      σε τέσσερις"];
 *   - the chunk's queries then attend over the valid FP8 window, 240 such
 *     calls per diffusion step [pttl.gr, same section];
 *   - the step must not synchronize with the host: one host read-back per step
 *     is reported to have raised the step time from 168.5 ms to 278 ms
 *     [aidose.in, fifth paragraph].
 * The pages give no API; the calls below are this library's own.
 *
 * Conventions for every call:
 *   - returns rtv_status: RTV_OK (0) or a negative RTV_ERR_* code;
 *   - validates all arguments before enqueuing anything; on error nothing is
 *     enqueued and the cache state is unchanged;
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream);
 *   - rtv_append_rope_quant / rtv_attend / rtv_advance never synchronize,
 *     never allocate, and only enqueue work on `stream`;
 *   - device pointers must be 16-byte aligned; token strides are in elements
 *     and must be multiples of 8;
 *   - bf16 = IEEE bfloat16 bit patterns, fp8 = OCP E4M3FN codes (bias 7,
 *     max 448, NaN = 0x7F/0xFF, no infinities);
 *   - a handle is not thread-safe; calls on one handle must be ordered.
 */
#ifndef RTV_H
#define RTV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t rtv_status;
#define RTV_OK 0
#define RTV_ERR_INVALID_ARG (-1)  /* a pointer, size, index or config field is out of range */
#define RTV_ERR_BUFFER (-2)       /* the caller's device buffer is too small or misaligned */
#define RTV_ERR_HIP (-3)          /* the HIP runtime reported an error (launch, copy, device) */
#define RTV_ERR_STATE (-4)        /* call out of order: attend/advance before append, RoPE table exhausted */
#define RTV_ERR_UNSUPPORTED (-5)  /* a shape the kernels do not implement (e.g. head_dim not 64/128) */

/* Opaque handle: one per session, holding the ring state of every layer. */
typedef struct rtv_cache rtv_cache;

/* Static description of one session's caches (all layers share it). */
typedef struct rtv_config {
  int32_t n_layers;          /* >= 1 */
  int32_t n_q_heads;         /* query heads; multiple of n_kv_heads (grouped-query attention) */
  int32_t n_kv_heads;        /* heads stored in the cache */
  int32_t head_dim;          /* D: 64 or 128 */
  int32_t tokens_per_frame;  /* T: latent tokens of one frame */
  int32_t chunk_frames;      /* F: frames appended per call (4 on the pages) */
  int32_t capacity_frames;   /* C: ring capacity in frames; multiple of F */
  int32_t max_global_frames; /* frames the session may ever append: extent of the RoPE table */
  int32_t query_terms;       /* e4m3 terms carrying each query through the matrix cores
                              * (each query with its own power-of-two scale, applied
                              * exactly by the matrix core):
                              * 1 (or 0): one term, relative rounding error 2^-4;
                              * 2: hi + 2^-4 lo, relative error about 2^-8, on every window
                              * (costs about 20% more attention time on long windows).
                              * Query tiles recomputed as peaked (prob_terms 0) and the
                              * two-term kernels always carry two terms. */
  int32_t prob_terms;        /* e4m3 terms carrying each attention weight P' into the PV
                              * product:
                              * 0 (default): one code read off the log domain (within one
                              * code step of the correctly rounded value, up to about 6%
                              * per weight), checked: every query row also measures how
                              * few keys carry its weight (sum of squared weights, on the
                              * matrix cores), and the query tiles holding a row above
                              * 5e-4 are recomputed in a second launch with queries and
                              * weights as two e4m3 terms (relative error about 2^-8).
                              * Rows whose weight spreads over many keys, where the
                              * one-code errors average out, cost one extra matrix-core
                              * product per tile; each recomputed query tile costs about
                              * twice its one-code time;
                              * 1: one code, unchecked, on windows of 8192 keys or more
                              * (two terms on shorter ones; in the device-state mode the
                              * choice follows the chunk length): outside the attention
                              * tolerance on peaked rows (a few keys carrying much of the
                              * weight);
                              * 2: two terms on every window, for callers that know their
                              * attention is peaked (about 1.8 times the one-code time on
                              * a 47872-key window). */
  double rope_base;          /* RoPE base (10000) */
  const float* rope_cos_sin_host;
                             /* optional host table [max_global_frames*T][D/2][2] of the
                              * (cos, sin) pairs of every position, read once by
                              * rtv_cache_create (the caller keeps ownership); NULL: the
                              * library computes it as rtv_rope_fill_host does.  Callers
                              * that check the codes against another implementation pass
                              * one table to both, so that no libm difference can move a
                              * code.  The arena holds the table for the whole session:
                              * max_global_frames * T * D * 4 bytes (1.53 MB per frame of
                              * 2992 tokens at D = 128; 132 GB for an hour at 24 frames
                              * per second), so max_global_frames bounds a session. */
} rtv_config;

/* Device layout of one layer's ring, for read-back and for callers that fuse
 * their own producers.  Slot s of the ring holds token t of global frame g
 * with s = (g mod C) * T + t.  S = C*T slots, padded to Sp = ceil(S/64)*64.
 *   k_codes  [n_kv_heads][Sp][D]        u8  RoPE-rotated K, e4m3, row per slot
 *   v_codes  [n_kv_heads][Sp/64][D][64] u8  V, e4m3, transposed per 64-slot tile;
 *            byte p of a tile row holds slot 64*tile + key(p) with
 *            h = p / 32, b = p % 32,
 *            key(p) = 32*(b >> 4) + 8*((b >> 2) & 3) + 4*h + (b & 3)
 *            (the key order of the attention kernel's matrix-core operands)
 *   k_scales [n_kv_heads][Sp]           f32 per-(slot, head) scale = amax/448
 *   v_scales [n_kv_heads][Sp]           f32
 * Dequantized value = decode(code) * scale; scale 0 means an all-zero row. */
typedef struct rtv_layout {
  void* k_codes;
  void* v_codes;
  float* k_scales;
  float* v_scales;
  int64_t slots;              /* S */
  int64_t slots_padded;       /* Sp */
  int64_t next_global_frame;  /* global frame of the chunk the next append writes */
  int32_t head_frame;         /* next_global_frame mod C: ring frame of that chunk */
  int32_t committed_frames;   /* valid frames before that chunk, at most C */
  int32_t appended;           /* 1 if a chunk was appended since the last advance */
  int32_t reserved;
} rtv_layout;

/* The window an attend reads, in slot space: at most two contiguous
 * segments [start, start+len) (the second exists when the window wraps). */
typedef struct rtv_window {
  int32_t window_frames;      /* W = min(committed + F, C, max_window or C) */
  int32_t n_segments;         /* 1 or 2 */
  int64_t seg_start[2];
  int64_t seg_len[2];
  int64_t write_slot;         /* first slot of the chunk being written: head_frame * T */
} rtv_window;

/* ---- sizing and lifetime ------------------------------------------------ */

/* Device bytes the caller must provide to rtv_cache_create for `cfg`:
 * the RoPE table (max_global_frames*T positions x D/2 (cos, sin) f32 pairs),
 * the attention workspace, 16 bytes of ring state per layer (device-state
 * mode) and, per layer, the codes and scales above.  Host-only; no GPU needed. */
rtv_status rtv_cache_bytes(const rtv_config* cfg, size_t* bytes);

/* Create a cache handle over the caller's device buffer `dev_buf` (>= the
 * size from rtv_cache_bytes, 256-byte aligned; the caller keeps ownership and
 * must keep it alive until rtv_destroy).  Builds the RoPE table on the host
 * (angle pos*base^(-2i/D) and its cosine/sine in double precision by the C
 * library, rounded once to float), uploads it, and zero-fills the ring; this
 * call synchronizes `stream` (not on the hot path).  All layers start empty at
 * global frame 0. */
rtv_status rtv_cache_create(const rtv_config* cfg, void* dev_buf, size_t bytes,
                            void* stream, rtv_cache** out);

/* Free the handle (host memory only); the device buffer stays the caller's. */
rtv_status rtv_destroy(rtv_cache* cache);

/* ---- the hot path ------------------------------------------------------- */

/* Cache upkeep for one layer: rotate the chunk's K by RoPE at global positions
 * next_global_frame*T + t, quantize K (rotated) and V per (token, head) to
 * e4m3 with an f32 scale amax/448 (codes = nearest e4m3 of f32(x/scale), ties
 * to even, saturating; scale 0 gives signed zero codes), and write codes and
 * scales to the ring slots of the current chunk.  A second append before
 * rtv_advance rewrites the same slots (the repeated calls of one step).
 *   k_bf16: [n_tokens][n_kv_heads][D] bf16, row stride k_tok_stride elements
 *   v_bf16: same shape, stride v_tok_stride
 *   n_tokens must equal chunk_frames * tokens_per_frame.
 * Errors: INVALID_ARG (layer, pointers, strides, n_tokens), STATE (the RoPE
 * table does not reach next_global_frame + chunk_frames). */
rtv_status rtv_append_rope_quant(rtv_cache* cache, int32_t layer,
                                 const void* k_bf16, int64_t k_tok_stride,
                                 const void* v_bf16, int64_t v_tok_stride,
                                 int32_t n_tokens, void* stream);

/* Chunk attention for one layer: RoPE the chunk's queries (same positions as
 * the appended chunk), then for each query head h (KV head h / (Hq/Hkv))
 * compute softmax(q.k / sqrt(D)) over every key of the window (the whole
 * current chunk included: no mask inside the chunk) and the weighted sum of
 * the dequantized V, written as bf16.  Queries and probabilities are carried
 * in e4m3 through the matrix cores with f32 accumulation (results are within
 * a tolerance of exact attention, not bit-exact).
 *   q_bf16:   [n_tokens][n_q_heads][D] bf16, row stride q_tok_stride (un-rotated)
 *   out_bf16: [n_tokens][n_q_heads][D] bf16, row stride out_tok_stride
 *   max_window_frames: 0 = all valid frames; otherwise caps W (>= chunk_frames)
 * The append of this step must be ordered before this call on `stream`.
 * Every attention call on one cache (any layer) uses the same workspace in the
 * cache's arena (per-window key factors and partial results of split key
 * ranges): calls that could overlap on the GPU must be ordered, e.g. on one
 * stream.
 * Errors: INVALID_ARG, STATE (no append since the last advance). */
rtv_status rtv_attend(rtv_cache* cache, int32_t layer,
                      const void* q_bf16, int64_t q_tok_stride,
                      void* out_bf16, int64_t out_tok_stride,
                      int32_t max_window_frames, void* stream);

/* Commit the current chunk of `layer` (-1 = every layer): the head index moves
 * by chunk_frames, committed = min(committed + F, C).  Host state only; no
 * device work is enqueued (in the device-state mode below: one small kernel on
 * `stream` that moves the state in the arena).  Errors: STATE (no append since
 * the last advance). */
rtv_status rtv_advance(rtv_cache* cache, int32_t layer, void* stream);

/* ---- device-resident ring state (for graph capture) ----------------------
 * The pages capture the forward pass in a CUDA graph [page "Runway partage la
 * construction de Runway Characters" (lhc.media), fourth paragraph].  A
 * captured graph freezes kernel arguments, while the ring state moves every
 * step.  Between rtv_device_state_begin and rtv_device_state_end the state of
 * every layer (next global frame, committed frames) lives in the arena:
 *   - rtv_append_rope_quant and rtv_attend enqueue kernels that read it (the
 *     chunk's slots, its RoPE rows, the window, the split schedule), with
 *     grids sized for the largest window;
 *   - rtv_advance enqueues a kernel that moves it;
 * so a sequence of these calls captured once (hipStreamBeginCapture, or
 * torch.cuda.graph) replays correctly step after step.  The results equal
 * the host-state calls' (same kernels and arithmetic; with prob_terms 1 the
 * two-term variant, which host-state calls take on windows under 8192 keys,
 * follows the shortest possible window, one chunk, instead of the current
 * one).
 * While the mode is on, rtv_cache_layout and rtv_cache_window report the
 * state as of rtv_device_state_begin, and the host checks only the argument
 * and call-order rules; a chunk past the end of the RoPE table makes the
 * kernels write nothing and is reported by rtv_device_state_end.
 * rtv_device_state_begin copies the host state into the arena and
 * synchronizes `stream`.  Errors: STATE (already on), HIP. */
rtv_status rtv_device_state_begin(rtv_cache* cache, void* stream);
/* Copy the state back to the host (synchronizes `stream`) and return to the
 * host-state mode.  Errors: STATE (the mode was off, or a call in the mode
 * found the RoPE table exhausted; the state is copied back either way), HIP. */
rtv_status rtv_device_state_end(rtv_cache* cache, void* stream);

/* ---- inspection (tests, fused producers) -------------------------------- */

rtv_status rtv_cache_layout(const rtv_cache* cache, int32_t layer, rtv_layout* out);

/* Number of query tiles (units of 256 queries of one query head) that the
 * latest rtv_attend on this cache flagged as peaked and recomputed with
 * two-term queries and weights (prob_terms 0; 0 for calls that took another
 * variant).  Copies one word from the arena and synchronizes `stream`: for
 * tests and monitoring, not the hot path. */
rtv_status rtv_cache_peaked_units(const rtv_cache* cache, int32_t* units, void* stream);

/* The window an attend of `layer` would read now. */
rtv_status rtv_cache_window(const rtv_cache* cache, int32_t layer,
                            int32_t max_window_frames, rtv_window* out);

/* Pure ring arithmetic (no handle, no GPU): the window of a layer whose next
 * chunk starts at global frame `next_global_frame` with `committed_frames`
 * valid frames before it. */
rtv_status rtv_ring_window(int64_t next_global_frame, int32_t committed_frames,
                           int32_t tokens_per_frame, int32_t chunk_frames,
                           int32_t capacity_frames, int32_t max_window_frames,
                           rtv_window* out);

/* Host fill of the RoPE table rows [pos0, pos0+npos): out[(p*D/2 + i)*2 + 0/1]
 * = cos/sin of p*base^(-2i/D), double precision then rounded to float; the
 * same values rtv_cache_create uploads.  No GPU needed. */
rtv_status rtv_rope_fill_host(int32_t head_dim, double rope_base, int64_t pos0,
                              int64_t npos, float* out);

/* Encode n floats to e4m3 codes on the device with the conversion the append
 * kernel uses (for exhaustive checks of its rounding). */
rtv_status rtv_encode_e4m3(const float* x_dev, uint8_t* codes_dev, int64_t n, void* stream);

const char* rtv_status_string(rtv_status status);

/* ---- projection (the largest workload) ----------------------------------- */

/* Per-tensor e4m3 quantization of n bf16 values, no host read-back:
 * scale = f32(amax/448) written to *scale_dev, codes = e4m3(f32(x/scale)).
 * `workspace` must hold rtv_quant_workspace_bytes(n) device bytes. */
size_t rtv_quant_workspace_bytes(int64_t n);
rtv_status rtv_quant_fp8_per_tensor(const void* x_bf16, int64_t n, uint8_t* codes_dev,
                                    float* scale_dev, void* workspace, void* stream);

/* For callers that cannot allocate device memory (code under graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the quantization
 * above with its workspace held by the library, a static device array of 1024
 * words per GPU (4 KiB, kept until the process ends; the first call on a
 * device looks up that device's copy).  Same results as
 * rtv_quant_fp8_per_tensor for every n >= 0: a launch uses at most 1024
 * partial maxima whatever n is, so no input is too large for the array.
 * Allocates nothing.  Calls that may overlap on one GPU race on the array:
 * order them (e.g. one stream).  Errors: INVALID_ARG (pointers, alignment,
 * n < 0), HIP (the array's address could not be found). */
rtv_status rtv_quant_fp8_per_tensor_static(const void* x_bf16, int64_t n, uint8_t* codes_dev,
                                           float* scale_dev, void* stream);

/* C[M][N] (bf16, row stride ldc) = (*sa) * (*sb) * A[M][K] * B[K][N], A and B
 * e4m3 codes, A row-major [M][K], B given TRANSPOSED as Bt[N][K] (row-major),
 * f32 accumulation, one rounding to bf16.  K must be a multiple of 64, M and N
 * any size. */
rtv_status rtv_gemm_fp8(const uint8_t* a, const float* sa_dev, const uint8_t* bt,
                        const float* sb_dev, void* c_bf16, int32_t M, int32_t N,
                        int32_t K, int64_t ldc, void* stream);

/* The projection GEMM fused with the cache upkeep (the fused FP8 matmul of
 * [aidose.in, fourth paragraph], whose K/V enter the cache with RoPE and FP8
 * applied at write time, same paragraph): for the n_tokens = chunk_frames *
 * tokens_per_frame tokens of the current chunk of `layer`,
 *   QKV[m][n] = (*sx_dev) * (*sw_dev) * sum_k dec(x_codes[m][k]) * dec(wt_codes[n][k])
 * with f32 accumulation, columns ordered [q_cols Q columns | n_kv_heads K heads
 * | n_kv_heads V heads] (head_dim columns per head).  Q columns are written
 * to q_bf16 ([n_tokens][q_tok_stride] bf16) exactly as rtv_gemm_fp8 writes
 * them.  K and V never go through bf16: from the f32 values the epilogue
 * applies RoPE to K at the chunk's positions and quantizes each (token, head)
 * row with the append's rule (scale = RN(amax/448), code = e4m3(RN(x/scale)))
 * into the chunk's ring slots, then counts as the layer's append.  It equals
 * rtv_gemm_fp8 followed by rtv_append_rope_quant except for the bf16 rounding
 * of K and V in between (codes may differ by one step).
 *   x_codes: [n_tokens][k_dim] e4m3; wt_codes: [q_cols + 2*n_kv_heads*head_dim][k_dim]
 *   e4m3 (the weight transposed); k_dim a multiple of 64; q_cols a multiple of
 *   head_dim (0 = no Q columns, q_bf16 may then be NULL).
 * Errors: INVALID_ARG (shapes, pointers, alignment), STATE (RoPE table
 * exhausted), UNSUPPORTED (a chunk that is not a multiple of 64 tokens, or
 * the device-state mode). */
rtv_status rtv_qkv_gemm_append(rtv_cache* cache, int32_t layer,
                               const uint8_t* x_codes, const float* sx_dev,
                               const uint8_t* wt_codes, const float* sw_dev,
                               int32_t n_tokens, int32_t k_dim, int32_t q_cols,
                               void* q_bf16, int64_t q_tok_stride, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* RTV_H */
