/*
 * libsinkattn -- frame-sink + short-window KV attention for one MI355X (gfx950).
 *
 * The operations follow two reviewed papers:
 *   [LongLive]  "LongLive: Real-time Interactive Long Video Generation",
 *               paper review page (xllm-io paper-review blog).
 *   [LoL]       "LoL: Longer than Longer, Scaling Video Generation to Hour",
 *               paper review page (rainbus paper reviews).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Tensors crossing the boundary are dense, row-major, in the [B, T, H, D]
 *   token-major layout the LoL review states for Q and K ("method steps" (1)):
 *   B streams, T tokens (latent frames x tokens per frame), H heads, D channels.
 *   Token i of a latent frame sits at grid row i / grid_w, column i % grid_w.
 * - Device pointers are plain device addresses (hipMalloc / torch CUDA
 *   tensors); host pointers are marked "host".  The library never frees or
 *   keeps a caller pointer beyond the call, except the two cache stores named
 *   in sa_cache_desc, which it borrows for the cache handle's lifetime.
 * - `stream` is a hipStream_t passed as void* (NULL = the legacy default
 *   stream).  Every launch is asynchronous on that stream; no call
 *   synchronises the host except sa_rope_create (one table upload).
 * - Element types: SA_BF16 (bfloat16, round-to-nearest-even on every store)
 *   or SA_F32.  All arithmetic is fp32 (bf16 MFMA inputs, fp32 accumulation);
 *   RoPE time-axis angles are formed and range-reduced in fp64 on the device,
 *   grid-axis sines and cosines are evaluated in fp64 once, on the host.
 * - Every function returns an sa_status.  Arguments and state are validated
 *   before anything is changed or launched: on error the handle is left as it
 *   was and sa_last_error() (thread-local) describes the problem.
 *   SA_ERR_HIP reports a HIP runtime / launch error; device faults surface at
 *   the caller's next synchronisation -- or, with SA_DEBUG_SYNC=1 in the
 *   environment when the library loads, at the call that caused them: every
 *   entry point then waits for its stream after launching and returns
 *   SA_ERR_HIP naming the launch (debugging only; it serialises the stream
 *   and must not be used under HIP graph capture).
 * - Handles are not thread-safe; distinct handles are independent.  A handle
 *   is bound to the device that was current at its creation.
 * - Alignment: every device pointer must be 16-byte aligned.
 * - A cache call's inputs and outputs must not overlap the cache's own two
 *   stores, and an output must not overlap that call's inputs
 *   (SA_ERR_RANGE, nothing changed or launched).
 */
#ifndef SINKATTN_H
#define SINKATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SA_OK = 0,
  SA_ERR_NULL = 1,   /* a required pointer is NULL */
  SA_ERR_SHAPE = 2,  /* sizes inconsistent or unsupported */
  SA_ERR_DTYPE = 3,  /* element type unsupported or mismatched */
  SA_ERR_ALIGN = 4,  /* pointer not 16-byte aligned */
  SA_ERR_STATE = 5,  /* the cache cannot do this now (e.g. attend on an empty cache) */
  SA_ERR_RANGE = 6,  /* a value is out of range (positions, chunk size, workspace) */
  SA_ERR_HIP = 7     /* HIP runtime or launch failure */
} sa_status;

/* SA_FP8 is a cache element type only: keys and values stored as OCP e4m3
 * (8 bits, max 448) with a per-tensor scale each (sa_cache_desc.k_scale,
 * v_scale); the tensors such a cache exchanges at the boundary (k, v, q, o)
 * are SA_BF16.  Supported with head_dim 128 by append, attention and read. */
typedef enum { SA_BF16 = 0, SA_F32 = 1, SA_FP8 = 2 } sa_dtype;

/* Attention mask inside a multi-frame query chunk.
 * SA_MASK_NONE: every query sees every resident frame.
 * SA_MASK_FRAME_CAUSAL: a query of latent frame f sees the resident frames
 * f' <= f in full (frame-level autoregression, [LongLive] section 2 "solution
 * overview"; chunk-wise generation compared in section 5's table). */
typedef enum { SA_MASK_NONE = 0, SA_MASK_FRAME_CAUSAL = 1 } sa_mask;

#define SA_AXIS_T 1u
#define SA_AXIS_H 2u
#define SA_AXIS_W 4u
#define SA_MAX_FRAMES 64 /* n_sink + n_local */

/* ------------------------------------------------------------------ RoPE --
 * 3D rotary position embedding with LoL's per-head jittered base.
 * [LoL] background "Rotary Position Embedding": channel pair p at position pos
 *   is rotated by R(phi) = [[cos phi, -sin phi], [sin phi, cos phi]],
 *   phi = pos * w_p, w = base^(-2j/d).
 * [LoL] "method steps" (2)-(7): per head h, theta_hat_h = theta0 (1 + sigma eps_h),
 *   eps_h ~ U[-1, 1] drawn by the caller (the library has no RNG).
 * Layout of the head dimension: adjacent pairs (2p, 2p+1); consecutive
 * segments [t | h | w] of dim_t, dim_h, dim_w channels; segment a uses
 * w_{a,j} = base_a^(-2j/dim_a), j = 0 .. dim_a/2 - 1, with base_a =
 * theta_hat_h on jittered axes (jitter_axes bitmask) and theta0 elsewhere.
 * Positions: t = the latent frame's time index; h = token / grid_w;
 * w = token % grid_w.
 * [LoL] results, position-interpolation (PI) baseline: positions compressed
 *   by a factor.  Here the time position becomes t * t_scale (grid positions
 *   unchanged); the library folds t_scale into the time-axis frequencies, so
 *   the angle is t * (w * t_scale).
 */
typedef struct {
  int32_t n_heads;      /* H >= 1 */
  int32_t head_dim;     /* D in {64, 128} */
  int32_t dim_t, dim_h, dim_w; /* even, sum = D */
  int32_t grid_h, grid_w;      /* tokens per latent frame = grid_h * grid_w, a multiple of 8 */
  double theta0;        /* > 1 */
  double sigma;         /* jitter scale, >= 0; every theta_hat must stay > 1 */
  const double* eps;    /* host [H], each in [-1, 1]; NULL = no jitter; copied */
  uint32_t jitter_axes; /* SA_AXIS_* bitmask; 0 is treated as SA_AXIS_T */
  double t_scale;       /* time-position scale (PI); 0 is treated as 1; else finite, > 0 */
  /* Optional per-head, per-axis bases, host [H*3] in (t, h, w) order per
   * head, each finite and > 1; copied.  When non-NULL it is theta_hat itself
   * ([LoL] "method steps" (4)) and theta0, sigma, eps and jitter_axes are
   * ignored, so any per-axis base can be expressed; NULL = build theta_hat
   * from theta0, sigma, eps and jitter_axes as above. */
  const double* theta;
} sa_rope_desc;

typedef struct sa_rope sa_rope;

/* Host-only: per-head bases theta_hat [H*3] (t, h, w) and frequencies
 * w [H*D/2] in fp64, as the device tables will hold them (time-axis entries
 * multiplied by t_scale).  No HIP call; either output may be NULL. */
sa_status sa_rope_tables(const sa_rope_desc* desc, double* theta_hat_out, double* freq_out);

/* Validates desc, builds the fp64 frequency table and the cos/sin table of
 * the grid-axis angles (row and column positions do not change from frame to
 * frame; evaluated in fp64, stored in fp32) and uploads them to the current
 * device (the only allocating / synchronising call of the library besides
 * this handle's destroy). */
sa_status sa_rope_create(const sa_rope_desc* desc, sa_rope** out);
void sa_rope_destroy(sa_rope* rope);

/* y = RoPE(x) for n_frames latent frames: x, y [B, n_frames*T_f, H, D] of
 * dtype; frame j of the token axis has time t0 + j.  y may be x itself
 * (in place); any other overlap of y with x is SA_ERR_RANGE. */
sa_status sa_rope3d_apply(const sa_rope* rope, const void* x, void* y, sa_dtype dtype,
                          int32_t batch, int32_t n_frames, int64_t t0, void* stream);

/* ----------------------------------------------------------------- cache --
 * [LongLive] section 3 "Frame Sink" and "Short-Window Attention": the KV of
 * the first n_sink latent frames is pinned for the whole stream; the other
 * frames live in a local window of the n_local most recent frames (the paper
 * uses 3 sink + 9 local = 12 frames, section 6 implementation table).
 * Frame f < n_sink goes to sink slot f; frame f >= n_sink to ring slot
 * (f - n_sink) mod n_local, evicting the frame that held it.
 * Logical order = sinks, then local frames oldest -> newest.
 *
 * Storage (library-internal layout, caller-allocated, borrowed):
 *   k_store: [n_sink + n_local][B][H][T_f][D]   keys, rotated at their frame time
 *   v_store: [n_sink + n_local][B][H][D][T_f]   values, transposed per (slot, b, h)
 * Each store is sa_cache_store_bytes(desc) bytes and must be below 4 GiB (the
 * kernels address a store with 32-bit byte offsets; larger caches fail with
 * SA_ERR_SHAPE).  Use sa_cache_read to view a frame in the boundary layout.
 */
typedef struct {
  int32_t batch;            /* B >= 1 */
  int32_t n_heads;          /* must equal the rope's */
  int32_t head_dim;         /* must equal the rope's */
  int32_t tokens_per_frame; /* must equal the rope's grid_h * grid_w */
  int32_t n_sink;           /* >= 0 */
  int32_t n_local;          /* >= 1, n_sink + n_local <= SA_MAX_FRAMES */
  sa_dtype dtype;
  void* k_store;            /* device */
  void* v_store;            /* device */
  /* SA_FP8 only: stored key = e4m3(rotated key / k_scale), stored value =
   * e4m3(value / v_scale), each clamped to +-448 first (round to nearest
   * even).  Finite and > 0; ignored for the other element types. */
  float k_scale;
  float v_scale;
} sa_cache_desc;

typedef struct sa_cache sa_cache;

typedef struct {
  int64_t frame;   /* frame number (0-based count of appended frames) */
  int64_t t;       /* time position the key was rotated with */
  int32_t segment; /* 0 sink, 1 ring */
  int32_t slot;    /* index inside its segment */
} sa_slot;

/* Bytes of ONE store (k or v) for desc; 0 if desc is invalid. */
size_t sa_cache_store_bytes(const sa_cache_desc* desc);
/* The same number under its short name: the caller allocates k_store and
 * v_store of sa_cache_bytes(desc) bytes each. */
size_t sa_cache_bytes(const sa_cache_desc* desc);

/* Host metadata only; makes no HIP call.  rope must outlive the cache. */
sa_status sa_cache_create(const sa_cache_desc* desc, const sa_rope* rope, sa_cache** out);
void sa_cache_destroy(sa_cache* cache);

/* Forget every frame (the "no KV cache" policy at a prompt switch,
 * [LongLive] section 3 "KV Recache", strategy comparison). */
sa_status sa_cache_reset(sa_cache* cache);

/* Append n_frames latent frames (a chunk) with times t0 .. t0+n_frames-1:
 * k, v [B, n_frames*T_f, H, D] un-rotated.  K is rotated at each frame's t and
 * stored; V is stored transposed.  Requires t0 > the newest cached t and the
 * chunk's non-sink frames to fit the ring (<= n_local), so a chunk never
 * evicts its own frames (SA_ERR_RANGE otherwise). */
sa_status sa_cache_append(sa_cache* cache, const void* k, const void* v, int32_t n_frames,
                          int64_t t0, void* stream);

/* KV recache at a prompt switch ([LongLive] section 3 "KV Recache"): for every
 * resident frame, K = RoPE(x . W_k, t_frame), V = x . W_v, written in place;
 * slots, order and times are unchanged.
 *   x    [B, n_resident*T_f, hidden]  hidden states of the resident frames in
 *                                     logical order (sinks, then local oldest -> newest)
 *   w_k, w_v [H*D, hidden]            projection weights in the nn.Linear
 *                                     [out, in] layout: row h*D+d makes channel d of head h
 * All of the cache's dtype (bf16 for an SA_FP8 cache, whose keys and values
 * are then the bf16-rounded results divided by k_scale / v_scale and rounded
 * to e4m3).  hidden must be a multiple of 32.  SA_ERR_STATE on an empty
 * cache. */
sa_status sa_cache_recache(sa_cache* cache, const void* x, const void* w_k, const void* w_v,
                           int32_t hidden, void* stream);

/* Per-frame projections of a new chunk, fused with its append ([LoL]
 * background "multi-head attention": each head's own query, key and value
 * projections; [LongLive] section 3 "KV Recache" re-runs the same key/value
 * maps over the cached frames):
 *   q = x . W_q^T (written to q_out, un-rotated: sa_window_attn rotates its
 *   queries), and the frames' k = x . W_k^T, v = x . W_v^T are appended with
 *   times t0 .. t0+n_frames-1 exactly as sa_cache_append would append them
 *   (K rotated, sinks pinned, ring eviction), without k and v ever being
 *   written to memory in between.
 *   x      [B, n_frames*T_f, hidden]  hidden states of the new frames
 *   w_q, w_k, w_v [H*D, hidden]       [out, in] layout; row h*D+d makes
 *                                     channel d of head h
 *   q_out  [B, n_frames*T_f, H, D]    may be NULL together with w_q (then
 *                                     only the cache is written)
 * All of the cache's dtype (bf16 for an SA_FP8 cache, as for the recache).
 * hidden must be a multiple of 32.  The same chunk and time rules as
 * sa_cache_append apply (SA_ERR_RANGE/SHAPE). */
sa_status sa_cache_project_append(sa_cache* cache, const void* x, const void* w_q, const void* w_k,
                                  const void* w_v, int32_t hidden, void* q_out, int32_t n_frames,
                                  int64_t t0, void* stream);

/* Plain linear map y = x . W^T, e.g. the output projection that follows the
 * attention in a multi-head attention block (the reviewed pages show none;
 * no bias):
 *   x [n_rows, in_features], w [out_features, in_features] ([out, in]
 *   layout), y [n_rows, out_features]; all of element type dtype.
 * in_features must be a multiple of 32, out_features a multiple of 16;
 * n_rows may be 0 (nothing is launched).  y must not overlap x or w. */
sa_status sa_linear(const void* x, const void* w, void* y, sa_dtype dtype, int64_t n_rows,
                    int32_t in_features, int32_t out_features, void* stream);

/* ----------------------------------------------------- 8-bit projections --
 * [LongLive] "INT8 quantized inference" table (the INT8 model: half the
 * size, 12.6 -> 16.4 FPS) and [LongLive model card] FP8 variant (24.8 FPS);
 * neither gives a scheme.  Here (W8A8) both operands of a projection are
 * 8-bit codes with one fp32 scale per row -- per token for x [n][C], per
 * output feature for W [F][C] ([out, in] layout):
 *   y[n][f] = bf16( (float(sum_c qx[n][c] qw[f][c]) * sx[n]) * sw[f] )
 * Codes are int8 (|q| <= 127; the sum is exact in int32) or OCP e4m3 (the
 * products are exact, summed in fp32).  bf16 rounding is to nearest even.
 * Every buffer is a device pointer, 16-byte aligned.
 */
typedef enum { SA_Q_INT8 = 0, SA_Q_E4M3 = 1 } sa_qtype;

/* Row-wise quantisation, every step in fp32: a = max_c |x[r][c]|,
 * scales[r] = a / Q, codes[r][c] = round(x[r][c] * (Q / a)) with Q = 127
 * (int8: nearest, ties to even) or 448 (e4m3: nearest even); a row of zeros
 * gets scale 0 and codes 0.  Serves activations (per token) and weights
 * [F][C] (per output feature) alike.
 *   x [n_rows, n_cols] bf16 (finite); codes [n_rows, n_cols] bytes (int8 or
 *   e4m3); scales [n_rows] fp32.  n_cols a multiple of 8 in [8, 65536];
 *   n_rows >= 0 (0 launches nothing).  x, codes and scales must not overlap
 *   one another (SA_ERR_RANGE). */
sa_status sa_quantize_rows(const void* x, void* codes, float* scales, sa_qtype qtype, int64_t n_rows,
                           int32_t n_cols, void* stream);

/* Plain W8A8 linear map: x codes [n_rows, in_features] with scales [n_rows],
 * w codes [out_features, in_features] with scales [out_features]; y
 * [n_rows, out_features] bf16 as above.  in_features a multiple of 64 in
 * [64, 65536], out_features a multiple of 16; y must not overlap the
 * inputs. */
sa_status sa_linear_q8(const void* x_codes, const float* x_scales, const void* w_codes,
                       const float* w_scales, void* y, sa_qtype qtype, int64_t n_rows,
                       int32_t in_features, int32_t out_features, void* stream);

/* sa_cache_recache with 8-bit operands: x codes [B*n_res*T_f, hidden]
 * (logical order, one scale per token), w_k / w_v codes [H*D, hidden] (one
 * scale per output feature).  The cache (SA_BF16 or SA_FP8) receives the
 * bf16-rounded products as in sa_cache_recache.  hidden a multiple of 64. */
sa_status sa_cache_recache_q8(sa_cache* cache, const void* x_codes, const float* x_scales,
                              const void* wk_codes, const float* wk_scales, const void* wv_codes,
                              const float* wv_scales, sa_qtype qtype, int32_t hidden, void* stream);

/* sa_cache_project_append with 8-bit operands (x codes one scale per token,
 * weights one scale per output feature); wq_codes, wq_scales and q_out
 * (bf16) are given together or all NULL.  hidden a multiple of 64. */
sa_status sa_cache_project_append_q8(sa_cache* cache, const void* x_codes, const float* x_scales,
                                     const void* wq_codes, const float* wq_scales, const void* wk_codes,
                                     const float* wk_scales, const void* wv_codes, const float* wv_scales,
                                     sa_qtype qtype, int32_t hidden, void* q_out, int32_t n_frames,
                                     int64_t t0, void* stream);

/* Workspace sa_window_attn needs for this cache state and n_q (may be 0). */
sa_status sa_window_attn_workspace(const sa_cache* cache, int32_t n_q, size_t* bytes);

/* Sink + window attention ([LongLive] section 3 "Short-Window Attention"
 * equation; [LoL] background "multi-head attention" equation):
 *   o = softmax(RoPE(q) K^T * scale) V per (stream, head), over the resident
 *   frames (all of them, or frame-causally with SA_MASK_FRAME_CAUSAL).
 *   q, o  [B, n_q*T_f, H, D]: un-rotated queries of the NEWEST n_q resident
 *         frames (append first, then attend); q is rotated at those frames' t.
 *   scale 0 => 1/sqrt(D).
 *   workspace: device scratch of at least sa_window_attn_workspace() bytes
 *         (NULL allowed when that is 0); SA_ERR_RANGE if too small.  It holds
 *         the key-split partial results of this call only and needs no
 *         initialisation.  Calls sharing a workspace must not run
 *         concurrently (stream order is enough).
 * q, o, the workspace and the cache's two stores must not overlap one
 * another (SA_ERR_RANGE, nothing launched). */
sa_status sa_window_attn(const sa_cache* cache, const void* q, void* o, int32_t n_q, float scale,
                         sa_mask mask, void* workspace, size_t workspace_bytes, void* stream);

/* sa_window_attn for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same operation, arguments, checks and results as sa_window_attn, with
 * the key-split partials kept in a 32 MiB scratch array the library holds on
 * each GPU (from the GPU's first use until the process ends); no workspace
 * argument, and no allocation of any kind.  SA_ERR_RANGE when this call's
 * partials exceed 32 MiB (sa_window_attn_workspace() gives the size; the
 * Wan-1.3B frame of 1560 queries over 12 frames needs 29.2 MB).  Every call
 * on one GPU shares that GPU's scratch, which keeps the last call's contents
 * (each call writes what it reads, so nothing needs clearing): calls that
 * overlap in time on one GPU -- on different streams, or from different host
 * threads -- race and give wrong results. */
sa_status sa_window_attn_noalloc(const sa_cache* cache, const void* q, void* o, int32_t n_q, float scale,
                                 sa_mask mask, void* stream);

/* LoL collapse diagnostic ([LoL] "core method" paragraph: at a sink collapse
 * several heads at once put abnormally high attention weight on the sink
 * frames).  Same arguments, workspace and output o as sa_window_attn, plus
 *   sink_mass [B, n_q*T_f, H] fp32: for each query row and head, the softmax
 *             probability mass the row puts on the keys of the resident sink
 *             frames (0 when no sink frame is resident); it must not
 *             overlap q, o, the workspace or the stores (SA_ERR_RANGE).
 * It runs the attention, which also records each row's log-sum-exp, then the
 * same rows over the sink keys only (about n_sink / (n_sink + n_local) of the
 * attention's work); mass = exp(LSE_sinks - LSE_all). */
sa_status sa_window_attn_sink_mass(const sa_cache* cache, const void* q, void* o, float* sink_mass,
                                   int32_t n_q, float scale, sa_mask mask, void* workspace,
                                   size_t workspace_bytes, void* stream);

/* Phase-coherence kernel per head ([LoL] "core innovation" paragraph), on the
 * host in fp64, from the same tables sa_rope_create builds:
 *   C_h(delta) = (1/K) sum_{i<K} exp(j w_{h,t,i} delta)
 * over head h's K = dim_t/2 time-axis frequencies, delta a frame offset
 * (with t_scale, a time-position offset of delta * t_scale).
 *   deltas [n] host; re, im [n_heads][n] host.  No HIP call.
 * SA_ERR_SHAPE if dim_t is 0. */
sa_status sa_rope_phase_coherence(const sa_rope_desc* desc, const double* deltas, int32_t n, double* re,
                                  double* im);

/* Resident frames in logical order (host, no sync): writes min(cap, n) entries,
 * *n_valid = n. */
sa_status sa_cache_slots(const sa_cache* cache, sa_slot* out, int32_t cap, int32_t* n_valid);

/* Copy logical frame `index` out in the boundary layout: k_out, v_out
 * [B, T_f, H, D] (either may be NULL).  K as stored (rotated). */
sa_status sa_cache_read(const sa_cache* cache, int32_t index, void* k_out, void* v_out,
                        void* stream);

/* Number of frames appended since creation / reset, and resident now. */
sa_status sa_cache_counts(const sa_cache* cache, int64_t* n_appended, int32_t* n_resident);

/* Test and tuning hook: force a launch shape for every later call in this
 * process, in place of the automatic choice (value 0 restores it).  Results
 * stay within the same tolerances whatever the shape; the parity tests use
 * this to cover every shape the automatic choice can take.  Not synchronised
 * with calls running on other host threads.
 *   SA_KNOB_ATTN_KERNEL  bf16 attention kernel: 1 = the default one, 2 = the
 *                        variant whose waves interleave their matrix
 *                        products and softmax in one instruction stream
 *                        (both: eight waves of 32 query rows per workgroup),
 *                        3 = that variant with four waves of 64 rows
 *   SA_KNOB_ATTN_SPLITS  key splits of the bf16 / e4m3 attention: 1 .. 16
 *                        (capped at one split per 8 key tiles)
 *   SA_KNOB_PROJ_TILE    projection GEMM tile (features x tokens):
 *                        1 = 256 x 128, 2 = 128 x 128, 3 = 128 x 64,
 *                        4 = 256 x 256 (eight waves, one workgroup per CU)
 * SA_ERR_RANGE for an unknown knob or a value outside its set. */
typedef enum { SA_KNOB_ATTN_KERNEL = 0, SA_KNOB_ATTN_SPLITS = 1, SA_KNOB_PROJ_TILE = 2 } sa_knob;
sa_status sa_set_launch_override(sa_knob knob, int32_t value);

const char* sa_status_str(sa_status status);
const char* sa_last_error(void); /* thread-local, "" when none */
const char* sa_version(void);

#ifdef __cplusplus
}
#endif
#endif /* SINKATTN_H */
