/*
 * vmla.h -- C ABI of the latent-KV chunk-attention library for AMD MI355X (gfx950).
 *
 * The library implements the inference hot path of VideoMLA (arXiv:2605.30351v1,
 * "VideoMLA: Low-Rank Latent KV Cache for Minute-Scale Autoregressive Video
 * Diffusion"; citations below refer to the paperlayer.ai section-by-section
 * summary of that paper as [PL]): every cached token keeps only a shared
 * content latent c (d_c scalars) and one head-shared 3D-RoPE positional key
 * k_R (d_rope scalars), and attention runs directly on those latents.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor pointers are DEVICE pointers owned by the caller (allocated and
 *    freed by the caller, e.g. through PyTorch). The library allocates nothing,
 *    keeps no global state, and is re-entrant. Every pointer must be 16-byte
 *    aligned. All tensors are dense and row-major ("C order").
 *  - Weights follow y = x @ W with W stored [in, out].
 *  - dtype: one element type per call for x, the weights, the cache and the
 *    output: VMLA_BF16 (bf16 storage; bf16 matrix-core products with fp32
 *    accumulation) or VMLA_F32 (fp32 storage; values are converted to bf16
 *    when they enter a matrix-core product, accumulation stays fp32).
 *  - stream: a hipStream_t passed as void* (NULL = the default stream). Calls
 *    are asynchronous on that stream and never synchronise the host.
 *  - Errors: every argument is validated on the host before any HIP call; a
 *    negative vmla_status is returned and nothing is launched. A failed launch
 *    returns VMLA_ERR_HIP. No exception or abort crosses the ABI.
 *  - Aliasing: a buffer that a call writes (the cache for the append; the
 *    workspace and out for the attention calls; the folded or packed weights)
 *    may share no byte with any other buffer argument of the same call, read
 *    or written. The byte range of each argument follows from the call's
 *    shapes (the whole cache, the workspace bytes the call needs). This is
 *    checked last, after every other check, and an overlap returns
 *    VMLA_ERR_OVERLAP with nothing launched.
 *  - Supported geometry in this version: d_v = 128, d_model a multiple of 64,
 *    1 <= n_heads <= 64, rope_pairs summing to d_rope / 2 (at most 48 pairs);
 *    d_nope / d_rope = 96 / 32 (the default of [PL] App. D.2-D.3) with d_c =
 *    192 (the default), or 64 / 128 / 256 / 512 for vmla_cache_append,
 *    vmla_chunk_attention and its two stages (the latent-budget sweep of [PL]
 *    §4 "Batch Scaling Under Fixed Memory" and App. F "Latent dimension");
 *    d_c = 256 and 512 take VMLA_BF16 storage and a cache with rope_at_read =
 *    0 and no sink frame.
 *    The NoPE/RoPE split variants d_nope / d_rope = 112 / 16, 64 / 64 and
 *    32 / 96 ([PL] App. F "NoPE/RoPE split") are accepted at d_c = 192 by the
 *    same three entry points and by vmla_pack_kv_weights /
 *    vmla_chunk_attention_explicit, with VMLA_BF16 storage and a cache with
 *    rope_at_read = 0 and no sink frame (VMLA_ERR_DTYPE / VMLA_ERR_SHAPE
 *    otherwise); cache and Qhat rows are then d_c + d_rope wide. The
 *    whole-layer, weight-fold and chunk-causal entry points take d_c = 192 and
 *    the default split only.
 *
 * Token and position convention: token n of a latent frame sits at grid
 * position (h, w) = (n / grid_w, n % grid_w); t is the absolute latent-frame
 * index counted from 0. T = grid_h * grid_w tokens per frame, W =
 * window_frames, S = sink_frames (0 or 1). Slot of token n of frame t:
 * t * T + n for t < S (the sink frame, kept for good), otherwise
 * (S + (t - S) mod W) * T + n (the ring of the most recent W frames).
 */
#ifndef VMLA_H
#define VMLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define VMLA_ABI_VERSION 9

typedef enum vmla_status {
  VMLA_OK = 0,
  VMLA_ERR_NULL = -1,       /* a required pointer is NULL */
  VMLA_ERR_SHAPE = -2,      /* unsupported or inconsistent dimensions */
  VMLA_ERR_DTYPE = -3,      /* unknown dtype, or cache dtype differs from the call's */
  VMLA_ERR_ALIGN = -4,      /* a pointer is not 16-byte aligned */
  VMLA_ERR_RANGE = -5,      /* t_first / n_frames / n_valid_frames / chunk or mask window out of range */
  VMLA_ERR_WORKSPACE = -6,  /* workspace NULL or smaller than vmla_attention_workspace_bytes */
  VMLA_ERR_HIP = -7,        /* a HIP launch failed (hipGetLastError after the launch) */
  VMLA_ERR_OVERLAP = -8     /* a buffer the call writes overlaps another buffer argument */
} vmla_status;

typedef enum vmla_dtype { VMLA_F32 = 0, VMLA_BF16 = 1 } vmla_dtype;

/* Layer geometry ([PL] §4, App. C.1, App. D.2-D.3). */
typedef struct vmla_dims {
  int32_t d_model;          /* hidden width of x (1536 for Wan2.1-T2V-1.3B) */
  int32_t n_heads;          /* attention heads (12) */
  int32_t d_nope;           /* per-head content width of q and k (96) */
  int32_t d_rope;           /* width of the head-shared positional key (32) */
  int32_t d_c;              /* width of the shared content latent (192) */
  int32_t d_v;              /* per-head value width (128) */
  int32_t rope_pairs[3];    /* complex pairs rotated by t, h, w: {6, 5, 5} ([PL] App. D.3) */
  int32_t rope_axis_dims[3];/* width D_a of each axis group in the frequency law
                               omega_i = theta^(-2 i / D_a), i = 0 .. pairs_a - 1: {12, 10, 10} */
  float rope_theta;         /* 10000 */
  float scale;              /* softmax scale applied to the full score, 1/sqrt(d_nope + d_rope) */
} vmla_dims;

/* Cache of latent frames ([PL] App. C.1, App. D.4-D.5): an optional sink
 * frame followed by a sliding-window ring with FIFO eviction.
 * data: [batch, (sink_frames + window_frames) * grid_h * grid_w, d_c + d_rope];
 * row of a slot = [c (d_c) | k_R (d_rope)].
 *  - rope_at_read = 0: k_R is stored rotated by 3D-RoPE at its absolute
 *    (t, h, w); queries use absolute t ([PL] App. C.1 clip-length window).
 *  - rope_at_read = 1: k_R is stored before RoPE (x W_KR) and rotated when the
 *    window is assembled: the frames of the active context (sink frames, then
 *    the window frames oldest first) are numbered 0, 1, 2, ... and that local
 *    number is the temporal coordinate of their keys and of the query chunk
 *    ([PL] App. D.5 "Long-Horizon RoPE Re-indexing"; App. E "RoPE branch").
 *    Equivalently a window frame t sits at t - shift with
 *    shift = max(0, t_first + n_frames - S - W), and the sink frame at 0.
 * sink_frames = 1 requires rope_at_read = 1 (the pages' long-horizon scheme:
 * one sink frame and a 6-frame window). */
typedef struct vmla_cache {
  void* data;
  int32_t dtype;            /* vmla_dtype */
  int32_t batch;
  int32_t window_frames;    /* W */
  int32_t grid_h;
  int32_t grid_w;
  int32_t sink_frames;      /* S: 0, or 1 (frame 0 is kept for good) */
  int32_t rope_at_read;     /* 0: k_R rotated at append (absolute t); 1: rotated at read */
} vmla_cache;

/* Fills *dims with the Wan2.1-T2V-1.3B VideoMLA defaults listed above. */
void vmla_default_dims(vmla_dims* dims);

/*
 * vmla_cache_append -- write the latent cache entries of one chunk of frames.
 *
 * Defined by: the shared content latent c_t = x_t W_down ([PL] §3 "Shared
 * low-rank KV cache"; App. D.2) and the head-shared positional key
 * k_R_t = RoPE3D(x_t W_KR, (t, h, w)) ([PL] §3 "Decoupled positional
 * encoding"; App. D.3); the pair (c_t, k_R_t) is what the cache stores
 * ([PL] App. D.2), in a fixed-size window of latent frames with FIFO eviction
 * ([PL] App. D.4).
 *
 *   x       [batch, n_frames * T, d_model]  activations of frames
 *                                           t_first .. t_first + n_frames - 1
 *   w_down  [d_model, d_c]
 *   w_kr    [d_model, d_rope]
 *   cache   written in place: exactly the slots of the chunk's frames (see
 *           the slot convention above) are (over)written; no other slot is
 *           touched. Appending a frame again (a later denoising step)
 *           overwrites it. With rope_at_read = 1 the k_R columns receive
 *           x W_KR unrotated ([PL] App. D.5).
 *
 * Errors: VMLA_ERR_NULL (any pointer NULL), VMLA_ERR_ALIGN, VMLA_ERR_DTYPE
 * (dtype invalid or != cache->dtype), VMLA_ERR_SHAPE (unsupported dims,
 * non-positive grid/batch/window, sink_frames not 0 or 1, rope_at_read not
 * 0 or 1, sink_frames = 1 with rope_at_read = 0,
 * (sink_frames + window_frames) * T >= 2^24 slots,
 * n_frames * T * d_model > 2^31 - 1 elements per batch element),
 * VMLA_ERR_RANGE (t_first < 0, n_frames < 1, n_frames > window_frames,
 * t_first + n_frames > 2^20), VMLA_ERR_HIP.
 */
int32_t vmla_cache_append(const vmla_dims* dims, const vmla_cache* cache, int32_t dtype,
                          const void* x, const void* w_down, const void* w_kr,
                          int32_t t_first, int32_t n_frames, void* stream);

/* Bytes of device workspace vmla_chunk_attention needs for batch and n_q query
 * tokens (the absorbed, pre-scaled bf16 queries [batch, n_heads, n_q, d_c + d_rope]).
 * Returns 0 for invalid arguments. */
size_t vmla_attention_workspace_bytes(const vmla_dims* dims, int32_t batch, int32_t n_q);

/*
 * vmla_chunk_attention -- attention of one query chunk over the latent window.
 *
 * Defined by: latent-form inference ([PL] App. E): queries q = x W_Q split per
 * head into q_nope (d_nope) and q_rope (d_rope, rotated by 3D-RoPE at the
 * token's absolute (t, h, w)); the content score uses the absorbed query
 * q_nope W_K_up[h]^T against c ("Content-path absorption"), the positional
 * score q_rope . k_R stays separate ("RoPE branch"); softmax over every valid
 * key of the window, the query chunk included (no mask: chunk-causal attention,
 * [PL] App. D.4); the softmax-weighted latents are accumulated and projected by
 * W_V_up[h] ("Value-path absorption"). The result equals explicit per-head
 * reconstruction k_nope = c W_K_up[h], v = c W_V_up[h] ([PL] §3) up to rounding.
 *
 *   x        [batch, n_q, d_model], n_q = n_frames * T: activations of the
 *            query chunk (frames t_first .. t_first + n_frames - 1)
 *   w_q      [d_model, n_heads * (d_nope + d_rope)]: head-major columns,
 *            each head [nope (d_nope) | rope (d_rope)]
 *   w_k_up   [n_heads, d_c, d_nope]
 *   w_v_up   [n_heads, d_c, d_v]
 *   n_valid_frames  must equal min(t_first + n_frames, sink_frames +
 *            window_frames): keys are the slots [0, n_valid_frames * T) of
 *            each batch element (the sink frame, then the ring)
 *   out      [batch, n_q, n_heads, d_v] (dtype of the call)
 *   workspace >= vmla_attention_workspace_bytes(dims, batch, n_q) bytes; its
 *            contents are scratch owned by the call until it completes on stream.
 *
 * With rope_at_read = 1 the queries and the cached k_R are rotated with the
 * local temporal coordinates of the active context (see vmla_cache).
 *
 * Errors: as vmla_cache_append, plus VMLA_ERR_RANGE when n_valid_frames is not
 * min(t_first + n_frames, sink_frames + window_frames), VMLA_ERR_WORKSPACE.
 */
int32_t vmla_chunk_attention(const vmla_dims* dims, const vmla_cache* cache, int32_t dtype,
                             const void* x, const void* w_q, const void* w_k_up,
                             const void* w_v_up, int32_t t_first, int32_t n_frames,
                             int32_t n_valid_frames, void* out, void* workspace,
                             size_t workspace_bytes, void* stream);

/* Size of the library-owned scratch array of vmla_chunk_attention_noalloc:
 * 32 MiB on each GPU the library runs on, held until the process ends. */
#define VMLA_NOALLOC_SCRATCH_BYTES (32u << 20)

/*
 * vmla_chunk_attention_noalloc -- vmla_chunk_attention without a workspace
 * argument, for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation. It
 * calls no hipMalloc, hipFree or allocating routine. The query rows go to a
 * library-owned array of VMLA_NOALLOC_SCRATCH_BYTES on the current device
 * (its address is looked up on the first call on that device).
 *
 * Arguments, results and errors as vmla_chunk_attention; the call needs
 * vmla_attention_workspace_bytes(dims, batch, n_q) <= VMLA_NOALLOC_SCRATCH_BYTES
 * (e.g. 4680 query tokens at batch 1 with the default widths: 25.2 MB) and
 * returns VMLA_ERR_WORKSPACE otherwise, before any HIP call.
 *
 * Every call on a GPU uses that GPU's one array: calls that overlap in time
 * on one GPU (concurrent streams, other host threads) race and corrupt each
 * other's results; serialize them. The array keeps the last call's contents;
 * nothing in it needs to start at zero.
 */
int32_t vmla_chunk_attention_noalloc(const vmla_dims* dims, const vmla_cache* cache, int32_t dtype,
                                     const void* x, const void* w_q, const void* w_k_up,
                                     const void* w_v_up, int32_t t_first, int32_t n_frames,
                                     int32_t n_valid_frames, void* out, void* stream);

/*
 * The two stages of vmla_chunk_attention, callable separately (same arguments,
 * same validation and errors; vmla_chunk_attention == the two in sequence).
 *
 * vmla_query_prologue -- queries in absorbed latent form ([PL] App. E
 * "Content-path absorption", "RoPE branch"; [PL] App. D.3): writes the
 * pre-scaled bf16 rows [q_nope W_K_up[h]^T | RoPE3D(q_rope)] * scale * log2(e)
 * of every (batch, head, token) into workspace, layout
 * [batch, n_heads, n_q, d_c + d_rope].
 *
 * vmla_latent_attention -- scores of those rows against the cached rows
 * [c | k_R] of slots [0, n_valid_frames * T) (k_R rotated as it is read when
 * rope_at_read = 1), online softmax, weighted sum
 * of the latents c, projection by W_V_up[h] ([PL] App. E "Value-path
 * absorption"). Reads the query rows from workspace; writes out.
 */
int32_t vmla_query_prologue(const vmla_dims* dims, const vmla_cache* cache, int32_t dtype,
                            const void* x, const void* w_q, const void* w_k_up,
                            int32_t t_first, int32_t n_frames, int32_t n_valid_frames,
                            void* workspace, size_t workspace_bytes, void* stream);

int32_t vmla_latent_attention(const vmla_dims* dims, const vmla_cache* cache, int32_t dtype,
                              const void* w_v_up, int32_t t_first, int32_t n_frames,
                              int32_t n_valid_frames, void* out, const void* workspace,
                              size_t workspace_bytes, void* stream);

/*
 * The whole attention layer: query latent and output mixer.
 * ---------------------------------------------------------
 * Defined by: queries from a d_q-wide query latent, c_q = x W_DQ, q = c_q W_UQ
 * ([PL] §4 "Implementation Details": d_q = 768 by default); the content score
 * applies a fixed per-head matrix A_h = W_UQ^nope[h] W_K_up[h]^T to the query
 * latent ([PL] App. E "Content-path absorption"); the softmax-weighted latents
 * are projected with B_h = W_V_up[h] folded into the output mixer W_O
 * ([PL] App. E "Value-path absorption"); the positional branch is not folded
 * ("RoPE branch"). The layer output is
 *   y = sum_h softmax_h(...) c W_V_up[h] W_O[h],
 * W_O[h] the d_v rows of W_O that mix head h, i.e. the concatenated head
 * outputs of vmla_chunk_attention (queries from c_q W_UQ) times W_O.
 *
 * Weight layouts (dtype of the call unless stated):
 *   w_dq  [d_model, d_q]
 *   w_uq  [d_q, n_heads * (d_nope + d_rope)]  head-major, each head [nope | rope]
 *   w_o   [n_heads * d_v, d_model]
 *   w_qa  [d_q, n_heads * (d_c + d_rope)]     bf16 always: per head [A_h | W_UQ^rope[h]]
 *   w_vo  [n_heads * d_c, d_model]            bf16 always: per head B_h W_O[h]
 * d_q: a multiple of 64 in [64, 8192].
 */

/* w_qa from w_uq and w_k_up (formed once per set of weights; fp32 accumulation,
 * bf16 result). Errors: VMLA_ERR_NULL, VMLA_ERR_DTYPE, VMLA_ERR_SHAPE (dims,
 * d_q), VMLA_ERR_ALIGN, VMLA_ERR_HIP. */
int32_t vmla_fold_query_weights(const vmla_dims* dims, int32_t dtype, int32_t d_q,
                                const void* w_uq, const void* w_k_up, void* w_qa, void* stream);

/* w_vo from w_v_up and w_o (formed once per set of weights; fp32 accumulation,
 * bf16 result). Errors as vmla_fold_query_weights. */
int32_t vmla_fold_output_weights(const vmla_dims* dims, int32_t dtype, const void* w_v_up,
                                 const void* w_o, void* w_vo, void* stream);

/* Bytes of device workspace the layer entry points need: the Qhat rows of
 * vmla_attention_workspace_bytes, then one bf16 region of
 * batch * n_q * max(d_q, n_heads * d_c) elements (its size rounded up to 256
 * bytes) that holds the query latent during the prologue and the normalized
 * latent outputs O_lat / l during the attention. Returns 0 for invalid
 * arguments. */
size_t vmla_layer_workspace_bytes(const vmla_dims* dims, int32_t d_q, int32_t batch, int32_t n_q);

/*
 * vmla_chunk_attention_layer -- one chunk step of the whole layer:
 *   vmla_layer_query_prologue: c_q = x W_DQ (bf16, workspace), then
 *     Qhat = [c_q A_h | RoPE3D(c_q W_UQ^rope[h])] * scale * log2(e) for every
 *     head (same Qhat rows and coordinates as vmla_query_prologue);
 *   vmla_layer_attention: scores, online softmax and weighted latents exactly as
 *     vmla_latent_attention, then O_lat / l of every head (bf16, workspace) and
 *     y = [O_lat,0 / l | ... | O_lat,H-1 / l] w_vo.
 *   x    [batch, n_q, d_model], n_q = n_frames * T
 *   out  [batch, n_q, d_model] (dtype of the call)
 * Cache, t_first, n_frames, n_valid_frames: as vmla_chunk_attention.
 * Errors: as vmla_chunk_attention (workspace checked against
 * vmla_layer_workspace_bytes), plus VMLA_ERR_SHAPE for d_q or more than 2^28
 * query rows. The two stages are callable separately with the same arguments;
 * vmla_layer_attention reads the Qhat rows the prologue left in workspace.
 */
int32_t vmla_chunk_attention_layer(const vmla_dims* dims, const vmla_cache* cache, int32_t dtype,
                                   const void* x, const void* w_dq, int32_t d_q, const void* w_qa,
                                   const void* w_vo, int32_t t_first, int32_t n_frames,
                                   int32_t n_valid_frames, void* out, void* workspace,
                                   size_t workspace_bytes, void* stream);

int32_t vmla_layer_query_prologue(const vmla_dims* dims, const vmla_cache* cache, int32_t dtype,
                                  const void* x, const void* w_dq, int32_t d_q, const void* w_qa,
                                  int32_t t_first, int32_t n_frames, int32_t n_valid_frames,
                                  void* workspace, size_t workspace_bytes, void* stream);

int32_t vmla_layer_attention(const vmla_dims* dims, const vmla_cache* cache, int32_t dtype,
                             int32_t d_q, const void* w_vo, int32_t t_first, int32_t n_frames,
                             int32_t n_valid_frames, void* out, void* workspace,
                             size_t workspace_bytes, void* stream);

/* out [m, d_model] = in [m, n_heads * d_v] w_o [n_heads * d_v, d_model]: the
 * output mixer applied to vmla_chunk_attention's head outputs (viewed as
 * [batch * n_q, n_heads * d_v]) without folding; the same product as the folded
 * path up to rounding. Errors: VMLA_ERR_NULL, VMLA_ERR_DTYPE, VMLA_ERR_SHAPE
 * (dims, m < 1 or m > 2^24), VMLA_ERR_ALIGN, VMLA_ERR_HIP. */
int32_t vmla_output_projection(const vmla_dims* dims, int32_t dtype, int64_t m, const void* in,
                               const void* w_o, void* out, void* stream);

/*
 * Explicit reconstruction: the comparison point of the latent form.
 * -----------------------------------------------------------------
 * Defined by: on-demand reconstruction of per-head keys k_h = [c W_K_up[h] |
 * k_R] and values v_h = c W_V_up[h] from the cached pair ([PL] §3 "On-demand
 * reconstruction"), then ordinary 128-dimensional multi-head attention over
 * them; App. E's latent form computes the same result without the rebuilt
 * rows. The output equals vmla_chunk_attention's up to rounding.
 *
 * w_kv [d_c, n_heads * (d_nope + d_v)] (dtype of the call): per head
 * [W_K_up[h] | W_V_up[h]], packed once by vmla_pack_kv_weights.
 * Workspace: the pre-scaled bf16 queries [batch, n_heads, n_q, d_nope + d_rope]
 * then the rebuilt bf16 rows [batch, n_heads, n_k, 2 (d_nope + d_rope)] with
 * row = [k_nope | k_R | v], n_k = n_valid_frames * T.
 * Only caches with rope_at_read = 0 (k_R rotated at append).
 * Errors: as vmla_chunk_attention (workspace against
 * vmla_explicit_workspace_bytes), plus VMLA_ERR_SHAPE for rope_at_read = 1 or
 * more than 2^31 rebuilt elements per batch element.
 */
int32_t vmla_pack_kv_weights(const vmla_dims* dims, int32_t dtype, const void* w_k_up,
                             const void* w_v_up, void* w_kv, void* stream);

size_t vmla_explicit_workspace_bytes(const vmla_dims* dims, int32_t batch, int32_t n_q, int32_t n_k);

int32_t vmla_chunk_attention_explicit(const vmla_dims* dims, const vmla_cache* cache, int32_t dtype,
                                      const void* x, const void* w_q, const void* w_kv,
                                      int32_t t_first, int32_t n_frames, int32_t n_valid_frames,
                                      void* out, void* workspace, size_t workspace_bytes,
                                      void* stream);

/*
 * A whole clip under the chunk-causal block mask.
 * -----------------------------------------------
 * Defined by: chunk-causal attention ([PL] App. D.4 "Chunk-Causal
 * Sliding-Window Attention": attention inside a chunk is allowed, an earlier
 * chunk never attends to a later one), the form in which causal block masks
 * run over the reconstructed heads ([PL] §3 "Integration with causal
 * attention"). Every token of the clip's frames 0 .. n_frames - 1 is a query
 * at its absolute (t, h, w); frames are cut into chunks of chunk_frames (the
 * last chunk may be shorter), and a query of chunk c attends to the key frames
 * [max(0, e - mask_window_frames), e), e = min((c + 1) * chunk_frames,
 * n_frames): its own chunk and the earlier frames of a window of
 * mask_window_frames frames, which are the keys a rolling cache of that many
 * frames holds right after chunk c is appended. mask_window_frames >= n_frames
 * is the plain block-causal mask. Row c of the result equals
 * vmla_chunk_attention for t_first = c * chunk_frames over such a cache.
 *
 *   cache  the clip's latent rows, written by vmla_cache_append for frames
 *          0 .. n_frames - 1 (slot t * T + n): window_frames >= n_frames,
 *          sink_frames = 0, rope_at_read = 0
 *   x      [batch, n_frames * T, d_model]: activations of every frame
 *   out    [batch, n_frames * T, n_heads, d_v] (dtype of the call)
 *   workspace  vmla_chunk_causal_attention, vmla_chunk_causal_latent_attention:
 *          >= vmla_attention_workspace_bytes(dims, batch, n_frames * T) (the
 *          Qhat rows of vmla_query_prologue with t_first = 0 and n_frames);
 *          vmla_chunk_causal_attention_explicit: >=
 *          vmla_explicit_workspace_bytes(dims, batch, n_frames * T, n_frames * T).
 * vmla_chunk_causal_latent_attention is the second stage alone: it reads the
 * Qhat rows that vmla_query_prologue (t_first = 0, n_frames, n_valid_frames =
 * n_frames) left in workspace. The explicit form takes d_c = 192 and w_kv of
 * vmla_pack_kv_weights.
 *
 * Errors: as vmla_chunk_attention, plus VMLA_ERR_SHAPE for sink_frames = 1,
 * rope_at_read = 1 or more than 65535 (chunk, batch element) pairs, and
 * VMLA_ERR_RANGE for n_frames < 1, n_frames > window_frames, chunk_frames
 * outside [1, n_frames] or mask_window_frames < chunk_frames.
 */
int32_t vmla_chunk_causal_attention(const vmla_dims* dims, const vmla_cache* cache, int32_t dtype,
                                    const void* x, const void* w_q, const void* w_k_up,
                                    const void* w_v_up, int32_t n_frames, int32_t chunk_frames,
                                    int32_t mask_window_frames, void* out, void* workspace,
                                    size_t workspace_bytes, void* stream);

int32_t vmla_chunk_causal_latent_attention(const vmla_dims* dims, const vmla_cache* cache,
                                           int32_t dtype, const void* w_v_up, int32_t n_frames,
                                           int32_t chunk_frames, int32_t mask_window_frames,
                                           void* out, const void* workspace,
                                           size_t workspace_bytes, void* stream);

int32_t vmla_chunk_causal_attention_explicit(const vmla_dims* dims, const vmla_cache* cache,
                                             int32_t dtype, const void* x, const void* w_q,
                                             const void* w_kv, int32_t n_frames,
                                             int32_t chunk_frames, int32_t mask_window_frames,
                                             void* out, void* workspace, size_t workspace_bytes,
                                             void* stream);

/* Static text for a status code (never NULL). */
const char* vmla_status_string(int32_t status);

/* VMLA_ABI_VERSION of the built library. */
int32_t vmla_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* VMLA_H */
