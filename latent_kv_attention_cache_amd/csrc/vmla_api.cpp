// Host side of the C ABI declared in include/vmla.h: argument validation (no
// HIP call before it passes), RoPE frequency table, kernel dispatch.
#include "vmla.h"

#include <cmath>
#include <climits>
#include <cstdint>
#include <initializer_list>

#include "kernels.h"

namespace {

using namespace vmla;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Largest t_first + n_frames accepted: keeps every token index below 2^24 for
// the exact float-reciprocal division (RoPE angles are exact fixed-point
// fractions of a revolution at any position).
constexpr int64_t kMaxFrameIndex = 1 << 20;

// NoPE/RoPE split of the 128-wide head: the default 96 / 32, or one of the
// split variants 64 / 64, 32 / 96, 112 / 16 (with d_c = 192).
bool split_ok(const vmla_dims* d) {
  if (d->d_nope + d->d_rope != kDHead) return false;
  return d->d_rope == kDRope || d->d_rope == 16 || d->d_rope == 64 || d->d_rope == 96;
}

int32_t check_dims(const vmla_dims* d) {
  if (!d) return VMLA_ERR_NULL;
  if (!split_ok(d) || d->d_v != kDV) return VMLA_ERR_SHAPE;
  // content width: the default 192, or 64 / 128 / 256 / 512 (latent-budget
  // sweep) for the append and the attention core; the split variants run at 192
  if (d->d_c != kDC && d->d_c != 64 && d->d_c != 128 && d->d_c != 256 && d->d_c != 512)
    return VMLA_ERR_SHAPE;
  if (d->d_rope != kDRope && d->d_c != kDC) return VMLA_ERR_SHAPE;
  if (d->d_model < 64 || d->d_model % 64 != 0 || d->d_model > (1 << 16)) return VMLA_ERR_SHAPE;
  if (d->n_heads < 1 || d->n_heads > 64) return VMLA_ERR_SHAPE;
  int pairs = 0;
  for (int i = 0; i < 3; ++i) {
    if (d->rope_pairs[i] < 0 || d->rope_axis_dims[i] < 1) return VMLA_ERR_SHAPE;
    pairs += d->rope_pairs[i];
  }
  if (2 * pairs != d->d_rope) return VMLA_ERR_SHAPE;
  if (!(d->rope_theta > 0.f) || !std::isfinite(d->rope_theta)) return VMLA_ERR_SHAPE;
  if (!(d->scale > 0.f) || !std::isfinite(d->scale)) return VMLA_ERR_SHAPE;
  return VMLA_OK;
}

// The explicit route runs at d_c = 192 (any split); the whole-layer and
// weight-fold entry points at d_c = 192 and the default split only.
int32_t check_dims_192(const vmla_dims* d) {
  const int32_t st = check_dims(d);
  if (st) return st;
  return d->d_c == kDC ? VMLA_OK : VMLA_ERR_SHAPE;
}

int32_t check_dims_default(const vmla_dims* d) {
  const int32_t st = check_dims_192(d);
  if (st) return st;
  return d->d_rope == kDRope ? VMLA_OK : VMLA_ERR_SHAPE;
}

// The split variants and the wide latents (d_c 256, 512) store bf16 and use
// neither read-time RoPE nor a sink.
int32_t check_split_cache(const vmla_dims* d, const vmla_cache* c, int32_t dtype) {
  if (d->d_rope == kDRope && d->d_c <= kDC) return VMLA_OK;
  if (dtype != VMLA_BF16) return VMLA_ERR_DTYPE;
  return c->rope_at_read || c->sink_frames ? VMLA_ERR_SHAPE : VMLA_OK;
}

int32_t check_cache(const vmla_cache* c, int32_t dtype, int row) {
  if (!c) return VMLA_ERR_NULL;
  if (!c->data) return VMLA_ERR_NULL;
  if (!aligned16(c->data)) return VMLA_ERR_ALIGN;
  if (dtype != VMLA_F32 && dtype != VMLA_BF16) return VMLA_ERR_DTYPE;
  if (c->dtype != dtype) return VMLA_ERR_DTYPE;
  if (c->batch < 1 || c->window_frames < 1 || c->grid_h < 1 || c->grid_w < 1) return VMLA_ERR_SHAPE;
  if ((c->sink_frames != 0 && c->sink_frames != 1) || (c->rope_at_read != 0 && c->rope_at_read != 1))
    return VMLA_ERR_SHAPE;
  if (c->sink_frames && !c->rope_at_read) return VMLA_ERR_SHAPE;
  const int64_t t = (int64_t)c->grid_h * c->grid_w;
  const int64_t rows = t * ((int64_t)c->sink_frames + c->window_frames);
  // every element offset handled by the kernels must fit in int32 per batch element
  if (rows * row > INT32_MAX || rows >= (1 << 24)) return VMLA_ERR_SHAPE;
  return VMLA_OK;
}

// omega_i = theta^(-2 i / D_a) for the pairs of each axis group, computed in
// double and passed as revolutions per position step (omega_i / 2 pi).
RopeTable rope_table(const vmla_dims* d) {
  RopeTable r{};
  const double two_pi = 6.283185307179586476925286766559;
  int j = 0;
  for (int ax = 0; ax < 3; ++ax) {
    for (int i = 0; i < d->rope_pairs[ax]; ++i, ++j) {
      if (j >= kMaxPairs) return r;           // excluded by check_dims
      const double omega = std::pow((double)d->rope_theta, -2.0 * i / (double)d->rope_axis_dims[ax]);
      // revolutions per step as a 64-bit binary fraction (only the fractional
      // revolution matters for the angle)
      const double rev = omega / two_pi;
      const uint64_t fx = (uint64_t)std::ldexp(rev - std::floor(rev), 64);
      r.rev_lo[j] = (uint32_t)fx;
      r.rev_hi[j] = (uint32_t)(fx >> 32);
      r.axis[j] = ax;
    }
  }
  return r;
}

int32_t hip_status(hipError_t e) { return e == hipSuccess ? VMLA_OK : VMLA_ERR_HIP; }

// ---- aliasing: the byte range of every tensor argument of a call

struct Span {
  uintptr_t lo, hi;   // [lo, hi)
};

Span bytes_at(const void* p, size_t n) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return {a, n > UINTPTR_MAX - a ? UINTPTR_MAX : a + n};
}

size_t esize(int32_t dtype) { return dtype == VMLA_F32 ? sizeof(float) : sizeof(uint16_t); }

Span cache_span(const vmla_dims* d, const vmla_cache* c) {
  const size_t rows = (size_t)c->grid_h * c->grid_w * ((size_t)c->sink_frames + c->window_frames);
  return bytes_at(c->data, (size_t)c->batch * rows * (d->d_c + d->d_rope) * esize(c->dtype));
}

// A buffer that a call writes may share no byte with any other buffer of the
// call, read or written: the kernels of one call read and write them
// concurrently, so an alias would corrupt results (or the cache) silently.
int32_t check_disjoint(std::initializer_list<Span> written, std::initializer_list<Span> read) {
  for (auto w = written.begin(); w != written.end(); ++w) {
    for (auto o = w + 1; o != written.end(); ++o)
      if (w->lo < o->hi && o->lo < w->hi) return VMLA_ERR_OVERLAP;
    for (const Span& r : read)
      if (w->lo < r.hi && r.lo < w->hi) return VMLA_ERR_OVERLAP;
  }
  return VMLA_OK;
}

// Spans of the attention-core arguments: activations x [B, n_q, d_model],
// W_Q [d_model, H (d_nope + d_rope)], W_K_up [H, d_c, d_nope], W_V_up
// [H, d_c, d_v], head outputs [B, n_q, H, d_v], and the Qhat workspace.
struct AttnSpans {
  Span x, w_q, w_k_up, w_v_up, out, ws, cache;
};

AttnSpans attn_spans(const vmla_dims* d, const vmla_cache* c, int32_t dtype, int64_t n_q, const void* x,
                     const void* w_q, const void* w_k_up, const void* w_v_up, const void* out,
                     const void* ws) {
  const size_t e = esize(dtype), m = (size_t)c->batch * n_q, h = d->n_heads;
  AttnSpans s;
  s.x = bytes_at(x, m * d->d_model * e);
  s.w_q = bytes_at(w_q, (size_t)d->d_model * h * (d->d_nope + d->d_rope) * e);
  s.w_k_up = bytes_at(w_k_up, h * d->d_c * d->d_nope * e);
  s.w_v_up = bytes_at(w_v_up, h * d->d_c * d->d_v * e);
  s.out = bytes_at(out, m * h * d->d_v * e);
  s.ws = bytes_at(ws, vmla_attention_workspace_bytes(d, c->batch, (int32_t)n_q));
  s.cache = cache_span(d, c);
  return s;
}

}  // namespace

extern "C" {

void vmla_default_dims(vmla_dims* d) {
  if (!d) return;
  d->d_model = 1536;
  d->n_heads = 12;
  d->d_nope = kDNope;
  d->d_rope = kDRope;
  d->d_c = kDC;
  d->d_v = kDV;
  d->rope_pairs[0] = 6; d->rope_pairs[1] = 5; d->rope_pairs[2] = 5;
  d->rope_axis_dims[0] = 12; d->rope_axis_dims[1] = 10; d->rope_axis_dims[2] = 10;
  d->rope_theta = 10000.f;
  d->scale = (float)(1.0 / std::sqrt((double)(kDNope + kDRope)));
}

int32_t vmla_abi_version(void) { return VMLA_ABI_VERSION; }

const char* vmla_status_string(int32_t s) {
  switch (s) {
    case VMLA_OK: return "ok";
    case VMLA_ERR_NULL: return "null pointer argument";
    case VMLA_ERR_SHAPE: return "unsupported or inconsistent dimensions";
    case VMLA_ERR_DTYPE: return "invalid dtype or dtype mismatch with the cache";
    case VMLA_ERR_ALIGN: return "pointer not 16-byte aligned";
    case VMLA_ERR_RANGE: return "t_first / n_frames / n_valid_frames / chunk or mask window out of range";
    case VMLA_ERR_WORKSPACE: return "workspace missing or too small";
    case VMLA_ERR_HIP: return "HIP launch failed";
    case VMLA_ERR_OVERLAP: return "a buffer the call writes overlaps another buffer of the call";
    default: return "unknown status";
  }
}

int32_t vmla_cache_append(const vmla_dims* dims, const vmla_cache* cache, int32_t dtype,
                          const void* x, const void* w_down, const void* w_kr,
                          int32_t t_first, int32_t n_frames, void* stream) {
  int32_t st = check_dims(dims);
  if (st) return st;
  if (!x || !w_down || !w_kr) return VMLA_ERR_NULL;
  st = check_cache(cache, dtype, dims->d_c + dims->d_rope);
  if (st) return st;
  st = check_split_cache(dims, cache, dtype);
  if (st) return st;
  if (!aligned16(x) || !aligned16(w_down) || !aligned16(w_kr)) return VMLA_ERR_ALIGN;
  if (t_first < 0 || n_frames < 1 || n_frames > cache->window_frames) return VMLA_ERR_RANGE;
  if ((int64_t)t_first + n_frames > kMaxFrameIndex) return VMLA_ERR_RANGE;
  const int64_t T = (int64_t)cache->grid_h * cache->grid_w;
  const int64_t n_tok = T * n_frames;
  if (n_tok * dims->d_model > INT32_MAX) return VMLA_ERR_SHAPE;
  const size_t e = esize(dtype);
  st = check_disjoint({cache_span(dims, cache)},
                      {bytes_at(x, (size_t)cache->batch * n_tok * dims->d_model * e),
                       bytes_at(w_down, (size_t)dims->d_model * dims->d_c * e),
                       bytes_at(w_kr, (size_t)dims->d_model * dims->d_rope * e)});
  if (st) return st;

  AppendArgs a{};
  a.x = x; a.w_down = w_down; a.w_kr = w_kr; a.cache = cache->data;
  a.batch = cache->batch; a.n_tok = (int)n_tok; a.d_model = dims->d_model;
  a.grid_w = cache->grid_w; a.tokens_per_frame = (int)T;
  a.window_frames = cache->window_frames; a.t_first = t_first;
  a.inv_grid_w = 1.f / (float)cache->grid_w;
  a.inv_tokens_per_frame = 1.f / (float)T;
  a.inv_window_frames = 1.f / (float)cache->window_frames;
  a.sink_frames = cache->sink_frames;
  a.rope_at_read = cache->rope_at_read;
  a.d_c = dims->d_c;
  a.d_rope = dims->d_rope;
  a.rope = rope_table(dims);
  return hip_status(launch_append(a, dtype == VMLA_F32, static_cast<hipStream_t>(stream)));
}

size_t vmla_attention_workspace_bytes(const vmla_dims* dims, int32_t batch, int32_t n_q) {
  if (check_dims(dims) != VMLA_OK || batch < 1 || n_q < 1) return 0;
  return (size_t)batch * dims->n_heads * (size_t)n_q * (dims->d_c + dims->d_rope) * sizeof(uint16_t);
}

namespace {

void fill_attention(const vmla_dims* dims, const vmla_cache* cache, const void* workspace,
                    int64_t n_q, int64_t t_q, int64_t n_k, int64_t shift, QArgs* q, AttnArgs* a);

// Shared validation of the attention stages; fills the launch arguments.
int32_t check_attention(const vmla_dims* dims, const vmla_cache* cache, int32_t dtype,
                        int32_t t_first, int32_t n_frames, int32_t n_valid_frames,
                        const void* workspace, size_t workspace_bytes, QArgs* q, AttnArgs* a) {
  int32_t st = check_dims(dims);
  if (st) return st;
  st = check_cache(cache, dtype, dims->d_c + dims->d_rope);
  if (st) return st;
  st = check_split_cache(dims, cache, dtype);
  if (st) return st;
  if (t_first < 0 || n_frames < 1 || n_frames > cache->window_frames) return VMLA_ERR_RANGE;
  if ((int64_t)t_first + n_frames > kMaxFrameIndex) return VMLA_ERR_RANGE;
  const int64_t t_end = (int64_t)t_first + n_frames;
  const int64_t span = (int64_t)cache->sink_frames + cache->window_frames;   // frames the cache holds
  const int64_t expect_valid = t_end < span ? t_end : span;
  if (n_valid_frames != expect_valid) return VMLA_ERR_RANGE;
  // Read-time RoPE: frames of the active context are renumbered from 0; a window
  // frame t sits at t - shift, the sink frame at 0.
  const int64_t shift = cache->rope_at_read && t_end > span ? t_end - span : 0;
  const int64_t T = (int64_t)cache->grid_h * cache->grid_w;
  const int64_t n_q = T * n_frames;
  if (n_q * dims->d_model > INT32_MAX || n_q * dims->n_heads * kDV > INT32_MAX) return VMLA_ERR_SHAPE;
  const size_t need = vmla_attention_workspace_bytes(dims, cache->batch, (int32_t)n_q);
  if (!workspace || workspace_bytes < need) return VMLA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return VMLA_ERR_ALIGN;
  fill_attention(dims, cache, workspace, n_q, t_first - shift, T * n_valid_frames, shift, q, a);
  return VMLA_OK;
}

// Launch arguments of the query prologue and the attention: n_q queries from
// absolute frame t_q, keys = slots [0, n_k), one query chunk over all of them.
void fill_attention(const vmla_dims* dims, const vmla_cache* cache, const void* workspace,
                    int64_t n_q, int64_t t_q, int64_t n_k, int64_t shift, QArgs* q, AttnArgs* a) {
  const int64_t T = (int64_t)cache->grid_h * cache->grid_w;
  const int64_t span = (int64_t)cache->sink_frames + cache->window_frames;
  *q = QArgs{};
  q->qhat = static_cast<uint16_t*>(const_cast<void*>(workspace));
  q->batch = cache->batch; q->n_q = (int)n_q; q->d_model = dims->d_model; q->n_heads = dims->n_heads;
  q->grid_w = cache->grid_w; q->tokens_per_frame = (int)T; q->t_first = (int)t_q;
  q->inv_grid_w = 1.f / (float)cache->grid_w;
  q->inv_tokens_per_frame = 1.f / (float)T;
  q->qscale = (float)((double)dims->scale * 1.4426950408889634);   // scale * log2(e)
  q->d_c = dims->d_c;
  q->d_rope = dims->d_rope;
  q->rope = rope_table(dims);

  *a = AttnArgs{};
  a->qhat = q->qhat; a->cache = cache->data;
  a->batch = cache->batch; a->n_q = (int)n_q; a->n_heads = dims->n_heads;
  a->n_k = (int)n_k; a->cache_rows = (int)(T * span);
  a->cm = ChunkMask{1, (int)n_q, (int)n_k, (int)n_k};
  a->rope_at_read = cache->rope_at_read;
  a->d_c = dims->d_c;
  a->d_rope = dims->d_rope;
  a->sink_frames = cache->sink_frames;
  a->window_frames = cache->window_frames;
  a->shift_mod_w = (int)(shift % cache->window_frames);
  a->tokens_per_frame = (int)T;
  a->grid_w = cache->grid_w;
  a->inv_tokens_per_frame = 1.f / (float)T;
  a->inv_grid_w = 1.f / (float)cache->grid_w;
  a->rope = q->rope;
}

}  // namespace

int32_t vmla_query_prologue(const vmla_dims* dims, const vmla_cache* cache, int32_t dtype,
                            const void* x, const void* w_q, const void* w_k_up,
                            int32_t t_first, int32_t n_frames, int32_t n_valid_frames,
                            void* workspace, size_t workspace_bytes, void* stream) {
  if (!x || !w_q || !w_k_up) return VMLA_ERR_NULL;
  QArgs q;
  AttnArgs a;
  int32_t st = check_attention(dims, cache, dtype, t_first, n_frames, n_valid_frames, workspace,
                               workspace_bytes, &q, &a);
  if (st) return st;
  if (!aligned16(x) || !aligned16(w_q) || !aligned16(w_k_up)) return VMLA_ERR_ALIGN;
  const AttnSpans sp = attn_spans(dims, cache, dtype, q.n_q, x, w_q, w_k_up, nullptr, nullptr, workspace);
  st = check_disjoint({sp.ws}, {sp.x, sp.w_q, sp.w_k_up, sp.cache});
  if (st) return st;
  q.x = x; q.w_q = w_q; q.w_k_up = w_k_up;
  return hip_status(launch_qprologue(q, dtype == VMLA_F32, static_cast<hipStream_t>(stream)));
}

int32_t vmla_latent_attention(const vmla_dims* dims, const vmla_cache* cache, int32_t dtype,
                              const void* w_v_up, int32_t t_first, int32_t n_frames,
                              int32_t n_valid_frames, void* out, const void* workspace,
                              size_t workspace_bytes, void* stream) {
  if (!w_v_up || !out) return VMLA_ERR_NULL;
  QArgs q;
  AttnArgs a;
  int32_t st = check_attention(dims, cache, dtype, t_first, n_frames, n_valid_frames, workspace,
                               workspace_bytes, &q, &a);
  if (st) return st;
  if (!aligned16(w_v_up) || !aligned16(out)) return VMLA_ERR_ALIGN;
  const AttnSpans sp = attn_spans(dims, cache, dtype, a.n_q, nullptr, nullptr, nullptr, w_v_up, out,
                                  workspace);
  st = check_disjoint({sp.out}, {sp.ws, sp.w_v_up, sp.cache});
  if (st) return st;
  a.w_v_up = w_v_up; a.out = out;
  return hip_status(launch_latent_attn(a, dtype == VMLA_F32, static_cast<hipStream_t>(stream)));
}

namespace {

// The attention core: the query prologue into the workspace, then the latent
// attention. With use_scratch the Qhat rows go to the library's scratch array
// instead of a caller's workspace: every host-side check runs first, against
// its size at a stand-in address, and its device address is looked up last.
int32_t chunk_attention_run(const vmla_dims* dims, const vmla_cache* cache, int32_t dtype,
                            const void* x, const void* w_q, const void* w_k_up, const void* w_v_up,
                            int32_t t_first, int32_t n_frames, int32_t n_valid_frames, void* out,
                            void* workspace, size_t workspace_bytes, bool use_scratch,
                            void* stream) {
  if (!x || !w_q || !w_k_up || !w_v_up || !out) return VMLA_ERR_NULL;
  QArgs q;
  AttnArgs a;
  void* ws = use_scratch ? reinterpret_cast<void*>(uintptr_t{256}) : workspace;
  const size_t ws_bytes = use_scratch ? (size_t)VMLA_NOALLOC_SCRATCH_BYTES : workspace_bytes;
  int32_t st = check_attention(dims, cache, dtype, t_first, n_frames, n_valid_frames, ws, ws_bytes,
                               &q, &a);
  if (st) return st;
  if (!aligned16(x) || !aligned16(w_q) || !aligned16(w_k_up) || !aligned16(w_v_up) || !aligned16(out))
    return VMLA_ERR_ALIGN;
  AttnSpans sp = attn_spans(dims, cache, dtype, q.n_q, x, w_q, w_k_up, w_v_up, out, workspace);
  if (use_scratch) sp.ws = Span{0, 0};        // library memory: no caller buffer can overlap it
  st = check_disjoint({sp.ws, sp.out}, {sp.x, sp.w_q, sp.w_k_up, sp.w_v_up, sp.cache});
  if (st) return st;
  if (use_scratch) {
    void* p = nullptr;
    if (scratch_buffer(&p) != hipSuccess) return VMLA_ERR_HIP;
    q.qhat = static_cast<uint16_t*>(p);
    a.qhat = q.qhat;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  q.x = x; q.w_q = w_q; q.w_k_up = w_k_up;
  st = hip_status(launch_qprologue(q, dtype == VMLA_F32, s));
  if (st) return st;
  a.w_v_up = w_v_up; a.out = out;
  return hip_status(launch_latent_attn(a, dtype == VMLA_F32, s));
}

}  // namespace

int32_t vmla_chunk_attention(const vmla_dims* dims, const vmla_cache* cache, int32_t dtype,
                             const void* x, const void* w_q, const void* w_k_up,
                             const void* w_v_up, int32_t t_first, int32_t n_frames,
                             int32_t n_valid_frames, void* out, void* workspace,
                             size_t workspace_bytes, void* stream) {
  return chunk_attention_run(dims, cache, dtype, x, w_q, w_k_up, w_v_up, t_first, n_frames,
                             n_valid_frames, out, workspace, workspace_bytes, false, stream);
}

int32_t vmla_chunk_attention_noalloc(const vmla_dims* dims, const vmla_cache* cache, int32_t dtype,
                                     const void* x, const void* w_q, const void* w_k_up,
                                     const void* w_v_up, int32_t t_first, int32_t n_frames,
                                     int32_t n_valid_frames, void* out, void* stream) {
  return chunk_attention_run(dims, cache, dtype, x, w_q, w_k_up, w_v_up, t_first, n_frames,
                             n_valid_frames, out, nullptr, 0, true, stream);
}

// ---- the whole attention layer: query latent and folded output mixer

static int32_t check_d_q(int32_t d_q) {
  return (d_q >= 64 && d_q <= 8192 && d_q % 64 == 0) ? VMLA_OK : VMLA_ERR_SHAPE;
}

int32_t vmla_fold_query_weights(const vmla_dims* dims, int32_t dtype, int32_t d_q,
                                const void* w_uq, const void* w_k_up, void* w_qa, void* stream) {
  int32_t st = check_dims_default(dims);
  if (st) return st;
  if (!w_uq || !w_k_up || !w_qa) return VMLA_ERR_NULL;
  if (dtype != VMLA_F32 && dtype != VMLA_BF16) return VMLA_ERR_DTYPE;
  st = check_d_q(d_q);
  if (st) return st;
  if (!aligned16(w_uq) || !aligned16(w_k_up) || !aligned16(w_qa)) return VMLA_ERR_ALIGN;
  const size_t e = esize(dtype), h = dims->n_heads;
  st = check_disjoint({bytes_at(w_qa, (size_t)d_q * h * kRow * sizeof(uint16_t))},
                      {bytes_at(w_uq, (size_t)d_q * h * kDHead * e), bytes_at(w_k_up, h * kDC * kDNope * e)});
  if (st) return st;
  FoldArgs f{};
  f.w_first = w_uq; f.w_second = w_k_up; f.out = w_qa;
  f.d_in = d_q; f.n_heads = dims->n_heads;
  return hip_status(launch_fold_query(f, dtype == VMLA_F32, static_cast<hipStream_t>(stream)));
}

int32_t vmla_fold_output_weights(const vmla_dims* dims, int32_t dtype, const void* w_v_up,
                                 const void* w_o, void* w_vo, void* stream) {
  int32_t st = check_dims_default(dims);
  if (st) return st;
  if (!w_v_up || !w_o || !w_vo) return VMLA_ERR_NULL;
  if (dtype != VMLA_F32 && dtype != VMLA_BF16) return VMLA_ERR_DTYPE;
  if (!aligned16(w_v_up) || !aligned16(w_o) || !aligned16(w_vo)) return VMLA_ERR_ALIGN;
  const size_t e = esize(dtype), h = dims->n_heads;
  st = check_disjoint({bytes_at(w_vo, h * kDC * dims->d_model * sizeof(uint16_t))},
                      {bytes_at(w_v_up, h * kDC * kDV * e), bytes_at(w_o, h * kDV * dims->d_model * e)});
  if (st) return st;
  FoldArgs f{};
  f.w_first = w_v_up; f.w_second = w_o; f.out = w_vo;
  f.d_out = dims->d_model; f.n_heads = dims->n_heads;
  return hip_status(launch_fold_output(f, dtype == VMLA_F32, static_cast<hipStream_t>(stream)));
}

size_t vmla_layer_workspace_bytes(const vmla_dims* dims, int32_t d_q, int32_t batch, int32_t n_q) {
  if (check_d_q(d_q) != VMLA_OK || check_dims_default(dims) != VMLA_OK) return 0;
  const size_t qhat = vmla_attention_workspace_bytes(dims, batch, n_q);
  if (!qhat) return 0;
  const size_t m = (size_t)batch * n_q;
  const size_t lat = (size_t)dims->n_heads * kDC;
  const size_t inner = m * ((size_t)d_q > lat ? (size_t)d_q : lat) * sizeof(uint16_t);
  return qhat + ((inner + 255) / 256) * 256;
}

namespace {

// Validation shared by the layer stages: the attention checks plus d_q and the
// layer workspace; *inner points just past the Qhat rows (a multiple of 448 bytes).
int32_t check_layer(const vmla_dims* dims, const vmla_cache* cache, int32_t dtype, int32_t d_q,
                    int32_t t_first, int32_t n_frames, int32_t n_valid_frames,
                    const void* workspace, size_t workspace_bytes, QArgs* q, AttnArgs* a,
                    uint16_t** inner) {
  int32_t st = check_d_q(d_q);
  if (st) return st;
  st = check_dims_default(dims);
  if (st) return st;
  st = check_attention(dims, cache, dtype, t_first, n_frames, n_valid_frames, workspace,
                       workspace_bytes, q, a);
  if (st) return st;
  const int64_t m = (int64_t)cache->batch * q->n_q;
  if (m > ((int64_t)1 << 28)) return VMLA_ERR_SHAPE;
  if (workspace_bytes < vmla_layer_workspace_bytes(dims, d_q, cache->batch, q->n_q))
    return VMLA_ERR_WORKSPACE;
  const size_t qhat = vmla_attention_workspace_bytes(dims, cache->batch, q->n_q);
  *inner = reinterpret_cast<uint16_t*>(static_cast<char*>(const_cast<void*>(workspace)) + qhat);
  return VMLA_OK;
}

int32_t launch_layer_prologue(const vmla_dims* dims, const vmla_cache* cache, int32_t dtype,
                              const void* x, const void* w_dq, int32_t d_q, const void* w_qa,
                              const QArgs& q, uint16_t* c_q, hipStream_t s) {
  // c_q = x W_DQ (bf16 rows of the workspace)
  GemmArgs g1{};
  g1.a = x; g1.w = w_dq; g1.out = c_q;
  g1.m = (int64_t)cache->batch * q.n_q; g1.k = dims->d_model; g1.n = d_q; g1.lda = dims->d_model;
  g1.mode = 0;
  int32_t st = hip_status(launch_gemm(g1, dtype == VMLA_F32, 0, s));
  if (st) return st;
  // Qhat = [c_q A_h | RoPE3D(c_q W_UQ^R[h])] * scale * log2(e), every head
  GemmArgs g2{};
  g2.a = c_q; g2.w = w_qa; g2.out = q.qhat;
  g2.m = g1.m; g2.k = d_q; g2.n = dims->n_heads * kRow; g2.lda = d_q; g2.mode = 1;
  g2.head_w = kRow; g2.rope_off = kDC;
  g2.n_q = q.n_q; g2.n_heads = q.n_heads; g2.grid_w = q.grid_w; g2.tokens_per_frame = q.tokens_per_frame;
  g2.t_first = q.t_first; g2.inv_grid_w = q.inv_grid_w; g2.inv_tokens_per_frame = q.inv_tokens_per_frame;
  g2.qscale = q.qscale; g2.rope = q.rope;
  return hip_status(launch_gemm(g2, 0, 0, s));
}

int32_t launch_layer_attention(const vmla_dims* dims, const vmla_cache* cache, int32_t dtype,
                               const void* w_vo, void* out, AttnArgs a, uint16_t* olat, hipStream_t s) {
  a.olat = olat;
  int32_t st = hip_status(launch_latent_attn(a, dtype == VMLA_F32, s));
  if (st) return st;
  // out = [O_lat,0 / l | ... | O_lat,H-1 / l] W_VO over all heads
  GemmArgs g{};
  g.a = olat; g.w = w_vo; g.out = out;
  g.m = (int64_t)cache->batch * a.n_q; g.k = dims->n_heads * kDC; g.n = dims->d_model;
  g.lda = g.k; g.mode = 0;
  return hip_status(launch_gemm(g, 0, dtype == VMLA_F32, s));
}

// Spans of the layer arguments: x [B, n_q, d_model], W_DQ [d_model, d_q],
// W_QA [d_q, H 224] and W_VO [H 192, d_model] (bf16), out [B, n_q, d_model],
// the layer workspace and the cache.
struct LayerSpans {
  Span x, w_dq, w_qa, w_vo, out, ws, cache;
};

LayerSpans layer_spans(const vmla_dims* d, const vmla_cache* c, int32_t dtype, int32_t d_q, int64_t n_q,
                       const void* x, const void* w_dq, const void* w_qa, const void* w_vo,
                       const void* out, const void* ws) {
  const size_t e = esize(dtype), m = (size_t)c->batch * n_q, h = d->n_heads;
  LayerSpans s;
  s.x = bytes_at(x, m * d->d_model * e);
  s.w_dq = bytes_at(w_dq, (size_t)d->d_model * d_q * e);
  s.w_qa = bytes_at(w_qa, (size_t)d_q * h * kRow * sizeof(uint16_t));
  s.w_vo = bytes_at(w_vo, h * kDC * d->d_model * sizeof(uint16_t));
  s.out = bytes_at(out, m * d->d_model * e);
  s.ws = bytes_at(ws, vmla_layer_workspace_bytes(d, d_q, c->batch, (int32_t)n_q));
  s.cache = cache_span(d, c);
  return s;
}

}  // namespace

int32_t vmla_layer_query_prologue(const vmla_dims* dims, const vmla_cache* cache, int32_t dtype,
                                  const void* x, const void* w_dq, int32_t d_q, const void* w_qa,
                                  int32_t t_first, int32_t n_frames, int32_t n_valid_frames,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  if (!x || !w_dq || !w_qa) return VMLA_ERR_NULL;
  QArgs q;
  AttnArgs a;
  uint16_t* inner;
  int32_t st = check_layer(dims, cache, dtype, d_q, t_first, n_frames, n_valid_frames, workspace,
                           workspace_bytes, &q, &a, &inner);
  if (st) return st;
  if (!aligned16(x) || !aligned16(w_dq) || !aligned16(w_qa)) return VMLA_ERR_ALIGN;
  const LayerSpans sp = layer_spans(dims, cache, dtype, d_q, q.n_q, x, w_dq, w_qa, nullptr, nullptr,
                                    workspace);
  st = check_disjoint({sp.ws}, {sp.x, sp.w_dq, sp.w_qa, sp.cache});
  if (st) return st;
  return launch_layer_prologue(dims, cache, dtype, x, w_dq, d_q, w_qa, q, inner,
                               static_cast<hipStream_t>(stream));
}

int32_t vmla_layer_attention(const vmla_dims* dims, const vmla_cache* cache, int32_t dtype,
                             int32_t d_q, const void* w_vo, int32_t t_first, int32_t n_frames,
                             int32_t n_valid_frames, void* out, void* workspace,
                             size_t workspace_bytes, void* stream) {
  if (!w_vo || !out) return VMLA_ERR_NULL;
  QArgs q;
  AttnArgs a;
  uint16_t* inner;
  int32_t st = check_layer(dims, cache, dtype, d_q, t_first, n_frames, n_valid_frames, workspace,
                           workspace_bytes, &q, &a, &inner);
  if (st) return st;
  if (!aligned16(w_vo) || !aligned16(out)) return VMLA_ERR_ALIGN;
  const LayerSpans sp = layer_spans(dims, cache, dtype, d_q, q.n_q, nullptr, nullptr, nullptr, w_vo, out,
                                    workspace);
  st = check_disjoint({sp.ws, sp.out}, {sp.w_vo, sp.cache});
  if (st) return st;
  return launch_layer_attention(dims, cache, dtype, w_vo, out, a, inner, static_cast<hipStream_t>(stream));
}

int32_t vmla_chunk_attention_layer(const vmla_dims* dims, const vmla_cache* cache, int32_t dtype,
                                   const void* x, const void* w_dq, int32_t d_q, const void* w_qa,
                                   const void* w_vo, int32_t t_first, int32_t n_frames,
                                   int32_t n_valid_frames, void* out, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  if (!x || !w_dq || !w_qa || !w_vo || !out) return VMLA_ERR_NULL;
  QArgs q;
  AttnArgs a;
  uint16_t* inner;
  int32_t st = check_layer(dims, cache, dtype, d_q, t_first, n_frames, n_valid_frames, workspace,
                           workspace_bytes, &q, &a, &inner);
  if (st) return st;
  if (!aligned16(x) || !aligned16(w_dq) || !aligned16(w_qa) || !aligned16(w_vo) || !aligned16(out))
    return VMLA_ERR_ALIGN;
  const LayerSpans sp = layer_spans(dims, cache, dtype, d_q, q.n_q, x, w_dq, w_qa, w_vo, out, workspace);
  st = check_disjoint({sp.ws, sp.out}, {sp.x, sp.w_dq, sp.w_qa, sp.w_vo, sp.cache});
  if (st) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = launch_layer_prologue(dims, cache, dtype, x, w_dq, d_q, w_qa, q, inner, s);
  if (st) return st;
  return launch_layer_attention(dims, cache, dtype, w_vo, out, a, inner, s);
}

// ---- explicit reconstruction: the comparison point of the latent form

int32_t vmla_pack_kv_weights(const vmla_dims* dims, int32_t dtype, const void* w_k_up,
                             const void* w_v_up, void* w_kv, void* stream) {
  int32_t st = check_dims_192(dims);
  if (st) return st;
  if (!w_k_up || !w_v_up || !w_kv) return VMLA_ERR_NULL;
  if (dtype != VMLA_F32 && dtype != VMLA_BF16) return VMLA_ERR_DTYPE;
  if (!aligned16(w_k_up) || !aligned16(w_v_up) || !aligned16(w_kv)) return VMLA_ERR_ALIGN;
  const size_t e = esize(dtype), h = dims->n_heads;
  st = check_disjoint({bytes_at(w_kv, kDC * h * (dims->d_nope + kDV) * e)},
                      {bytes_at(w_k_up, h * kDC * dims->d_nope * e), bytes_at(w_v_up, h * kDC * kDV * e)});
  if (st) return st;
  FoldArgs f{};
  f.w_first = w_k_up; f.w_second = w_v_up; f.out = w_kv; f.n_heads = dims->n_heads;
  f.d_nope = dims->d_nope;
  return hip_status(launch_pack_kv(f, dtype == VMLA_F32, static_cast<hipStream_t>(stream)));
}

size_t vmla_explicit_workspace_bytes(const vmla_dims* dims, int32_t batch, int32_t n_q, int32_t n_k) {
  if (check_dims_192(dims) != VMLA_OK || batch < 1 || n_q < 1 || n_k < 1) return 0;
  const size_t per = (size_t)batch * dims->n_heads * sizeof(uint16_t);
  return per * ((size_t)n_q * kDHead + (size_t)n_k * 2 * kDHead);
}

namespace {

// The explicit route writes its workspace (queries, then per-head K/V rows)
// and out; it reads x, W_Q, the packed [W_K_up[h] | W_V_up[h]] and the cache.
int32_t check_explicit_disjoint(const vmla_dims* d, const vmla_cache* c, int32_t dtype, int64_t n_q,
                                int64_t n_k, const void* x, const void* w_q, const void* w_kv,
                                const void* out, const void* ws) {
  const size_t e = esize(dtype), m = (size_t)c->batch * n_q, h = d->n_heads;
  return check_disjoint(
      {bytes_at(ws, vmla_explicit_workspace_bytes(d, c->batch, (int32_t)n_q, (int32_t)n_k)),
       bytes_at(out, m * h * d->d_v * e)},
      {bytes_at(x, m * d->d_model * e), bytes_at(w_q, (size_t)d->d_model * h * kDHead * e),
       bytes_at(w_kv, kDC * h * (d->d_nope + kDV) * e), cache_span(d, c)});
}

// Query GEMM, per-head K/V rebuild of slots [0, a.n_k), explicit attention
// with a's query chunks.
int32_t run_explicit(const vmla_dims* dims, const vmla_cache* cache, int32_t dtype, const void* x,
                     const void* w_q, const void* w_kv, const QArgs& q, const AttnArgs& a, void* out,
                     void* workspace, hipStream_t s) {
  int32_t st;
  const bool f32 = dtype == VMLA_F32;
  uint16_t* qbuf = static_cast<uint16_t*>(workspace);
  uint16_t* kvbuf = qbuf + (size_t)cache->batch * dims->n_heads * a.n_q * kDHead;
  // queries: [q_nope | RoPE3D(q_rope)] * scale * log2(e), per head
  GemmArgs g{};
  g.a = x; g.w = w_q; g.out = qbuf;
  g.m = (int64_t)cache->batch * a.n_q; g.k = dims->d_model; g.n = dims->n_heads * kDHead;
  g.lda = dims->d_model; g.mode = 1; g.head_w = kDHead; g.rope_off = dims->d_nope;
  g.n_q = q.n_q; g.n_heads = q.n_heads; g.grid_w = q.grid_w; g.tokens_per_frame = q.tokens_per_frame;
  g.t_first = q.t_first; g.inv_grid_w = q.inv_grid_w; g.inv_tokens_per_frame = q.inv_tokens_per_frame;
  g.qscale = q.qscale; g.rope = q.rope;
  st = hip_status(launch_gemm(g, f32, 0, s));
  if (st) return st;
  // per-head keys and values of every valid slot, one batch element at a time
  const size_t elem = f32 ? sizeof(float) : sizeof(uint16_t);
  for (int b = 0; b < cache->batch; ++b) {
    GemmArgs r{};
    const int row = dims->d_c + dims->d_rope;
    r.a = static_cast<const char*>(cache->data) + (size_t)b * a.cache_rows * row * elem;
    r.w = w_kv; r.out = kvbuf + (size_t)b * dims->n_heads * a.n_k * 2 * kDHead;
    r.m = a.n_k; r.k = kDC; r.n = dims->n_heads * (dims->d_nope + kDV); r.lda = row; r.mode = 2;
    r.d_nope = dims->d_nope;
    st = hip_status(launch_gemm(r, f32, 0, s));
    if (st) return st;
  }
  ExplicitArgs e{};
  e.q = qbuf; e.kv = kvbuf; e.out = out;
  e.batch = cache->batch; e.n_q = a.n_q; e.n_heads = dims->n_heads; e.n_k = a.n_k;
  e.cm = a.cm;
  return hip_status(launch_explicit_attn(e, f32, s));
}

}  // namespace

int32_t vmla_chunk_attention_explicit(const vmla_dims* dims, const vmla_cache* cache, int32_t dtype,
                                      const void* x, const void* w_q, const void* w_kv,
                                      int32_t t_first, int32_t n_frames, int32_t n_valid_frames,
                                      void* out, void* workspace, size_t workspace_bytes,
                                      void* stream) {
  if (!x || !w_q || !w_kv || !out) return VMLA_ERR_NULL;
  QArgs q;
  AttnArgs a;
  // the attention checks, with the workspace size checked below
  int32_t st = check_dims_192(dims);
  if (st) return st;
  st = check_attention(dims, cache, dtype, t_first, n_frames, n_valid_frames, workspace,
                       SIZE_MAX, &q, &a);
  if (st) return st;
  if (cache->rope_at_read) return VMLA_ERR_SHAPE;
  if ((int64_t)a.n_k * 2 * kDHead * dims->n_heads > INT32_MAX) return VMLA_ERR_SHAPE;
  if (workspace_bytes < vmla_explicit_workspace_bytes(dims, cache->batch, a.n_q, a.n_k))
    return VMLA_ERR_WORKSPACE;
  if (!aligned16(x) || !aligned16(w_q) || !aligned16(w_kv) || !aligned16(out)) return VMLA_ERR_ALIGN;
  st = check_explicit_disjoint(dims, cache, dtype, a.n_q, a.n_k, x, w_q, w_kv, out, workspace);
  if (st) return st;
  return run_explicit(dims, cache, dtype, x, w_q, w_kv, q, a, out, workspace,
                      static_cast<hipStream_t>(stream));
}


// ---- a whole clip under the chunk-causal block mask

namespace {

// Validation of the whole-clip form. Frames 0 .. n_frames - 1 sit in slots
// t T + n (a cache of at least n_frames frames, no sink frame, k_R rotated at
// append); every token of the clip is a query at its absolute position; chunk
// c (chunk_frames frames) sees the slots of frames [e - W, e), e its end.
int32_t check_clip(const vmla_dims* dims, const vmla_cache* cache, int32_t dtype, int32_t n_frames,
                   int32_t chunk_frames, int32_t mask_window_frames, const void* workspace,
                   QArgs* q, AttnArgs* a) {
  int32_t st = check_dims(dims);
  if (st) return st;
  if (dims->d_rope != kDRope || dims->d_c > kDC) return VMLA_ERR_SHAPE;   // default split, d_c <= 192
  st = check_cache(cache, dtype, dims->d_c + dims->d_rope);
  if (st) return st;
  if (cache->sink_frames || cache->rope_at_read) return VMLA_ERR_SHAPE;
  if (n_frames < 1 || n_frames > cache->window_frames) return VMLA_ERR_RANGE;
  if (chunk_frames < 1 || chunk_frames > n_frames || mask_window_frames < chunk_frames)
    return VMLA_ERR_RANGE;
  const int64_t T = (int64_t)cache->grid_h * cache->grid_w;
  const int64_t n_q = T * n_frames;
  if (n_q * dims->d_model > INT32_MAX || n_q * dims->n_heads * kDV > INT32_MAX) return VMLA_ERR_SHAPE;
  const int64_t n_chunks = (n_frames + chunk_frames - 1) / chunk_frames;
  if (n_chunks * cache->batch > 65535) return VMLA_ERR_SHAPE;   // one grid z index per (chunk, element)
  if (!workspace) return VMLA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return VMLA_ERR_ALIGN;
  fill_attention(dims, cache, workspace, n_q, 0, n_q, 0, q, a);
  const int64_t span = mask_window_frames < n_frames ? mask_window_frames : n_frames;
  a->cm = ChunkMask{(int)n_chunks, (int)(T * chunk_frames), (int)(T * chunk_frames), (int)(T * span)};
  return VMLA_OK;
}

}  // namespace

int32_t vmla_chunk_causal_attention(const vmla_dims* dims, const vmla_cache* cache, int32_t dtype,
                                    const void* x, const void* w_q, const void* w_k_up,
                                    const void* w_v_up, int32_t n_frames, int32_t chunk_frames,
                                    int32_t mask_window_frames, void* out, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  if (!x || !w_q || !w_k_up || !w_v_up || !out) return VMLA_ERR_NULL;
  QArgs q;
  AttnArgs a;
  int32_t st = check_clip(dims, cache, dtype, n_frames, chunk_frames, mask_window_frames, workspace,
                          &q, &a);
  if (st) return st;
  if (workspace_bytes < vmla_attention_workspace_bytes(dims, cache->batch, a.n_q))
    return VMLA_ERR_WORKSPACE;
  if (!aligned16(x) || !aligned16(w_q) || !aligned16(w_k_up) || !aligned16(w_v_up) || !aligned16(out))
    return VMLA_ERR_ALIGN;
  const AttnSpans sp = attn_spans(dims, cache, dtype, q.n_q, x, w_q, w_k_up, w_v_up, out, workspace);
  st = check_disjoint({sp.ws, sp.out}, {sp.x, sp.w_q, sp.w_k_up, sp.w_v_up, sp.cache});
  if (st) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  q.x = x; q.w_q = w_q; q.w_k_up = w_k_up;
  st = hip_status(launch_qprologue(q, dtype == VMLA_F32, s));
  if (st) return st;
  a.w_v_up = w_v_up; a.out = out;
  return hip_status(launch_latent_attn(a, dtype == VMLA_F32, s));
}

int32_t vmla_chunk_causal_latent_attention(const vmla_dims* dims, const vmla_cache* cache,
                                           int32_t dtype, const void* w_v_up, int32_t n_frames,
                                           int32_t chunk_frames, int32_t mask_window_frames,
                                           void* out, const void* workspace,
                                           size_t workspace_bytes, void* stream) {
  if (!w_v_up || !out) return VMLA_ERR_NULL;
  QArgs q;
  AttnArgs a;
  int32_t st = check_clip(dims, cache, dtype, n_frames, chunk_frames, mask_window_frames, workspace,
                          &q, &a);
  if (st) return st;
  if (workspace_bytes < vmla_attention_workspace_bytes(dims, cache->batch, a.n_q))
    return VMLA_ERR_WORKSPACE;
  if (!aligned16(w_v_up) || !aligned16(out)) return VMLA_ERR_ALIGN;
  const AttnSpans sp = attn_spans(dims, cache, dtype, a.n_q, nullptr, nullptr, nullptr, w_v_up, out,
                                  workspace);
  st = check_disjoint({sp.out}, {sp.ws, sp.w_v_up, sp.cache});
  if (st) return st;
  a.w_v_up = w_v_up; a.out = out;
  return hip_status(launch_latent_attn(a, dtype == VMLA_F32, static_cast<hipStream_t>(stream)));
}

int32_t vmla_chunk_causal_attention_explicit(const vmla_dims* dims, const vmla_cache* cache,
                                             int32_t dtype, const void* x, const void* w_q,
                                             const void* w_kv, int32_t n_frames,
                                             int32_t chunk_frames, int32_t mask_window_frames,
                                             void* out, void* workspace, size_t workspace_bytes,
                                             void* stream) {
  if (!x || !w_q || !w_kv || !out) return VMLA_ERR_NULL;
  int32_t st = check_dims_192(dims);
  if (st) return st;
  QArgs q;
  AttnArgs a;
  st = check_clip(dims, cache, dtype, n_frames, chunk_frames, mask_window_frames, workspace, &q, &a);
  if (st) return st;
  if ((int64_t)a.n_k * 2 * kDHead * dims->n_heads > INT32_MAX) return VMLA_ERR_SHAPE;
  if (workspace_bytes < vmla_explicit_workspace_bytes(dims, cache->batch, a.n_q, a.n_k))
    return VMLA_ERR_WORKSPACE;
  if (!aligned16(x) || !aligned16(w_q) || !aligned16(w_kv) || !aligned16(out)) return VMLA_ERR_ALIGN;
  st = check_explicit_disjoint(dims, cache, dtype, a.n_q, a.n_k, x, w_q, w_kv, out, workspace);
  if (st) return st;
  return run_explicit(dims, cache, dtype, x, w_q, w_kv, q, a, out, workspace,
                      static_cast<hipStream_t>(stream));
}

int32_t vmla_output_projection(const vmla_dims* dims, int32_t dtype, int64_t m, const void* in,
                               const void* w_o, void* out, void* stream) {
  int32_t st = check_dims_default(dims);
  if (st) return st;
  if (!in || !w_o || !out) return VMLA_ERR_NULL;
  if (dtype != VMLA_F32 && dtype != VMLA_BF16) return VMLA_ERR_DTYPE;
  if (m < 1 || m > ((int64_t)1 << 31) / 128) return VMLA_ERR_SHAPE;
  if (!aligned16(in) || !aligned16(w_o) || !aligned16(out)) return VMLA_ERR_ALIGN;
  const size_t e = esize(dtype), hv = (size_t)dims->n_heads * kDV;
  st = check_disjoint({bytes_at(out, (size_t)m * dims->d_model * e)},
                      {bytes_at(in, (size_t)m * hv * e), bytes_at(w_o, hv * dims->d_model * e)});
  if (st) return st;
  GemmArgs g{};
  g.a = in; g.w = w_o; g.out = out;
  g.m = m; g.k = dims->n_heads * kDV; g.n = dims->d_model; g.lda = g.k; g.mode = 0;
  const int f32 = dtype == VMLA_F32;
  return hip_status(launch_gemm(g, f32, f32, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
