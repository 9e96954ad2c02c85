// Internal launch interface between the C-ABI host layer (vmla_api.cpp) and the
// gfx950 kernels. Arguments are validated by the host layer before any launcher
// is called; launchers only configure grids and launch.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vmla {

// Widths of the default configuration (VideoMLA: 96/32 NoPE/RoPE split,
// 192-wide content latent, 128-wide values). The head width d_nope + d_rope
// is always 128; the split variants move the boundary (64/64, 32/96, 112/16).
constexpr int kDNope = 96;
constexpr int kDRope = 32;
constexpr int kDC = 192;
constexpr int kDV = 128;
constexpr int kDHead = kDNope + kDRope;   // 128
constexpr int kRow = kDC + kDRope;        // 224 cached scalars per token
constexpr int kPairs = kDRope / 2;        // 16 complex RoPE pairs
constexpr int kMaxPairs = 48;             // the RoPE-heavy 32/96 split

// Rate of each RoPE pair in revolutions per position step (omega / 2 pi) as a
// 64-bit binary fraction rate * 2^64 = (rev_hi << 32) | rev_lo, and its axis
// (0 = t, 1 = h, 2 = w).
struct RopeTable {
  uint32_t rev_lo[kMaxPairs];
  uint32_t rev_hi[kMaxPairs];
  int axis[kMaxPairs];
};

// Query chunks of one attention launch. Each batch element's n_q queries are
// cut into n_chunks chunks of chunk_q (the last may be shorter); chunk c
// attends to the keys [max(0, e - key_span), e) with e = min(n_k, (c + 1) *
// key_step). n_chunks = 1, chunk_q = n_q, key_step = key_span = n_k is one
// query chunk over all n_k keys.
struct ChunkMask {
  int n_chunks, chunk_q, key_step, key_span;
};

struct AppendArgs {
  const void* x;        // [batch, n_tok, d_model]
  const void* w_down;   // [d_model, kDC]
  const void* w_kr;     // [d_model, kDRope]
  void* cache;          // [batch, window_frames * T, kRow]
  int batch, n_tok, d_model;
  int grid_w, tokens_per_frame, window_frames, t_first;
  float inv_grid_w, inv_tokens_per_frame, inv_window_frames;   // 1/x as float
  int sink_frames;      // 0 or 1: frame 0 kept in slots [0, T)
  int rope_at_read;     // 1: k_R stored unrotated
  int d_c;              // content width: 64, 128, kDC, 256 or 512 (rows are d_c + d_rope wide)
  int d_rope;           // positional width: kDRope, or 16 / 64 / 96 (split variants, d_c = kDC)
  RopeTable rope;
};

struct QArgs {
  const void* x;        // [batch, n_q, d_model]
  const void* w_q;      // [d_model, n_heads * kDHead]
  const void* w_k_up;   // [n_heads, kDC, kDNope]
  uint16_t* qhat;       // [batch, n_heads, n_q, kRow] bf16 (workspace)
  int batch, n_q, d_model, n_heads;
  int grid_w, tokens_per_frame, t_first;
  float inv_grid_w, inv_tokens_per_frame;   // 1/x as float
  float qscale;         // softmax scale * log2(e)
  int d_c;              // content width: 64, 128 or kDC (Qhat rows are d_c + d_rope wide)
  int d_rope;           // positional width; the head's first kDHead - d_rope columns are NoPE
  RopeTable rope;
};

struct AttnArgs {
  const uint16_t* qhat; // [batch, n_heads, n_q, kRow] bf16
  const void* cache;    // [batch, cache_rows, kRow]
  const void* w_v_up;   // [n_heads, kDC, kDV]
  void* out;            // [batch, n_q, n_heads, kDV]
  uint16_t* olat;       // null, or [batch * n_q, n_heads * kDC] bf16: O_lat / l instead of out
  int batch, n_q, n_heads, n_k, cache_rows;
  int d_c;              // content width: 64, 128 or kDC (rows are d_c + d_rope wide)
  int d_rope;           // positional width of the rows
  // Read-time RoPE of k_R (rope_at_read = 1): the key in slot frame fs sits at
  // temporal coordinate fs when fs < sink_frames, otherwise at
  // sink_frames + ((fs - sink_frames - shift_mod_w) mod window_frames).
  int rope_at_read, sink_frames, window_frames, shift_mod_w, tokens_per_frame, grid_w;
  float inv_tokens_per_frame, inv_grid_w;
  RopeTable rope;
  ChunkMask cm;
};

// out = A W over row-major operands; A [m][lda >= k], W [k][n]. mode 0:
// out [m][n]; mode 1: per-head query rows out[b][h][n][head_w] (n = n_heads *
// head_w, RoPE from column rope_off on, times qscale); mode 2: explicit K/V
// rows out[h][m][2 kDHead] from W = per-head [W_K_up | W_V_up] and the k_R
// columns of A.
struct GemmArgs {
  const void* a;
  const void* w;
  void* out;
  int64_t m;
  int k, n, lda, mode;
  // mode 2: NoPE width of a head's key (the k_R copy fills the rest of kDHead)
  int d_nope;
  // mode 1 only
  int n_q, n_heads, grid_w, tokens_per_frame, t_first, head_w, rope_off;
  float inv_grid_w, inv_tokens_per_frame, qscale;
  RopeTable rope;
};

struct ExplicitArgs {
  const uint16_t* q;    // [batch, n_heads, n_q, kDHead] bf16, pre-scaled by scale * log2(e)
  const uint16_t* kv;   // [batch, n_heads, n_k, 2 kDHead] bf16: [k (128) | v (128)]
  void* out;            // [batch, n_q, n_heads, kDV]
  int batch, n_q, n_heads, n_k;
  ChunkMask cm;
};

// One-time weight folds (bf16 results). Query: w_first = W_UQ [d_in][n_heads
// kDHead], w_second = W_K_up [n_heads][kDC][kDNope], out [d_in][n_heads kRow].
// Output: w_first = W_V_up [n_heads][kDC][kDV], w_second = W_O [n_heads kDV][d_out],
// out [n_heads kDC][d_out].
struct FoldArgs {
  const void* w_first;
  const void* w_second;
  void* out;
  int d_in, d_out, n_heads;
  int d_nope;           // NoPE width of a head (the K/V weight pack)
};

hipError_t launch_append(const AppendArgs& a, bool f32, hipStream_t s);
int append_plan(int64_t m, int cus, int max_rows, int* nrb);   // append workgroups; row blocks per wave
hipError_t launch_qprologue(const QArgs& a, bool f32, hipStream_t s);
hipError_t launch_latent_attn(const AttnArgs& a, bool f32, hipStream_t s);
hipError_t launch_latent_attn_wide(const AttnArgs& a, hipStream_t s);   // d_c 256 / 512, bf16
hipError_t launch_gemm(const GemmArgs& a, int a_f32, int out_f32, hipStream_t s);
hipError_t launch_fold_query(const FoldArgs& a, bool f32, hipStream_t s);
hipError_t launch_fold_output(const FoldArgs& a, bool f32, hipStream_t s);
hipError_t launch_explicit_attn(const ExplicitArgs& a, bool f32, hipStream_t s);
hipError_t launch_pack_kv(const FoldArgs& a, bool f32, hipStream_t s);
// Device address of this GPU's library-owned scratch array
// (VMLA_NOALLOC_SCRATCH_BYTES), looked up once per device.
hipError_t scratch_buffer(void** ptr);

}  // namespace vmla
