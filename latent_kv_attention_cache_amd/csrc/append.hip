// Latent cache append for gfx950: [c | k_R] = x @ [W_down | W_KR], 3D-RoPE on
// the k_R columns, store into the ring slots of the appended frames.
//
// VideoMLA (paperlayer.ai summary of arXiv:2605.30351v1): the cached pair per
// token is the shared content latent and the head-shared positional key
// (§3 "Shared low-rank KV cache", "Decoupled positional encoding"; App. D.2);
// the positional key is rotated by 3D-RoPE with 6/5/5 complex pairs on t/h/w
// (App. D.3); the cache is a fixed-size window of latent frames with FIFO
// eviction (App. D.4).
//
// One workgroup (4 waves) computes a 128-token x 224-column tile; wave w owns
// tokens [32w, 32w+32) of the tile and all seven 32-column output blocks. The
// K loop stages a 64-deep slice of x and of [W_down | W_KR] in LDS, row-major;
// x fragments are read row-wise, weight fragments with the LDS transpose read.
#include "device_common.h"
#include "kernels.h"

namespace vmla {
namespace {

constexpr int kTok = 128;            // tokens per workgroup
constexpr int kKc = 64;              // K slice per stage
constexpr int kXLd = kKc + 8;        // padded LDS row of the x slice
constexpr int kWLd = kRow + 8;       // padded LDS row of the weight slice
constexpr int kThreads = 256;
constexpr int kColTiles = kRow / 32; // 7

template <typename T>
__global__ __launch_bounds__(kThreads)
void append_kernel(AppendArgs a) {
  __shared__ __attribute__((aligned(16))) bf16_t xs[kTok * kXLd];
  __shared__ __attribute__((aligned(16))) bf16_t ws[kKc * kWLd];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int b = blockIdx.y;
  const int tok0 = blockIdx.x * kTok;
  const T* x = static_cast<const T*>(a.x) + (size_t)b * a.n_tok * a.d_model;
  const T* wd = static_cast<const T*>(a.w_down);
  const T* wr = static_cast<const T*>(a.w_kr);

  f32x16 acc[kColTiles];
#pragma unroll
  for (int c = 0; c < kColTiles; ++c) acc[c] = f32x16{};

  for (int k0 = 0; k0 < a.d_model; k0 += kKc) {
    // stage x[tok0 .. tok0+127][k0 .. k0+63]: 1024 chunks of 8
#pragma unroll
    for (int i = 0; i < (kTok * kKc / 8) / kThreads; ++i) {
      const int c = tid + i * kThreads;
      const int row = c >> 3, kc = c & 7;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (tok0 + row < a.n_tok) v = load8_bf16<T>(x + (size_t)(tok0 + row) * a.d_model + k0 + 8 * kc);
      *reinterpret_cast<uint4*>(&xs[row * kXLd + 8 * kc]) = v;
    }
    // stage [W_down | W_KR][k0 .. k0+63][0 .. 223]: 1792 chunks of 8
#pragma unroll
    for (int i = 0; i < (kKc * kRow / 8 + kThreads - 1) / kThreads; ++i) {
      const int c = tid + i * kThreads;
      if (c < kKc * kRow / 8) {
        const int kr = c / (kRow / 8), cc = c % (kRow / 8);
        const T* src = cc < kDC / 8 ? wd + (size_t)(k0 + kr) * kDC + 8 * cc
                                    : wr + (size_t)(k0 + kr) * kDRope + 8 * (cc - kDC / 8);
        *reinterpret_cast<uint4*>(&ws[kr * kWLd + 8 * cc]) = load8_bf16<T>(src);
      }
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < kKc / 16; ++ks) {
      const bf16x8 av = lds_row8(&xs[(32 * wave + (lane & 31)) * kXLd + ks * 16 + 8 * half]);
      const int ka = ks * 16 + 8 * half;
#pragma unroll
      for (int c = 0; c < kColTiles; ++c) {
        const bf16x8 bv = lds_tr8(ws, kWLd, ka, ka + 4, 32 * c, lane);
        acc[c] = mfma32(av, bv, acc[c]);
      }
    }
    __syncthreads();
  }

  // Epilogue. Register r of lane l holds token row 8(r/4) + 4*half + r%4 of the
  // wave's 32 tokens and column 32c + l%32.
  const int col = lane & 31;
  const int pair = col >> 1;
  const bool odd = col & 1;
  const float omega = a.rope.omega[pair];
  const int axis = a.rope.axis[pair];
  T* cache = static_cast<T*>(a.cache);
  const size_t ring_rows = (size_t)a.window_frames * a.tokens_per_frame;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = 32 * wave + 8 * (r >> 2) + 4 * half + (r & 3);
    const int n = tok0 + row;
    // the RoPE lane exchange runs in every lane so that partners are always live
    const float v = acc[kColTiles - 1][r];
    const float partner = swap_adjacent(v);
    if (n >= a.n_tok) continue;
    const int f = n / a.tokens_per_frame;
    const int n_in = n - f * a.tokens_per_frame;
    const int t = a.t_first + f;
    const int hh = n_in / a.grid_w;
    const int ww = n_in - hh * a.grid_w;
    const int pos = axis == 0 ? t : (axis == 1 ? hh : ww);
    float sn, cs;
    sincosf((float)pos * omega, &sn, &cs);
    // pair (a0, a1) -> (a0 cos - a1 sin, a0 sin + a1 cos)
    const float rot = odd ? partner * sn + v * cs : v * cs - partner * sn;
    const size_t slot = (size_t)(t % a.window_frames) * a.tokens_per_frame + n_in;
    T* dst = cache + ((size_t)b * ring_rows + slot) * kRow;
#pragma unroll
    for (int c = 0; c < kColTiles - 1; ++c) dst[32 * c + col] = from_f32<T>(acc[c][r]);
    dst[32 * (kColTiles - 1) + col] = from_f32<T>(rot);
  }
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, bool f32, hipStream_t s) {
  dim3 grid((a.n_tok + kTok - 1) / kTok, a.batch);
  if (f32) hipLaunchKernelGGL(append_kernel<float>, grid, dim3(kThreads), 0, s, a);
  else hipLaunchKernelGGL(append_kernel<bf16_t>, grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace vmla
