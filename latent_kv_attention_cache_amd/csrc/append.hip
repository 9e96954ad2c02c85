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
// One workgroup (7 waves) computes a 64-token x 224-column tile; wave w owns
// the 32-column block w (blocks 0-5: c from W_down, block 6: k_R from W_KR)
// for all 64 tokens. The d_model contraction runs as a pipeline of 64-deep
// stages (kStages buffers fetched by LDS-DMA kStages-1 stages ahead, one
// barrier per stage); x, W_down and W_KR slices sit in separate LDS regions.
#include "device_common.h"
#include "kernels.h"
#include "staging.h"

namespace vmla {
namespace {

constexpr int kTok = 64;               // tokens per workgroup
constexpr int kWaves = kRow / 32;      // 7: one per 32-column block
constexpr int kThreads = 64 * kWaves;
constexpr int kStages = 4;
constexpr int kAElems = kTok * kStageK;          // x slice        (8 KB)
constexpr int kB1Elems = kStageK * kDC;          // W_down slice   (24 KB)
constexpr int kB2Elems = kStageK * kDRope;       // W_KR slice     (4 KB)
constexpr int kStageElems = kAElems + kB1Elems + kB2Elems;
constexpr int kALoads = kAElems * 2 / 1024;      // 8
constexpr int kB1Loads = kB1Elems * 2 / 1024;    // 24
constexpr int kB2Loads = kB2Elems * 2 / 1024;    // 4
constexpr int kLoads = kALoads + kB1Loads + kB2Loads;   // 36
// wave w issues loads w, w + 7, ...: wave 0 issues 6 per stage, waves 1-6 issue 5
constexpr int kLoadsWave0 = (kLoads + kWaves - 1) / kWaves;
constexpr int kLoadsOther = kLoads / kWaves;
static_assert(kLoads % kWaves == 1, "load split assumed: wave 0 takes one extra load");

template <typename T>
__global__ __launch_bounds__(kThreads)
void append_kernel(AppendArgs a) {
  __shared__ __attribute__((aligned(16))) bf16_t smem[kStages * kStageElems];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int b = blockIdx.y;
  const int tok0 = blockIdx.x * kTok;
  const T* x = static_cast<const T*>(a.x) + (size_t)b * a.n_tok * a.d_model;
  const T* wd = static_cast<const T*>(a.w_down);
  const T* wr = static_cast<const T*>(a.w_kr);
  const int nst = a.d_model / kStageK;

  auto issue = [&](int s) {
    bf16_t* st = smem + (s % kStages) * kStageElems;
    for (int n = wave; n < kLoads; n += kWaves) {
      if (n < kALoads) stage_a_load<T>(st, x, a.d_model, tok0, a.n_tok, s * kStageK, n, lane);
      else if (n < kALoads + kB1Loads)
        stage_b_load<T, kDC>(st + kAElems, wd, kDC, 0, s * kStageK, n - kALoads, lane);
      else
        stage_b_load<T, kDRope>(st + kAElems + kB1Elems, wr, kDRope, 0, s * kStageK,
                                n - kALoads - kB1Loads, lane);
    }
  };
  auto wait = [&](int stages) {
    if (wave == 0) wait_stages<kLoadsWave0>(stages);
    else wait_stages<kLoadsOther>(stages);
  };

  for (int s = 0; s < kStages - 1 && s < nst; ++s) issue(s);

  f32x16 acc[2] = {f32x16{}, f32x16{}};
  for (int s = 0; s < nst; ++s) {
    wait(min(kStages - 2, nst - 1 - s));                  // stage s has landed
    __syncthreads();
    if (s + kStages - 1 < nst) issue(s + kStages - 1);    // into the buffer of stage s-1
    const bf16_t* A = smem + (s % kStages) * kStageElems;
#pragma unroll
    for (int ks = 0; ks < kStageK / 16; ++ks) {
      bf16x8 bv;
      if (wave < kWaves - 1) bv = b_frag<kDC>(A + kAElems, ks, 32 * wave, lane);
      else bv = b_frag<kDRope>(A + kAElems + kB1Elems, ks, 0, lane);
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const bf16x8 av = a_frag(A, 32 * tt + (lane & 31), ks, half);
        acc[tt] = mfma32(av, bv, acc[tt]);
      }
    }
  }

  // Epilogue. Register r of lane l holds token row 32 tt + 8(r/4) + 4 half + r%4
  // and column 32 wave + l%32; wave 6 holds the k_R columns and rotates them.
  const int col = lane & 31;
  const int pair = col >> 1;
  const bool odd = col & 1;
  const bool rope = wave == kWaves - 1;
  const float rev = a.rope.rev[pair];
  const int axis = a.rope.axis[pair];
  T* cache = static_cast<T*>(a.cache);
  const size_t ring_rows = (size_t)a.window_frames * a.tokens_per_frame;
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = 32 * tt + 8 * (r >> 2) + 4 * half + (r & 3);
      const int n = tok0 + row;
      float v = acc[tt][r];
      // the RoPE lane exchange runs in every lane so that partners are always live
      const float partner = swap_adjacent(v);
      if (n >= a.n_tok) continue;
      int n_in, ww, tw;
      const int f = div_small(n, a.tokens_per_frame, a.inv_tokens_per_frame, &n_in);
      const int t = a.t_first + f;
      if (rope) {
        const int hh = div_small(n_in, a.grid_w, a.inv_grid_w, &ww);
        const int pos = axis == 0 ? t : (axis == 1 ? hh : ww);
        float sn, cs;
        sincos_rev(pos, rev, &sn, &cs);
        // pair (a0, a1) -> (a0 cos - a1 sin, a0 sin + a1 cos)
        v = odd ? partner * sn + v * cs : v * cs - partner * sn;
      }
      div_small(t, a.window_frames, a.inv_window_frames, &tw);
      const size_t slot = (size_t)tw * a.tokens_per_frame + n_in;
      cache[((size_t)b * ring_rows + slot) * kRow + 32 * wave + col] = from_f32<T>(v);
    }
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
