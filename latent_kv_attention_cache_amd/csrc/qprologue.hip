// Query prologue for gfx950: per head h,
//   q_h     = x @ W_Q[:, h*128 : h*128+128]            (nope 96 | rope 32)
//   q_rope  = RoPE3D(q_h[96:128], (t, h, w))
//   q_lat   = q_h[0:96] @ W_K_up[h]^T                   (96 -> 192)
//   Qhat_h  = (scale * log2 e) * [q_lat | q_rope]       stored bf16
//
// VideoMLA (paperlayer.ai summary of arXiv:2605.30351v1), App. E
// "Content-path absorption": the content score is taken against the cached
// latent through a fixed matrix applied to the query side, so no per-head key
// is built; "RoPE branch": the positional part stays separate and is rotated
// with the token's (t, h, w) (App. D.3). Folding log2 e into the scale lets the
// attention kernel use exp2 directly.
//
// One workgroup (4 waves) handles 64 tokens of one head. Wave w computes output
// columns [32w, 32w+32) of q_h for all 64 tokens; wave 3 therefore holds the
// rope channels. The absorption GEMM then splits its 2 x 6 output blocks
// three per wave. The [64 x 224] result is assembled in LDS and written with
// 16-byte row stores.
#include "device_common.h"
#include "kernels.h"

namespace vmla {
namespace {

constexpr int kTok = 64;
constexpr int kKc = 64;
constexpr int kThreads = 256;
constexpr int kXLd = kKc + 8;          // x slice row (elements)
constexpr int kWLd = kDHead + 8;       // W_Q slice row
constexpr int kQnLd = kDNope + 8;      // q_nope staging row
constexpr int kOutLd = kRow + 8;       // output tile row
constexpr int kLoopElems = kTok * kXLd + kKc * kWLd;
constexpr int kEpiElems = kTok * kQnLd + kTok * kOutLd;
constexpr int kSmemElems = kLoopElems > kEpiElems ? kLoopElems : kEpiElems;

template <typename T>
__global__ __launch_bounds__(kThreads)
void qprologue_kernel(QArgs a) {
  __shared__ __attribute__((aligned(16))) bf16_t smem[kSmemElems];
  bf16_t* xs = smem;                       // [kTok][kXLd]
  bf16_t* ws = smem + kTok * kXLd;         // [kKc][kWLd]
  bf16_t* qn = smem;                       // [kTok][kQnLd]   (after the K loop)
  bf16_t* ot = smem + kTok * kQnLd;        // [kTok][kOutLd]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int tok0 = blockIdx.x * kTok;
  const int wq_ld = a.n_heads * kDHead;
  const T* x = static_cast<const T*>(a.x) + (size_t)b * a.n_q * a.d_model;
  const T* wq = static_cast<const T*>(a.w_q) + (size_t)h * kDHead;

  f32x16 acc[2] = {f32x16{}, f32x16{}};
  for (int k0 = 0; k0 < a.d_model; k0 += kKc) {
#pragma unroll
    for (int i = 0; i < kTok * kKc / 8 / kThreads; ++i) {
      const int c = tid + i * kThreads;
      const int row = c >> 3, kc = c & 7;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (tok0 + row < a.n_q) v = load8_bf16<T>(x + (size_t)(tok0 + row) * a.d_model + k0 + 8 * kc);
      *reinterpret_cast<uint4*>(&xs[row * kXLd + 8 * kc]) = v;
    }
#pragma unroll
    for (int i = 0; i < kKc * kDHead / 8 / kThreads; ++i) {
      const int c = tid + i * kThreads;
      const int kr = c >> 4, cc = c & 15;
      *reinterpret_cast<uint4*>(&ws[kr * kWLd + 8 * cc]) =
          load8_bf16<T>(wq + (size_t)(k0 + kr) * wq_ld + 8 * cc);
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < kKc / 16; ++ks) {
      const int ka = ks * 16 + 8 * half;
      const bf16x8 bv = lds_tr8(ws, kWLd, ka, ka + 4, 32 * wave, lane);
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const bf16x8 av = lds_row8(&xs[(32 * tt + (lane & 31)) * kXLd + ka]);
        acc[tt] = mfma32(av, bv, acc[tt]);
      }
    }
    __syncthreads();
  }

  // Register r of lane l: token row 32*tt + 8(r/4) + 4*half + r%4, column 32*wave + l%32.
  const int col = lane & 31;
  if (wave == 3) {
    const int pair = col >> 1;
    const bool odd = col & 1;
    const float omega = a.rope.omega[pair];
    const int axis = a.rope.axis[pair];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 32 * tt + 8 * (r >> 2) + 4 * half + (r & 3);
        const float v = acc[tt][r];
        const float partner = swap_adjacent(v);
        const int n = min(tok0 + row, a.n_q - 1);
        const int f = n / a.tokens_per_frame;
        const int n_in = n - f * a.tokens_per_frame;
        const int hh = n_in / a.grid_w;
        const int pos = axis == 0 ? a.t_first + f : (axis == 1 ? hh : n_in - hh * a.grid_w);
        float sn, cs;
        sincosf((float)pos * omega, &sn, &cs);
        const float rot = odd ? partner * sn + v * cs : v * cs - partner * sn;
        ot[row * kOutLd + kDC + col] = f2bf(rot * a.qscale);
      }
    }
  } else {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 32 * tt + 8 * (r >> 2) + 4 * half + (r & 3);
        qn[row * kQnLd + 32 * wave + col] = f2bf(acc[tt][r]);
      }
    }
  }
  __syncthreads();

  // q_lat[64][192] = q_nope[64][96] @ W_K_up[h]^T: B[k = n][col = c] = W_K_up[h][c][n]
  const T* wku = static_cast<const T*>(a.w_k_up) + (size_t)h * kDC * kDNope;
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const int tile = wave + 4 * i;         // 0..11
    const int tt = tile / 6, ct = tile % 6;
    f32x16 q = f32x16{};
#pragma unroll
    for (int ks = 0; ks < kDNope / 16; ++ks) {
      const bf16x8 av = lds_row8(&qn[(32 * tt + (lane & 31)) * kQnLd + ks * 16 + 8 * half]);
      const uint4 braw = load8_bf16<T>(wku + (size_t)(32 * ct + (lane & 31)) * kDNope + ks * 16 + 8 * half);
      q = mfma32(av, __builtin_bit_cast(bf16x8, braw), q);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = 32 * tt + 8 * (r >> 2) + 4 * half + (r & 3);
      ot[row * kOutLd + 32 * ct + col] = f2bf(q[r] * a.qscale);
    }
  }
  __syncthreads();

  uint16_t* dst = a.qhat + (((size_t)b * a.n_heads + h) * a.n_q + tok0) * kRow;
#pragma unroll
  for (int i = 0; i < (kTok * kRow / 8 + kThreads - 1) / kThreads; ++i) {
    const int c = tid + i * kThreads;
    if (c < kTok * kRow / 8) {
      const int row = c / (kRow / 8), cc = c % (kRow / 8);
      if (tok0 + row < a.n_q)
        *reinterpret_cast<uint4*>(dst + (size_t)row * kRow + 8 * cc) =
            *reinterpret_cast<const uint4*>(&ot[row * kOutLd + 8 * cc]);
    }
  }
}

}  // namespace

hipError_t launch_qprologue(const QArgs& a, bool f32, hipStream_t s) {
  dim3 grid((a.n_q + kTok - 1) / kTok, a.n_heads, a.batch);
  if (f32) hipLaunchKernelGGL(qprologue_kernel<float>, grid, dim3(kThreads), 0, s, a);
  else hipLaunchKernelGGL(qprologue_kernel<bf16_t>, grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace vmla
