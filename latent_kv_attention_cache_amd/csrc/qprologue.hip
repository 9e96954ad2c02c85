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
// One workgroup (4 waves) handles 64 tokens of one head (XCD-aware order, see
// the kernel). The d_model
// contraction runs as a pipeline of 64-deep stages (kStages buffers, fetched
// by LDS-DMA kStages-1 stages ahead, one barrier per stage). Wave w computes
// output columns [32w, 32w+32) of q_h for all 64 tokens; wave 3 therefore holds
// the rope channels. The absorption GEMM then splits its 2 x 6 output blocks
// three per wave, and the [64 x 224] result is assembled in LDS and written
// with 16-byte row stores.
#include "device_common.h"
#include "kernels.h"
#include "staging.h"

namespace vmla {
namespace {

constexpr int kTok = 64;
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kStages = 3;
constexpr int kAElems = kTok * kStageK;                 // 4096
constexpr int kBElems = kStageK * kDHead;               // 8192
constexpr int kStageElems = kAElems + kBElems;
constexpr int kALoads = kAElems * 2 / 1024;             // 8
constexpr int kBLoads = kBElems * 2 / 1024;             // 16
constexpr int kLoadsPerWave = (kALoads + kBLoads) / kWaves;   // 6
constexpr int kQnLd = kDNope + 8;      // q_nope staging row
constexpr int kOutLd = kRow + 8;       // output tile row
constexpr int kEpiElems = kTok * kQnLd + kTok * kOutLd;
constexpr int kSmemElems = kStages * kStageElems > kEpiElems ? kStages * kStageElems : kEpiElems;
static_assert((kALoads + kBLoads) % kWaves == 0, "stage loads must split evenly");

template <typename T>
__global__ __launch_bounds__(kThreads)
void qprologue_kernel(QArgs a) {
  __shared__ __attribute__((aligned(16))) bf16_t smem[kSmemElems];
  bf16_t* qn = smem;                       // [kTok][kQnLd]   (after the K loop)
  bf16_t* ot = smem + kTok * kQnLd;        // [kTok][kOutLd]

  // Workgroups are dispatched round-robin over the 8 XCDs; id = 8 (H q + h) + x8
  // keeps all heads of token block 8 q + x8 on XCD x8, so that block's x rows
  // are fetched into that XCD's L2 once and shared by its heads.
  const int ntb = (a.n_q + kTok - 1) / kTok;
  const int x8 = blockIdx.x & 7;
  const int rest = blockIdx.x >> 3;
  const int h = rest % a.n_heads;
  const int tb = 8 * (rest / a.n_heads) + x8;
  if (tb >= ntb) return;                   // whole workgroup: no barrier is skipped
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int b = blockIdx.z;
  const int tok0 = tb * kTok;
  const int wq_ld = a.n_heads * kDHead;
  const T* x = static_cast<const T*>(a.x) + (size_t)b * a.n_q * a.d_model;
  const T* wq = static_cast<const T*>(a.w_q) + (size_t)h * kDHead;
  const int nst = a.d_model / kStageK;

  // Wave w issues loads n = w, w + 4, ... of every stage. For bf16 sources the
  // lane offsets of those loads are computed once; a stage only moves the
  // scalar source pointer and the LDS destination.
  uint32_t voff[kLoadsPerWave];
  if constexpr (std::is_same_v<T, bf16_t>) {
#pragma unroll
    for (int i = 0; i < kLoadsPerWave; ++i) {
      const int n = wave + kWaves * i;
      voff[i] = n < kALoads ? stage_a_voff(a.d_model, tok0, a.n_q, n, lane)
                            : stage_b_voff<kDHead>(wq_ld, n - kALoads, lane);
    }
  }
  auto issue = [&](int s, int i0 = 0, int i1 = kLoadsPerWave) {   // this wave's loads i0 <= i < i1
    bf16_t* st = smem + (s % kStages) * kStageElems;
    const int k0 = s * kStageK;
#pragma unroll
    for (int i = 0; i < kLoadsPerWave; ++i) {
      if (i < i0 || i >= i1) continue;
      const int n = wave + kWaves * i;
      if constexpr (std::is_same_v<T, bf16_t>) {
        if (n < kALoads) dma16_lds(x + k0, voff[i], lds_u32(st + 512 * n));
        else dma16_lds(wq + (size_t)k0 * wq_ld, voff[i], lds_u32(st + 512 * n));
      } else {
        if (n < kALoads) stage_a_load<T>(st, x, a.d_model, tok0, a.n_q, k0, n, lane);
        else stage_b_load<T, kDHead>(st + kAElems, wq, wq_ld, 0, k0, n - kALoads, lane);
      }
    }
  };

  for (int s = 0; s < kStages - 1 && s < nst; ++s) issue(s);

  f32x16 acc[2] = {f32x16{}, f32x16{}};
  for (int s = 0; s < nst; ++s) {
    wait_stages<kLoadsPerWave>(min(kStages - 2, nst - 1 - s));   // stage s has landed
    __syncthreads();
    const bool more = s + kStages - 1 < nst;                      // loads into the buffer of stage s-1
    const bf16_t* A = smem + (s % kStages) * kStageElems;
    const bf16_t* B = A + kAElems;
#pragma unroll
    for (int ks = 0; ks < kStageK / 16; ++ks) {
      const bf16x8 bv = b_frag<kDHead>(B, ks, 32 * wave, lane);
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const bf16x8 av = a_frag(A, 32 * tt + (lane & 31), ks, half);
        acc[tt] = mfma32(av, bv, acc[tt]);
      }
      // the wave's next-stage loads, spread over the k-steps so that their
      // issue overlaps the MFMAs already in flight
      if (more) issue(s + kStages - 1, (kLoadsPerWave * ks) / 4, (kLoadsPerWave * (ks + 1)) / 4);
    }
  }
  __syncthreads();

  // Register r of lane l: token row 32*tt + 8(r/4) + 4*half + r%4, column 32*wave + l%32.
  const int col = lane & 31;
  if (wave == 3) {
    const int pair = col >> 1;
    const bool odd = col & 1;
    const float rev = a.rope.rev[pair];
    const int axis = a.rope.axis[pair];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 32 * tt + 8 * (r >> 2) + 4 * half + (r & 3);
        const float v = acc[tt][r];
        const float partner = swap_adjacent(v);
        const int n = min(tok0 + row, a.n_q - 1);
        int n_in, ww;
        const int f = div_small(n, a.tokens_per_frame, a.inv_tokens_per_frame, &n_in);
        const int hh = div_small(n_in, a.grid_w, a.inv_grid_w, &ww);
        const int pos = axis == 0 ? a.t_first + f : (axis == 1 ? hh : ww);
        float sn, cs;
        sincos_rev(pos, rev, &sn, &cs);
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
  const int ntb = (a.n_q + kTok - 1) / kTok;
  dim3 grid(8 * a.n_heads * ((ntb + 7) / 8), 1, a.batch);
  if (f32) hipLaunchKernelGGL(qprologue_kernel<float>, grid, dim3(kThreads), 0, s, a);
  else hipLaunchKernelGGL(qprologue_kernel<bf16_t>, grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace vmla
