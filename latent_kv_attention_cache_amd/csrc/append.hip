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
// A skinny GEMM (N = 224, K = d_model) over all tokens of the chunk. One
// workgroup (7 waves) computes a TM-token x 224-column tile; wave w owns the
// 32-column block w (blocks 0-5: c from W_down, block 6: k_R from W_KR) for all
// TM tokens. The d_model contraction runs as a pipeline of 64-deep stages
// (kStages buffers fetched by LDS-DMA kStages-1 stages ahead, one barrier per
// stage); x, W_down and W_KR slices sit in separate LDS regions. All 7 waves
// issue a share of each stage's loads (the LDS-DMA issue rate grows with the
// number of issuing waves), spread between the MFMAs of the current stage, and
// each load costs only a scalar base update: the lane offsets are fixed.
//
// Tile height. Every workgroup streams all of W_down / W_KR (688 KB at
// d_model = 1536) from L2 next to its TM x d_model slice of x from HBM, so a
// tall tile amortises the weight stream, while a short tile spreads a small
// chunk over more compute units. The launcher picks TM in {32, ..., 160} from
// the token count (one workgroup per compute unit at a time, see below).
#include "device_common.h"
#include "kernels.h"
#include "staging.h"

namespace vmla {
namespace {

constexpr int kWaves = kRow / 32;      // 7: one per 32-column block
constexpr int kThreads = 64 * kWaves;
constexpr int kB1Elems = kStageK * kDC;          // W_down slice   (24 KB)
constexpr int kB2Elems = kStageK * kDRope;       // W_KR slice     (4 KB)
constexpr int kB1Loads = kB1Elems * 2 / 1024;    // 24
constexpr int kB2Loads = kB2Elems * 2 / 1024;    // 4

template <int TM>
struct Tile {
  static constexpr int kTB = TM / 32;                        // 32-token blocks per wave
  static constexpr int kAElems = TM * kStageK;               // x slice
  static constexpr int kALoads = kAElems * 2 / 1024;         // TM / 8
  static constexpr int kStageElems = kAElems + kB1Elems + kB2Elems;
  static constexpr int kStages = TM >= 96 ? 3 : 4;           // <= 144 KB of LDS
  static constexpr int kLoads = kALoads + kB1Loads + kB2Loads;
  // wave w issues loads w, w + 7, ...: the first kLoads % 7 waves issue one more
  static constexpr int kLoadsHi = (kLoads + kWaves - 1) / kWaves;
  static constexpr int kLoadsLo = kLoads / kWaves;
  static constexpr int kHiWaves = kLoads % kWaves;
  static_assert(TM % 32 == 0 && TM >= 32 && TM <= 160, "tile height");
  static_assert(kStages * kStageElems * 2 <= 160 * 1024, "LDS budget");
};

template <typename T, int TM>
__global__ __launch_bounds__(kThreads)
void append_kernel(AppendArgs a) {
  using Tl = Tile<TM>;
  __shared__ __attribute__((aligned(16))) bf16_t smem[Tl::kStages * Tl::kStageElems];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int b = blockIdx.y;
  const int tok0 = blockIdx.x * TM;
  const T* x = static_cast<const T*>(a.x) + (size_t)b * a.n_tok * a.d_model;
  const T* wd = static_cast<const T*>(a.w_down);
  const T* wr = static_cast<const T*>(a.w_kr);
  const int nst = a.d_model / kStageK;

  // Wave w issues loads n = w, w + 7, ... of every stage. For bf16 sources the
  // lane offsets of those loads are computed once; a stage only moves the
  // scalar source pointer and the LDS destination.
  uint32_t voff[Tl::kLoadsHi];
  if constexpr (std::is_same_v<T, bf16_t>) {
#pragma unroll
    for (int i = 0; i < Tl::kLoadsHi; ++i) {
      const int n = wave + kWaves * i;
      if (n < Tl::kALoads) voff[i] = stage_a_voff(a.d_model, tok0, a.n_tok, n, lane);
      else if (n < Tl::kALoads + kB1Loads) voff[i] = stage_b_voff<kDC>(kDC, n - Tl::kALoads, lane);
      else voff[i] = stage_b_voff<kDRope>(kDRope, n - Tl::kALoads - kB1Loads, lane);
    }
  }
  auto issue = [&](int s, int i0 = 0, int i1 = Tl::kLoadsHi) {   // this wave's loads i0 <= i < i1 of stage s
    bf16_t* st = smem + (s % Tl::kStages) * Tl::kStageElems;
    const int k0 = s * kStageK;
#pragma unroll
    for (int i = 0; i < Tl::kLoadsHi; ++i) {
      const int n = wave + kWaves * i;
      if (i < i0 || i >= i1 || n >= Tl::kLoads) continue;
      if constexpr (std::is_same_v<T, bf16_t>) {
        if (n < Tl::kALoads) dma16_lds(x + k0, voff[i], lds_u32(st + 512 * n));
        else if (n < Tl::kALoads + kB1Loads) dma16_lds(wd + (size_t)k0 * kDC, voff[i], lds_u32(st + 512 * n));
        else dma16_lds(wr + (size_t)k0 * kDRope, voff[i], lds_u32(st + 512 * n));
      } else {
        if (n < Tl::kALoads) stage_a_load<T>(st, x, a.d_model, tok0, a.n_tok, k0, n, lane);
        else if (n < Tl::kALoads + kB1Loads)
          stage_b_load<T, kDC>(st + Tl::kAElems, wd, kDC, 0, k0, n - Tl::kALoads, lane);
        else
          stage_b_load<T, kDRope>(st + Tl::kAElems + kB1Elems, wr, kDRope, 0, k0,
                                  n - Tl::kALoads - kB1Loads, lane);
      }
    }
  };
  auto wait = [&](int stages) {      // own loads of all but the newest `stages` stages landed
    if constexpr (Tl::kHiWaves == 0) {
      wait_stages<Tl::kLoadsLo>(stages);
    } else {
      if (wave < Tl::kHiWaves) wait_stages<Tl::kLoadsHi>(stages);
      else wait_stages<Tl::kLoadsLo>(stages);
    }
  };

  for (int s = 0; s < Tl::kStages - 1 && s < nst; ++s) issue(s);

  f32x16 acc[Tl::kTB];
#pragma unroll
  for (int tt = 0; tt < Tl::kTB; ++tt) acc[tt] = f32x16{};
  for (int s = 0; s < nst; ++s) {
    wait(min(Tl::kStages - 2, nst - 1 - s));                   // stage s has landed
    __syncthreads();
    const bool more = s + Tl::kStages - 1 < nst;               // loads into the buffer of stage s-1
    const bf16_t* A = smem + (s % Tl::kStages) * Tl::kStageElems;
#pragma unroll
    for (int ks = 0; ks < kStageK / 16; ++ks) {
      bf16x8 bv;
      if (wave < kWaves - 1) bv = b_frag<kDC>(A + Tl::kAElems, ks, 32 * wave, lane);
      else bv = b_frag<kDRope>(A + Tl::kAElems + kB1Elems, ks, 0, lane);
#pragma unroll
      for (int tt = 0; tt < Tl::kTB; ++tt) {
        const bf16x8 av = a_frag(A, 32 * tt + (lane & 31), ks, half);
        acc[tt] = mfma32(av, bv, acc[tt]);
      }
      // the wave's next-stage loads, spread over the k-steps so that their
      // issue overlaps the MFMAs already in flight
      if (more) issue(s + Tl::kStages - 1, 2 * ks, ks == 3 ? Tl::kLoadsHi : 2 * ks + 2);
    }
  }

  // Epilogue. Register r of lane l holds token row 32 tt + 8(r/4) + 4 half + r%4
  // and column 32 wave + l%32; wave 6 holds the k_R columns.
  const int col = lane & 31;
  T* cache = static_cast<T*>(a.cache) + (size_t)b * a.window_frames * a.tokens_per_frame * kRow;
  if constexpr (std::is_same_v<T, bf16_t>) {
    // The tile is assembled in LDS: c as bf16 rows of 224 + 8, k_R unrotated in
    // fp32; per row the ring slot and (t, h, w) are computed once. The store
    // pass rotates k_R (each (row, pair) once, spread over all threads) and
    // writes whole 448-byte cache rows as 16-byte stores.
    constexpr int kOutLd = kRow + 8;
    constexpr int kKrLd = kDRope + 1;
    static_assert(TM * kOutLd * 2 + TM * kKrLd * 4 + TM * 16 <= Tl::kStages * Tl::kStageElems * 2,
                  "epilogue tile fits");
    __syncthreads();                            // all stage reads done; the buffers are free
    bf16_t* ot = smem;                                                     // [TM][kOutLd]
    float* kr = reinterpret_cast<float*>(smem + TM * kOutLd);             // [TM][kKrLd]
    int* rowinfo = reinterpret_cast<int*>(kr + TM * kKrLd);               // [TM][4]: slot, t, h, w
    for (int row = tid; row < TM; row += kThreads) {
      const int n = tok0 + row;
      int n_in, ww, tw;
      const int f = div_small(min(n, a.n_tok - 1), a.tokens_per_frame, a.inv_tokens_per_frame, &n_in);
      const int hh = div_small(n_in, a.grid_w, a.inv_grid_w, &ww);
      div_small(a.t_first + f, a.window_frames, a.inv_window_frames, &tw);
      rowinfo[4 * row] = n < a.n_tok ? tw * a.tokens_per_frame + n_in : -1;
      rowinfo[4 * row + 1] = a.t_first + f;
      rowinfo[4 * row + 2] = hh;
      rowinfo[4 * row + 3] = ww;
    }
#pragma unroll
    for (int tt = 0; tt < Tl::kTB; ++tt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 32 * tt + 8 * (r >> 2) + 4 * half + (r & 3);
        if (wave < kWaves - 1) ot[row * kOutLd + 32 * wave + col] = f2bf(acc[tt][r]);
        else kr[row * kKrLd + col] = acc[tt][r];
      }
    }
    __syncthreads();
    for (int c = tid; c < TM * (kRow / 8); c += kThreads) {
      const int row = c / (kRow / 8), cc = c - row * (kRow / 8);
      const int slot = rowinfo[4 * row];
      if (slot < 0) continue;
      uint4 v;
      if (cc < kDC / 8) {
        v = *reinterpret_cast<const uint4*>(&ot[row * kOutLd + 8 * cc]);
      } else {                                  // k_R pairs 4 j .. 4 j + 3
        const int j = cc - kDC / 8;
        uint32_t w[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int pr = 4 * j + q;
          const float a0 = kr[row * kKrLd + 2 * pr], a1 = kr[row * kKrLd + 2 * pr + 1];
          float sn, cs;
          sincos_rev(rowinfo[4 * row + 1 + a.rope.axis[pr]], a.rope.rev[pr], &sn, &cs);
          // pair (a0, a1) -> (a0 cos - a1 sin, a0 sin + a1 cos)
          w[q] = pack2(a0 * cs - a1 * sn, a0 * sn + a1 * cs);
        }
        v = uint4{w[0], w[1], w[2], w[3]};
      }
      *reinterpret_cast<uint4*>(cache + (size_t)slot * kRow + 8 * cc) = v;
    }
  } else {
    // fp32 storage keeps the fp32 result: per-element stores, RoPE in wave 6
    const int pair = col >> 1;
    const bool odd = col & 1;
    const bool rope = wave == kWaves - 1;
    const float rev = a.rope.rev[pair];
    const int axis = a.rope.axis[pair];
#pragma unroll
    for (int tt = 0; tt < Tl::kTB; ++tt) {
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
          v = odd ? partner * sn + v * cs : v * cs - partner * sn;
        }
        div_small(t, a.window_frames, a.inv_window_frames, &tw);
        cache[((size_t)tw * a.tokens_per_frame + n_in) * kRow + 32 * wave + col] = v;
      }
    }
  }
}

template <typename T, int TM>
void launch_tm(const AppendArgs& a, hipStream_t s) {
  dim3 grid((a.n_tok + TM - 1) / TM, a.batch);
  hipLaunchKernelGGL((append_kernel<T, TM>), grid, dim3(kThreads), 0, s, a);
}

template <typename T>
void launch_t(const AppendArgs& a, int tm, hipStream_t s) {
  switch (tm) {
    case 160: launch_tm<T, 160>(a, s); break;
    case 128: launch_tm<T, 128>(a, s); break;
    case 96: launch_tm<T, 96>(a, s); break;
    case 64: launch_tm<T, 64>(a, s); break;
    default: launch_tm<T, 32>(a, s); break;
  }
}

}  // namespace

// Tile height: one workgroup fits a compute unit (LDS), so a launch runs in
// ceil(workgroups / CUs) rounds of one tile each; a tile costs about TM + 32
// token-rows of work (the weight stream is the fixed part). Pick the TM with
// the least rounds x (TM + 32).
int append_tile_rows(int n_tok, int batch, int cus) {
  int best = 32;
  int64_t best_cost = -1;
  for (int tm : {160, 128, 96, 64, 32}) {
    const int64_t wgs = (int64_t)((n_tok + tm - 1) / tm) * batch;
    const int64_t rounds = (wgs + cus - 1) / cus;
    const int64_t cost = rounds * (tm + 32);
    if (best_cost < 0 || cost < best_cost) { best_cost = cost; best = tm; }
  }
  return best;
}

hipError_t launch_append(const AppendArgs& a, bool f32, hipStream_t s) {
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const int tm = append_tile_rows(a.n_tok, a.batch, cus > 0 ? cus : 1);
  if (f32) launch_t<float>(a, tm, s);
  else launch_t<bf16_t>(a, tm, s);
  return hipGetLastError();
}

}  // namespace vmla
