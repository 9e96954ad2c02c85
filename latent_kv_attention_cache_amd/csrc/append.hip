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
// With a cache that keeps k_R before RoPE (read-time rotation, App. D.5) the
// k_R columns are stored as computed; with a sink frame, frame 0 keeps slots
// [0, T) and the ring of the most recent frames follows it.
//
// A skinny GEMM: M = batch x tokens rows (the batch elements are contiguous in
// x, so they form one row range), N = 224, K = d_model. The M rows are split
// into one contiguous range per workgroup, at most 160 rows, as evenly as the
// device's compute units allow (a workgroup fills one compute unit's LDS).
// Every workgroup streams all of W_down / W_KR (688 KB at d_model = 1536) from
// L2 next to its slice of x from HBM.
//
// Four waves, one per SIMD, split the tile 2 x 2: wave (rh, ch) owns row half
// rh (up to 5 blocks of 16 rows) and column half ch (7 blocks of 16 columns;
// half 1 holds c columns 112-191 and the 32 k_R columns), with
// v_mfma_f32_16x16x32_bf16 computing the transposed block out^T = W^T x^T, so
// that a lane ends up with four consecutive columns of one token row. Per
// 32-deep step a wave reads 5 x and 7 W fragments from LDS for 35 MFMAs, so
// LDS traffic per MFMA is low and the four SIMDs carry equal work.
//
// The d_model contraction runs as a pipeline of 64-deep stages (3-4 buffers,
// fetched by 16-byte LDS-DMA loads kStages-1 stages ahead, one barrier per
// stage); each wave issues its share of the next stage's loads between its
// MFMAs, and each load costs a scalar base update only (fixed lane offsets).
// LDS layouts of a stage:
//   x tile: row-major, 64 bf16 (8 chunks of 16 B) per row, chunk c of row r at
//           position c ^ swz_a(r): the row-wise operand reads of 16 consecutive
//           rows hit distinct banks;
//   W tiles: W_down [64][192] and W_KR [64][32], row-major, so that a DMA load
//           reads 1 KB of contiguous weight. The 16-byte chunks of row k are
//           XOR-permuted, chunk c at position c ^ 2 t(k) with
//           t(k) = bit1(k) | bit3(k) << 1 for W_down and t(k) = bit3(k) for
//           W_KR: a transposed B read of 32 lanes (rows k0 .. k0+3 and
//           k0+8 .. k0+11, two chunks each) then covers all 64 banks once.
#include <algorithm>

#include "device_common.h"
#include "kernels.h"
#include "staging.h"

namespace vmla {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxRows = 160;

// Weight-tile shape for a content width DC (192 by default; 64 and 128 for
// the latent-budget sweep) and a positional width DR (32 by default; 16, 64,
// 96 for the NoPE/RoPE split variants): a row of [W_down | W_KR] is DC + DR
// wide. Column half 0 takes the first kColBlocks 16-wide blocks, half 1 the
// other kColBlocks1 (one fewer when the row has an odd number of blocks).
template <int DC, int DR>
struct WShape {
  static constexpr int kRow = DC + DR;
  static constexpr int kWChunks = kRow / 8;               // 28 chunks per weight row at DC 192
  static constexpr int kWdElems = kStageK * DC;           // W_down tile
  static constexpr int kWElems = kStageK * kRow;          // W_down + W_KR tiles
  static constexpr int kWdLoads = kWdElems * 2 / 1024;    // 24 wave-wide loads at DC 192
  static constexpr int kColBlocks = (kRow / 16 + 1) / 2;  // 16-wide column blocks of half 0 (7)
  static constexpr int kColBlocks1 = kRow / 16 - kColBlocks;
  static constexpr int kWPerWave = (kWChunks + 3) / 4;    // W loads per wave (the last may repeat)
  static_assert(kRow % 16 == 0 && 16 * kColBlocks <= DC, "half 0 holds content columns only");
};

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// chunk permutation masks of W_down / W_KR row k (an involution per row)
__device__ __forceinline__ int swz_wd(int k) { return 2 * (((k >> 1) & 1) | (((k >> 3) & 1) << 1)); }
template <int DR>   // W_KR rows of DR / 8 chunks: flip bit 1 (4, 8 or 12 chunks), none for 2
__device__ __forceinline__ int swz_wr(int k) { return DR == 16 ? 0 : 2 * ((k >> 3) & 1); }

template <typename T, int NRB, int DC, int DR>
struct Tile {
  static constexpr int kRow = WShape<DC, DR>::kRow;
  static constexpr int kWChunks = WShape<DC, DR>::kWChunks;
  static constexpr int kWElems = WShape<DC, DR>::kWElems;
  static constexpr int kRows = 32 * NRB;                   // rows of a workgroup at most
  static constexpr int kXElems = kRows * kStageK;
  static constexpr int kXLoads = kXElems * 2 / 1024;       // 4 NRB
  static constexpr int kStageElems = kXElems + kWElems;
  static constexpr int kStages = 4 * kStageElems * 2 <= 160 * 1024 ? 4
                                 : (3 * kStageElems * 2 <= 160 * 1024 ? 3 : 2);
  static constexpr int kLoadsPerWave = NRB + WShape<DC, DR>::kWPerWave;   // NRB x loads + 7 W chunks
  // epilogue: bf16 storage keeps c as bf16 rows of 224 + 8 and k_R in fp32;
  // fp32 storage keeps all 224 columns in fp32 rows of 228; 5 ints of row info
  static constexpr int kOutLd = std::is_same_v<T, bf16_t> ? kRow + 8 : kRow + 4;
  static constexpr int kKrLd = DR + 4;
  static constexpr int kEpiBytes = std::is_same_v<T, bf16_t>
      ? kRows * (kOutLd * 2 + kKrLd * 4 + 20) : kRows * (kOutLd * 4 + 20);
  static constexpr int kSmemElems = std::max(kStages * kStageElems, (kEpiBytes + 1) / 2);
  static_assert(NRB >= 1 && NRB <= 5, "row blocks per wave");
  static_assert(kXLoads == kWaves * NRB, "load split");
  static_assert(kSmemElems * 2 <= 160 * 1024, "LDS budget");
};

template <typename T, int NRB, int DC, int DR>
__global__ __launch_bounds__(kThreads)
void append_kernel(AppendArgs a) {
  using Tl = Tile<T, NRB, DC, DR>;
  constexpr int kDC = DC;
  constexpr int kDRope = DR;
  constexpr int kRow = WShape<DC, DR>::kRow;
  constexpr int kWdElems = WShape<DC, DR>::kWdElems;
  constexpr int kWdLoads = WShape<DC, DR>::kWdLoads;
  constexpr int kColBlocks = WShape<DC, DR>::kColBlocks;
  constexpr int kColBlocks1 = WShape<DC, DR>::kColBlocks1;
  constexpr int kWPerWave = WShape<DC, DR>::kWPerWave;
  constexpr int kWChunks = WShape<DC, DR>::kWChunks;
  // W load index of load i >= NRB of wave wv (a repeat of the last chunk when
  // the chunks do not split evenly over the four waves)
  auto w_load = [&](int wv_, int i) {
    const int n = kWPerWave * wv_ + (i - NRB);
    if constexpr (kWChunks % kWaves == 0) return n;
    else return min(n, kWChunks - 1);
  };
  constexpr bool kBf16 = std::is_same_v<T, bf16_t>;
  __shared__ __attribute__((aligned(16))) bf16_t smem[Tl::kSmemElems];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int g = lane >> 4;                  // 16-lane group: k sub-range of an MFMA operand
  const int rh = wv >> 1, ch = wv & 1;      // wave-uniform

  // This workgroup's rows [m0, m0 + rows) of the flattened batch x tokens.
  const int64_t M = (int64_t)a.batch * a.n_tok;
  const int64_t m0 = (int64_t)blockIdx.x * M / gridDim.x;
  const int rows = (int)((int64_t)(blockIdx.x + 1) * M / gridDim.x - m0);
  const int nb = (rows + 15) / 16;          // 16-row blocks of the tile
  const int nb0 = (nb + 1) / 2;             // blocks of row half 0 (<= NRB)
  const int rbase = rh ? 16 * nb0 : 0;

  const T* xw = static_cast<const T*>(a.x) + m0 * a.d_model;
  const T* wd = static_cast<const T*>(a.w_down);
  const T* wr = static_cast<const T*>(a.w_kr);
  const int nst = a.d_model / kStageK;

  // Loads of a stage: x loads n = NRB wv + i (i < NRB), W chunks c = 7 wv + j
  // (j < 7). For bf16 sources the lane offsets are fixed; a stage moves only
  // the scalar source pointers and the LDS destinations.
  uint32_t voff[Tl::kLoadsPerWave];
  if constexpr (kBf16) {
#pragma unroll
    for (int i = 0; i < Tl::kLoadsPerWave; ++i) {
      if (i < NRB) {
        voff[i] = stage_a_voff(a.d_model, 0, rows, NRB * wv + i, lane);
      } else {
        // W load n: 1 KB of the W_down tile (n < 24) or of the W_KR tile; LDS
        // slot q holds chunk position q % rowchunks of row q / rowchunks
        const int n = w_load(wv, i);
        if (n < kWdLoads) {
          const int q = 64 * n + lane, k = q / (kDC / 8), cp = q - k * (kDC / 8);
          voff[i] = (uint32_t)(k * (kDC / 8) + (cp ^ swz_wd(k))) * 16u;
        } else {
          const int q = 64 * (n - kWdLoads) + lane, k = q / (kDRope / 8), cp = q - k * (kDRope / 8);
          voff[i] = (uint32_t)(k * (kDRope / 8) + (cp ^ swz_wr<DR>(k))) * 16u;
        }
      }
    }
  }
  // this wave's loads i0 <= i < i1: data of stage sd into the buffer of stage sb
  auto issue = [&](int sb, int sd, int i0, int i1) {
    bf16_t* st = smem + (sb % Tl::kStages) * Tl::kStageElems;
    const int k0 = sd * kStageK;
#pragma unroll
    for (int i = 0; i < Tl::kLoadsPerWave; ++i) {
      if (i < i0 || i >= i1) continue;
      if (i < NRB) {
        const int n = NRB * wv + i;
        if constexpr (kBf16) dma16_lds(xw + k0, voff[i], lds_u32(st + 512 * n));
        else stage_a_load<T>(st, xw, a.d_model, 0, rows, k0, n, lane);
      } else {
        const int n = w_load(wv, i);
        bf16_t* dst = st + Tl::kXElems + 512 * n;
        if constexpr (kBf16) {
          const bf16_t* src = n < kWdLoads ? wd + (size_t)k0 * kDC : wr + (size_t)k0 * kDRope;
          dma16_lds(src, voff[i], lds_u32(dst));
        } else {
          const T* src;
          if (n < kWdLoads) {
            const int q = 64 * n + lane, k = q / (kDC / 8), cp = q - k * (kDC / 8);
            src = wd + (size_t)(k0 + k) * kDC + 8 * (cp ^ swz_wd(k));
          } else {
            const int q = 64 * (n - kWdLoads) + lane, k = q / (kDRope / 8), cp = q - k * (kDRope / 8);
            src = wr + (size_t)(k0 + k) * kDRope + 8 * (cp ^ swz_wr<DR>(k));
          }
          *reinterpret_cast<uint4*>(dst + 8 * lane) = load8_bf16<T>(src);
        }
      }
    }
  };

  // Per-lane operand offsets (elements, relative to a stage's tile).
  // A (x, row-major swizzled): lane = row (lane % 16) of block rb, chunk 4 kk + g.
  int a_off[NRB][2];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    const int row = rbase + 16 * rb + (lane & 15);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) a_off[rb][kk] = 64 * row + 8 * ((4 * kk + g) ^ swz_a(row));
  }
  // B (W) by ds_read_b64_tr_b16: lane j of 16-lane group g points at k row
  // 32 kk + 8 g + j/4 (+4 for the upper half of the fragment) and columns
  // col0 + 4 (j%4) .. +3, i.e. logical chunk col0/8 + (j%4)/2, element 4 (j%2).
  // Bits 1 and 3 of that row (the swizzle bits) depend on the lane only, so one
  // offset per column block serves every (kk, half).
  const int j = lane & 15;
  int b_off[kColBlocks];
  {
    const int k = 8 * g + (j >> 2);
#pragma unroll
    for (int cb = 0; cb < kColBlocks; ++cb) {
      const int gcb = kColBlocks * ch + cb;            // 16-column block of [c | k_R]
      const int c = (gcb < kDC / 16 ? 2 * gcb : 2 * (gcb - kDC / 16)) + ((j & 3) >> 1);
      b_off[cb] = gcb < kDC / 16 ? k * kDC + 8 * (c ^ swz_wd(k)) + 4 * (j & 1)
                                 : kWdElems + k * kDRope + 8 * (c ^ swz_wr<DR>(k)) + 4 * (j & 1);
    }
  }

  for (int s = 0; s < Tl::kStages - 1 && s < nst; ++s) issue(s, s, 0, Tl::kLoadsPerWave);

  f32x4 acc[NRB][kColBlocks];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
    for (int cb = 0; cb < kColBlocks; ++cb) acc[rb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};

  constexpr int kL = Tl::kLoadsPerWave;
  // Stage s: two 32-deep steps of NRB x 7 MFMAs. The A fragment of the next
  // row block and the B fragments of the second step are read while the
  // current MFMAs run, and the wave's share of the loads of stage
  // s + kStages - 1 goes out after every row block. Past the last stage those
  // loads repeat the last stage's (cached) data into the buffer of stage s-1,
  // which is not read again, so the stage body has no branch.
  // Every iteration issues one stage, so min(kStages - 2, nst - 1) stages are in
  // flight behind stage s at the top of each iteration.
  const int behind = min(Tl::kStages - 2, nst - 1);
  for (int s = 0; s < nst; ++s) {
    wait_stages<kL>(behind);                                     // stage s has landed
    __syncthreads();
    const int sn = min(s + Tl::kStages - 1, nst - 1);           // source stage of the loads
    const bf16_t* X = smem + (s % Tl::kStages) * Tl::kStageElems;
    const bf16_t* W = X + Tl::kXElems;
    auto read_b = [&](int kk, bf16x8* bf) {
#pragma unroll
      for (int cb = 0; cb < kColBlocks; ++cb) {
        if (cb >= kColBlocks1 && ch != 0) {      // half 1 may hold one block fewer
          bf[cb] = bf16x8{};
          continue;
        }
        const bf16_t* p = W + b_off[cb] + 32 * kk * (cb + kColBlocks * ch < kDC / 16 ? kDC : kDRope);
        const int up = 4 * (cb + kColBlocks * ch < kDC / 16 ? kDC : kDRope);
        const bf16x4 lo = lds_tr4(p);
        const bf16x4 hi = lds_tr4(p + up);
        bf[cb] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
    };
    bf16x8 b0[kColBlocks], b1[kColBlocks];
    read_b(0, b0);
    bf16x8 av = lds_row8(X + a_off[0][0]);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        const int q = kk * NRB + rb;
        bf16x8 an = av;
        if (q + 1 < 2 * NRB) an = lds_row8(X + a_off[(q + 1) % NRB][(q + 1) / NRB]);
        if (kk == 0 && rb == NRB - 1) read_b(1, b1);
        issue(s + Tl::kStages - 1, sn, q * kL / (2 * NRB), (q + 1) * kL / (2 * NRB));
#pragma unroll
        for (int cb = 0; cb < kColBlocks; ++cb)
          if (cb < kColBlocks1 || ch == 0)        // half 1 may hold one block fewer
            acc[rb][cb] = mfma16(kk == 0 ? b0[cb] : b1[cb], av, acc[rb][cb]);
        av = an;
      }
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");    // the trailing loads have landed

  // ---- epilogue. Register r of acc[rb][cb] in lane l: token row
  // rbase + 16 rb + l%16, column 112 ch + 16 cb + 4 g + r. Per row the batch element, the ring slot and
  // (t, h, w) are computed once; the store pass rotates each (row, k_R pair)
  // once, spread over all threads, and writes whole cache rows in 16-byte stores.
  __syncthreads();                          // all stage reads done; the buffers are free
  constexpr int kOutLd = Tl::kOutLd;
  constexpr int kKrLd = Tl::kKrLd;
  using OutT = std::conditional_t<kBf16, bf16_t, float>;
  OutT* ot = reinterpret_cast<OutT*>(smem);                                 // [kRows][kOutLd]
  float* kr = reinterpret_cast<float*>(ot + Tl::kRows * kOutLd);            // bf16: [kRows][kKrLd]
  int* ri = kBf16 ? reinterpret_cast<int*>(kr + Tl::kRows * kKrLd)
                  : reinterpret_cast<int*>(ot + Tl::kRows * kOutLd);        // [kRows][5]
  const int64_t cache_rows = ((int64_t)a.sink_frames + a.window_frames) * a.tokens_per_frame;
  for (int row = tid; row < rows; row += kThreads) {
    const int64_t m = m0 + row;
    const int bb = (int)(m / a.n_tok);
    const int n = (int)(m - (int64_t)bb * a.n_tok);
    int n_in, ww, tw;
    const int f = div_small(n, a.tokens_per_frame, a.inv_tokens_per_frame, &n_in);
    const int hh = div_small(n_in, a.grid_w, a.inv_grid_w, &ww);
    const int t = a.t_first + f;
    if (t < a.sink_frames) {                // the sink frame keeps slots [0, T)
      tw = t;
    } else {                                // ring of the most recent frames after it
      div_small(t - a.sink_frames, a.window_frames, a.inv_window_frames, &tw);
      tw += a.sink_frames;
    }
    ri[5 * row] = bb;
    ri[5 * row + 1] = tw * a.tokens_per_frame + n_in;
    ri[5 * row + 2] = a.t_first + f;
    ri[5 * row + 3] = hh;
    ri[5 * row + 4] = ww;
  }
  {
    const int row0 = rbase + (lane & 15);
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const int row = row0 + 16 * rb;
#pragma unroll
      for (int cb = 0; cb < kColBlocks; ++cb) {
        if (cb >= kColBlocks1 && ch != 0) continue;   // half 1 may hold one block fewer
        const int col = 16 * kColBlocks * ch + 16 * cb + 4 * g;
        const f32x4 v = acc[rb][cb];
        if constexpr (kBf16) {
          if (ch == 0 || cb < kDC / 16 - kColBlocks)   // c columns (half 1 ends with k_R)
            *reinterpret_cast<uint2*>(&ot[row * kOutLd + col]) = uint2{pack2(v[0], v[1]), pack2(v[2], v[3])};
          else
            *reinterpret_cast<f32x4*>(&kr[row * kKrLd + col - kDC]) = v;
        } else {
          *reinterpret_cast<f32x4*>(&ot[row * kOutLd + col]) = v;
        }
      }
    }
  }
  __syncthreads();
  T* cache = static_cast<T*>(a.cache);
  constexpr int kPer = 16 / sizeof(T);      // elements per 16-byte store
  constexpr int kChunksRow = kRow / kPer;
  constexpr int kCChunks = kDC / kPer;
  for (int c = tid; c < rows * kChunksRow; c += kThreads) {
    const int row = c / kChunksRow, cc = c - row * kChunksRow;
    T* dst = cache + ((size_t)ri[5 * row] * cache_rows + ri[5 * row + 1]) * kRow + kPer * cc;
    uint4 v;
    if (cc < kCChunks) {
      v = *reinterpret_cast<const uint4*>(&ot[row * kOutLd + kPer * cc]);
    } else {                                // k_R pairs kPer/2 (cc - kCChunks) ...
      const int p0 = kPer / 2 * (cc - kCChunks);
      const float* src = kBf16 ? kr + row * kKrLd + kPer * (cc - kCChunks)
                               : reinterpret_cast<const float*>(ot) + row * kOutLd + kPer * cc;
      float o[kPer];
#pragma unroll
      for (int q = 0; q < kPer / 2; ++q) {
        const int pr = p0 + q;
        const float a0 = src[2 * q], a1 = src[2 * q + 1];
        float sn = 0.f, cs = 1.f;           // keys kept before RoPE: stored as computed
        if (!a.rope_at_read) sincos_rev(ri[5 * row + 2 + a.rope.axis[pr]], a.rope.rev_lo[pr], a.rope.rev_hi[pr], &sn, &cs);
        // pair (a0, a1) -> (a0 cos - a1 sin, a0 sin + a1 cos)
        o[2 * q] = a0 * cs - a1 * sn;
        o[2 * q + 1] = a0 * sn + a1 * cs;
      }
      if constexpr (kBf16) {
        v = uint4{pack2(o[0], o[1]), pack2(o[2], o[3]), pack2(o[4], o[5]), pack2(o[6], o[7])};
      } else {
        v = uint4{__float_as_uint(o[0]), __float_as_uint(o[1]), __float_as_uint(o[2]),
                  __float_as_uint(o[3])};
      }
    }
    *reinterpret_cast<uint4*>(dst) = v;
  }
}

template <typename T, int DC, int DR>
void launch_t(const AppendArgs& a, int groups, int nrb, hipStream_t s) {
  const dim3 grid(groups), block(kThreads);
  switch (nrb) {
    case 5: hipLaunchKernelGGL((append_kernel<T, 5, DC, DR>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((append_kernel<T, 4, DC, DR>), grid, block, 0, s, a); break;
    case 3: hipLaunchKernelGGL((append_kernel<T, 3, DC, DR>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((append_kernel<T, 2, DC, DR>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((append_kernel<T, 1, DC, DR>), grid, block, 0, s, a); break;
  }
}

template <typename T>
void launch_dc(const AppendArgs& a, int groups, int nrb, hipStream_t s) {
  if (a.d_rope != kDRope) {                 // split variants: d_c = kDC, bf16 storage
    if constexpr (std::is_same_v<T, bf16_t>) {
      switch (a.d_rope) {
        case 16: launch_t<T, kDC, 16>(a, groups, nrb, s); break;
        case 64: launch_t<T, kDC, 64>(a, groups, nrb, s); break;
        default: launch_t<T, kDC, 96>(a, groups, nrb, s); break;
      }
    }
    return;
  }
  switch (a.d_c) {
    case 64: launch_t<T, 64, kDRope>(a, groups, nrb, s); break;
    case 128: launch_t<T, 128, kDRope>(a, groups, nrb, s); break;
    case 256:                                 // wide latents: bf16 storage only
      if constexpr (std::is_same_v<T, bf16_t>) launch_t<T, 256, kDRope>(a, groups, nrb, s);
      break;
    case 512:                                 // at most 2 row blocks per wave (64-row ranges)
      if constexpr (std::is_same_v<T, bf16_t>) {
        const dim3 grid(groups), block(kThreads);
        if (nrb == 2) hipLaunchKernelGGL((append_kernel<T, 2, 512, kDRope>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((append_kernel<T, 1, 512, kDRope>), grid, block, 0, s, a);
      }
      break;
    default: launch_t<T, kDC, kDRope>(a, groups, nrb, s); break;
  }
}

}  // namespace

// Workgroups and row blocks per wave for m rows on `cus` compute units: one
// workgroup per compute unit while the ranges stay within 160 rows (more
// workgroups, in rounds, beyond that), but no range below 32 rows, since each
// workgroup streams the whole weight. A range of r rows is 16-row blocks split
// over the two row halves: ceil(ceil(r / 16) / 2) blocks per wave.
int append_plan(int64_t m, int cus, int max_rows, int* nrb) {
  const int64_t lo = (m + max_rows - 1) / max_rows;
  const int64_t groups = std::max<int64_t>(lo, std::min<int64_t>(cus, (m + 31) / 32));
  const int64_t rows = (m + groups - 1) / groups;
  *nrb = (int)(((rows + 15) / 16 + 1) / 2);
  return (int)groups;
}

hipError_t launch_append(const AppendArgs& a, bool f32, hipStream_t s) {
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  int nrb = 1;
  // d_c = 512: row ranges of at most 64 rows, so two 64-deep stages fit the LDS
  const int max_rows = a.d_c == 512 ? 64 : kMaxRows;
  const int groups = append_plan((int64_t)a.batch * a.n_tok, cus > 0 ? cus : 1, max_rows, &nrb);
  if (a.d_rope != kDRope && (f32 || a.d_c != kDC)) return hipErrorInvalidValue;   // not instantiated
  if ((a.d_c == 256 || a.d_c == 512) && f32) return hipErrorInvalidValue;
  if (f32) launch_dc<float>(a, groups, nrb, s);
  else launch_dc<bf16_t>(a, groups, nrb, s);
  return hipGetLastError();
}

}  // namespace vmla
