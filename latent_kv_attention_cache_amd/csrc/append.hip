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
// x, so they form one row range), N = d_c + d_rope (224), K = d_model. The M
// rows are split into one contiguous range per workgroup, at most 160 rows, as
// evenly as the device's compute units allow (a workgroup fills one compute
// unit's LDS). Every workgroup streams all of W_down / W_KR (688 KB at
// d_model = 1536) from L2 next to its slice of x from HBM.
//
// Eight waves, two per SIMD. The output tile [rows x 224] is cut 2 x 2 into
// four wave tiles: tile (rh, ch) is row half rh (up to 5 blocks of 16 rows)
// by column half ch (7 blocks of 16 columns; half 1 holds c columns 112-191
// and the k_R columns). The two waves of a SIMD (waves t and t + 4, "teams" 0
// and 1) own the same tile and split the contraction: team 0 takes the even
// 32-deep stages, team 1 the odd ones, each with its own fp32 accumulators.
// At the end each team hands the other, through LDS, the partial sums of the
// half of the tile's column blocks that the other finalises. So while one
// wave of a SIMD waits for LDS operands or at the barrier, its partner issues
// matrix instructions, and the LDS operand traffic stays that of one 80 x 112
// tile per SIMD (46 flops per LDS byte).
//
// v_mfma_f32_16x16x32_bf16 computes the transposed block out^T = W^T x^T, so a
// lane ends up with four consecutive columns of one token row.
//
// Pipeline: a round is two 32-deep stages (one per team); LDS holds kRing
// rounds (3 of 48 KB for ranges of 160 rows at the default widths, 4 for
// ranges of up to 64 rows, whose rounds take 32-37 KB), filled by 16-byte
// LDS-DMA loads kRing - 1 rounds ahead, one barrier per round. The loads of a round
// are spread evenly over the eight waves (six each at the default widths) and
// issued between the matrix instructions; each costs a scalar base update
// only (fixed lane offsets). LDS layouts of a round:
//   x tile: row-major [rows][64] (both stages), 128 bytes per row, so a DMA
//           load reads whole cache lines of 8 rows; chunk c of row r at
//           c ^ swz_a(r), so the 16-row operand reads hit distinct banks;
//   W tiles, one per stage: W_down [32][d_c] and W_KR [32][d_rope],
//           row-major, so that a DMA load reads 1 KB of contiguous weight.
//           The 16-byte chunks of row k are XOR-permuted, chunk c at position
//           c ^ 2 t(k) with t(k) = bit1(k) | bit3(k) << 1 for W_down and
//           t(k) = bit3(k) for W_KR: a transposed operand read of 32 lanes
//           (rows k0 .. k0+3 and k0+8 .. k0+11, two chunks each) then covers
//           all 64 banks once.
//
// Epilogue: the k_R columns are rotated in registers before the rows are
// staged in LDS; every RoPE rate and row position is read from LDS (the rates
// copied there once at the start with uniform kernel-argument loads), since a
// kernel argument indexed per lane compiles to per-lane loads from the
// kernel-argument segment on the epilogue's critical path.
#include <algorithm>

#include "device_common.h"
#include "kernels.h"
#include "staging.h"

namespace vmla {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxRows = 160;
constexpr int kSK = 32;                     // contraction depth of a stage
constexpr int kLdsBytes = 160 * 1024;

// Weight-tile shape for a content width DC (192 by default; 64, 128, 256, 512
// for the latent-budget sweep) and a positional width DR (32 by default; 16,
// 64, 96 for the NoPE/RoPE split variants): a row of [W_down | W_KR] is
// DC + DR wide. Column half 0 takes the first kColBlocks 16-wide blocks, half 1
// the other kColBlocks1 (one fewer when the row has an odd number of blocks).
template <int DC, int DR>
struct WShape {
  static constexpr int kRow = DC + DR;
  static constexpr int kWdElems = kSK * DC;               // W_down tile of a stage
  static constexpr int kWElems = kSK * kRow;              // W_down + W_KR tiles
  static constexpr int kWdLoads = kWdElems * 2 / 1024;    // wave-wide 1 KB loads: 12 at DC 192
  static constexpr int kWrLoads = kSK * DR * 2 / 1024;    // 2 at DR 32
  static constexpr int kColBlocks = (kRow / 16 + 1) / 2;  // 16-wide column blocks of half 0 (7)
  static constexpr int kColBlocks1 = kRow / 16 - kColBlocks;
  static_assert(kRow % 16 == 0 && 16 * kColBlocks <= DC, "half 0 holds content columns only");
  static_assert(DR % 16 == 0 && kWrLoads >= 1, "W_KR tile of whole 1 KB loads");
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
  using WS = WShape<DC, DR>;
  static constexpr int kRow = WS::kRow;
  static constexpr int kRows = 32 * NRB;                   // rows of a workgroup at most
  static constexpr int kXElems = kRows * 2 * kSK;          // x tile of a round: both stages
  static constexpr int kXLoads = kXElems * 2 / 1024;       // 4 NRB (8 rows of 128 B each)
  static constexpr int kWStageLoads = WS::kWdLoads + WS::kWrLoads;
  static constexpr int kRoundElems = kXElems + 2 * WS::kWElems;
  static constexpr int kRoundLoads = kXLoads + 2 * kWStageLoads;
  static constexpr int kLPW = (kRoundLoads + kWaves - 1) / kWaves;   // loads per wave per round
  // rounds held in LDS: 4 where they fit with a margin for the RoPE table
  // (one or two row blocks per wave), else 3, else 2
  static constexpr int kRing = 4 * kRoundElems * 2 <= kLdsBytes - 1024 ? 4
                               : (3 * kRoundElems * 2 <= kLdsBytes ? 3 : 2);
  static constexpr int kRingElems = kRing * kRoundElems;
  // epilogue LDS: the RoPE table (its own array, for the whole kernel); five
  // ints of row info per row (batch element, slot, t, h, w) at kRiOff, past
  // both the partial sums exchanged by the teams (register order, kPassRB row
  // blocks of all four tiles per pass) and the output rows (kRow + 8 bf16 or
  // kRow + 4 fp32 wide) that reuse the same bytes afterwards
  static constexpr int kTabBytes = 3 * (DR / 2) * 4;
  static constexpr int kRiBytes = kRows * 5 * 4;
  static constexpr int kAccBytesRB = 4 * WS::kColBlocks * 64 * 16;
  static constexpr int kPassRB = std::min(NRB, (kLdsBytes - kTabBytes - kRiBytes) / kAccBytesRB);
  static constexpr int kOutLd = std::is_same_v<T, bf16_t> ? kRow + 8 : kRow + 4;
  static constexpr int kRiOff = std::max(kPassRB * kAccBytesRB, kRows * kOutLd * (int)sizeof(T));
  static constexpr int kSmemElems = std::max(kRingElems, (kRiOff + kRiBytes) / 2);
  static_assert(NRB >= 1 && NRB <= 5, "row blocks per wave");
  static_assert(kPassRB >= 1, "one row block of partial sums fits the LDS");
  static_assert(kRiOff % 16 == 0, "row info alignment");
  static_assert(kSmemElems * 2 + kTabBytes <= kLdsBytes, "LDS budget");
};

template <typename T, int NRB, int DC, int DR>
__global__ __launch_bounds__(kThreads)
void append_kernel(AppendArgs a) {
  using Tl = Tile<T, NRB, DC, DR>;
  using WS = WShape<DC, DR>;
  constexpr int kRow = WS::kRow;
  constexpr int kColBlocks = WS::kColBlocks;
  constexpr int kColBlocks1 = WS::kColBlocks1;
  constexpr int kLPW = Tl::kLPW;
  constexpr int kRing = Tl::kRing;
  constexpr bool kBf16 = std::is_same_v<T, bf16_t>;
  // W fragments held at once: all column blocks of the wave's half up to 256-wide
  // rows; two passes over them for wider rows (x fragments read once per pass)
  constexpr int kCBP = kRow <= 256 ? kColBlocks : (kColBlocks + 1) / 2;
  constexpr int kPasses = (kColBlocks + kCBP - 1) / kCBP;
  constexpr int kSteps = kPasses * NRB;     // slots that the round's loads are spread over
  __shared__ __attribute__((aligned(16))) bf16_t smem[Tl::kSmemElems];
  __shared__ uint32_t rtab[3 * (DR / 2)];   // rev_lo, rev_hi, axis of every k_R pair

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tile = wv & 3, team = wv >> 2;  // wave-uniform; waves t and t + 4 share a SIMD
  const int g = lane >> 4;                  // 16-lane group: k sub-range of an MFMA operand
  const int rh = tile >> 1, ch = tile & 1;

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
  const int nrounds = a.d_model / (2 * kSK);
  // With ranges of three or more row blocks per wave, each workgroup runs
  // the rounds in its own rotated order, starting at round rot: workgroups
  // are dealt round-robin to the 8 XCDs, so the 32 or so on one XCD start at
  // different rounds and read different weight lines from its L2 at any
  // moment (about 1 % faster at the batch-8 chunk shape than all starting at
  // round 0; 2 % slower for the 32-row ranges of a batch-1 chunk, which keep
  // the plain order). The fp32 sums only change order.
  const int rot = NRB >= 3 ? (int)((blockIdx.x / 8) % (unsigned)nrounds) : 0;

  // Load n of a round (0 <= n < kRoundLoads): first the x loads (8 rows of
  // 128 bytes each: both stages' k columns, so every load reads whole cache
  // lines), then the W_down and W_KR loads of stage 0, then those of stage 1.
  // Wave wv issues n = kLPW wv + i; the last wave repeats the round's last
  // load when the loads do not split evenly (same data to the same LDS
  // bytes). The LDS destination (elements from the round's buffer), the
  // source and the lane offset depend on the wave only.
  int ldst[kLPW], kind[kLPW], half[kLPW];
  uint32_t voff[kLPW];
#pragma unroll
  for (int i = 0; i < kLPW; ++i) {
    const int n = min(kLPW * wv + i, Tl::kRoundLoads - 1);
    if (n < Tl::kXLoads) {
      kind[i] = 0;
      half[i] = 0;
      ldst[i] = 512 * n;
      voff[i] = stage_a_voff(a.d_model, 0, rows, n, lane);
    } else {
      const int v = n - Tl::kXLoads;
      const int h = v / Tl::kWStageLoads, u = v - h * Tl::kWStageLoads;
      half[i] = h;
      if (u < WS::kWdLoads) {
        kind[i] = 1;
        ldst[i] = Tl::kXElems + h * WS::kWElems + 512 * u;
        const int q = 64 * u + lane, k = q / (DC / 8), cp = q - k * (DC / 8);
        voff[i] = (uint32_t)(k * DC + 8 * (cp ^ swz_wd(k))) * 2u;
      } else {
        kind[i] = 2;
        ldst[i] = Tl::kXElems + h * WS::kWElems + WS::kWdElems + 512 * (u - WS::kWdLoads);
        const int q = 64 * (u - WS::kWdLoads) + lane, k = q / (DR / 8), cp = q - k * (DR / 8);
        voff[i] = (uint32_t)(k * DR + 8 * (cp ^ swz_wr<DR>(k))) * 2u;
      }
    }
  }
  // this wave's loads i0 <= i < i1 of round rs (data) into the buffer of round rb
  auto issue = [&](int rb, int rs, int i0, int i1) {
    bf16_t* base = smem + (rb % kRing) * Tl::kRoundElems;
#pragma unroll
    for (int i = 0; i < kLPW; ++i) {
      if (i < i0 || i >= i1) continue;
      const int rk = rs + rot < nrounds ? rs + rot : rs + rot - nrounds;   // round of the data
      const int k0 = kind[i] == 0 ? rk * 2 * kSK : (2 * rk + half[i]) * kSK;
      bf16_t* dst = base + ldst[i];
      if constexpr (kBf16) {
        const bf16_t* src = kind[i] == 0 ? xw + k0 : (kind[i] == 1 ? wd + (size_t)k0 * DC
                                                                   : wr + (size_t)k0 * DR);
        dma16_lds(src, voff[i], lds_u32(dst));
      } else {
        // fp32 sources: through registers, converted to bf16, same layout
        // (voff holds the bf16 byte offset, i.e. twice the element offset)
        const uint32_t e = voff[i] / 2u;
        const T* src = kind[i] == 0 ? xw + k0 + e : (kind[i] == 1 ? wd + (size_t)k0 * DC + e
                                                                  : wr + (size_t)k0 * DR + e);
        *reinterpret_cast<uint4*>(dst + 8 * lane) = load8_bf16<T>(src);
      }
    }
  };

  // Per-lane operand offsets (elements, relative to a round's buffer).
  // x (B operand): lane = row (lane % 16) of block rb, k 8 g .. 8 g + 7 of the
  // team's stage, i.e. logical chunk 4 team + g of the row's 8 (x tile rows
  // are 64 wide with the chunk permutation swz_a).
  int a_off[NRB];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    const int row = rbase + 16 * rb + (lane & 15);
    a_off[rb] = 2 * kSK * row + 8 * ((4 * team + g) ^ swz_a(row));
  }
  // W^T (A operand) by ds_read_b64_tr_b16: lane j of 16-lane group g points at
  // k row 8 g + j/4 (+4 for the upper half of the fragment) and columns
  // col0 + 4 (j%4) .. +3, i.e. logical chunk col0/8 + (j%4)/2, element 4 (j%2).
  const int j = lane & 15;
  int b_off[kColBlocks], b_up[kColBlocks];
  {
    const int k = 8 * g + (j >> 2);
#pragma unroll
    for (int cb = 0; cb < kColBlocks; ++cb) {
      const int gcb = kColBlocks * ch + cb;            // 16-column block of [c | k_R]
      const bool content = gcb < DC / 16;
      const int c = (content ? 2 * gcb : 2 * (gcb - DC / 16)) + ((j & 3) >> 1);
      b_off[cb] = Tl::kXElems + team * WS::kWElems +
                  (content ? k * DC + 8 * (c ^ swz_wd(k)) + 4 * (j & 1)
                           : WS::kWdElems + k * DR + 8 * (c ^ swz_wr<DR>(k)) + 4 * (j & 1));
      b_up[cb] = 4 * (content ? DC : DR);
    }
  }

  for (int r = 0; r < kRing - 1; ++r) issue(r, min(r, nrounds - 1), 0, kLPW);
  // The RoPE rates of the k_R pairs, copied once from the kernel arguments
  // with uniform loads (compile-time indices): read per lane in the epilogue,
  // and fetched now, while the first loads are in flight, not on the
  // epilogue's critical path. The round barriers order these writes.
  if (wv == kWaves - 1) {
#pragma unroll
    for (int p = 0; p < DR / 2; ++p) {
      if (lane == 0) {
        rtab[p] = a.rope.rev_lo[p];
        rtab[DR / 2 + p] = a.rope.rev_hi[p];
        rtab[DR + p] = (uint32_t)a.rope.axis[p];
      }
    }
  }

  f32x4 acc[NRB][kColBlocks];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
    for (int cb = 0; cb < kColBlocks; ++cb) acc[rb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Round r: each wave runs its team's stage (NRB x 7 MFMAs), reading its W
  // fragments and the first x fragment up front and the next x fragment under
  // the current MFMAs, and issues its share of the loads of round
  // r + kRing - 1 (into the buffers of round r - 1, free after this round's
  // barrier) after every row block. Past the last round those loads repeat
  // the last round's data into buffers that are not read again, so the round
  // body has no branch; every wave issues kLPW loads per round.
  for (int r = 0; r < nrounds; ++r) {
    // round r has landed: the loads of the kRing - 2 later rounds may be in flight
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"((kRing - 2) * kLPW) : "memory");
    __syncthreads();
    const int rn = min(r + kRing - 1, nrounds - 1);           // source round of the loads
    const bf16_t* S = smem + (r % kRing) * Tl::kRoundElems;
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
      bf16x8 bw[kCBP];
#pragma unroll
      for (int c = 0; c < kCBP; ++c) {
        const int cb = kCBP * p + c;
        if (cb >= kColBlocks || (cb >= kColBlocks1 && ch != 0)) {   // half 1 may hold one block fewer
          bw[c] = bf16x8{};
          continue;
        }
        const bf16x4 lo = lds_tr4(S + b_off[cb]);
        const bf16x4 hi = lds_tr4(S + b_off[cb] + b_up[cb]);
        bw[c] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
      bf16x8 av = lds_row8(S + a_off[0]);
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        const int q = NRB * p + rb;
        bf16x8 an = av;
        if (rb + 1 < NRB) an = lds_row8(S + a_off[rb + 1]);
        issue(r + kRing - 1, rn, q * kLPW / kSteps, (q + 1) * kLPW / kSteps);
#pragma unroll
        for (int c = 0; c < kCBP; ++c) {
          const int cb = kCBP * p + c;
          if (cb < kColBlocks && (cb < kColBlocks1 || ch == 0))
            acc[rb][cb] = mfma16(bw[c], av, acc[rb][cb]);
        }
        av = an;
      }
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");    // the trailing loads have landed
  __syncthreads();                                    // every stage read is done

  // ---- row info: threads tid < rows compute their row's batch element,
  // ring slot and (t, h, w), into LDS bytes that the exchange below leaves
  // alone (its barriers order them before their use)
  int* ri = reinterpret_cast<int*>(reinterpret_cast<char*>(smem) + Tl::kRiOff);   // [kRows][5]
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
    ri[5 * row + 2] = t;
    ri[5 * row + 3] = hh;
    ri[5 * row + 4] = ww;
  }

  // ---- the two teams' partial sums. Team 0 finalises column blocks
  // cb < kCBh of its tile, team 1 the rest: each team writes the partials of
  // the blocks the other finalises (register order, kPassRB row blocks per
  // pass) and adds the other's partials into its own blocks.
  constexpr int kCBh = (kColBlocks + 1) / 2;
  auto mine = [&](int cb) { return team == 0 ? cb < kCBh : cb >= kCBh; };
  {
    f32x4* part = reinterpret_cast<f32x4*>(smem);
#pragma unroll
    for (int p0 = 0; p0 < NRB; p0 += Tl::kPassRB) {
#pragma unroll
      for (int rb = p0; rb < std::min(NRB, p0 + Tl::kPassRB); ++rb)
#pragma unroll
        for (int cb = 0; cb < kColBlocks; ++cb)
          if (!mine(cb)) part[(((rb - p0) * kColBlocks + cb) * 4 + tile) * 64 + lane] = acc[rb][cb];
      __syncthreads();
#pragma unroll
      for (int rb = p0; rb < std::min(NRB, p0 + Tl::kPassRB); ++rb)
#pragma unroll
        for (int cb = 0; cb < kColBlocks; ++cb)
          if (mine(cb)) acc[rb][cb] += part[(((rb - p0) * kColBlocks + cb) * 4 + tile) * 64 + lane];
      __syncthreads();
    }
  }

  // ---- epilogue. Register r of acc[rb][cb] in lane l: token row
  // rbase + 16 rb + l%16, column 16 (kColBlocks ch + cb) + 4 g + r. Each team
  // writes its finalised blocks to LDS rows (bf16, or fp32 for fp32 storage),
  // rotating the k_R blocks in registers first (the lane's two pairs at its
  // row's (t, h, w)); then all threads copy whole cache rows out of LDS in
  // 16-byte stores.
  constexpr int kOutLd = Tl::kOutLd;
  using OutT = std::conditional_t<kBf16, bf16_t, float>;
  OutT* ot = reinterpret_cast<OutT*>(smem);                                 // [kRows][kOutLd]
  const int64_t cache_rows = ((int64_t)a.sink_frames + a.window_frames) * a.tokens_per_frame;
#pragma unroll
  for (int cb = 0; cb < kColBlocks; ++cb) {
    if (!mine(cb) || (cb >= kColBlocks1 && ch != 0)) continue;   // half 1 may hold one block fewer
    const int gcb = kColBlocks * ch + cb;
    const bool rot = gcb >= DC / 16 && !a.rope_at_read;
    const int p0 = (16 * gcb - DC) / 2 + 2 * g;                 // the lane's pairs p0, p0 + 1
    const int col = 16 * gcb + 4 * g;
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const int row = rbase + 16 * rb + (lane & 15);
      f32x4 v = acc[rb][cb];
      if (rot) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {       // (a0, a1) -> (a0 cos - a1 sin, a0 sin + a1 cos)
          const int p = p0 + q;
          float sn, cs;
          sincos_rev(ri[5 * row + 2 + (int)rtab[DR + p]], rtab[p], rtab[DR / 2 + p], &sn, &cs);
          const float a0 = v[2 * q], a1 = v[2 * q + 1];
          v[2 * q] = a0 * cs - a1 * sn;
          v[2 * q + 1] = a0 * sn + a1 * cs;
        }
      }
      if constexpr (kBf16)
        *reinterpret_cast<uint2*>(&ot[row * kOutLd + col]) = uint2{pack2(v[0], v[1]), pack2(v[2], v[3])};
      else
        *reinterpret_cast<f32x4*>(&ot[row * kOutLd + col]) = v;
    }
  }
  __syncthreads();
  // Non-temporal 16-byte stores: every workgroup writes its rows at the end of
  // the kernel, and streaming them out as they are issued (rather than
  // leaving up to 16.8 MB of dirty lines in the L2s at the kernel's end) made
  // the batch-8 append ~7 % faster; the attention that reads the rows next
  // measured the same.
  typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
  T* cache = static_cast<T*>(a.cache);
  constexpr int kPer = 16 / sizeof(T);      // elements per 16-byte store
  constexpr int kChunksRow = kRow / kPer;
  for (int c = tid; c < rows * kChunksRow; c += kThreads) {
    const int row = c / kChunksRow, cc = c - row * kChunksRow;
    T* dst = cache + ((size_t)ri[5 * row] * cache_rows + ri[5 * row + 1]) * kRow + kPer * cc;
    __builtin_nontemporal_store(*reinterpret_cast<const u32x4_t*>(&ot[row * kOutLd + kPer * cc]),
                                reinterpret_cast<u32x4_t*>(dst));
  }
}

// Rows of a range: 160 (5 row blocks per wave); 128 for 288-wide rows, whose
// five-block instances would exceed the registers of two waves per SIMD; 64
// for d_c = 512.
constexpr int max_rows_for(int d_c, int d_rope) {
  return d_c == 512 ? 64 : (d_c + d_rope > 256 ? 128 : kMaxRows);
}

template <typename T, int DC, int DR>
void launch_t(const AppendArgs& a, int groups, int nrb, hipStream_t s) {
  const dim3 grid(groups), block(kThreads);
  switch (nrb) {
    case 5:
      if constexpr (max_rows_for(DC, DR) >= 160) hipLaunchKernelGGL((append_kernel<T, 5, DC, DR>), grid, block, 0, s, a);
      break;
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
  const int max_rows = max_rows_for(a.d_c, a.d_rope);
  const int groups = append_plan((int64_t)a.batch * a.n_tok, cus > 0 ? cus : 1, max_rows, &nrb);
  if (a.d_rope != kDRope && (f32 || a.d_c != kDC)) return hipErrorInvalidValue;   // not instantiated
  if ((a.d_c == 256 || a.d_c == 512) && f32) return hipErrorInvalidValue;
  if (f32) launch_dc<float>(a, groups, nrb, s);
  else launch_dc<bf16_t>(a, groups, nrb, s);
  return hipGetLastError();
}

}  // namespace vmla
