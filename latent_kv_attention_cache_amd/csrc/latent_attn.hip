// Latent-form chunk attention for gfx950.
//
// VideoMLA (paperlayer.ai summary of arXiv:2605.30351v1), App. E
// "Inference-Time Reparameterization": scores are taken directly against the
// cached rows [c | k_R] with absorbed, pre-scaled queries Qhat_h = [q_lat | q_rope]
// (built by the query prologue), the softmax-weighted latents c are
// accumulated ("Value-path absorption") and projected by W_V_up[h] at the end.
// Every query of the chunk attends to every valid key of the window, its own
// chunk included (App. D.4: chunk-causal, so no mask inside the window).
//
// Work split. The queries of a batch element are cut into units of 32 tokens
// of one head, numbered head-major (U = ceil(n_q / 32) units per head, at
// least 8). A workgroup of 8 waves (two per SIMD) takes 8 consecutive units,
// one per wave; since the cache rows are shared by all heads, a workgroup may
// span two heads, and only the last unit of a head can be partial. Each wave
// keeps its 32 queries' Qhat rows in registers. The waves walk the key window
// in tiles of 64 keys. A tile [64][224] is copied once from global memory
// straight into LDS (16-byte LDS-DMA loads, no VGPR staging) and read by all 8
// waves, so every cache read is shared by all 256 queries of the block.
//
// Two schedules share this layout and arithmetic. The split-role schedule
// (latent_attn_pair_kernel, further below) runs the content widths 128 and 192
// at the default positional width: the two waves of a SIMD divide the work of
// 64 queries by role, so every LDS operand fragment feeds two MFMAs. The
// ping-pong schedule (latent_attn_kernel) runs d_c = 64 and the NoPE/RoPE
// split variants, whose wider rows leave no LDS for the split-role hand-over.
//
// Ping-pong schedule. Time is cut into phases separated by workgroup barriers.
// Waves 0-3 ("X") and 4-7 ("Y", one per SIMD next to an X wave) run the same
// program, Y one phase behind X. In its matrix phase for tile j a wave runs
//   O^T += C^T(j-1) P^T(j-1)   and   S^T(j) = K(j) Qhat^T      (52 MFMA 32x32x16)
// and in its vector phase it runs the online softmax of S^T(j) and packs
// P^T(j) to bf16. While one wave of a SIMD is in its matrix phase the other is
// in its vector phase, so matrix cores and VALU overlap by construction. Every
// wave executes exactly one barrier per phase, outside all branches, with the
// same trip count. Within a matrix phase the LDS operand reads run two MFMA
// steps ahead of the MFMAs (scheduling groups below).
//
// Tile buffers. Tile t is read in phases 2t .. 2t+3 (X scores, Y scores, X and Y
// P.C). The X waves fetch tile t+2 during their vector phase 2t+1 into the
// buffer of tile t-2 (four buffers) and make sure it has landed before the
// barrier that precedes its first reader (phase 2t+4).
//
// LDS tile layout, chunk-major: the 16-byte chunk c (features 8c .. 8c+7) of
// key row r sits at slot c * 68 + r. One wave-wide LDS-DMA load moves chunk c of
// all 64 rows (lane = row), so a lane's source address is its row plus a
// scalar column offset. A score operand read (chunk c of 32 consecutive rows)
// is contiguous; the 4-slot pad per chunk column places chunk c+1 of a row 16
// banks after chunk c, so the transpose reads of 4 rows x 2 chunks that a
// 16-lane group issues cover distinct banks.
//
// MFMA formulation (keys on MFMA rows): S^T[key][q] = K[key][:] . Qhat[q][:];
// per query (= per lane) max and sum over the lane's own keys, the other half
// of the keys sitting in lane l^32 (one permlane32 swap). The score
// accumulators start at -m (m the running reference max), so the MFMAs deliver
// s - m and the exp2 needs no subtraction unless m moves; at d_c = 64, where
// the VALU bounds the loop, the row sum comes from 4 more MFMAs per tile
// against a register fragment of ones instead of VALU adds. O^T[d][q] +=
// C^T[d][key] . P^T[key][q] with C^T read straight from the row-major tile by
// the LDS transpose read and P^T the S^T accumulator packed to bf16 in place
// (the MFMA contraction order of keys is permuted identically on both sides).
// Epilogue: out^T[e][q] = W_V_up[h]^T[e][:] . (O^T / l)[:][q], W_V_up[h]
// staged in LDS and read transposed.
//
// Folded output (template flag kFold; App. E "Value-path absorption" with B_h
// folded into the output mixer): the epilogue writes the normalized latent
// O_lat / l of each (token, head) as bf16 to olat[b n_q + n][h d_c ..] and the
// folded mixer weights are applied by a separate GEMM over all heads.
//
// Read-time RoPE (caches that keep k_R before rotation, [PL] App. D.5 and
// App. E "RoPE branch"; template flag kRot): loading wave w moves chunk column
// 24 + w of every tile, i.e. RoPE pairs 4w .. 4w+3 of k_R. Once its own loads
// of a tile have landed it rotates that column in LDS, in place (lane = key
// row), with the key's local coordinate in the active context, before the
// barrier that publishes the tile.
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace vmla {
namespace {

constexpr int kKT = 64;                     // keys per tile
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kSlots = kKT + 4;             // slots per chunk column (padded)
constexpr int kLoaders = kWaves / 2;        // the X waves issue the tile loads
constexpr int kBufs = 4;
constexpr int kVLd = kDV + 8;               // padded LDS row of W_V_up[h] (epilogue)
constexpr float kLazy = 8.f;                // lazy-rescale threshold (log2 units)

// Shape of the latent row for a content width DC (192 by default; 64 and 128
// for the latent-budget sweep) and a positional width DR (32 by default; 16,
// 64, 96 for the NoPE/RoPE split variants): [c (DC) | k_R (DR)].
template <int DC, int DR>
struct AttnShape {
  static constexpr int kDC = DC;
  static constexpr int kRow = DC + DR;
  static constexpr int kChunks = kRow / 8;          // 16-byte chunks per key row (28 at DC 192)
  static constexpr int kTileElems = kChunks * kSlots * 8;
  // one load per chunk column; with 26 columns (DR = 16) the last two loads of
  // waves 2 and 3 are skipped
  static constexpr int kLoadsPerWave = (kChunks + kLoaders - 1) / kLoaders;
  static constexpr int kFeatSteps = kRow / 16;      // 14
  static constexpr int kLatTiles = DC / 32;         // 6
  static_assert(kRow % 16 == 0, "whole 16-feature MFMA steps");
  static_assert(kBufs * kTileElems * 2 <= 160 * 1024, "LDS budget");
  static_assert(2 * DC * kVLd <= kBufs * kTileElems, "W_V_up of two heads must fit in the tile buffers");
  static_assert(DC % 32 == 0 && DC * kDV / 8 % kThreads == 0, "content width");
};

// Scheduling-group masks (instruction classes of sched_group_barrier).
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;

// 16-byte LDS-DMA load: lane i's 16 bytes from base + voff (bytes; base
// wave-uniform) land at LDS byte address lds_addr + 16 i (lds_addr
// wave-uniform). Issued as inline assembly so the compiler does not serialize
// unrelated LDS reads behind it; completion is waited for explicitly with
// s_waitcnt vmcnt. No register output; M0 is set inside the statement.
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(voff), "s"(base), "s"(__builtin_amdgcn_readfirstlane(lds_addr)) : "memory");
}

template <typename T, bool kRot, bool kFold, int DC, bool kChunked, int DR>
__global__ __launch_bounds__(kThreads)
void latent_attn_kernel(AttnArgs a) {
  using Sh = AttnShape<DC, DR>;
  static_assert(!kRot || DR == kDRope, "read-time RoPE rotates the default 32 positional columns");
  constexpr int kDC = Sh::kDC;
  constexpr int kRow = Sh::kRow;
  constexpr int kTileElems = Sh::kTileElems;
  constexpr int kLoadsPerWave = Sh::kLoadsPerWave;
  constexpr int kFeatSteps = Sh::kFeatSteps;
  constexpr int kLatTiles = Sh::kLatTiles;
  // At narrow latents one phase covers kSub 64-key sub-tiles (128 keys), so
  // the two barriers and the phase starts of a step are spread over twice the
  // work; the sub-tiles keep the 64-key LDS layout, kBufs * kSub buffers.
  constexpr int kSub = DC <= 64 ? 2 : 1;
  constexpr int kNB = kBufs * kSub;                 // sub-tile buffers
  static_assert(kNB * kTileElems * 2 <= 160 * 1024, "LDS budget");
  __shared__ __attribute__((aligned(16))) bf16_t kt[kNB * kTileElems];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int qi = lane & 31;
  const int lag = wave >= kLoaders ? 1 : 0;   // Y waves run one phase behind
  // Query chunk of this workgroup (kChunked): blockIdx.z = (n_chunks - 1 - c) *
  // batch + b, so the chunks with the most keys are dispatched first. Without
  // chunks: all n_q queries over keys [0, n_k).
  int b = blockIdx.z, q0 = 0, nq = a.n_q, k0 = 0, nk = a.n_k, chunk_q = a.n_q;
  if constexpr (kChunked) {
    const int rc = blockIdx.z / a.batch;
    const int c = a.cm.n_chunks - 1 - rc;
    b = blockIdx.z - rc * a.batch;
    chunk_q = a.cm.chunk_q;
    q0 = c * chunk_q;                                     // first query of the chunk
    nq = min(chunk_q, a.n_q - q0);
    const int k_end = min(a.n_k, (c + 1) * a.cm.key_step);
    k0 = max(0, k_end - a.cm.key_span);                   // first key of the chunk
    nk = k_end - k0;
  }
  // This wave's unit: head h, chunk query rows 32 qb .. 32 qb + 31.
  const int units = (nq + 31) / 32;
  const int umax = (chunk_q + 31) / 32;
  const int upad = umax > kWaves ? umax : kWaves;        // units per head, padded to >= 8
  const int u0 = blockIdx.x * kWaves;
  const int u = u0 + wave;
  const int h_lo = u0 / upad;                             // heads of this workgroup: h_lo, h_lo + 1
  const int h = min(u / upad, a.n_heads - 1);
  const int qb = u - (u / upad) * upad;
  const int qrow = 32 * qb + qi;
  // A wave without queries (past the last head, or a pad unit of a head with
  // fewer than 8 units) keeps the barriers and its share of the tile loads but
  // skips the math: on a power-limited chip idle matrix cores raise the
  // others' clock.
  const bool live = u / upad < a.n_heads && qb < units;
  const bool qvalid = live && qrow < nq;

  // Qhat fragments (B operand of S^T): lane holds features ks*16 + 8*half + e of its query.
  bf16x8 qf[kFeatSteps];
  {
    const bf16_t* qp = a.qhat + (((size_t)b * a.n_heads + h) * a.n_q + q0 + (qvalid ? qrow : nq - 1)) * kRow;
#pragma unroll
    for (int ks = 0; ks < kFeatSteps; ++ks)
      qf[ks] = *reinterpret_cast<const bf16x8*>(qp + ks * 16 + 8 * half);
    // Re-define the fragments by an (empty) register statement: the memory
    // wait for the loads is then placed here, once. Otherwise the compiler
    // keeps vmcnt waits for them in front of every score MFMA of the loop,
    // where they would also wait for the tile prefetches in flight.
#pragma unroll
    for (int ks = 0; ks < kFeatSteps; ++ks) asm volatile("" : "+v"(qf[ks]));
  }

  const T* cache = static_cast<const T*>(a.cache) + ((size_t)b * a.cache_rows + k0) * kRow;
  constexpr int kTileKeys = kKT * kSub;             // keys per step
  const int ntiles = (nk + kTileKeys - 1) / kTileKeys;
  // sub-tile st of the window sits in buffer st % kNB
  auto sub_buf = [&](int st) { return kt + (st % kNB) * kTileElems; };

  // ---- tile staging (X waves only). Wave-wide load n moves chunk column n:
  // lane r reads features 8n .. 8n+7 of key 64 st + r (sub-tile st) into slot
  // n * kSlots + r. Keys past the window are clamped to the last valid key
  // (finite data; their scores are masked).
  const uint32_t kt_lds = (uint32_t)(uintptr_t)(VMLA_LDS bf16_t*)kt;
  auto issue_tile = [&](int j) {
    const int wv = __builtin_amdgcn_readfirstlane(wave);   // scalar load index and LDS address
#pragma unroll
    for (int sb = 0; sb < kSub; ++sb) {
      const int st = j * kSub + sb;
      const int buf = st % kNB;
      const int kg = min(st * kKT + lane, nk - 1);
#pragma unroll
      for (int i = 0; i < kLoadsPerWave; ++i) {
        const int n = wv + kLoaders * i;
        if (Sh::kChunks % kLoaders != 0 && n >= Sh::kChunks) continue;   // wave-uniform
        if constexpr (std::is_same_v<T, bf16_t>) {
          dma16(cache, (uint32_t)(kg * (kRow * 2)) + (uint32_t)(16 * n),
                kt_lds + 2u * (uint32_t)(buf * kTileElems + n * kSlots * 8));
        } else {
          const T* src = cache + (size_t)kg * kRow + 8 * n;
          *reinterpret_cast<uint4*>(kt + buf * kTileElems + (n * kSlots + lane) * 8) = load8_bf16<T>(src);
        }
      }
    }
  };

  // Read-time RoPE of this loading wave's k_R column of sub-tile st (kRot only).
  auto rotate_sub = [&](int st) {
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    bf16_t* p = sub_buf(st) + ((kDC / 8 + wv) * kSlots + lane) * 8;
    const int kg = k0 + min(st * kKT + lane, nk - 1);       // cache slot
    int n_in, ww;
    const int fs = div_small(kg, a.tokens_per_frame, a.inv_tokens_per_frame, &n_in);
    const int hh = div_small(n_in, a.grid_w, a.inv_grid_w, &ww);
    int tl = fs;                                  // sink frame: its own index
    if (fs >= a.sink_frames) {
      int r = fs - a.sink_frames - a.shift_mod_w;
      if (r < 0) r += a.window_frames;
      tl = a.sink_frames + r;
    }
    const uint4 raw = *reinterpret_cast<const uint4*>(p);
    const uint32_t in[4] = {raw.x, raw.y, raw.z, raw.w};
    uint32_t o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int pr = 4 * wv + q;
      const int ax = a.rope.axis[pr];
      const float a0 = __uint_as_float(in[q] << 16), a1 = __uint_as_float(in[q] & 0xffff0000u);
      float sn, cs;
      sincos_rev(ax == 0 ? tl : (ax == 1 ? hh : ww), a.rope.rev_lo[pr], a.rope.rev_hi[pr], &sn, &cs);
      o[q] = pack2(a0 * cs - a1 * sn, a0 * sn + a1 * cs);
    }
    *reinterpret_cast<uint4*>(p) = uint4{o[0], o[1], o[2], o[3]};
  };
  auto rotate_tile = [&](int j) {
#pragma unroll
    for (int sb = 0; sb < kSub; ++sb) rotate_sub(j * kSub + sb);
  };

  // Per-lane LDS element offsets (relative to a tile) of the operand reads; a
  // key row advances by 8 elements. Score A operand: row qi (+32 for the second
  // key block), features 16 ks + 8 half, i.e. chunk 2 ks + half.
  const int a_base = (half * kSlots + qi) * 8;
  // Transpose reads of C^T: lane j of a 16-lane group points at row
  // kbase + rb + j/4 (rb = 4*half, or 8 + 4*half for the second read), elements
  // 32 t + nsub + 4 (j%4) .. +3 with nsub = 16 ((lane / 16) % 2), i.e. chunk
  // 4 t + x4 at element offset sub inside the chunk.
  const int jl = lane & 15;
  const int x4 = ((lane & 16) >> 3) + ((jl & 3) >> 1);   // chunk within the 4-chunk group
  const int sub = 4 * (jl & 1);
  const int v_off1 = (x4 * kSlots + 4 * half + (jl >> 2)) * 8 + sub;
  const int v_off2 = v_off1 + 8 * 8;

  f32x16 o[kLatTiles];
#pragma unroll
  for (int t = 0; t < kLatTiles; ++t) o[t] = f32x16{};
  // m: reference max of this query (log2 units), identical in lanes l and l^32;
  // l: running sum over this lane's half of the keys, relative to m.
  float m = -INFINITY;
  float l = 0.f;
  // Narrow latents keep the matrix cores idle half the time; there the row
  // sum l comes from 4 more MFMAs per tile against a constant fragment whose
  // row 0 is all ones (O_sum^T[0][q] = sum over keys of P^T[key][q]), off the
  // VALU, which bounds those widths.
  constexpr bool kSumMfma = DC <= 64;
  f32x16 osum = f32x16{};
  bf16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = (__bf16)(qi == 0 ? 1.f : 0.f);
  // S^T of the current step, per sub-tile and key block: register r holds
  // key 32 kb + 8(r/4) + 4 half + r%4 of the sub-tile
  f32x16 s[kSub][2];
  bf16x8 pb[kSub][2][2];  // P^T of the previous step, bf16, per (sub-tile, key block, 16-key step)

  // O^T += C^T(step j) P^T: 4 kLatTiles MFMAs per sub-tile (24 at d_c 192),
  // the transpose reads issued two MFMAs ahead.
  auto accumulate = [&](int j) {
#pragma unroll
    for (int sb = 0; sb < kSub; ++sb) {
      const bf16_t* K = sub_buf(j * kSub + sb);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          const bf16_t* Kb = K + (kb * 32 + jj * 16) * 8;
#pragma unroll
          for (int t = 0; t < kLatTiles; ++t) {
            const bf16x4 lo = lds_tr4(Kb + v_off1 + 4 * kSlots * 8 * t);
            const bf16x4 hi = lds_tr4(Kb + v_off2 + 4 * kSlots * 8 * t);
            const bf16x8 av = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            o[t] = mfma32(av, pb[sb][kb][jj], o[t]);
          }
          if constexpr (kSumMfma) osum = mfma32(ones, pb[sb][kb][jj], osum);
        }
      }
    }
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 4, 0);
#pragma unroll
    for (int i = 0; i < 4 * kLatTiles * kSub - 2; ++i) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2 + (kSumMfma ? 4 * kSub : 0), 0);
  };
  // S^T of one step: 2 kFeatSteps MFMAs per sub-tile (28 at d_c 192), the row
  // reads issued two feature steps ahead. The score accumulators start at
  // -mo, mo = the reference max m (0 before the first tile): the MFMAs deliver
  // s - m, and the softmax needs no subtraction unless m moves.
  auto scores = [&](int j) {
    const float mo = m > -INFINITY ? -m : 0.f;
#pragma unroll
    for (int sb = 0; sb < kSub; ++sb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[sb][0][r] = mo;
        s[sb][1][r] = mo;
      }
#pragma unroll
    for (int sb = 0; sb < kSub; ++sb) {
      const bf16_t* K = sub_buf(j * kSub + sb);
#pragma unroll
      for (int ks = 0; ks < kFeatSteps; ++ks) {
        const int off = a_base + 2 * kSlots * 8 * ks;
        const bf16x8 a0 = lds_row8(K + off);
        const bf16x8 a1 = lds_row8(K + off + 32 * 8);
        s[sb][0] = mfma32(a0, qf[ks], s[sb][0]);
        s[sb][1] = mfma32(a1, qf[ks], s[sb][1]);
      }
    }
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 4, 1);
#pragma unroll
    for (int i = 0; i < kFeatSteps * kSub - 2; ++i) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2, 1);
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 1);
    }
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 4, 1);
  };
  // Online softmax of the current step; leaves P^T (bf16) in pb.
  auto softmax = [&](int key0) {
#pragma unroll
    for (int sb = 0; sb < kSub; ++sb) {
      const int ks0 = key0 + sb * kKT;          // first key of the sub-tile
      if (ks0 + kKT > nk) {        // the keys end inside this sub-tile (wave-uniform)
        // register r of key block kb holds key ks0 + 32 kb + 8(r/4) + 4 half + r%4
        const int lim = nk - ks0 - 4 * half;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int k = 8 * (r >> 2) + (r & 3);
          if (k >= lim) s[sb][0][r] = -INFINITY;
          if (k + 32 >= lim) s[sb][1][r] = -INFINITY;
        }
      }
    }
    // the registers hold s - mo with mo = m (0 before the first tile)
    const float mo = m > -INFINITY ? m : 0.f;
    float mx = -INFINITY;
#pragma unroll
    for (int sb = 0; sb < kSub; ++sb) {
      float ms = fmaxf(s[sb][0][0], s[sb][1][0]);
#pragma unroll
      for (int r = 1; r < 16; ++r) ms = fmaxf(ms, fmaxf(s[sb][0][r], s[sb][1][r]));
      mx = sb == 0 ? ms : fmaxf(mx, ms);
    }
    mx = max_across_halves(mx) + mo;
    // Lazy rescaling: the reference max only moves when a score exceeds it by
    // more than 2^kLazy, so exp2(s - m) <= 2^kLazy stays exact in fp32/bf16 and
    // the O / l rescale runs on few tiles. Wave-uniform branch.
    const bool grow = mx > m + kLazy;
    if (__builtin_amdgcn_ballot_w64(grow)) {
      const float m_new = grow ? mx : m;
      const float alpha = __builtin_amdgcn_exp2f(m - m_new);
      l *= alpha;
      osum *= alpha;
#pragma unroll
      for (int t = 0; t < kLatTiles; ++t) o[t] *= alpha;
      const float dm = m_new - mo;             // scores to the new reference
#pragma unroll
      for (int sb = 0; sb < kSub; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          s[sb][0][r] -= dm;
          s[sb][1][r] -= dm;
        }
      m = m_new;
    }
    if constexpr (kSumMfma) {
#pragma unroll
      for (int sb = 0; sb < kSub; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          s[sb][0][r] = __builtin_amdgcn_exp2f(s[sb][0][r]);
          s[sb][1][r] = __builtin_amdgcn_exp2f(s[sb][1][r]);
        }
    } else {
      float ls = 0.f;
#pragma unroll
      for (int sb = 0; sb < kSub; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          s[sb][0][r] = __builtin_amdgcn_exp2f(s[sb][0][r]);
          s[sb][1][r] = __builtin_amdgcn_exp2f(s[sb][1][r]);
          ls += s[sb][0][r] + s[sb][1][r];
        }
      l += ls;
    }
#pragma unroll
    for (int sb = 0; sb < kSub; ++sb)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
          for (int e = 0; e < 8; ++e) pb[sb][kb][jj][e] = (__bf16)s[sb][kb][8 * jj + e];
  };

  if (!lag) {
    issue_tile(0);
    if (ntiles > 1) issue_tile(1);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    // tile 1 is rotated in the vector phase of tile 0, like every later tile
    if constexpr (kRot) rotate_tile(0);
  }
  __syncthreads();

  // Phases p = 0 .. 2 ntiles + 1; wave-local phase q = p - lag. In its vector
  // phase for tile jt (phase 2 jt + 1) an X wave first waits for all of its
  // loads, i.e. its part of tile jt + 1 (requested in phase 2 jt - 1), so that
  // the barrier closing this phase publishes tile jt + 1 to its first readers
  // (phase 2 jt + 2); it then requests tile jt + 2 into the buffer of tile
  // jt - 2, whose last readers ran in phase 2 jt - 1. The requests stay off the
  // matrix phases.
  const int nphases = 2 * ntiles + 2;
  for (int p = 0; p < nphases; ++p) {
    const int q = p - lag;
    if (q >= 0) {
      const int jt = q >> 1;
      if ((q & 1) == 0) {          // matrix phase for tile jt
        __builtin_amdgcn_s_setprio(1);
        if (live) {
          if (jt >= 1) accumulate(jt - 1);
          if (jt < ntiles) scores(jt);
        }
        __builtin_amdgcn_s_setprio(0);
      } else if (jt < ntiles) {    // vector phase for tile jt
        if (!lag) {
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
          if constexpr (kRot) {
            if (jt + 1 < ntiles) rotate_tile(jt + 1);
          }
          if (jt + 2 < ntiles) issue_tile(jt + 2);
        }
        if (live) softmax(jt * kTileKeys);
      }
    }
    __syncthreads();
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // osum register 0: row 0 (the sum) in lanes 0-31, row 4 (zero) in lanes 32-63
  const float inv = 1.f / sum_across_halves(kSumMfma ? osum[0] : l);
  if constexpr (kFold) {
    // ---- epilogue: olat = O / l. Register 8 jj + e of latent tile t holds
    // latent dim 32 t + 16 jj + 8 (e / 4) + 4 half + e % 4 of query qrow.
    if (!qvalid) return;   // no barrier follows
    uint16_t* dst = a.olat + ((size_t)b * a.n_q + q0 + qrow) * ((size_t)a.n_heads * kDC) + (size_t)h * kDC;
#pragma unroll
    for (int t = 0; t < kLatTiles; ++t)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int e4 = 0; e4 < 2; ++e4) {
          const int r = 8 * jj + 4 * e4;
          *reinterpret_cast<uint2*>(dst + 32 * t + 16 * jj + 8 * e4 + 4 * half) =
              uint2{pack2(o[t][r] * inv, o[t][r + 1] * inv), pack2(o[t][r + 2] * inv, o[t][r + 3] * inv)};
        }
    return;
  }

  // ---- epilogue: out = (O / l) @ W_V_up[h]; W_V_up of the workgroup's one or
  // two heads staged in LDS, [kDC][kVLd] each.
  const int nh = min((u0 + kWaves - 1) / upad, a.n_heads - 1) - h_lo + 1;   // 1 or 2 (upad >= 8)
  const T* wsrc = static_cast<const T*>(a.w_v_up) + (size_t)h_lo * kDC * kDV;
  for (int hh = 0; hh < nh; ++hh) {
#pragma unroll
    for (int i = 0; i < kDC * kDV / 8 / kThreads; ++i) {
      const int c = tid + i * kThreads;
      const int row = c / (kDV / 8), cc = c % (kDV / 8);
      *reinterpret_cast<uint4*>(&kt[(hh * kDC + row) * kVLd + 8 * cc]) =
          load8_bf16<T>(wsrc + ((size_t)hh * kDC + row) * kDV + 8 * cc);
    }
  }
  __syncthreads();
  const bf16_t* wv = kt + (h - h_lo) * kDC * kVLd;

  if (!live) return;   // no barrier follows
  bf16x8 ob[kLatTiles][2];
#pragma unroll
  for (int t = 0; t < kLatTiles; ++t)
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
      for (int e = 0; e < 8; ++e) ob[t][jj][e] = (__bf16)(o[t][8 * jj + e] * inv);

  T* out = static_cast<T*>(a.out) + (((size_t)b * a.n_q + q0 + (qvalid ? qrow : 0)) * a.n_heads + h) * kDV;
#pragma unroll
  for (int et = 0; et < kDV / 32; ++et) {
    f32x16 acc = f32x16{};
#pragma unroll
    for (int t = 0; t < kLatTiles; ++t) {
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int dbase = 32 * t + 16 * jj;
        const bf16x8 av = lds_tr8(wv, kVLd, dbase + 4 * half, dbase + 8 + 4 * half, 32 * et, lane);
        acc = mfma32(av, ob[t][jj], acc);
      }
    }
    if (qvalid) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int e0 = 32 * et + 8 * g + 4 * half;
#pragma unroll
        for (int e = 0; e < 4; ++e) out[e0 + e] = from_f32<T>(acc[4 * g + e]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Split-role schedule (content widths 128 and 192, default positional width):
// the two waves of a SIMD share two 32-query units (64 queries) and split the
// work by role instead of by query.
//   X (waves 0-3): scores of both units, S^T(j) = K(j) Qhat^T: each K fragment
//       read from LDS feeds two MFMAs (56 per tile); then the online softmax
//       of both units, handing P^T(j) (bf16) and each query's rescale factor
//       to its partner through LDS.
//   Y (waves 4-7): the tile loads (and the read-time rotation), then
//       O^T += C^T(j-1) P^T(j-1) for both units: each C^T fragment feeds two
//       MFMAs (48 per tile); Y also keeps the row sums l (from the same bf16
//       P^T that multiplies the latents) and at the end runs the W_V_up
//       epilogue of both units.
// Phase A(j): X issues the score MFMAs while Y issues the next tile's loads,
// reads P^T(j-1) into registers, applies the (rare) rescale of O and l and
// adds P^T(j-1)'s row sums to l.
// Phase B(j): Y issues the P.C MFMAs while
// X runs the softmax of tile j, so X's vector work overlaps Y's matrix work.
// X is the busier role (its score MFMAs and its softmax run in series), so
// every vector operation that does not need the scores runs on Y.
// Every wave executes one barrier per phase; the role branches are wave-
// uniform (scalar) branches around loops of the same trip count. LDS operand
// traffic per tile and SIMD: 28 KB of K, 24 KB of C^T and 16 KB of P^T, where
// two waves of 32 queries each would read 104 KB.
//
// Buffers: tile j is read in B(j-1) (X's first K fragments), A(j) (K) and
// B(j+1) (C^T); four tile buffers. Y requests tile j+2 at the start of A(j)
// into the buffer of tile j-2 (last read in B(j-1)) and waits for tile j+1
// (requested in A(j-1)) at the end of A(j), before the barrier that publishes
// it; X then reads the first K fragments of tile j+1 in B(j), next to its
// softmax, so A(j+1) starts with MFMAs.
// The hand-over region of a pair holds P^T of one tile (8 fragments per lane)
// and one float per lane and unit (the rescale factor): X writes it in B(j);
// Y reads it into registers in A(j+1), where it has no matrix work, together
// with the first two C^T fragments of its next P.C, so B(j+1) starts without
// waiting for LDS.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
constexpr int kPairs = 4;
constexpr int kHandPBytes = 8 * 64 * 16;                       // P^T of one tile
constexpr int kHandBytes = kHandPBytes + 2 * 64 * 4;            // + one float per lane and unit

template <typename T, bool kRot, bool kFold, int DC, bool kChunked>
__global__ __launch_bounds__(kThreads)
void latent_attn_pair_kernel(AttnArgs a) {
  using Sh = AttnShape<DC, kDRope>;
  constexpr int kDC = Sh::kDC;
  constexpr int kRow = Sh::kRow;
  constexpr int kTileElems = Sh::kTileElems;
  constexpr int kLoadsPerWave = Sh::kLoadsPerWave;
  constexpr int kFeatSteps = Sh::kFeatSteps;
  constexpr int kLatTiles = Sh::kLatTiles;
  constexpr int kHandElems = kHandBytes / 2;
  constexpr int kHandOff = kBufs * kTileElems;            // elements
  static_assert(Sh::kChunks % kLoaders == 0, "every loading wave moves the same number of chunk columns");
  static_assert((kHandOff + kPairs * kHandElems) * 2 <= 160 * 1024, "LDS budget");
  static_assert(2 * DC * kVLd <= kHandOff, "W_V_up staging inside the tile buffers");
  __shared__ __attribute__((aligned(16))) bf16_t kt[kHandOff + kPairs * kHandElems];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave-uniform by construction; readfirstlane makes it uniform to the
  // compiler, so the role branches (which hold barriers) are scalar branches
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int qi = lane & 31;
  const int pair = wave & (kPairs - 1);
  const bool is_y = wave >= kPairs;
  int b = blockIdx.z, q0 = 0, nq = a.n_q, k0 = 0, nk = a.n_k, chunk_q = a.n_q;
  if constexpr (kChunked) {
    const int rc = blockIdx.z / a.batch;
    const int c = a.cm.n_chunks - 1 - rc;
    b = blockIdx.z - rc * a.batch;
    chunk_q = a.cm.chunk_q;
    q0 = c * chunk_q;
    nq = min(chunk_q, a.n_q - q0);
    const int k_end = min(a.n_k, (c + 1) * a.cm.key_step);
    k0 = max(0, k_end - a.cm.key_span);
    nk = k_end - k0;
  }
  // The pair's units u0 + 2 pair + i, i = 0, 1: head hu[i], query rows qrow[i].
  const int units = (nq + 31) / 32;
  const int umax = (chunk_q + 31) / 32;
  const int upad = umax > kWaves ? umax : kWaves;
  const int u0 = blockIdx.x * kWaves;
  const int h_lo = u0 / upad;
  int hu[2], qrow[2];
  bool live_u[2], qvalid[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int u = u0 + 2 * pair + i;
    const int qb = u - (u / upad) * upad;
    hu[i] = min(u / upad, a.n_heads - 1);
    qrow[i] = 32 * qb + qi;
    live_u[i] = u / upad < a.n_heads && qb < units;
    qvalid[i] = live_u[i] && qrow[i] < nq;
  }
  const bool live = live_u[0] || live_u[1];

  const T* cache = static_cast<const T*>(a.cache) + ((size_t)b * a.cache_rows + k0) * kRow;
  const int ntiles = (nk + kKT - 1) / kKT;
  // the pair's hand-over region: P^T at hand_p, the floats at hand_f
  bf16_t* const hand_p = kt + kHandOff + pair * kHandElems;
  float* const hand_f = reinterpret_cast<float*>(hand_p + kHandPBytes / 2);

  // W_V_up of the workgroup's one or two heads into the tile buffers, [kDC][kVLd] each.
  auto stage_w_v_up = [&]() {
    const int nh = min((u0 + kWaves - 1) / upad, a.n_heads - 1) - h_lo + 1;
    const T* wsrc = static_cast<const T*>(a.w_v_up) + (size_t)h_lo * kDC * kDV;
    for (int hh = 0; hh < nh; ++hh) {
#pragma unroll
      for (int i = 0; i < kDC * kDV / 8 / kThreads; ++i) {
        const int c = tid + i * kThreads;
        const int row = c / (kDV / 8), cc = c % (kDV / 8);
        *reinterpret_cast<uint4*>(&kt[(hh * kDC + row) * kVLd + 8 * cc]) =
            load8_bf16<T>(wsrc + ((size_t)hh * kDC + row) * kDV + 8 * cc);
      }
    }
  };

  if (!is_y) {
    // ================= X: scores and softmax of the pair's two units
    bf16x8 qf[2][kFeatSteps];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const bf16_t* qp = a.qhat + (((size_t)b * a.n_heads + hu[i]) * a.n_q + q0 + (qvalid[i] ? qrow[i] : nq - 1)) * kRow;
#pragma unroll
      for (int ks = 0; ks < kFeatSteps; ++ks)
        qf[i][ks] = *reinterpret_cast<const bf16x8*>(qp + ks * 16 + 8 * half);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int ks = 0; ks < kFeatSteps; ++ks) asm volatile("" : "+v"(qf[i][ks]));
    const int a_base = (half * kSlots + qi) * 8;
    float m[2] = {-INFINITY, -INFINITY};
    f32x16 s[2][2];     // [unit][key block]: register r holds key 32 kb + 8(r/4) + 4 half + r%4

    // K fragment (key block kb, feature step ks) of a tile
    auto k_frag = [&](const bf16_t* K, int ks, int kb) {
      return lds_row8(K + a_base + 2 * kSlots * 8 * ks + kb * 32 * 8);
    };
    // score accumulators start at -m (m the running reference max; 0 before
    // the first key), so the MFMAs deliver s - m: the first MFMA of each key
    // block takes the block negm[unit] as its addend. The block is built in
    // the softmax phase; pinning it there keeps the 32 moves out of the score
    // phase, whose matrix work would otherwise wait for them.
    f32x16 negm[2];
    auto init_scores = [&]() {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const float mo = m[i] > -INFINITY ? -m[i] : 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) negm[i][r] = mo;
        asm volatile("" : "+v"(negm[i]));
      }
    };
    // S^T of one tile for both units: 56 MFMAs; the fragments of feature
    // steps 0 and 1 come in already read, later ones are read two steps ahead.
    bf16x8 kpre[2][2];
    auto scores = [&](const bf16_t* K) {
      bf16x8 fr[3][2];
      fr[0][0] = kpre[0][0];
      fr[0][1] = kpre[0][1];
      fr[1][0] = kpre[1][0];
      fr[1][1] = kpre[1][1];
#pragma unroll
      for (int ks = 0; ks < kFeatSteps; ++ks) {
        if (ks + 2 < kFeatSteps) {
          fr[(ks + 2) % 3][0] = k_frag(K, ks + 2, 0);
          fr[(ks + 2) % 3][1] = k_frag(K, ks + 2, 1);
        }
        s[0][0] = mfma32(fr[ks % 3][0], qf[0][ks], ks == 0 ? negm[0] : s[0][0]);
        s[1][0] = mfma32(fr[ks % 3][0], qf[1][ks], ks == 0 ? negm[1] : s[1][0]);
        s[0][1] = mfma32(fr[ks % 3][1], qf[0][ks], ks == 0 ? negm[0] : s[0][1]);
        s[1][1] = mfma32(fr[ks % 3][1], qf[1][ks], ks == 0 ? negm[1] : s[1][1]);
      }
#pragma unroll
      for (int i = 0; i < kFeatSteps - 2; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 4, 0);
      }
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 8, 0);
    };
    auto prefetch_k = [&](const bf16_t* K) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        kpre[ks][0] = k_frag(K, ks, 0);
        kpre[ks][1] = k_frag(K, ks, 1);
      }
    };
    // Online softmax of both units; hands P^T and the rescale factors over.
    auto softmax = [&](int key0) {
      if (key0 + kKT > nk) {       // the keys end inside this tile (wave-uniform)
        const int lim = nk - key0 - 4 * half;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int k = 8 * (r >> 2) + (r & 3);
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            if (k >= lim) s[i][0][r] = -INFINITY;
            if (k + 32 >= lim) s[i][1][r] = -INFINITY;
          }
        }
      }
      // both units side by side (two independent max trees, one wave-uniform
      // rescale check, then the exps and bf16 packing of both), so the
      // dependent steps of one unit overlap those of the other
      float mo[2], mx[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        mo[i] = m[i] > -INFINITY ? m[i] : 0.f;
        float t[4];
#pragma unroll
        for (int c = 0; c < 4; ++c)
          t[c] = fmaxf(fmaxf(fmaxf(s[i][0][4 * c], s[i][1][4 * c]), fmaxf(s[i][0][4 * c + 1], s[i][1][4 * c + 1])),
                       fmaxf(fmaxf(s[i][0][4 * c + 2], s[i][1][4 * c + 2]), fmaxf(s[i][0][4 * c + 3], s[i][1][4 * c + 3])));
        mx[i] = fmaxf(fmaxf(t[0], t[1]), fmaxf(t[2], t[3]));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) mx[i] = max_across_halves(mx[i]) + mo[i];
      const bool grow0 = mx[0] > m[0] + kLazy, grow1 = mx[1] > m[1] + kLazy;
      float alpha[2] = {1.f, 1.f};
      if (__builtin_amdgcn_ballot_w64(grow0 || grow1)) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const float m_new = (i ? grow1 : grow0) ? mx[i] : m[i];
          alpha[i] = __builtin_amdgcn_exp2f(m[i] - m_new);
          const float dm = m_new - mo[i];
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            s[i][0][r] -= dm;
            s[i][1][r] -= dm;
          }
          m[i] = m_new;
        }
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) hand_f[i * 64 + lane] = alpha[i];
#pragma unroll
      for (int r = 0; r < 16; ++r)
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          s[i][0][r] = __builtin_amdgcn_exp2f(s[i][0][r]);
          s[i][1][r] = __builtin_amdgcn_exp2f(s[i][1][r]);
        }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            bf16x8 v;
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = (__bf16)s[i][kb][8 * jj + e];
            *reinterpret_cast<bf16x8*>(hand_p + ((4 * i + 2 * kb + jj) * 64 + lane) * 8) = v;
          }
    };

    __syncthreads();               // tile 0 published
    // per tile j: A(j) scores, B(j) softmax (and the head of tile j+1's
    // scores); then A(ntiles), B(ntiles) idle
    if (live) {
      prefetch_k(kt);
      init_scores();
      for (int j = 0; j < ntiles; ++j) {
        __builtin_amdgcn_s_setprio(1);
        scores(kt + (j % kBufs) * kTileElems);
        __builtin_amdgcn_s_setprio(0);
        __syncthreads();
        if (j + 1 < ntiles) prefetch_k(kt + ((j + 1) % kBufs) * kTileElems);
        softmax(j * kKT);
        init_scores();
        __syncthreads();
      }
    } else {
      for (int j = 0; j < ntiles; ++j) {
        __syncthreads();
        __syncthreads();
      }
    }
    __syncthreads();
    __syncthreads();
    if constexpr (!kFold) {
      stage_w_v_up();
      __syncthreads();
    }
    return;
  }

  // ================= Y: tile loads, P.C of the pair's two units, epilogue
  const int wl = wave - kPairs;     // loading wave index 0..3
  const uint32_t kt_lds = (uint32_t)(uintptr_t)(VMLA_LDS bf16_t*)kt;
  auto issue_tile = [&](int j) {
    const int buf = j % kBufs;
    const int kg = min(j * kKT + lane, nk - 1);
#pragma unroll
    for (int i = 0; i < kLoadsPerWave; ++i) {
      const int n = wl + kLoaders * i;
      if constexpr (std::is_same_v<T, bf16_t>) {
        dma16(cache, (uint32_t)(kg * (kRow * 2)) + (uint32_t)(16 * n),
              kt_lds + 2u * (uint32_t)(buf * kTileElems + n * kSlots * 8));
      } else {
        const T* src = cache + (size_t)kg * kRow + 8 * n;
        *reinterpret_cast<uint4*>(kt + buf * kTileElems + (n * kSlots + lane) * 8) = load8_bf16<T>(src);
      }
    }
  };
  auto rotate_tile = [&](int j) {
    bf16_t* p = kt + (j % kBufs) * kTileElems + ((kDC / 8 + wl) * kSlots + lane) * 8;
    const int kg = k0 + min(j * kKT + lane, nk - 1);
    int n_in, ww;
    const int fs = div_small(kg, a.tokens_per_frame, a.inv_tokens_per_frame, &n_in);
    const int hh = div_small(n_in, a.grid_w, a.inv_grid_w, &ww);
    int tl = fs;
    if (fs >= a.sink_frames) {
      int r = fs - a.sink_frames - a.shift_mod_w;
      if (r < 0) r += a.window_frames;
      tl = a.sink_frames + r;
    }
    const uint4 raw = *reinterpret_cast<const uint4*>(p);
    const uint32_t in[4] = {raw.x, raw.y, raw.z, raw.w};
    uint32_t o4[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int pr = 4 * wl + q;
      const int ax = a.rope.axis[pr];
      const float a0 = __uint_as_float(in[q] << 16), a1 = __uint_as_float(in[q] & 0xffff0000u);
      float sn, cs;
      sincos_rev(ax == 0 ? tl : (ax == 1 ? hh : ww), a.rope.rev_lo[pr], a.rope.rev_hi[pr], &sn, &cs);
      o4[q] = pack2(a0 * cs - a1 * sn, a0 * sn + a1 * cs);
    }
    *reinterpret_cast<uint4*>(p) = uint4{o4[0], o4[1], o4[2], o4[3]};
  };

  const int jl = lane & 15;
  const int x4 = ((lane & 16) >> 3) + ((jl & 3) >> 1);
  const int sub = 4 * (jl & 1);
  const int v_off1 = (x4 * kSlots + 4 * half + (jl >> 2)) * 8 + sub;
  const int v_off2 = v_off1 + 8 * 8;

  f32x16 o[2][kLatTiles];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int t = 0; t < kLatTiles; ++t) o[i][t] = f32x16{};
  // row sums l of both units over this lane's keys, from the bf16 P^T
  float lsum[2] = {0.f, 0.f};

  const bf16x2 one2 = {(__bf16)1.f, (__bf16)1.f};
  bf16x8 pb[2][4];        // P^T of the tile being accumulated: [unit][(key block, 16-key step)]
  // C^T fragment f = g * kLatTiles + t of a tile: key group g = (key block,
  // 16-key step), latent block t; two transpose reads.
  constexpr int kFrags = 4 * kLatTiles;
  auto ct_frag = [&](const bf16_t* K, int f) {
    const int g = f / kLatTiles, t = f % kLatTiles;
    const bf16_t* Kb = K + ((g >> 1) * 32 + (g & 1) * 16) * 8 + 4 * kSlots * 8 * t;
    const bf16x4 lo = lds_tr4(Kb + v_off1);
    const bf16x4 hi = lds_tr4(Kb + v_off2);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  };
  // O^T += C^T P^T for both units: kFrags fragments, each feeding two MFMAs.
  // Fragments 0 and 1 are read into the ring fr (slot f % 3) before the
  // phase's barrier; later ones are read two fragments ahead.
  bf16x8 fr[3];
  auto accumulate = [&](const bf16_t* K) {
#pragma unroll
    for (int f = 0; f < kFrags; ++f) {
      if (f + 2 < kFrags) fr[(f + 2) % 3] = ct_frag(K, f + 2);
      const int g = f / kLatTiles, t = f % kLatTiles;
      o[0][t] = mfma32(fr[f % 3], pb[0][g], o[0][t]);
      o[1][t] = mfma32(fr[f % 3], pb[1][g], o[1][t]);
    }
#pragma unroll
    for (int f = 0; f < kFrags - 2; ++f) {
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 4, 0);
  };

  issue_tile(0);
  if (ntiles > 1) issue_tile(1);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if constexpr (kRot) rotate_tile(0);
  __syncthreads();

  // A(j) ends by publishing tile j+1: this wave waits for its loads of it
  // (requested in A(j-1); tile j+2's, requested at the start of A(j), may
  // still be in flight) and rotates its column
  auto publish_next = [&](int j) {
    if (j + 1 < ntiles) {
      if (j + 2 < ntiles) asm volatile("s_waitcnt vmcnt(%0)" :: "n"(kLoadsPerWave) : "memory");
      else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      if constexpr (kRot) rotate_tile(j + 1);
    }
  };
  // A(0), B(0): no P.C yet
  if (2 < ntiles) issue_tile(2);
  publish_next(0);
  __syncthreads();
  __syncthreads();
  if (live) {
    for (int j = 1; j <= ntiles; ++j) {
      // A(j): request tile j+2; P^T(j-1), its rescale factors and the first
      // two C^T fragments of tile j-1 into registers; publish tile j+1
      if (j + 2 < ntiles) issue_tile(j + 2);
      const bf16_t* K = kt + ((j - 1) % kBufs) * kTileElems;
      // the read-time rotation runs before P^T occupies its registers
      if constexpr (kRot) publish_next(j);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) pb[i][g] = lds_row8(hand_p + ((4 * i + g) * 64 + lane) * 8);
      const float al0 = hand_f[lane], al1 = hand_f[64 + lane];
      fr[0] = ct_frag(K, 0);
      fr[1] = ct_frag(K, 1);
      if constexpr (!kRot) publish_next(j);
      // the (rare) rescale of O by the factors of tile j-1 also runs here
      if (__builtin_amdgcn_ballot_w64(al0 != 1.f || al1 != 1.f)) {
#pragma unroll
        for (int t = 0; t < kLatTiles; ++t) {
          o[0][t] *= al0;
          o[1][t] *= al1;
        }
        lsum[0] *= al0;
        lsum[1] *= al1;
      }
      // row sums of P^T(j-1): a lane's 32 bf16 values per unit (8 keys of
      // each 16-key step, one query), by dot products with (1, 1)
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        float part[2] = {0.f, 0.f};
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          part[g & 1] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[i][g], pb[i][g], 0, 1), one2, part[g & 1], false);
          part[g & 1] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[i][g], pb[i][g], 2, 3), one2, part[g & 1], false);
          part[g & 1] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[i][g], pb[i][g], 4, 5), one2, part[g & 1], false);
          part[g & 1] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[i][g], pb[i][g], 6, 7), one2, part[g & 1], false);
        }
        lsum[i] += part[0] + part[1];
      }
      __syncthreads();
      // B(j): P.C of tile j-1
      __builtin_amdgcn_s_setprio(1);
      accumulate(K);
      __builtin_amdgcn_s_setprio(0);
      __syncthreads();
    }
  } else {
    for (int j = 1; j <= ntiles; ++j) {
      if (j + 2 < ntiles) issue_tile(j + 2);
      publish_next(j);
      __syncthreads();
      __syncthreads();
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  // lanes l and l + 32 hold the sums over the two key halves of one query
  float inv[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) inv[i] = 1.f / sum_across_halves(lsum[i]);

  if constexpr (kFold) {
    // olat = O / l; register 8 jj + e of latent tile t holds latent dim
    // 32 t + 16 jj + 8 (e / 4) + 4 half + e % 4 of the unit's query.
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if (!qvalid[i]) continue;
      uint16_t* dst = a.olat + ((size_t)b * a.n_q + q0 + qrow[i]) * ((size_t)a.n_heads * kDC) + (size_t)hu[i] * kDC;
#pragma unroll
      for (int t = 0; t < kLatTiles; ++t)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
          for (int e4 = 0; e4 < 2; ++e4) {
            const int r = 8 * jj + 4 * e4;
            *reinterpret_cast<uint2*>(dst + 32 * t + 16 * jj + 8 * e4 + 4 * half) =
                uint2{pack2(o[i][t][r] * inv[i], o[i][t][r + 1] * inv[i]),
                      pack2(o[i][t][r + 2] * inv[i], o[i][t][r + 3] * inv[i])};
          }
    }
    return;
  } else {
    stage_w_v_up();
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if (!live_u[i]) continue;
      const bf16_t* wv = kt + (hu[i] - h_lo) * kDC * kVLd;
      bf16x8 ob[kLatTiles][2];
#pragma unroll
      for (int t = 0; t < kLatTiles; ++t)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
          for (int e = 0; e < 8; ++e) ob[t][jj][e] = (__bf16)(o[i][t][8 * jj + e] * inv[i]);
      T* out = static_cast<T*>(a.out) + (((size_t)b * a.n_q + q0 + (qvalid[i] ? qrow[i] : 0)) * a.n_heads + hu[i]) * kDV;
#pragma unroll
      for (int et = 0; et < kDV / 32; ++et) {
        f32x16 acc = f32x16{};
#pragma unroll
        for (int t = 0; t < kLatTiles; ++t) {
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            const int dbase = 32 * t + 16 * jj;
            const bf16x8 av = lds_tr8(wv, kVLd, dbase + 4 * half, dbase + 8 + 4 * half, 32 * et, lane);
            acc = mfma32(av, ob[t][jj], acc);
          }
        }
        if (qvalid[i]) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int e0 = 32 * et + 8 * g + 4 * half;
#pragma unroll
            for (int e = 0; e < 4; ++e) out[e0 + e] = from_f32<T>(acc[4 * g + e]);
          }
        }
      }
    }
  }
}

template <int DC>
hipError_t launch_dc_pingpong(const AttnArgs& a, bool f32, hipStream_t s) {
  const int units = (a.cm.chunk_q + 31) / 32;
  const int upad = units > kWaves ? units : kWaves;
  dim3 grid((a.n_heads * upad + kWaves - 1) / kWaves, 1, a.batch * a.cm.n_chunks);
  if (a.cm.n_chunks > 1) {
    // query chunks come only with append-time RoPE and the W_V_up epilogue
    if (a.rope_at_read || a.olat) return hipErrorInvalidValue;
    if (f32) hipLaunchKernelGGL((latent_attn_kernel<float, false, false, DC, true, kDRope>), grid, dim3(kThreads), 0, s, a);
    else hipLaunchKernelGGL((latent_attn_kernel<bf16_t, false, false, DC, true, kDRope>), grid, dim3(kThreads), 0, s, a);
  } else if (a.olat) {
    if (a.rope_at_read) {
      if (f32) hipLaunchKernelGGL((latent_attn_kernel<float, true, true, DC, false, kDRope>), grid, dim3(kThreads), 0, s, a);
      else hipLaunchKernelGGL((latent_attn_kernel<bf16_t, true, true, DC, false, kDRope>), grid, dim3(kThreads), 0, s, a);
    } else {
      if (f32) hipLaunchKernelGGL((latent_attn_kernel<float, false, true, DC, false, kDRope>), grid, dim3(kThreads), 0, s, a);
      else hipLaunchKernelGGL((latent_attn_kernel<bf16_t, false, true, DC, false, kDRope>), grid, dim3(kThreads), 0, s, a);
    }
  } else if (a.rope_at_read) {
    if (f32) hipLaunchKernelGGL((latent_attn_kernel<float, true, false, DC, false, kDRope>), grid, dim3(kThreads), 0, s, a);
    else hipLaunchKernelGGL((latent_attn_kernel<bf16_t, true, false, DC, false, kDRope>), grid, dim3(kThreads), 0, s, a);
  } else {
    if (f32) hipLaunchKernelGGL((latent_attn_kernel<float, false, false, DC, false, kDRope>), grid, dim3(kThreads), 0, s, a);
    else hipLaunchKernelGGL((latent_attn_kernel<bf16_t, false, false, DC, false, kDRope>), grid, dim3(kThreads), 0, s, a);
  }
  return hipGetLastError();
}


template <int DC>
hipError_t launch_dc_pair(const AttnArgs& a, bool f32, hipStream_t s) {
  const int units = (a.cm.chunk_q + 31) / 32;
  const int upad = units > kWaves ? units : kWaves;
  dim3 grid((a.n_heads * upad + kWaves - 1) / kWaves, 1, a.batch * a.cm.n_chunks);
  if (a.cm.n_chunks > 1) {
    // query chunks come only with append-time RoPE and the W_V_up epilogue
    if (a.rope_at_read || a.olat) return hipErrorInvalidValue;
    if (f32) hipLaunchKernelGGL((latent_attn_pair_kernel<float, false, false, DC, true>), grid, dim3(kThreads), 0, s, a);
    else hipLaunchKernelGGL((latent_attn_pair_kernel<bf16_t, false, false, DC, true>), grid, dim3(kThreads), 0, s, a);
  } else if (a.olat) {
    if (a.rope_at_read) {
      if (f32) hipLaunchKernelGGL((latent_attn_pair_kernel<float, true, true, DC, false>), grid, dim3(kThreads), 0, s, a);
      else hipLaunchKernelGGL((latent_attn_pair_kernel<bf16_t, true, true, DC, false>), grid, dim3(kThreads), 0, s, a);
    } else {
      if (f32) hipLaunchKernelGGL((latent_attn_pair_kernel<float, false, true, DC, false>), grid, dim3(kThreads), 0, s, a);
      else hipLaunchKernelGGL((latent_attn_pair_kernel<bf16_t, false, true, DC, false>), grid, dim3(kThreads), 0, s, a);
    }
  } else if (a.rope_at_read) {
    if (f32) hipLaunchKernelGGL((latent_attn_pair_kernel<float, true, false, DC, false>), grid, dim3(kThreads), 0, s, a);
    else hipLaunchKernelGGL((latent_attn_pair_kernel<bf16_t, true, false, DC, false>), grid, dim3(kThreads), 0, s, a);
  } else {
    if (f32) hipLaunchKernelGGL((latent_attn_pair_kernel<float, false, false, DC, false>), grid, dim3(kThreads), 0, s, a);
    else hipLaunchKernelGGL((latent_attn_pair_kernel<bf16_t, false, false, DC, false>), grid, dim3(kThreads), 0, s, a);
  }
  return hipGetLastError();
}


// d_c 128 and 192: the split-role schedule; d_c 64, where the softmax's
// vector work bounds either schedule, the ping-pong one measured faster.
template <int DC>
hipError_t launch_dc(const AttnArgs& a, bool f32, hipStream_t s) {
  if constexpr (DC <= 64) return launch_dc_pingpong<DC>(a, f32, s);
  else return launch_dc_pair<DC>(a, f32, s);
}

template <int DR>
hipError_t launch_split(const AttnArgs& a, bool f32, hipStream_t s) {
  const int units = (a.cm.chunk_q + 31) / 32;
  const int upad = units > kWaves ? units : kWaves;
  dim3 grid((a.n_heads * upad + kWaves - 1) / kWaves, 1, a.batch);
  if (f32) hipLaunchKernelGGL((latent_attn_kernel<float, false, false, kDC, false, DR>), grid, dim3(kThreads), 0, s, a);
  else hipLaunchKernelGGL((latent_attn_kernel<bf16_t, false, false, kDC, false, DR>), grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_latent_attn(const AttnArgs& a, bool f32, hipStream_t s) {
  if (a.d_c == 256 || a.d_c == 512) {
    // wide latents: bf16, one query chunk, k_R rotated at append, W_V_up epilogue
    if (f32 || a.cm.n_chunks != 1 || a.rope_at_read || a.olat || a.d_rope != kDRope)
      return hipErrorInvalidValue;
    return launch_latent_attn_wide(a, s);
  }
  if (a.d_rope != kDRope) {
    // split variants: d_c = kDC, one query chunk, k_R rotated at append, W_V_up epilogue
    if (a.d_c != kDC || a.cm.n_chunks != 1 || a.rope_at_read || a.olat) return hipErrorInvalidValue;
    switch (a.d_rope) {
      case 16: return launch_split<16>(a, f32, s);
      case 64: return launch_split<64>(a, f32, s);
      case 96: return launch_split<96>(a, f32, s);
      default: return hipErrorInvalidValue;
    }
  }
  switch (a.d_c) {
    case 64: return launch_dc<64>(a, f32, s);
    case 128: return launch_dc<128>(a, f32, s);
    default: return launch_dc<kDC>(a, f32, s);
  }
}

}  // namespace vmla
