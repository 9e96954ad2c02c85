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
// of the keys sitting in lane l^32 (one permlane32 swap); O^T[d][q] +=
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
  __shared__ __attribute__((aligned(16))) bf16_t kt[kBufs * kTileElems];

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
  const int ntiles = (nk + kKT - 1) / kKT;

  // ---- tile staging (X waves only). Wave-wide load n moves chunk column n:
  // lane r reads features 8n .. 8n+7 of key 64 j + r into slot n * kSlots + r.
  // Keys past the window are clamped to the last valid key (finite data; their
  // scores are masked).
  const uint32_t kt_lds = (uint32_t)(uintptr_t)(VMLA_LDS bf16_t*)kt;
  auto issue_tile = [&](int j) {
    const int buf = j % kBufs;
    const int kg = min(j * kKT + lane, nk - 1);
    const int wv = __builtin_amdgcn_readfirstlane(wave);   // scalar load index and LDS address
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
  };

  // Read-time RoPE of this loading wave's k_R column of tile j (kRot only).
  auto rotate_tile = [&](int j) {
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    bf16_t* p = kt + (j % kBufs) * kTileElems + ((kDC / 8 + wv) * kSlots + lane) * 8;
    const int kg = k0 + min(j * kKT + lane, nk - 1);        // cache slot
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
  f32x16 s0, s1;          // S^T of the current tile: register r holds key 32 kb + 8(r/4) + 4 half + r%4
  bf16x8 pb[2][2];        // P^T of the previous tile, bf16, per (key block, 16-key step)

  // O^T += C^T(tile) P^T: 24 MFMAs, 48 transpose reads issued two MFMAs ahead.
  auto accumulate = [&](const bf16_t* K) {
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
          o[t] = mfma32(av, pb[kb][jj], o[t]);
        }
      }
    }
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 4, 0);
#pragma unroll
    for (int i = 0; i < 4 * kLatTiles - 2; ++i) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2, 0);
  };
  // S^T of one tile: 28 MFMAs, 28 row reads issued two steps ahead.
  auto scores = [&](const bf16_t* K) {
    s0 = f32x16{};
    s1 = f32x16{};
#pragma unroll
    for (int ks = 0; ks < kFeatSteps; ++ks) {
      const int off = a_base + 2 * kSlots * 8 * ks;
      const bf16x8 a0 = lds_row8(K + off);
      const bf16x8 a1 = lds_row8(K + off + 32 * 8);
      s0 = mfma32(a0, qf[ks], s0);
      s1 = mfma32(a1, qf[ks], s1);
    }
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 4, 1);
#pragma unroll
    for (int i = 0; i < kFeatSteps - 2; ++i) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2, 1);
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 1);
    }
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 4, 1);
  };
  // Online softmax of the current tile; leaves P^T (bf16) in pb.
  auto softmax = [&](int key0) {
    if (key0 + kKT > nk) {       // the keys end inside this tile (wave-uniform)
      // register r of key block kb holds key key0 + 32 kb + 8(r/4) + 4 half + r%4
      const int lim = nk - key0 - 4 * half;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int k = 8 * (r >> 2) + (r & 3);
        if (k >= lim) s0[r] = -INFINITY;
        if (k + 32 >= lim) s1[r] = -INFINITY;
      }
    }
    float mx = fmaxf(s0[0], s1[0]);
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, fmaxf(s0[r], s1[r]));
    mx = max_across_halves(mx);
    // Lazy rescaling: the reference max only moves when a score exceeds it by
    // more than 2^kLazy, so exp2(s - m) <= 2^kLazy stays exact in fp32/bf16 and
    // the O / l rescale runs on few tiles. Wave-uniform branch.
    const bool grow = mx > m + kLazy;
    if (__builtin_amdgcn_ballot_w64(grow)) {
      const float m_new = grow ? mx : m;
      const float alpha = __builtin_amdgcn_exp2f(m - m_new);
      l *= alpha;
#pragma unroll
      for (int t = 0; t < kLatTiles; ++t) o[t] *= alpha;
      m = m_new;
    }
    float ls = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s0[r] = __builtin_amdgcn_exp2f(s0[r] - m);
      s1[r] = __builtin_amdgcn_exp2f(s1[r] - m);
      ls += s0[r] + s1[r];
    }
    l += ls;
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pb[0][jj][e] = (__bf16)s0[8 * jj + e];
        pb[1][jj][e] = (__bf16)s1[8 * jj + e];
      }
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
          if (jt >= 1) accumulate(kt + ((jt - 1) % kBufs) * kTileElems);
          if (jt < ntiles) scores(kt + (jt % kBufs) * kTileElems);
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
        if (live) softmax(jt * kKT);
      }
    }
    __syncthreads();
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  const float inv = 1.f / sum_across_halves(l);
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

template <int DC>
hipError_t launch_dc(const AttnArgs& a, bool f32, hipStream_t s) {
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
