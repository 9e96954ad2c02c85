// Latent-form chunk attention for wide content latents (d_c = 256, 512) on
// gfx950.
//
// VideoMLA (paperlayer.ai summary of arXiv:2605.30351v1): the latent widths of
// the batch-scaling measurement (§4 "Batch Scaling Under Fixed Memory", d_c up
// to 512) and the latent-dimension ablation (App. F). The math is the one of
// latent_attn_kernel (App. E "Inference-Time Reparameterization"): scores of the
// absorbed queries Qhat_h = [q_lat | q_rope] against the cached rows [c | k_R],
// online softmax, O_lat += P c, out = (O_lat / l) W_V_up[h].
//
// Why a second kernel. Per wave of 32 queries the O^T accumulators take d_c x 32
// fp32 (128 or 256 registers per lane) and the Qhat fragments d_c + 32 bf16
// (72 or 136): more than the 256 registers of a wave when two waves share a
// SIMD. Here a workgroup is four waves, one per SIMD, each with the SIMD's
// whole register file (the O^T accumulators live in the accumulation
// registers). Without a partner wave there is no ping-pong; at d_c = 256 a
// wave instead pipelines its own tiles: the exps, row sums and bf16 packing of
// tile j - 1 run between the score MFMAs of tile j (a wave's vector work next
// to its own MFMAs costs little), then P.C of tile j - 1, then the max and
// rescale decision of tile j, while tile j + 1 streams into a third buffer.
//
// Work split. Units of 32 queries of one head, numbered head-major with the
// units of a head padded to a multiple of the units per workgroup, so that a
// workgroup's units belong to one head (its W_V_up[h] is staged once for the
// epilogue). At d_c = 256 each of the four waves takes one unit. At d_c = 512
// the whole O^T (256 registers) and Qhat (136) still do not fit one wave
// without spills, so two waves share a unit: wave k of the pair scores keys
// 32 k .. 32 k + 31 of each tile, the pair swaps its maxima through LDS (both
// then hold the same reference max), each wave packs its P^T to bf16 and
// swaps it too, and each accumulates one half of the latent dimensions over
// all 64 keys (128 accumulation registers). The exponent sums and the two
// halves of (O / l) W_V_up[h] are combined through LDS in the epilogue. Per
// unit and tile the pair issues the 132 MFMAs of one wave with the whole
// row, at three barriers per tile instead of one.
//
// Tile. 64 keys, chunk-major and padded in LDS as in latent_attn_kernel (chunk
// c of key row r at slot c * 68 + r), copied by 16-byte LDS-DMA loads that all
// four waves share; three buffers at d_c = 256 (117 KB), two at 512 (148 KB).
//
// Per tile, per wave: S^T = K Qhat^T (2 x (d_c + 32) / 16 MFMAs 32x32x16, in
// four accumulation chains at d_c = 256), softmax of its 64 keys with the lazy
// reference max, P^T packed to bf16 in place, O^T += C^T P^T (d_c / 32 x 4
// MFMAs) with C^T read by the LDS transpose read. One barrier per tile.
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace vmla {
namespace {

constexpr int kKT = 64;                     // keys per tile
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kSlots = kKT + 4;             // slots per chunk column (padded)
constexpr int kVLd = kDV + 8;               // padded LDS row of W_V_up[h] (epilogue)
constexpr float kLazy = 8.f;                // lazy-rescale threshold (log2 units)
// Scheduling-group masks (instruction classes of sched_group_barrier).
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;

template <int DC>
struct WideShape {
  static constexpr bool kPair = DC > 256;                  // two waves per unit (latent halves)
  static constexpr int kUnitsWG = kPair ? kWaves / 2 : kWaves;
  static constexpr int kRow = DC + kDRope;
  static constexpr int kChunks = kRow / 8;                 // 36 / 68
  static constexpr int kTileElems = kChunks * kSlots * 8;
  static constexpr int kLoadsPerWave = kChunks / kWaves;   // 9 / 17
  static constexpr int kFeatSteps = kRow / 16;             // 18 / 34
  static constexpr int kLatTiles = DC / 32;                // 8 / 16
  static constexpr int kOTiles = kPair ? kLatTiles / 2 : kLatTiles;   // latent tiles of one wave
  static_assert(kChunks % kWaves == 0, "tile loads split evenly over the four waves");
  static_assert(!kPair || (DC / 2) * kVLd * 2 + kUnitsWG * (kDV / 32) * 16 * 64 * 4 <= 2 * kTileElems * 2,
                "epilogue staging of one W_V_up half and the partial outputs fits the tile buffers");
  // pair exchange area after the tile buffers: maxima [wave][lane] (fp32)
  // and packed P^T [wave][step][lane] (16 bytes)
  static constexpr int kXchElems = kPair ? (kWaves * 64 * 4 + kWaves * 2 * 64 * 16) / 2 : 0;
  // one wave per unit pipelines tiles (C^T of tile j - 1, K of tile j, tile
  // j + 1 in flight): three buffers; the wave pair keeps two
  static constexpr int kBufs = kPair ? 2 : 3;
  static_assert(kBufs * kTileElems * 2 + kXchElems * 2 <= 160 * 1024, "tile buffers in LDS");
  static_assert((kPair ? DC / 2 : DC) * kVLd <= 2 * kTileElems, "staged W_V_up rows fit the tile buffers");
};

__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(voff), "s"(base), "s"(__builtin_amdgcn_readfirstlane(lds_addr)) : "memory");
}

template <int DC>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void latent_attn_wide_kernel(AttnArgs a) {
  using Sh = WideShape<DC>;
  constexpr int kRow = Sh::kRow;
  constexpr int kTileElems = Sh::kTileElems;
  constexpr int kFeatSteps = Sh::kFeatSteps;
  constexpr int kOTiles = Sh::kOTiles;
  constexpr int kUnitsWG = Sh::kUnitsWG;
  __shared__ __attribute__((aligned(16))) bf16_t kt[Sh::kBufs * kTileElems + Sh::kXchElems];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int qi = lane & 31;
  const int b = blockIdx.z;
  const int unit = Sh::kPair ? wave >> 1 : wave;             // unit of this wave in the workgroup
  const int lat_half = Sh::kPair ? wave & 1 : 0;             // latent half of this wave (d_c 512)
  const int units = (a.n_q + 31) / 32;
  const int upad = (units + kUnitsWG - 1) / kUnitsWG * kUnitsWG;   // units per head, padded
  const int h = (blockIdx.x * kUnitsWG) / upad;              // one head per workgroup
  const int qb = blockIdx.x * kUnitsWG - h * upad + unit;
  const int qrow = 32 * qb + qi;
  const bool live = qb < units;                              // wave-uniform
  const bool qvalid = live && qrow < a.n_q;

  // Qhat fragments (B operand of S^T): lane holds features 16 ks + 8 half .. +7 of its query.
  bf16x8 qf[kFeatSteps];
  {
    const bf16_t* qp = a.qhat + (((size_t)b * a.n_heads + h) * a.n_q + (qvalid ? qrow : a.n_q - 1)) * kRow;
#pragma unroll
    for (int ks = 0; ks < kFeatSteps; ++ks)
      qf[ks] = *reinterpret_cast<const bf16x8*>(qp + ks * 16 + 8 * half);
#pragma unroll
    for (int ks = 0; ks < kFeatSteps; ++ks) asm volatile("" : "+v"(qf[ks]));
  }

  const bf16_t* cache = static_cast<const bf16_t*>(a.cache) + (size_t)b * a.cache_rows * kRow;
  const int nk = a.n_k;
  const int ntiles = (nk + kKT - 1) / kKT;
  const uint32_t kt_lds = (uint32_t)(uintptr_t)(VMLA_LDS bf16_t*)kt;
  // Wave-wide load n moves chunk column n of tile j: lane r reads features
  // 8n .. 8n+7 of key 64 j + r (clamped to the last key; masked scores).
  auto issue_tile = [&](int j) {
    const int kg = min(j * kKT + lane, nk - 1);
    const int wv = __builtin_amdgcn_readfirstlane(wave);
#pragma unroll
    for (int i = 0; i < Sh::kLoadsPerWave; ++i) {
      const int n = wv + kWaves * i;
      dma16(cache, (uint32_t)(kg * (kRow * 2)) + (uint32_t)(16 * n),
            kt_lds + 2u * (uint32_t)((j % Sh::kBufs) * kTileElems + n * kSlots * 8));
    }
  };

  const int a_base = (half * kSlots + qi) * 8;
  const int jl = lane & 15;
  const int x4 = ((lane & 16) >> 3) + ((jl & 3) >> 1);
  const int sub = 4 * (jl & 1);
  const int v_off1 = (x4 * kSlots + 4 * half + (jl >> 2)) * 8 + sub;
  const int v_off2 = v_off1 + 8 * 8;

  f32x16 o[kOTiles];                     // this wave's latent tiles: kOTiles lat_half + t
#pragma unroll
  for (int t = 0; t < kOTiles; ++t) o[t] = f32x16{};
  float m = -INFINITY;
  float l = 0.f;

  issue_tile(0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if constexpr (Sh::kPair) {
    float* xmax = reinterpret_cast<float*>(kt + 2 * kTileElems);          // [wave][lane]
    uint4* xp = reinterpret_cast<uint4*>(xmax + kWaves * 64);             // [wave][step][lane]
    const int partner = wave ^ 1;
    const int kb_own = lat_half;                                          // this wave's key block
    for (int jt = 0; jt < ntiles; ++jt) {
      if (jt + 1 < ntiles) issue_tile(jt + 1);     // into the buffer read in tile jt - 1
      const bf16_t* K = kt + (jt & 1) * kTileElems;
      f32x16 sc = f32x16{};                        // S^T of keys 32 kb_own + 8(r/4) + 4 half + r%4
      float mx = -INFINITY;
      if (live) {
#pragma unroll
        for (int ks = 0; ks < kFeatSteps; ++ks)
          sc = mfma32(lds_row8(K + a_base + 2 * kSlots * 8 * ks + 32 * 8 * kb_own), qf[ks], sc);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 4, 0);
#pragma unroll
        for (int i = 0; i < kFeatSteps - 4; ++i) {
          __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
          __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 4, 0);
        const int key0 = jt * kKT;
        if (key0 + kKT > nk) {
          const int lim = nk - key0 - 4 * half;
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (32 * kb_own + 8 * (r >> 2) + (r & 3) >= lim) sc[r] = -INFINITY;
        }
        mx = sc[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sc[r]);
        mx = max_across_halves(mx);
        xmax[wave * 64 + lane] = mx;
      }
      __syncthreads();                             // both halves' maxima visible
      bf16x8 pown[2];
      if (live) {
        mx = fmaxf(mx, xmax[partner * 64 + lane]); // the same value in both waves of the pair
        const bool grow = mx > m + kLazy;
        if (__builtin_amdgcn_ballot_w64(grow)) {
          const float m_new = grow ? mx : m;
          const float alpha = __builtin_amdgcn_exp2f(m - m_new);
          l *= alpha;
#pragma unroll
          for (int t = 0; t < kOTiles; ++t) o[t] *= alpha;
          m = m_new;
        }
        float ls = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          sc[r] = __builtin_amdgcn_exp2f(sc[r] - m);
          ls += sc[r];
        }
        l += ls;
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
#pragma unroll
          for (int e = 0; e < 8; ++e) pown[jj][e] = (__bf16)sc[8 * jj + e];
          xp[(wave * 2 + jj) * 64 + lane] = __builtin_bit_cast(uint4, pown[jj]);
        }
      }
      __syncthreads();                             // both halves' P^T visible
      if (live) {
        bf16x8 ppart[2];
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) ppart[jj] = __builtin_bit_cast(bf16x8, xp[(partner * 2 + jj) * 64 + lane]);
        // O^T(latent half) += C^T(tile) P^T over all 64 keys
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            const bf16_t* Kb = K + (kb * 32 + jj * 16) * 8;
            const bf16x8 pv = kb == kb_own ? pown[jj] : ppart[jj];
#pragma unroll
            for (int t = 0; t < kOTiles; ++t) {
              const int ct = 4 * kSlots * 8 * (t + kOTiles * lat_half);
              const bf16x4 lo = lds_tr4(Kb + v_off1 + ct);
              const bf16x4 hi = lds_tr4(Kb + v_off2 + ct);
              o[t] = mfma32(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7), pv, o[t]);
            }
          }
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 8, 1);
#pragma unroll
        for (int i = 0; i < 4 * kOTiles - 4; ++i) {
          __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 1);
          __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 1);
        }
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 4, 1);
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's loads of tile jt + 1
      __syncthreads();                                    // tile jt + 1 complete, buffer jt free
    }
    // the exponent sums of the two key halves: l of the pair = l + l(partner)
    xmax[wave * 64 + lane] = l;
    __syncthreads();
    l += xmax[partner * 64 + lane];
    __syncthreads();                               // the exchange area is free again
  } else {
    // Software pipeline over tiles. Iteration jt issues the score MFMAs of tile
    // jt with the exps, row sums and bf16 packing of tile jt - 1 spread between
    // them (one wave per SIMD, so the exps sit between this wave's own MFMAs),
    // then P.C of tile jt - 1, then the max and lazy rescale of tile jt.
    // S^T of tile jt sits in set jt % 2: register r of key block kb holds key
    // 32 kb + 8(r/4) + 4 half + r%4.
    f32x16 sc[2][2];
    bf16x8 pb[2][2];
    auto buf = [&](int j) { return kt + (j % Sh::kBufs) * kTileElems; };
    // items n0 .. n1 - 1 of set Q: exp of register n % 16 of key block n / 16
    // against the reference max, its row sum, and every eighth a bf16 fragment
    float ls[2] = {0.f, 0.f};
    auto items = [&](auto qc, int n0, int n1) {
      constexpr int Q = decltype(qc)::value;
#pragma unroll
      for (int n = n0; n < n1; ++n) {
        const int kb = n / 16, r = n % 16;
        sc[Q][kb][r] = __builtin_amdgcn_exp2f(sc[Q][kb][r] - m);
        ls[n & 1] += sc[Q][kb][r];
        if (r % 8 == 7) {
#pragma unroll
          for (int e = 0; e < 8; ++e) pb[kb][r / 8][e] = (__bf16)sc[Q][kb][8 * (r / 8) + e];
        }
      }
    };
    // S^T of tile j into set P; with kExp the items of set P ^ 1 between the
    // 2 kFeatSteps MFMAs. Operand rows are read kAhead feature steps ahead.
    constexpr int kAhead = 3;
    auto scores = [&](auto pc, auto ec, const bf16_t* K) {
      constexpr int P = decltype(pc)::value;
      constexpr bool kExp = decltype(ec)::value;
      constexpr int nm = 2 * kFeatSteps;
      // four accumulation chains: even feature steps into sc, odd ones into
      // sx, added at the end (two dependent chains leave the matrix core
      // waiting on each MFMA's result)
      f32x16 sx[2];
      sc[P][0] = f32x16{};
      sc[P][1] = f32x16{};
      sx[0] = f32x16{};
      sx[1] = f32x16{};
      bf16x8 fa[kAhead + 1][2];
#pragma unroll
      for (int ks = 0; ks < kAhead; ++ks) {
        fa[ks][0] = lds_row8(K + a_base + 2 * kSlots * 8 * ks);
        fa[ks][1] = lds_row8(K + a_base + 2 * kSlots * 8 * ks + 32 * 8);
      }
#pragma unroll
      for (int ks = 0; ks < kFeatSteps; ++ks) {
        if (ks + kAhead < kFeatSteps) {
          fa[(ks + kAhead) % (kAhead + 1)][0] = lds_row8(K + a_base + 2 * kSlots * 8 * (ks + kAhead));
          fa[(ks + kAhead) % (kAhead + 1)][1] = lds_row8(K + a_base + 2 * kSlots * 8 * (ks + kAhead) + 32 * 8);
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          if (ks & 1) sx[kb] = mfma32(fa[ks % (kAhead + 1)][kb], qf[ks], sx[kb]);
          else sc[P][kb] = mfma32(fa[ks % (kAhead + 1)][kb], qf[ks], sc[P][kb]);
          if constexpr (kExp) items(std::integral_constant<int, P ^ 1>{}, 32 * (2 * ks + kb) / nm, 32 * (2 * ks + kb + 1) / nm);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      sc[P][0] += sx[0];
      sc[P][1] += sx[1];
    };
    // O^T += C^T(tile) P^T
    auto accumulate = [&](const bf16_t* K) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          const bf16_t* Kb = K + (kb * 32 + jj * 16) * 8;
#pragma unroll
          for (int t = 0; t < kOTiles; ++t) {
            const int ct = 4 * kSlots * 8 * t;
            const bf16x4 lo = lds_tr4(Kb + v_off1 + ct);
            const bf16x4 hi = lds_tr4(Kb + v_off2 + ct);
            o[t] = mfma32(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7), pb[kb][jj], o[t]);
          }
        }
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 8, 1);
#pragma unroll
      for (int i = 0; i < 4 * kOTiles - 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 1);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 1);
      }
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 4, 1);
    };
    // mask, max and lazy rescale of tile j (set P)
    auto decide = [&](auto pc, int j) {
      constexpr int P = decltype(pc)::value;
      const int key0 = j * kKT;
      if (key0 + kKT > nk) {
        const int lim = nk - key0 - 4 * half;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int k = 8 * (r >> 2) + (r & 3);
          if (k >= lim) sc[P][0][r] = -INFINITY;
          if (k + 32 >= lim) sc[P][1][r] = -INFINITY;
        }
      }
      float mx = fmaxf(sc[P][0][0], sc[P][1][0]);
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, fmaxf(sc[P][0][r], sc[P][1][r]));
      mx = max_across_halves(mx);
      const bool grow = mx > m + kLazy;
      if (__builtin_amdgcn_ballot_w64(grow)) {
        const float m_new = grow ? mx : m;
        const float alpha = __builtin_amdgcn_exp2f(m - m_new);
        l *= alpha;
#pragma unroll
        for (int t = 0; t < kOTiles; ++t) o[t] *= alpha;
        m = m_new;
      }
    };
    auto iteration = [&](auto pc, auto ec, int jt) {
      constexpr int P = decltype(pc)::value;
      constexpr bool kExp = decltype(ec)::value;
      if (jt + 1 < ntiles) issue_tile(jt + 1);     // into the buffer of tile jt - 2
      if (live) {
        scores(pc, ec, buf(jt));
        if constexpr (kExp) {
          l += ls[0] + ls[1];
          ls[0] = ls[1] = 0.f;
          accumulate(buf(jt - 1));
        }
        decide(pc, jt);
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's loads of tile jt + 1
      __syncthreads();                                    // tile jt + 1 complete, tile jt - 2 free
    };
    iteration(std::integral_constant<int, 0>{}, std::false_type{}, 0);
    for (int jt = 1; jt < ntiles; jt += 2) {
      iteration(std::integral_constant<int, 1>{}, std::true_type{}, jt);
      if (jt + 1 < ntiles) iteration(std::integral_constant<int, 0>{}, std::true_type{}, jt + 1);
    }
    if (live) {                                     // the last tile's exps and P.C
      if ((ntiles - 1) & 1) items(std::integral_constant<int, 1>{}, 0, 32);
      else items(std::integral_constant<int, 0>{}, 0, 32);
      l += ls[0] + ls[1];
      accumulate(buf(ntiles - 1));
    }
    __syncthreads();                                // every tile read before the staging
  }

  // ---- epilogue: out = (O / l) @ W_V_up[h]. The W_V_up[h] rows of a latent
  // half, [DC / 2][kVLd] (or all DC rows), are staged in LDS; with two waves
  // per unit the half-0 wave leaves its partial product in LDS (fp32) and the
  // half-1 wave adds it before the store.
  const float inv = 1.f / sum_across_halves(l);
  bf16x8 ob[kOTiles][2];
#pragma unroll
  for (int t = 0; t < kOTiles; ++t)
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
      for (int e = 0; e < 8; ++e) ob[t][jj][e] = (__bf16)(o[t][8 * jj + e] * inv);
  bf16_t* out = static_cast<bf16_t*>(a.out) + (((size_t)b * a.n_q + (qvalid ? qrow : 0)) * a.n_heads + h) * kDV;
  constexpr int kStageRows = kOTiles * 32;                   // W_V_up rows staged per phase
  constexpr int kPhases = Sh::kPair ? 2 : 1;
  float* xch = reinterpret_cast<float*>(kt + kStageRows * kVLd);   // [unit][et][r][lane] partials
  const bf16_t* wsrc = static_cast<const bf16_t*>(a.w_v_up) + (size_t)h * DC * kDV;
  for (int ph = 0; ph < kPhases; ++ph) {
    for (int c = tid; c < kStageRows * kDV / 8; c += kThreads) {
      const int row = c / (kDV / 8), cc = c % (kDV / 8);
      *reinterpret_cast<uint4*>(&kt[row * kVLd + 8 * cc]) =
          *reinterpret_cast<const uint4*>(wsrc + ((size_t)ph * kStageRows + row) * kDV + 8 * cc);
    }
    __syncthreads();
    if (live && lat_half == ph) {
#pragma unroll
      for (int et = 0; et < kDV / 32; ++et) {
        f32x16 acc = f32x16{};
#pragma unroll
        for (int t = 0; t < kOTiles; ++t)
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            const int dbase = 32 * t + 16 * jj;
            acc = mfma32(lds_tr8(kt, kVLd, dbase + 4 * half, dbase + 8 + 4 * half, 32 * et, lane), ob[t][jj], acc);
          }
        float* xp = xch + ((unit * (kDV / 32) + et) * 16) * 64 + lane;
        if (ph + 1 < kPhases) {                              // half 0 of a pair: leave the partial
#pragma unroll
          for (int r = 0; r < 16; ++r) xp[64 * r] = acc[r];
          continue;
        }
        if constexpr (Sh::kPair) {
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[r] += xp[64 * r];
        }
        if (qvalid) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int e0 = 32 * et + 8 * g + 4 * half;
            *reinterpret_cast<uint2*>(out + e0) =
                uint2{pack2(acc[4 * g], acc[4 * g + 1]), pack2(acc[4 * g + 2], acc[4 * g + 3])};
          }
        }
      }
    }
    __syncthreads();                                         // staging area and partials reused
  }
}

template <int DC>
hipError_t launch_wide_dc(const AttnArgs& a, hipStream_t s) {
  constexpr int kU = WideShape<DC>::kUnitsWG;
  const int units = (a.n_q + 31) / 32;
  const int upad = (units + kU - 1) / kU * kU;
  const dim3 grid((unsigned)(a.n_heads * upad / kU), 1, (unsigned)a.batch);
  hipLaunchKernelGGL(latent_attn_wide_kernel<DC>, grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

// bf16 cache, one query chunk, k_R rotated at append, W_V_up epilogue, the
// default 96/32 split (validated by the host layer).
hipError_t launch_latent_attn_wide(const AttnArgs& a, hipStream_t s) {
  switch (a.d_c) {
    case 256: return launch_wide_dc<256>(a, s);
    case 512: return launch_wide_dc<512>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace vmla
