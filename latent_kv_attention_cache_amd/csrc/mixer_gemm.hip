// Projections of the whole attention layer for gfx950 (query latent and output
// mixer), as one tiled bf16 GEMM with two epilogues, plus the one-time weight
// folds.
//
// VideoMLA (paperlayer.ai summary of arXiv:2605.30351v1): the layer's queries
// come from a d_q-wide query latent (§4 "Implementation Details", d_q = 768);
// App. E "Content-path absorption" applies a fixed per-head matrix A_h to that
// latent, so the content score is taken against the cached latent c directly;
// "Value-path absorption" projects the softmax-weighted latents with B_h folded
// into the output mixer; "RoPE branch" keeps the positional columns separate.
//
//   gemm_kernel<TA, TO, kPlain>: out[m][n] = sum_k A[m][k] W[k][n]   (TO storage)
//   gemm_kernel<TA, bf16, kHead>: per-head query rows. The columns are head_w
//     wide per head, the last ones from rope_off on are RoPE pairs; the
//     epilogue rotates them with the token's (t, h, w), multiplies everything
//     by scale * log2(e) and scatters each head's row to out[b][h][n]. Over the
//     folded query weights [A_h | W_UQ^R[h]] (head_w 224) this is the latent
//     attention's Qhat; over W_Q (head_w 128) the explicit form's queries.
//   gemm_kernel<TA, bf16, kKV>: explicit reconstruction ([PL] §3 "On-demand
//     reconstruction") over the cache rows of one batch element and the packed
//     per-head [W_K_up[h] | W_V_up[h]] (224 columns per head): row m of head h
//     becomes kv[h][m] = [c W_K_up[h] (96) | k_R of row m (32) | c W_V_up[h] (128)].
//
// Tile: 128 rows x 256 columns, four waves, one per SIMD; wave (rh, ch) owns
// rows 64 rh .. +63 and columns 128 ch .. +127 of the tile and computes
// out^T = W^T A^T with v_mfma_f32_16x16x32_bf16, so a lane ends with four
// consecutive columns of one row (a RoPE pair never straddles lanes). The K
// loop is a 3-stage pipeline of 64-deep slices fetched by LDS-DMA two stages
// ahead: A row-major with the chunk swizzle of staging.h; W row-major, 512-byte
// rows, chunk c of row k at position c ^ 2 t(k), t(k) = (k & 3) | bit3(k) << 2,
// so that a transposed operand read of 32 lanes (rows k0 .. k0+3 and
// k0+8 .. k0+11) covers all 64 banks once. Columns past n are loaded from
// column n - 8 (any finite data; their results are not stored); rows past m
// repeat the last row.
#include "device_common.h"
#include "kernels.h"
#include "staging.h"

namespace vmla {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kColsT = 256;                       // columns per workgroup
constexpr int kCB = 8;                            // 16-column blocks per wave
constexpr int kWElems = kStageK * kColsT;         // W slice of a stage
constexpr int kWLoads = kWElems * 2 / 1024;       // 32
constexpr int kStages = 3;
constexpr int kWPerWave = kWLoads / kWaves;       // 8
constexpr int kWChunks = kColsT / 8;              // 32 chunks per W tile row

// Row tile of NRB 16-row blocks per wave: 128 rows (NRB = 4), or 64 rows
// (NRB = 2) for launches that would otherwise leave most compute units idle.
template <int NRB>
struct GShape {
  static constexpr int kRowsT = 32 * NRB;                 // rows per workgroup
  static constexpr int kXElems = kRowsT * kStageK;        // A slice of a stage
  static constexpr int kXPerWave = kXElems * 2 / 1024 / kWaves;   // NRB wave-wide 1 KB loads
  static constexpr int kStageElems = kXElems + kWElems;
  static constexpr int kL = kXPerWave + kWPerWave;        // loads per wave per stage
  static_assert(kXElems * 2 / 1024 % kWaves == 0 && kWLoads % kWaves == 0, "loads split evenly");
  static_assert(kStages * kStageElems * 2 <= 160 * 1024, "LDS budget");
};

enum { kPlain = 0, kHead = 1, kKV = 2 };

__device__ __forceinline__ float to_f32(bf16_t v) { return bf2f(v); }
__device__ __forceinline__ float to_f32(float v) { return v; }

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// chunk permutation mask of W tile row k (an involution on the chunks of a row)
__device__ __forceinline__ int swz_w(int k) { return 2 * ((k & 3) | (((k >> 3) & 1) << 2)); }

template <typename T> __device__ __forceinline__ void store4(T* p, float a, float b, float c, float d);
template <> __device__ __forceinline__ void store4<bf16_t>(bf16_t* p, float a, float b, float c, float d) {
  *reinterpret_cast<uint2*>(p) = uint2{pack2(a, b), pack2(c, d)};
}
template <> __device__ __forceinline__ void store4<float>(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<float4*>(p) = float4{a, b, c, d};
}

template <typename TA, typename TO, int kMode, int NRB>
__global__ __launch_bounds__(kThreads)
void gemm_kernel(GemmArgs a) {
  constexpr int kNRB = NRB;
  constexpr int kRowsT = GShape<NRB>::kRowsT;
  constexpr int kXElems = GShape<NRB>::kXElems;
  constexpr int kXPerWave = GShape<NRB>::kXPerWave;
  constexpr int kStageElems = GShape<NRB>::kStageElems;
  constexpr int kL = GShape<NRB>::kL;
  __shared__ __attribute__((aligned(16))) bf16_t smem[kStages * kStageElems];
  constexpr bool kBf16 = std::is_same_v<TA, bf16_t>;

  // Workgroups are dispatched round-robin over the 8 XCDs; id = 8 (NC q + ct) + x8
  // keeps every column tile of row tile 8 q + x8 on XCD x8, so that tile's A rows
  // are fetched into that XCD's L2 once and shared by its column tiles.
  const int n_rt = (int)((a.m + kRowsT - 1) / kRowsT);
  const int n_ct = (a.n + kColsT - 1) / kColsT;
  const int x8 = blockIdx.x & 7;
  const int rest = blockIdx.x >> 3;
  const int ct = rest % n_ct;
  const int rt = 8 * (rest / n_ct) + x8;
  if (rt >= n_rt) return;                   // whole workgroup: no barrier is skipped

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int g = lane >> 4;
  const int j = lane & 15;
  const int rh = wv >> 1, ch = wv & 1;      // wave-uniform
  const int64_t m0 = (int64_t)rt * kRowsT;
  const int rows = (int)min<int64_t>(kRowsT, a.m - m0);
  const int col0 = kColsT * ct;
  const TA* xw = static_cast<const TA*>(a.a) + m0 * a.lda;
  const TA* ww = static_cast<const TA*>(a.w);
  const int nst = a.k / kStageK;

  // W load n = 8 wv + i moves rows 2n, 2n+1 of the slice; lane q = 64 n + lane
  // fills stored chunk position cp of row k with logical chunk cp ^ swz_w(k).
  auto w_col = [&](int i) {
    const int q = 64 * (kWPerWave * wv + i) + lane, k = q / kWChunks, cp = q - k * kWChunks;
    const int col = min(col0 + 8 * (cp ^ swz_w(k)), a.n - 8);
    return k * a.n + col;                   // element offset within the slice
  };
  uint32_t voff[kL];
  if constexpr (kBf16) {
#pragma unroll
    for (int i = 0; i < kXPerWave; ++i) voff[i] = stage_a_voff(a.lda, 0, rows, kXPerWave * wv + i, lane);
#pragma unroll
    for (int i = 0; i < kWPerWave; ++i) voff[kXPerWave + i] = (uint32_t)w_col(i) * 2u;
  }
  auto issue = [&](int sb, int sd, int i0, int i1) {   // loads i0 <= i < i1: data of stage sd, buffer of sb
    bf16_t* st = smem + (sb % kStages) * kStageElems;
    const int k0 = sd * kStageK;
#pragma unroll
    for (int i = 0; i < kL; ++i) {
      if (i < i0 || i >= i1) continue;
      if (i < kXPerWave) {
        const int n = kXPerWave * wv + i;
        if constexpr (kBf16) dma16_lds(xw + k0, voff[i], lds_u32(st + 512 * n));
        else stage_a_load<TA>(st, xw, a.lda, 0, rows, k0, n, lane);
      } else {
        const int n = kWPerWave * wv + (i - kXPerWave);
        bf16_t* dst = st + kXElems + 512 * n;
        if constexpr (kBf16) {
          dma16_lds(ww + (size_t)k0 * a.n, voff[i], lds_u32(dst));
        } else {
          *reinterpret_cast<uint4*>(dst + 8 * lane) =
              load8_bf16<TA>(ww + (size_t)k0 * a.n + w_col(i - kXPerWave));
        }
      }
    }
  };

  // Operand offsets (elements, relative to a stage's tiles).
  // A (B operand of the MFMA): lane (j, g) of block rb = row 64 rh + 16 rb + j, chunk 4 kk + g.
  int a_off[kNRB][2];
#pragma unroll
  for (int rb = 0; rb < kNRB; ++rb) {
    const int row = 16 * kNRB * rh + 16 * rb + j;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) a_off[rb][kk] = 64 * row + 8 * ((4 * kk + g) ^ swz_a(row));
  }
  // W (A operand) by ds_read_b64_tr_b16: lane j of group g points at row
  // 32 kk + 8 g + j/4 (+4 for the upper half) and columns col + 4 (j%4) .. +3
  // of column block cb of half ch. The swizzle bits of that row (bits 0, 1, 3)
  // depend on the lane only.
  int b_off[kCB];
  {
    const int k = 8 * g + (j >> 2);
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb) {
      const int c = 2 * (kCB * ch + cb) + ((j & 3) >> 1);
      b_off[cb] = k * kColsT + 8 * (c ^ swz_w(k)) + 4 * (j & 1);
    }
  }

  for (int s = 0; s < kStages - 1 && s < nst; ++s) issue(s, s, 0, kL);

  f32x4 acc[kNRB][kCB];
#pragma unroll
  for (int rb = 0; rb < kNRB; ++rb)
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb) acc[rb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Stage s: two 32-deep steps of 4 x 8 MFMAs; the next A fragment and the W
  // fragments of the second step are read while the current MFMAs run. Past
  // the last stage the loads repeat the last stage into a buffer that is not
  // read again, so the stage body has no branch; every iteration issues one
  // stage, so min(kStages - 2, nst - 1) stages are in flight behind stage s.
  const int behind = min(kStages - 2, nst - 1);
  for (int s = 0; s < nst; ++s) {
    wait_stages<kL>(behind);                                    // stage s has landed
    __syncthreads();
    const int sn = min(s + kStages - 1, nst - 1);
    const bf16_t* X = smem + (s % kStages) * kStageElems;
    const bf16_t* W = X + kXElems;
    auto read_w = [&](int kk, bf16x8* bw) {
#pragma unroll
      for (int cb = 0; cb < kCB; ++cb) {
        const bf16_t* p = W + b_off[cb] + 32 * kk * kColsT;
        const bf16x4 lo = lds_tr4(p);
        const bf16x4 hi = lds_tr4(p + 4 * kColsT);
        bw[cb] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
    };
    bf16x8 b0[kCB], b1[kCB];
    read_w(0, b0);
    bf16x8 av = lds_row8(X + a_off[0][0]);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int rb = 0; rb < kNRB; ++rb) {
        const int q = kk * kNRB + rb;
        bf16x8 an = av;
        if (q + 1 < 2 * kNRB) an = lds_row8(X + a_off[(q + 1) % kNRB][(q + 1) / kNRB]);
        if (kk == 0 && rb == kNRB - 1) read_w(1, b1);
        issue(s + kStages - 1, sn, q * kL / (2 * kNRB), (q + 1) * kL / (2 * kNRB));
#pragma unroll
        for (int cb = 0; cb < kCB; ++cb)
          acc[rb][cb] = mfma16(kk == 0 ? b0[cb] : b1[cb], av, acc[rb][cb]);
        av = an;
      }
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");    // the trailing loads have landed

  // ---- epilogue. Register r of acc[rb][cb] in lane (j, g): row 64 rh + 16 rb + j
  // of the tile, column col0 + 128 ch + 16 cb + 4 g + r.
  const int cbase = col0 + 128 * ch + 4 * g;
  if constexpr (kMode == kPlain) {
    TO* out = static_cast<TO*>(a.out);
#pragma unroll
    for (int rb = 0; rb < kNRB; ++rb) {
      const int64_t m = m0 + 16 * kNRB * rh + 16 * rb + j;
      if (m >= a.m) continue;
#pragma unroll
      for (int cb = 0; cb < kCB; ++cb) {
        const int col = cbase + 16 * cb;
        if (col >= a.n) continue;
        const f32x4 v = acc[rb][cb];
        store4<TO>(out + m * a.n + col, v[0], v[1], v[2], v[3]);
      }
    }
  } else if constexpr (kMode == kKV) {
    // column col = h (d_nope + kDV) + ci: ci < d_nope key part, else value part;
    // the lanes holding ci < d_rope = kDHead - d_nope also copy k_R (A columns
    // kDC .. kDC + d_rope - 1).
    const int d_nope = a.d_nope, d_rope = kDHead - a.d_nope;
    const int kCols = d_nope + kDV;
    uint16_t* kv = static_cast<uint16_t*>(a.out);
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb) {
      const int col = cbase + 16 * cb;
      if (col >= a.n) continue;
      const int h = col / kCols;
      const int ci = col - h * kCols;
      const int dst = ci < d_nope ? ci : ci + d_rope;
#pragma unroll
      for (int rb = 0; rb < kNRB; ++rb) {
        const int64_t m = m0 + 16 * kNRB * rh + 16 * rb + j;
        if (m >= a.m) continue;
        uint16_t* row = kv + ((int64_t)h * a.m + m) * (2 * kDHead);
        const f32x4 v = acc[rb][cb];
        store4<bf16_t>(row + dst, v[0], v[1], v[2], v[3]);
        if (ci < d_rope) {
          const TA* kr = static_cast<const TA*>(a.a) + m * a.lda + kDC + ci;
          store4<bf16_t>(row + d_nope + ci, to_f32(kr[0]), to_f32(kr[1]), to_f32(kr[2]), to_f32(kr[3]));
        }
      }
    }
  } else {
    // per-head rows: column col = head_w h + ci of head h; ci < rope_off plain
    // (scaled), ci >= rope_off rope pairs (ci - rope_off) / 2 and +1 (rotated,
    // then scaled).
    int64_t qrow[kNRB];                                // row of Qhat for head 0, -1 past m
    int pos[kNRB][3];                                  // (t, h, w) of each row
#pragma unroll
    for (int rb = 0; rb < kNRB; ++rb) {
      const int64_t m = m0 + 16 * kNRB * rh + 16 * rb + j;
      const int64_t mc = m < a.m ? m : a.m - 1;
      const int b = (int)(mc / a.n_q);
      const int n = (int)(mc - (int64_t)b * a.n_q);
      int n_in, ww2;
      const int f = div_small(n, a.tokens_per_frame, a.inv_tokens_per_frame, &n_in);
      const int hpos = div_small(n_in, a.grid_w, a.inv_grid_w, &ww2);
      pos[rb][0] = a.t_first + f;
      pos[rb][1] = hpos;
      pos[rb][2] = ww2;
      qrow[rb] = m < a.m ? (int64_t)b * a.n_heads * a.n_q + n : -1;
    }
    uint16_t* qhat = static_cast<uint16_t*>(a.out);
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb) {
      const int col = cbase + 16 * cb;
      if (col >= a.n) continue;
      const int h = col / a.head_w;
      const int ci = col - h * a.head_w;
      const bool rope = ci >= a.rope_off;
      // first of the lane's two pairs: (ci - rope_off) / 2 = pb + 2 g, pb the
      // 16-column block's first pair (blocks never straddle a head)
      const int pb = (ci - 4 * g - a.rope_off) >> 1;
#pragma unroll
      for (int rb = 0; rb < kNRB; ++rb) {
        if (qrow[rb] < 0) continue;
        f32x4 v = acc[rb][cb];
        if (rope) {
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            uint32_t lo, hi;
            int ax;
            rope_rate_by_group(a.rope, pb + q, g, &lo, &hi, &ax);
            float sn, cs;
            sincos_rev(pos[rb][ax], lo, hi, &sn, &cs);
            const float x0 = v[2 * q], x1 = v[2 * q + 1];
            v[2 * q] = x0 * cs - x1 * sn;
            v[2 * q + 1] = x0 * sn + x1 * cs;
          }
        }
        store4<bf16_t>(qhat + (qrow[rb] + (int64_t)h * a.n_q) * a.head_w + ci, v[0] * a.qscale,
                       v[1] * a.qscale, v[2] * a.qscale, v[3] * a.qscale);
      }
    }
  }
}

// ---- one-time weight folds (fp32 accumulation, bf16 results)

// W_QA[k][h kRow + c] = sum_n W_UQ[k][h kDHead + n] W_K_up[h][c][n]   (c < kDC)
//                     = W_UQ[k][h kDHead + kDNope + c - kDC]           (c >= kDC)
template <typename T>
__global__ __launch_bounds__(256)
void fold_query_kernel(FoldArgs a) {
  const int64_t total = (int64_t)a.d_in * a.n_heads * kRow;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int k = (int)(i / (a.n_heads * kRow));
  const int col = (int)(i - (int64_t)k * a.n_heads * kRow);
  const int h = col / kRow, c = col - h * kRow;
  const T* uq = static_cast<const T*>(a.w_first) + (size_t)k * a.n_heads * kDHead + (size_t)h * kDHead;
  float v;
  if (c < kDC) {
    const T* ku = static_cast<const T*>(a.w_second) + ((size_t)h * kDC + c) * kDNope;
    v = 0.f;
    for (int n = 0; n < kDNope; ++n) v = fmaf(to_f32(uq[n]), to_f32(ku[n]), v);
  } else {
    v = to_f32(uq[kDNope + c - kDC]);
  }
  static_cast<bf16_t*>(a.out)[i] = f2bf(v);
}

// W_VO[h kDC + c][j] = sum_e W_V_up[h][c][e] W_O[h kDV + e][j]
template <typename T>
__global__ __launch_bounds__(256)
void fold_output_kernel(FoldArgs a) {
  const int64_t total = (int64_t)a.n_heads * kDC * a.d_out;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int r = (int)(i / a.d_out);
  const int jc = (int)(i - (int64_t)r * a.d_out);
  const int h = r / kDC;
  const T* vu = static_cast<const T*>(a.w_first) + (size_t)r * kDV;
  const T* wo = static_cast<const T*>(a.w_second) + (size_t)h * kDV * a.d_out + jc;
  float v = 0.f;
  for (int e = 0; e < kDV; ++e) v = fmaf(to_f32(vu[e]), to_f32(wo[(size_t)e * a.d_out]), v);
  static_cast<bf16_t*>(a.out)[i] = f2bf(v);
}

template <int NRB>
void launch_nrb(const GemmArgs& a, int a_f32, int out_f32, hipStream_t s) {
  const int64_t n_rt = (a.m + GShape<NRB>::kRowsT - 1) / GShape<NRB>::kRowsT;
  const int n_ct = (a.n + kColsT - 1) / kColsT;
  const dim3 grid((unsigned)(8 * n_ct * ((n_rt + 7) / 8)));
  if (a.mode == kHead) {
    if (a_f32) hipLaunchKernelGGL((gemm_kernel<float, bf16_t, kHead, NRB>), grid, dim3(kThreads), 0, s, a);
    else hipLaunchKernelGGL((gemm_kernel<bf16_t, bf16_t, kHead, NRB>), grid, dim3(kThreads), 0, s, a);
  } else if (a.mode == kKV) {
    if (a_f32) hipLaunchKernelGGL((gemm_kernel<float, bf16_t, kKV, NRB>), grid, dim3(kThreads), 0, s, a);
    else hipLaunchKernelGGL((gemm_kernel<bf16_t, bf16_t, kKV, NRB>), grid, dim3(kThreads), 0, s, a);
  } else if (a_f32) {
    if (out_f32) hipLaunchKernelGGL((gemm_kernel<float, float, kPlain, NRB>), grid, dim3(kThreads), 0, s, a);
    else hipLaunchKernelGGL((gemm_kernel<float, bf16_t, kPlain, NRB>), grid, dim3(kThreads), 0, s, a);
  } else {
    if (out_f32) hipLaunchKernelGGL((gemm_kernel<bf16_t, float, kPlain, NRB>), grid, dim3(kThreads), 0, s, a);
    else hipLaunchKernelGGL((gemm_kernel<bf16_t, bf16_t, kPlain, NRB>), grid, dim3(kThreads), 0, s, a);
  }
}

}  // namespace

// 128-row tiles, unless they would occupy at most half of the compute units:
// then 64-row tiles, twice as many workgroups in the same single round.
hipError_t launch_gemm(const GemmArgs& a, int a_f32, int out_f32, hipStream_t s) {
  const int64_t tiles = (a.m + 127) / 128 * ((a.n + kColsT - 1) / kColsT);
  if (tiles <= 128) launch_nrb<2>(a, a_f32, out_f32, s);
  else launch_nrb<4>(a, a_f32, out_f32, s);
  return hipGetLastError();
}

hipError_t launch_fold_query(const FoldArgs& a, bool f32, hipStream_t s) {
  const int64_t total = (int64_t)a.d_in * a.n_heads * kRow;
  const dim3 grid((unsigned)((total + 255) / 256));
  if (f32) hipLaunchKernelGGL(fold_query_kernel<float>, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(fold_query_kernel<bf16_t>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_fold_output(const FoldArgs& a, bool f32, hipStream_t s) {
  const int64_t total = (int64_t)a.n_heads * kDC * a.d_out;
  const dim3 grid((unsigned)((total + 255) / 256));
  if (f32) hipLaunchKernelGGL(fold_output_kernel<float>, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(fold_output_kernel<bf16_t>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace vmla
