// Query prologue for gfx950: per head h, with the NoPE/RoPE split DN / 128 - DN
// (96 / 32 by default; 64 / 64, 32 / 96 and 112 / 16 are the split variants),
//   q_h     = x @ W_Q[:, h*128 : h*128+128]            (nope DN | rope 128 - DN)
//   q_rope  = RoPE3D(q_h[DN:128], (t, h, w))
//   q_lat   = q_h[0:DN] @ W_K_up[h]^T                   (DN -> d_c)
//   Qhat_h  = (scale * log2 e) * [q_lat | q_rope]       stored bf16
//
// VideoMLA (paperlayer.ai summary of arXiv:2605.30351v1), App. E
// "Content-path absorption": the content score is taken against the cached
// latent through a fixed matrix applied to the query side, so no per-head key
// is built; "RoPE branch": the positional part stays separate and is rotated
// with the token's (t, h, w) (App. D.3). Folding log2 e into the scale lets the
// attention kernel use exp2 directly.
//
// Tile: 128 query rows (256 for large grids; batch x tokens flattened, so a
// tile may span two batch elements) x two heads (256 columns of W_Q). Per
// output the L2 traffic of the projection is (1/128 + 1/256) of the operand
// bytes (1/256 + 1/256 with 256-row tiles). Eight waves, two per SIMD (one
// wave's LDS and barrier waits overlap the other's MFMAs): wave (rh, hh)
// computes rows R rh .. R rh + R - 1 (R = 32 or 64) and the 128 columns of head hh of
// the pair with v_mfma_f32_16x16x32_bf16 as out^T = W^T x^T, so that
// a lane holds four consecutive columns of one row (a RoPE pair sits in one
// lane). The d_model contraction runs as a pipeline of 64-deep slices of x
// (row-major, chunk-swizzled) and W_Q (row-major, 512-byte rows, chunk c of
// row k at position c ^ 2 t(k), t(k) = (k & 3) | bit3(k) << 2, so that a
// transposed operand read of 32 lanes, rows k0 .. k0+3 and k0+8 .. k0+11,
// covers all 64 banks once), three stages in LDS fetched by LDS-DMA two
// stages ahead, each wave issuing its share of the next loads between its
// MFMAs (256-row tiles: two stages, the next one's loads all issued as the
// current one starts).
//
// Epilogue, per wave and in registers: RoPE on the 32 rope columns and their
// store; q_nope goes to LDS as bf16, and q_lat^T = W_K_up[h] q_nope^T by MFMA
// with the W_K_up rows (contiguous in the contraction index) read straight
// from global memory; results are stored 8 bytes per lane.
#include "device_common.h"
#include "kernels.h"
#include "staging.h"

namespace vmla {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kHeadsT = 2;                        // heads per workgroup
constexpr int kColsT = kHeadsT * kDHead;          // 256 columns of W_Q
constexpr int kCB = kDHead / 16;                  // 8 column blocks per wave
constexpr int kWElems = kStageK * kColsT;         // W_Q slice of a stage
constexpr int kWLoads = kWElems * 2 / 1024;       // 32
constexpr int kWPerWave = kWLoads / kWaves;       // 4
constexpr int kWChunks = kColsT / 8;              // 32 chunks per W_Q tile row
static_assert(kWLoads % kWaves == 0, "loads split evenly");

// Row tile of NRB 16-row blocks per wave: 128 rows (NRB = 2, three stages in
// LDS) or, for grids of more than two rounds of workgroups, 256 rows (NRB = 4,
// two stages: each W_Q fragment read from LDS then feeds twice the MFMAs).
template <int NRB>
struct QTile {
  static constexpr int kNRB = NRB;                          // 16-row blocks per wave
  static constexpr int kRowsW = 16 * NRB;                   // query rows per wave
  static constexpr int kRowsT = 4 * kRowsW;                 // query rows per workgroup
  static constexpr int kXElems = kRowsT * kStageK;          // x slice of a stage
  static constexpr int kXLoads = kXElems * 2 / 1024;        // wave-wide 1 KB loads
  static constexpr int kStageElems = kXElems + kWElems;
  static constexpr int kStages = NRB == 2 ? 3 : 2;
  static constexpr int kXPerWave = kXLoads / kWaves;
  static constexpr int kL = kXPerWave + kWPerWave;          // loads per wave per stage
  static_assert(kXLoads % kWaves == 0, "loads split evenly");
  static_assert(kStages * kStageElems * 2 <= 160 * 1024, "LDS budget");
};

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// chunk permutation mask of W_Q tile row k (an involution on the chunks of a row)
__device__ __forceinline__ int swz_q(int k) { return 2 * ((k & 3) | (((k >> 3) & 1) << 2)); }

template <typename T, int DC, int DN, int NRB>
__global__ __launch_bounds__(kThreads)
void qprologue_kernel(QArgs a) {
  using QT = QTile<NRB>;
  constexpr int kNRB = QT::kNRB, kRowsW = QT::kRowsW, kRowsT = QT::kRowsT;
  constexpr int kXElems = QT::kXElems, kStageElems = QT::kStageElems, kStages = QT::kStages;
  constexpr int kXPerWave = QT::kXPerWave, kL = QT::kL;
  constexpr int kDC = DC;                   // content width (192 by default; 64, 128 in the sweep)
  constexpr int kDNope = DN;                // NoPE width of a head (96 by default)
  constexpr int kRow = DC + kDHead - DN;    // Qhat row: [q_lat (DC) | q_rope (128 - DN)]
  constexpr int kQnLd = kDNope + 8;         // q_nope staging row (bf16)
  static_assert(DN % 16 == 0 && DN > 0 && DN < kDHead, "NoPE width");
  static_assert(kWaves * kRowsW * kQnLd <= kStages * kStageElems, "epilogue staging fits");
  __shared__ __attribute__((aligned(16))) bf16_t smem[kStages * kStageElems];

  // Workgroups are dispatched round-robin over the 8 XCDs; id = 8 (HP q + hp) + x8
  // keeps every head pair of row tile 8 q + x8 on XCD x8, so that tile's x rows
  // are fetched into that XCD's L2 once and shared by its head pairs.
  const int64_t M = (int64_t)a.batch * a.n_q;
  const int n_rt = (int)((M + kRowsT - 1) / kRowsT);
  const int n_hp = (a.n_heads + kHeadsT - 1) / kHeadsT;
  const int x8 = blockIdx.x & 7;
  const int rest = blockIdx.x >> 3;
  const int hp = rest % n_hp;
  const int rt = 8 * (rest / n_hp) + x8;
  if (rt >= n_rt) return;                   // whole workgroup: no barrier is skipped

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int g = lane >> 4;
  const int j = lane & 15;
  const int rh = wv >> 1, hh = wv & 1;      // wave-uniform
  const int64_t m0 = (int64_t)rt * kRowsT;
  const int rows = (int)min<int64_t>(kRowsT, M - m0);
  const int wq_ld = a.n_heads * kDHead;
  const int col0 = kColsT * hp;             // first W_Q column of the pair
  const T* xw = static_cast<const T*>(a.x) + m0 * a.d_model;
  const T* wq = static_cast<const T*>(a.w_q) + col0;
  const int nst = a.d_model / kStageK;

  // Load offsets (bytes; bf16 sources). x load n = 2 wv + i moves rows
  // 8n .. 8n+7 of the tile (clamped to the last row); W load n = 4 wv + i moves
  // rows 2n, 2n+1 of the W_Q slice. A head pair with one head (odd head count)
  // reads the existing head's columns in place of the missing one.
  uint32_t voff[kL];
  if constexpr (std::is_same_v<T, bf16_t>) {
#pragma unroll
    for (int i = 0; i < kXPerWave; ++i) voff[i] = stage_a_voff(a.d_model, 0, rows, kXPerWave * wv + i, lane);
#pragma unroll
    for (int i = 0; i < kWPerWave; ++i) {
      const int q = 64 * (kWPerWave * wv + i) + lane, k = q / kWChunks, cp = q - k * kWChunks;
      int c = cp ^ swz_q(k);
      if (col0 + 8 * c >= wq_ld) c -= kDHead / 8;
      voff[kXPerWave + i] = (uint32_t)(k * wq_ld + 8 * c) * 2u;
    }
  }
  auto issue = [&](int sb, int sd, int i0, int i1) {   // loads i0 <= i < i1: data of stage sd, buffer of sb
    bf16_t* st = smem + (sb % kStages) * kStageElems;
    const int k0 = sd * kStageK;
#pragma unroll
    for (int i = 0; i < kL; ++i) {
      if (i < i0 || i >= i1) continue;
      if (i < kXPerWave) {
        const int n = kXPerWave * wv + i;
        if constexpr (std::is_same_v<T, bf16_t>) dma16_lds(xw + k0, voff[i], lds_u32(st + 512 * n));
        else stage_a_load<T>(st, xw, a.d_model, 0, rows, k0, n, lane);
      } else {
        const int n = kWPerWave * wv + (i - kXPerWave);
        bf16_t* dst = st + kXElems + 512 * n;
        if constexpr (std::is_same_v<T, bf16_t>) {
          dma16_lds(wq + (size_t)k0 * wq_ld, voff[i], lds_u32(dst));
        } else {
          const int q = 64 * n + lane, k = q / kWChunks, cp = q - k * kWChunks;
          int c = cp ^ swz_q(k);
          if (col0 + 8 * c >= wq_ld) c -= kDHead / 8;
          *reinterpret_cast<uint4*>(dst + 8 * lane) = load8_bf16<T>(wq + (size_t)(k0 + k) * wq_ld + 8 * c);
        }
      }
    }
  };

  // Operand offsets (elements, relative to a stage's tiles).
  // x (B operand): lane (j, g) of block rb = row 32 rh + 16 rb + j, chunk 4 kk + g.
  int a_off[kNRB][2];
#pragma unroll
  for (int rb = 0; rb < kNRB; ++rb) {
    const int row = kRowsW * rh + 16 * rb + j;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) a_off[rb][kk] = 64 * row + 8 * ((4 * kk + g) ^ swz_a(row));
  }
  // W_Q (A operand) by ds_read_b64_tr_b16: lane j of group g points at row
  // 32 kk + 8 g + j/4 (+4 for the upper half) and columns col + 4 (j%4) .. +3
  // of column block cb of head hh. The swizzle bits of that row (bits 0, 1, 3)
  // depend on the lane only.
  int b_off[kCB];
  {
    const int k = 8 * g + (j >> 2);
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb) {
      const int c = 2 * (kCB * hh + cb) + ((j & 3) >> 1);
      b_off[cb] = k * kColsT + 8 * (c ^ swz_q(k)) + 4 * (j & 1);
    }
  }

  for (int s = 0; s < kStages - 1 && s < nst; ++s) issue(s, s, 0, kL);

  f32x4 acc[kNRB][kCB];
#pragma unroll
  for (int rb = 0; rb < kNRB; ++rb)
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb) acc[rb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Stage s: two 32-deep steps of 2 x 8 MFMAs; the next x fragment and the W
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
        if constexpr (kStages == 2) {       // one stage ahead: all loads at its start
          if (q == 0) issue(s + kStages - 1, sn, 0, kL);
        } else {
          issue(s + kStages - 1, sn, q * kL / (2 * kNRB), (q + 1) * kL / (2 * kNRB));
        }
#pragma unroll
        for (int cb = 0; cb < kCB; ++cb)
          acc[rb][cb] = mfma16(kk == 0 ? b0[cb] : b1[cb], av, acc[rb][cb]);
        av = an;
      }
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");    // the trailing loads have landed
  __syncthreads();                                     // the stage buffers are free

  // ---- epilogue. Register r of acc[rb][cb] in lane (j, g): row 32 rh + 16 rb + j
  // of the tile, column 16 cb + 4 g + r of head h.
  const int h = kHeadsT * hp + hh;
  if (h >= a.n_heads) return;                         // no barrier follows
  // W_K_up[h] fragments of the absorption, A operand: lane (j, g) of column
  // tile ct holds row 16 ct + j, n = 32 ks + 8 g .. +7. The first kWkD tiles
  // are requested now and land during the RoPE and q_nope work; each register
  // set is refilled with tile ct + kWkD once tile ct has been consumed.
  constexpr int kCT = kDC / 16;                        // 12 column tiles of q_lat
  constexpr int kKS = (kDNope + 31) / 32;              // 3 steps (DN = 112: 4, the last half empty)
  constexpr int kWkD = kCT / 2 < 6 ? kCT / 2 : (kKS > 3 ? 4 : 6);   // tiles in flight
  // lanes whose n = 32 ks + 8 g .. +7 lies past the NoPE width (DN % 32 = 16,
  // last step) contribute zeros on both operands
  auto n_live = [&](int ks) { return kDNope % 32 == 0 || 32 * ks + 8 * g < kDNope; };
  const T* wku = static_cast<const T*>(a.w_k_up) + (size_t)h * kDC * kDNope;
  auto load_wk = [&](int ct, bf16x8 (&w)[kKS]) {
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks)
      w[ks] = n_live(ks) ? __builtin_bit_cast(bf16x8, load8_bf16<T>(wku + (size_t)(16 * ct + j) * kDNope + 32 * ks + 8 * g))
                         : bf16x8{};
  };
  bf16x8 wk[kWkD][kKS];
#pragma unroll
  for (int c = 0; c < kWkD; ++c) load_wk(c, wk[c]);
  int64_t qrow[kNRB];                                  // Qhat row index, -1 past the last row
  int pos[kNRB][3];                                    // (t, h, w) of each row
#pragma unroll
  for (int rb = 0; rb < kNRB; ++rb) {
    const int64_t m = m0 + kRowsW * rh + 16 * rb + j;
    const int64_t mc = m < M ? m : M - 1;
    const int b = (int)(mc / a.n_q);
    const int n = (int)(mc - (int64_t)b * a.n_q);
    int n_in, ww;
    const int f = div_small(n, a.tokens_per_frame, a.inv_tokens_per_frame, &n_in);
    const int hpos = div_small(n_in, a.grid_w, a.inv_grid_w, &ww);
    pos[rb][0] = a.t_first + f;
    pos[rb][1] = hpos;
    pos[rb][2] = ww;
    qrow[rb] = m < M ? ((int64_t)b * a.n_heads + h) * a.n_q + n : -1;
  }
  uint16_t* qhat = a.qhat;
  // RoPE: columns DN + 16 (cb - DN/16) + 4 g + r, pairs 8 (cb - DN/16) + 2 g + {0, 1}
#pragma unroll
  for (int cb = kDNope / 16; cb < kCB; ++cb) {
#pragma unroll
    for (int rb = 0; rb < kNRB; ++rb) {
      const f32x4 v = acc[rb][cb];
      float o[4];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        uint32_t lo, hi;
        int ax;
        rope_rate_by_group(a.rope, 8 * (cb - kDNope / 16) + q, g, &lo, &hi, &ax);   // pair 8 (cb - DN/16) + 2 g + q
        float sn, cs;
        sincos_rev(pos[rb][ax], lo, hi, &sn, &cs);
        o[2 * q] = v[2 * q] * cs - v[2 * q + 1] * sn;
        o[2 * q + 1] = v[2 * q] * sn + v[2 * q + 1] * cs;
      }
      if (qrow[rb] >= 0) {
        const int col = kDC + 16 * (cb - kDNope / 16) + 4 * g;
        *reinterpret_cast<uint2*>(qhat + qrow[rb] * kRow + col) =
            uint2{pack2(o[0] * a.qscale, o[1] * a.qscale), pack2(o[2] * a.qscale, o[3] * a.qscale)};
      }
    }
  }
  // q_nope of this wave's kRowsW rows to LDS: qn[row][0..DN-1] (bf16)
  bf16_t* qn = smem + wv * kRowsW * kQnLd;
#pragma unroll
  for (int rb = 0; rb < kNRB; ++rb)
#pragma unroll
    for (int cb = 0; cb < kDNope / 16; ++cb) {
      const f32x4 v = acc[rb][cb];
      *reinterpret_cast<uint2*>(&qn[(16 * rb + j) * kQnLd + 16 * cb + 4 * g]) =
          uint2{pack2(v[0], v[1]), pack2(v[2], v[3])};
    }
  // q_lat^T[c][row] = sum_n W_K_up[h][c][n] q_nope[row][n]: A = W_K_up rows,
  // B = q_nope rows from LDS (lane (j, g): row 16 rb + j, n = 32 ks + 8 g .. +7).
  bf16x8 qb[kNRB][kKS];
#pragma unroll
  for (int rb = 0; rb < kNRB; ++rb)
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks)
      qb[rb][ks] = n_live(ks) ? lds_row8(&qn[(16 * rb + j) * kQnLd + 32 * ks + 8 * g]) : bf16x8{};
#pragma unroll
  for (int ct = 0; ct < kCT; ++ct) {
    bf16x8 (&w)[kKS] = wk[ct % kWkD];
#pragma unroll
    for (int rb = 0; rb < kNRB; ++rb) {
      f32x4 ql = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < kKS; ++ks) ql = mfma16(w[ks], qb[rb][ks], ql);
      // register r: c = 16 ct + 4 g + r of row 16 rb + j
      if (qrow[rb] >= 0)
        *reinterpret_cast<uint2*>(qhat + qrow[rb] * kRow + 16 * ct + 4 * g) =
            uint2{pack2(ql[0] * a.qscale, ql[1] * a.qscale), pack2(ql[2] * a.qscale, ql[3] * a.qscale)};
    }
    if (ct + kWkD < kCT) load_wk(ct + kWkD, w);
  }
}

template <int DC, int DN, int NRB>
void launch_t(const QArgs& a, bool f32, dim3 grid, hipStream_t s) {
  if (f32) hipLaunchKernelGGL((qprologue_kernel<float, DC, DN, NRB>), grid, dim3(kThreads), 0, s, a);
  else hipLaunchKernelGGL((qprologue_kernel<bf16_t, DC, DN, NRB>), grid, dim3(kThreads), 0, s, a);
}

template <int NRB>
hipError_t launch_nrb(const QArgs& a, bool f32, hipStream_t s) {
  const int64_t M = (int64_t)a.batch * a.n_q;
  const int64_t n_rt = (M + QTile<NRB>::kRowsT - 1) / QTile<NRB>::kRowsT;
  const int n_hp = (a.n_heads + kHeadsT - 1) / kHeadsT;
  const dim3 grid((unsigned)(8 * n_hp * ((n_rt + 7) / 8)));
  if (a.d_rope != kDRope) {                 // split variants: d_c = kDC
    switch (a.d_rope) {
      case 16: launch_t<kDC, 112, NRB>(a, f32, grid, s); break;
      case 64: launch_t<kDC, 64, NRB>(a, f32, grid, s); break;
      case 96: launch_t<kDC, 32, NRB>(a, f32, grid, s); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  switch (a.d_c) {
    case 64: launch_t<64, kDNope, NRB>(a, f32, grid, s); break;
    case 128: launch_t<128, kDNope, NRB>(a, f32, grid, s); break;
    case 256:
    case 512:                                 // wide latents: bf16 storage only
      if (f32) return hipErrorInvalidValue;
      if (a.d_c == 256) hipLaunchKernelGGL((qprologue_kernel<bf16_t, 256, kDNope, NRB>), grid, dim3(kThreads), 0, s, a);
      else hipLaunchKernelGGL((qprologue_kernel<bf16_t, 512, kDNope, NRB>), grid, dim3(kThreads), 0, s, a);
      break;
    default: launch_t<kDC, kDNope, NRB>(a, f32, grid, s); break;
  }
  return hipGetLastError();
}

}  // namespace

// 256-row tiles (bf16 sources) once the 128-row grid would take more than two
// rounds of the device's compute units (batch 8 of the 4680-token chunk: 12%
// faster; batch 1 keeps 222 workgroups of 128 rows on 256 CUs).
hipError_t launch_qprologue(const QArgs& a, bool f32, hipStream_t s) {
  if (!f32) {
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    const int64_t M = (int64_t)a.batch * a.n_q;
    const int64_t n_hp = (a.n_heads + kHeadsT - 1) / kHeadsT;
    if ((M + QTile<2>::kRowsT - 1) / QTile<2>::kRowsT * n_hp > 2 * (int64_t)cus) return launch_nrb<4>(a, f32, s);
  }
  return launch_nrb<2>(a, f32, s);
}

}  // namespace vmla
