// Explicit-reconstruction chunk attention for gfx950: the comparison point of
// the latent form.
//
// VideoMLA (paperlayer.ai summary of arXiv:2605.30351v1), §3 "On-demand
// reconstruction": per-head keys k_h = [c W_K_up[h] | k_R] and values
// v_h = c W_V_up[h] are rebuilt from the cached latents and attention runs as
// ordinary 128-dimensional multi-head attention; App. E notes that inference
// can instead stay in latent form. This kernel runs the ordinary attention
// over the rebuilt per-head rows [k_h (128) | v_h (128)] (built by the
// reconstruction GEMM): 2 * 128 + 2 * 128 = 512 flops per (query, key, head)
// against the latent form's 832, at the price of writing and reading the
// rebuilt rows (H * 512 bytes per key instead of 448).
//
// The schedule is that of the latent kernel: 8 waves, each with 32 queries of
// one head (all 8 units of a workgroup belong to the same head, since the
// rebuilt rows are per head); tiles of 64 keys x 256 values copied by LDS-DMA
// into 4 chunk-major buffers two tiles ahead; ping-pong of matrix phases
// (S^T = K Q^T: 16 MFMAs; O^T += V^T P^T: 16 MFMAs, V^T by transposed LDS
// reads) and vector phases (online softmax with lazy rescaling) between the
// wave halves of each SIMD.
#include "device_common.h"
#include "kernels.h"

namespace vmla {
namespace {

constexpr int kKT = 64;                     // keys per tile
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kD = kDHead;                  // 128: score width and value width
constexpr int kKVRow = 2 * kD;              // rebuilt row [k (128) | v (128)]
constexpr int kChunks = kKVRow / 8;         // 32 chunks of 16 bytes
constexpr int kSlots = kKT + 4;             // slots per chunk column (padded)
constexpr int kTileElems = kChunks * kSlots * 8;
constexpr int kLoaders = kWaves / 2;
constexpr int kLoadsPerWave = kChunks / kLoaders;   // 8
constexpr int kBufs = 4;
constexpr int kFeatSteps = kD / 16;         // 8
constexpr int kValTiles = kD / 32;          // 4
constexpr float kLazy = 8.f;
static_assert(kBufs * kTileElems * 2 <= 160 * 1024, "LDS budget");

constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;

__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(voff), "s"(base), "s"(__builtin_amdgcn_readfirstlane(lds_addr)) : "memory");
}

template <typename T> __device__ __forceinline__ void store4(T* p, float a, float b, float c, float d);
template <> __device__ __forceinline__ void store4<bf16_t>(bf16_t* p, float a, float b, float c, float d) {
  *reinterpret_cast<uint2*>(p) = uint2{pack2(a, b), pack2(c, d)};
}
template <> __device__ __forceinline__ void store4<float>(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<float4*>(p) = float4{a, b, c, d};
}

template <typename T>
__global__ __launch_bounds__(kThreads)
void explicit_attn_kernel(ExplicitArgs a) {
  __shared__ __attribute__((aligned(16))) bf16_t kt[kBufs * kTileElems];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int qi = lane & 31;
  const int lag = wave >= kLoaders ? 1 : 0;
  // Query chunk: blockIdx.z = (n_chunks - 1 - c) * batch + b (most keys first).
  const int rc = blockIdx.z / a.batch;
  const int b = blockIdx.z - rc * a.batch;
  const int c = a.cm.n_chunks - 1 - rc;
  const int q0 = c * a.cm.chunk_q;
  const int nq = min(a.cm.chunk_q, a.n_q - q0);
  const int k_end = min(a.n_k, (c + 1) * a.cm.key_step);
  const int k0 = max(0, k_end - a.cm.key_span);
  const int nk = k_end - k0;
  // Workgroup g of head h = blockIdx.x / G takes units 8 g .. 8 g + 7 of that
  // head's chunk (G = ceil(units / 8) workgroups per head for the longest chunk).
  const int units = (nq + 31) / 32;
  const int groups = ((a.cm.chunk_q + 31) / 32 + kWaves - 1) / kWaves;
  const int h = blockIdx.x / groups;
  const int qb = (blockIdx.x - h * groups) * kWaves + wave;
  const int qrow = 32 * qb + qi;
  const bool live = qb < units;
  const bool qvalid = live && qrow < nq;

  bf16x8 qf[kFeatSteps];
  {
    const bf16_t* qp = a.q + (((size_t)b * a.n_heads + h) * a.n_q + q0 + (qvalid ? qrow : nq - 1)) * kD;
#pragma unroll
    for (int ks = 0; ks < kFeatSteps; ++ks)
      qf[ks] = *reinterpret_cast<const bf16x8*>(qp + ks * 16 + 8 * half);
#pragma unroll
    for (int ks = 0; ks < kFeatSteps; ++ks) asm volatile("" : "+v"(qf[ks]));
  }

  const bf16_t* kv = a.kv + (((size_t)b * a.n_heads + h) * (size_t)a.n_k + k0) * kKVRow;
  const int ntiles = (nk + kKT - 1) / kKT;

  // Tile staging (X waves): load n moves chunk column n, lane r = key 64 j + r.
  const uint32_t kt_lds = (uint32_t)(uintptr_t)(VMLA_LDS bf16_t*)kt;
  auto issue_tile = [&](int j) {
    const int buf = j % kBufs;
    const int kg = min(j * kKT + lane, nk - 1);
    const int wv = __builtin_amdgcn_readfirstlane(wave);
#pragma unroll
    for (int i = 0; i < kLoadsPerWave; ++i) {
      const int n = wv + kLoaders * i;
      dma16(kv, (uint32_t)(kg * (kKVRow * 2)) + (uint32_t)(16 * n),
            kt_lds + 2u * (uint32_t)(buf * kTileElems + n * kSlots * 8));
    }
  };

  const int a_base = (half * kSlots + qi) * 8;
  const int jl = lane & 15;
  const int x4 = ((lane & 16) >> 3) + ((jl & 3) >> 1);
  const int sub = 4 * (jl & 1);
  const int v_off1 = ((kD / 8 + x4) * kSlots + 4 * half + (jl >> 2)) * 8 + sub;   // value chunks 16..31
  const int v_off2 = v_off1 + 8 * 8;

  f32x16 o[kValTiles];
#pragma unroll
  for (int t = 0; t < kValTiles; ++t) o[t] = f32x16{};
  float m = -INFINITY;
  float l = 0.f;
  f32x16 s0, s1;
  bf16x8 pb[2][2];

  // O^T += V^T(tile) P^T: 16 MFMAs, 32 transpose reads issued ahead.
  auto accumulate = [&](const bf16_t* K) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const bf16_t* Kb = K + (kb * 32 + jj * 16) * 8;
#pragma unroll
        for (int t = 0; t < kValTiles; ++t) {
          const bf16x4 lo = lds_tr4(Kb + v_off1 + 4 * kSlots * 8 * t);
          const bf16x4 hi = lds_tr4(Kb + v_off2 + 4 * kSlots * 8 * t);
          const bf16x8 av = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          o[t] = mfma32(av, pb[kb][jj], o[t]);
        }
      }
    }
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 4, 0);
#pragma unroll
    for (int i = 0; i < 14; ++i) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2, 0);
  };
  // S^T of one tile: 16 MFMAs, 16 row reads issued ahead.
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
    for (int i = 0; i < 6; ++i) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2, 1);
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 1);
    }
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 4, 1);
  };
  auto softmax = [&](int key0) {
    if (key0 + kKT > nk) {
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
    const bool grow = mx > m + kLazy;
    if (__builtin_amdgcn_ballot_w64(grow)) {
      const float m_new = grow ? mx : m;
      const float alpha = __builtin_amdgcn_exp2f(m - m_new);
      l *= alpha;
#pragma unroll
      for (int t = 0; t < kValTiles; ++t) o[t] *= alpha;
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
  }
  __syncthreads();

  const int nphases = 2 * ntiles + 2;
  for (int p = 0; p < nphases; ++p) {
    const int q = p - lag;
    if (q >= 0) {
      const int jt = q >> 1;
      if ((q & 1) == 0) {
        __builtin_amdgcn_s_setprio(1);
        if (live) {
          if (jt >= 1) accumulate(kt + ((jt - 1) % kBufs) * kTileElems);
          if (jt < ntiles) scores(kt + (jt % kBufs) * kTileElems);
        }
        __builtin_amdgcn_s_setprio(0);
      } else if (jt < ntiles) {
        if (!lag) {
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
          if (jt + 2 < ntiles) issue_tile(jt + 2);
        }
        if (live) softmax(jt * kKT);
      }
    }
    __syncthreads();
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // out[b][n][h][d] = O^T[d][n] / l; register 4 g + e of value tile t holds
  // dim 32 t + 8 g + 4 half + e.
  if (!qvalid) return;
  const float inv = 1.f / sum_across_halves(l);
  T* out = static_cast<T*>(a.out) + (((size_t)b * a.n_q + q0 + qrow) * a.n_heads + h) * kD;
#pragma unroll
  for (int t = 0; t < kValTiles; ++t)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      store4<T>(out + 32 * t + 8 * g + 4 * half, o[t][4 * g] * inv, o[t][4 * g + 1] * inv,
                o[t][4 * g + 2] * inv, o[t][4 * g + 3] * inv);
}

// W_KV[c][h (d_nope + d_v) + j] = W_K_up[h][c][j] (j < d_nope), W_V_up[h][c][j - d_nope]
// (W_K_up[h] is [kDC][d_nope])
template <typename T>
__global__ __launch_bounds__(256)
void pack_kv_kernel(FoldArgs a) {
  const int dn = a.d_nope;                  // NoPE width of a head's key
  const int kCols = dn + kDV;
  const int64_t total = (int64_t)kDC * a.n_heads * kCols;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int c = (int)(i / (a.n_heads * kCols));
  const int col = (int)(i - (int64_t)c * a.n_heads * kCols);
  const int h = col / kCols, j = col - h * kCols;
  const T* src = j < dn ? static_cast<const T*>(a.w_first) + ((size_t)h * kDC + c) * dn + j
                        : static_cast<const T*>(a.w_second) + ((size_t)h * kDC + c) * kDV + (j - dn);
  static_cast<T*>(a.out)[i] = *src;
}

}  // namespace

hipError_t launch_explicit_attn(const ExplicitArgs& a, bool f32, hipStream_t s) {
  const int units = (a.cm.chunk_q + 31) / 32;
  const int groups = (units + kWaves - 1) / kWaves;
  const dim3 grid((unsigned)(a.n_heads * groups), 1, (unsigned)(a.batch * a.cm.n_chunks));
  if (f32) hipLaunchKernelGGL(explicit_attn_kernel<float>, grid, dim3(kThreads), 0, s, a);
  else hipLaunchKernelGGL(explicit_attn_kernel<bf16_t>, grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_pack_kv(const FoldArgs& a, bool f32, hipStream_t s) {
  const int64_t total = (int64_t)kDC * a.n_heads * (a.d_nope + kDV);
  const dim3 grid((unsigned)((total + 255) / 256));
  if (f32) hipLaunchKernelGGL(pack_kv_kernel<float>, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(pack_kv_kernel<bf16_t>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace vmla
